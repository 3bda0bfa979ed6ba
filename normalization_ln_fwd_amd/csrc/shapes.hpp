// shapes.hpp -- the row-kernel shapes instantiated for each dtype, as
// X(T, VEC, LPR, VPL, TEAMS) lists ordered by row capacity LPR * VPL * VEC.
// The host picks the first shape whose capacity covers N.
//
// 16-byte path (VEC = 16 / sizeof(T)); narrow rows in workgroups of 256
// threads (the forward adds 512-thread variants), wide rows in teams of
// 320 to 1024 threads (softmax has tables of its own, in softmax.hip):
//   bf16 capacities: 64 128 256 384 512 768 1024 1536 2048 2560 3072 4096
//                    (backward: 5120 6144) 8192 10240 12288 16384; the forward
//                    adds 2560 on one wave per row
//   fp32 capacities: 32 64 128 192 256 384 512 768 1024 1280 1536 2048 4096
//                    (forward: 5120 6144) 8192 16384
// Rows that are not whole 16-byte vectors, or pointers that are not 16-byte
// aligned, take the widest of 8-byte vectors (bf16, N % 4 == 0, the fp32
// layouts), 4-byte vectors of 2 elements (N even) or single elements that
// N and the alignment allow.  Element-wise capacities: 256 512 1024 2048
// 4096 5120 6144 8192 16384.  (Steps of 2x capacity and 8 elements per lane beyond 1024 columns:
// with steps of 4x and 16 per lane, 32768 x 1500 bf16 took 205 / 254 us
// forward / backward, now 117 / 164 us.)
#pragma once

// Teams of at most one wave per row (bf16 rows <= 2048, fp32 <= 1024).
#define NF_SHAPES_NARROW(X, T, VEC)                                                              \
    X(T, VEC, 8, 1, 32)                                                                          \
    X(T, VEC, 16, 1, 16)                                                                         \
    X(T, VEC, 16, 2, 16)                                                                         \
    X(T, VEC, 16, 3, 16)                                                                         \
    X(T, VEC, 16, 4, 16)                                                                         \
    X(T, VEC, 32, 3, 8)                                                                          \
    X(T, VEC, 32, 4, 8)                                                                          \
    X(T, VEC, 64, 3, 4)                                                                          \
    X(T, VEC, 64, 4, 4)

// Wide rows, several waves per row: teams of 320, 384 or 512 lanes holding
// one vector each, two rows per workgroup, up to twice the narrow capacity;
// beyond that one team of 512 lanes per workgroup, holding 2 or 4 vectors
// per lane.  (Rows of 2304-3072 bf16 columns on teams of 320 or 384 lanes
// instead of 512 with idle lanes, measured on MI355X at 32768 rows: forward
// 61-73% -> 70-75% of peak, backward 56-71% -> 68-79%.)  (Teams of 256 lanes
// holding 4 vectors, measured on MI355X for the 8192-column bf16 rows: the
// backward at 32768 x 8192 took 299 us against 252 us, the forward at
// 8192 x 8192 90 us against 87 us; their 212 registers leave 2 waves per
// SIMD.)
#define NF_SHAPES_WIDE_ONE_VEC(X, T, VEC)                                                        \
    X(T, VEC, 320, 1, 2)                                                                         \
    X(T, VEC, 384, 1, 2)                                                                         \
    X(T, VEC, 512, 1, 2)
#define NF_SHAPES_WIDE_MULTI_VEC(X, T, VEC)                                                      \
    X(T, VEC, 512, 2, 1)                                                                         \
    X(T, VEC, 512, 4, 1)
#define NF_SHAPES_WIDE(X, T, VEC) NF_SHAPES_WIDE_ONE_VEC(X, T, VEC) NF_SHAPES_WIDE_MULTI_VEC(X, T, VEC)
// Teams of 640 and 768 lanes holding two vectors each, between 512 lanes
// holding two and 512 holding four (up to half of whose lanes would idle).
// Measured on MI355X, 512 x 4 against these (us): bf16 forward 8192 x 9216
// 123.9 -> 114.4, 8192 x 10240 130.8 -> 121.2, 32768 x 12288 569.9 ->
// 546.0; bf16 backward 8192 x 9216 103.9 -> 81.2, 8192 x 10240 104.2 ->
// 85.2, 32768 x 12288 420.8 -> 392.9; fp32 forward 32768 x 5120 466.5 ->
// 456.8, 32768 x 6144 559.1 -> 540.8, 10922 x 6144 184.1 -> 178.0.  (The
// fp32 backward went either way, by up to 15%, and keeps 512 x 4; teams of
// 1024 lanes holding two lost to 512 holding four at 16384 columns.)
#define NF_SHAPES_WIDE_TWO_VEC_FINE(X, T, VEC)                                                   \
    X(T, VEC, 512, 2, 1)                                                                         \
    X(T, VEC, 640, 2, 1)                                                                         \
    X(T, VEC, 768, 2, 1)                                                                         \
    X(T, VEC, 512, 4, 1)
// The forward's 16-byte tables (fp32 adds 1024 x 4 for 16384 columns).
#define NF_SHAPES_FWD_VEC(X, T, VEC)                                                             \
    NF_SHAPES_NARROW(X, T, VEC)                                                                  \
    NF_SHAPES_WIDE_ONE_VEC(X, T, VEC)                                                            \
    NF_SHAPES_WIDE_TWO_VEC_FINE(X, T, VEC)
// bf16 adds one wave per row holding five vectors for 2049-2560 columns,
// taken where it leaves at least 2048 row groups (the host's fwd_entry):
// measured on MI355X against 320 lanes x 1 (us), 16384 x 2560 57.9 ->
// 53.2, 65536 x 2304 212.0 -> 194.6, 8192 x 2560 28.9 -> 27.8; with fewer
// rows its 256-thread workgroups hold too few waves (4096 x 2560: 18.3
// against 16.2).
#define NF_SHAPES_FWD_BF16_VEC(X)                                                                \
    NF_SHAPES_NARROW(X, bf16, 8)                                                                 \
    X(bf16, 8, 64, 5, 4)                                                                         \
    NF_SHAPES_WIDE_ONE_VEC(X, bf16, 8)                                                           \
    NF_SHAPES_WIDE_TWO_VEC_FINE(X, bf16, 8)

// The bf16 backward also runs rows of 4097-6144 columns on teams that leave
// fewer lanes idle than 512 lanes holding two vectors: two teams of 320
// lanes holding two each up to 5120 columns, one team of 768 lanes holding
// one up to 6144.  Measured on MI355X against 512 x 2: 32768 x 5120 219 ->
// 158 us, 32768 x 6144 230 -> 193 us, 8192 x 5120 62 -> 45 us; 320 x 2 x 2
// against 640 lanes holding one: 32768 x 5120 176 -> 158 us, 16384 x 4608
// 92.5 -> 77.0 us (at 6144 columns 384 x 2 x 2 and 768 x 1 were within 2%
// either way).  The forward gains nothing from 640 or 768 lanes holding
// one vector (-7% to +2%), nor does either direction in fp32.
#define NF_SHAPES_BF16_BWD_VEC(X)                                                                \
    NF_SHAPES_NARROW(X, bf16, 8)                                                                 \
    NF_SHAPES_WIDE_ONE_VEC(X, bf16, 8)                                                           \
    X(bf16, 8, 320, 2, 2)                                                                        \
    X(bf16, 8, 768, 1, 1)                                                                        \
    NF_SHAPES_WIDE_TWO_VEC_FINE(X, bf16, 8)
#define NF_SHAPES_F32_VEC(X)                                                                     \
    NF_SHAPES_NARROW(X, float, 4) NF_SHAPES_WIDE(X, float, 4) X(float, 4, 1024, 4, 1)

// Forward only: the same team shapes in 512-thread workgroups (twice the
// rows per workgroup), preferred when there are rows enough to fill the GPU.
#define NF_SHAPES_NARROW_2X(X, T, VEC)                                                             \
    X(T, VEC, 8, 1, 64)                                                                          \
    X(T, VEC, 16, 1, 32)                                                                         \
    X(T, VEC, 16, 2, 32)                                                                         \
    X(T, VEC, 16, 3, 32)                                                                         \
    X(T, VEC, 16, 4, 32)                                                                         \
    X(T, VEC, 32, 3, 16)                                                                         \
    X(T, VEC, 32, 4, 16)                                                                         \
    X(T, VEC, 64, 3, 8)                                                                          \
    X(T, VEC, 64, 4, 8)

#define NF_SHAPES_ELEM(X, T)                                                                     \
    NF_SHAPES_SHORT_VEC_FINE(X, T, 1)                                                            \
    X(T, 1, 1024, 16, 1)
// Element-wise-like layouts for 4-byte vectors of 2 elements (bf16 rows of
// an even N, fp32 rows of an even N on 8-byte alignment): capacities 512 to
// 16384.
#define NF_SHAPES_SHORT_VEC(X, T, VEC)                                                            \
    X(T, VEC, 64, 4, 4)                                                                          \
    X(T, VEC, 64, 8, 4)                                                                          \
    X(T, VEC, 64, 16, 4)                                                                         \
    X(T, VEC, 256, 8, 1)                                                                         \
    X(T, VEC, 512, 8, 1)                                                                         \
    X(T, VEC, 1024, 8, 1)
// The same with teams of 640 and 768 lanes between 512 and 1024, for the
// single-element path and bf16 pairs: rows just past a power of two no
// longer leave up to half of the lanes idle.  Measured on MI355X (forward /
// backward): 16384 x 4097 bf16 252 / 166 -> 204 / 142 us, 16384 x 6001 bf16
// 270 / 186 -> 229 / 174 us, 8192 x 9002 bf16 160 / 120 -> 137 / 112 us,
// 16384 x 4097 fp32 272 / 185 -> 233 / 179 us.  (fp32 pairs are left out:
// their forward with the next group's loads in flight spilled on these
// teams.)
#define NF_SHAPES_SHORT_VEC_FINE(X, T, VEC)                                                       \
    X(T, VEC, 64, 4, 4)                                                                          \
    X(T, VEC, 64, 8, 4)                                                                          \
    X(T, VEC, 64, 16, 4)                                                                         \
    X(T, VEC, 256, 8, 1)                                                                         \
    X(T, VEC, 512, 8, 1)                                                                         \
    X(T, VEC, 640, 8, 1)                                                                         \
    X(T, VEC, 768, 8, 1)                                                                         \
    X(T, VEC, 1024, 8, 1)
// bf16 rows of a multiple of 4 elements on 8-byte alignment: the fp32
// layouts (4 elements per vector).
#define NF_SHAPES_BF16_VEC4(X)                                                                   \
    NF_SHAPES_NARROW(X, bf16, 4) NF_SHAPES_WIDE(X, bf16, 4) X(bf16, 4, 1024, 4, 1)
// Forward and backward on 8-byte bf16 vectors also run rows of 4097-6144
// columns on one team of 640 or 768 lanes holding two vectors each, instead
// of 512 lanes holding four with up to half of them idle (as the 16-byte
// backward does with one vector per lane).  Measured on MI355X at
// 16384 x 4100: forward 135.5 -> 121.5 us, backward 151.3 -> 123.0 us.
#define NF_SHAPES_BF16_VEC4_FINE(X)                                                               \
    NF_SHAPES_NARROW(X, bf16, 4)                                                                 \
    NF_SHAPES_WIDE_ONE_VEC(X, bf16, 4)                                                           \
    X(bf16, 4, 512, 2, 1)                                                                        \
    X(bf16, 4, 640, 2, 1)                                                                        \
    X(bf16, 4, 768, 2, 1)                                                                        \
    X(bf16, 4, 512, 4, 1)                                                                        \
    X(bf16, 4, 1024, 4, 1)
