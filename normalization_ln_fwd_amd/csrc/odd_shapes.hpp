// odd_shapes.hpp -- shapes of the kernels for rows of an odd multiple of a
// unit of U elements (odd.hpp), as X(T, 2U, LPR, VPL, TEAMS) lists ordered
// by capacity LPR * VPL * 2U, the elements of a row's vectors (N - U).
// Unit 1 (odd N) below, in steps of a third to a half: a row just past one
// capacity leaves at most a third of the lanes of the next idle (16384 x
// 6001 bf16 on 512 lanes holding 8 pairs each, 73% of them busy: 250 us
// against 230 us on the single-element kernels).  Units 2 and 4 take the
// vector layouts of shapes.hpp for their vector width, the backward's with
// an even number of teams.
#pragma once

#include "shapes.hpp"

#define NF_SHAPES_ODD(X, T)                                                                      \
    X(T, 2, 16, 4, 16)                                                                           \
    X(T, 2, 32, 4, 8)                                                                            \
    X(T, 2, 64, 3, 4)                                                                            \
    X(T, 2, 64, 4, 4)                                                                            \
    X(T, 2, 64, 6, 4)                                                                            \
    X(T, 2, 64, 8, 4)                                                                            \
    X(T, 2, 64, 12, 4)                                                                           \
    X(T, 2, 64, 16, 4)                                                                           \
    X(T, 2, 192, 8, 1)                                                                           \
    X(T, 2, 256, 8, 1)                                                                           \
    X(T, 2, 320, 8, 1)                                                                           \
    X(T, 2, 384, 8, 1)                                                                           \
    X(T, 2, 512, 8, 1)
// The bf16 forward's: the wide teams two to a workgroup (they share the
// staged per-column vectors and hold twice the waves).  Measured on MI355X
// against one team per workgroup (us): 32760 x 4097 263.7 -> 224.2, 26209 x
// 5121 331.1 -> 265.3, 21841 x 6145 302.5 -> 256.3, 16382 x 8193 266.2 ->
// 234.5, 8192 x 4097 84.9 -> 68.6.  (Teams of twice the lanes holding four
// pairs instead were slower: 16382 x 8193 on 1024 lanes, 296.2 us.)
#define NF_SHAPES_ODD_FWD_BF16(X)                                                                \
    X(bf16, 2, 16, 4, 16)                                                                        \
    X(bf16, 2, 32, 4, 8)                                                                         \
    X(bf16, 2, 64, 3, 4)                                                                         \
    X(bf16, 2, 64, 4, 4)                                                                         \
    X(bf16, 2, 64, 6, 4)                                                                         \
    X(bf16, 2, 64, 8, 4)                                                                         \
    X(bf16, 2, 64, 12, 4)                                                                        \
    X(bf16, 2, 64, 16, 4)                                                                        \
    X(bf16, 2, 192, 8, 2)                                                                        \
    X(bf16, 2, 256, 8, 2)                                                                        \
    X(bf16, 2, 320, 8, 2)                                                                        \
    X(bf16, 2, 384, 8, 2)                                                                        \
    X(bf16, 2, 512, 8, 2)
// The bf16 softmax's likewise, but for the 320-lane teams (measured (us),
// one team / two: 43676 x 3073 106.7 / 92.0, 32760 x 4097 101.4 / 89.9,
// 16382 x 8193 104.9 / 98.0; 26209 x 5121 105.3 / 110.1).
#define NF_SHAPES_ODD_SOFTMAX_BF16(X)                                                            \
    X(bf16, 2, 16, 4, 16)                                                                        \
    X(bf16, 2, 32, 4, 8)                                                                         \
    X(bf16, 2, 64, 3, 4)                                                                         \
    X(bf16, 2, 64, 4, 4)                                                                         \
    X(bf16, 2, 64, 6, 4)                                                                         \
    X(bf16, 2, 64, 8, 4)                                                                         \
    X(bf16, 2, 64, 12, 4)                                                                        \
    X(bf16, 2, 64, 16, 4)                                                                        \
    X(bf16, 2, 192, 8, 2)                                                                        \
    X(bf16, 2, 256, 8, 2)                                                                        \
    X(bf16, 2, 320, 8, 1)                                                                        \
    X(bf16, 2, 384, 8, 2)                                                                        \
    X(bf16, 2, 512, 8, 2)
// Up to 16385 columns (the forward's per-column vectors take 6 bytes per
// column of LDS for bf16; fp32's 12 would not fit past 8193 columns beside
// the rows in flight).
#define NF_SHAPES_ODD_WIDE(X, T)                                                                 \
    X(T, 2, 640, 8, 1)                                                                           \
    X(T, 2, 768, 8, 1)                                                                           \
    X(T, 2, 1024, 8, 1)

// The backward's: an even number of teams per workgroup (each team keeps
// one row parity), teams of whole waves, up to 8193 columns in workgroups
// of at most 1024 threads.  Beyond 8 pairs per lane, two teams of 128
// lanes instead of four of 64: 16 pairs per lane took 256 registers with
// dbias (one wave per SIMD).
#define NF_SHAPES_ODD_BWD(X, T)                                                                  \
    X(T, 2, 64, 1, 4)                                                                            \
    X(T, 2, 64, 2, 4)                                                                            \
    X(T, 2, 64, 3, 4)                                                                            \
    X(T, 2, 64, 4, 4)                                                                            \
    X(T, 2, 64, 6, 4)                                                                            \
    X(T, 2, 64, 8, 4)                                                                            \
    X(T, 2, 128, 6, 2)                                                                           \
    X(T, 2, 128, 8, 2)                                                                           \
    X(T, 2, 192, 8, 2)                                                                           \
    X(T, 2, 256, 8, 2)                                                                           \
    X(T, 2, 320, 8, 2)                                                                           \
    X(T, 2, 384, 8, 2)                                                                           \
    X(T, 2, 512, 8, 2)

// Units 2 and 4 with 16-byte vectors (bf16 unit 4, fp32 unit 2): the
// narrow layouts of shapes.hpp, wide teams holding one vector per lane,
// then one team of 512, 640 or 768 lanes holding 2 or 4 vectors (bf16 rows
// of unit 2 have tables of their own, below).  Measured on MI355X (bf16, us):
// one vector per lane on 640 or 768 lanes is slower than two on 512
// (8192 x 5124 forward 78 against 67, 8192 x 6004 softmax 43 against 35),
// and so are 1024 lanes holding 4 (8192 x 9002 forward 163 against 139 on
// 640 lanes).  The softmax, with no parameters to stage, prefers 4 vectors
// on 512 lanes to 2 on 768 (8192 x 6002: 36 against 43 us).
// bf16 rows of unit 4 take one wave per row holding five vectors up to
// 2564 columns instead of 320 lanes holding one (58153 x 2308 forward
// 225.1 -> 193.8 us, 52347 x 2564 215.6 -> 198.5 us).
#define NF_SHAPES_ODD_U4_BF16(X)                                                                 \
    NF_SHAPES_NARROW(X, bf16, 8)                                                                 \
    X(bf16, 8, 64, 5, 4)                                                                         \
    X(bf16, 8, 384, 1, 2)                                                                        \
    X(bf16, 8, 512, 1, 2)                                                                        \
    X(bf16, 8, 512, 2, 1)                                                                        \
    X(bf16, 8, 640, 2, 1)                                                                        \
    X(bf16, 8, 768, 2, 1)                                                                        \
    X(bf16, 8, 512, 4, 1)
#define NF_SHAPES_ODD_U2_FWD(X, T)                                                               \
    NF_SHAPES_NARROW(X, T, 4)                                                                    \
    NF_SHAPES_WIDE_ONE_VEC(X, T, 4)                                                              \
    X(T, 4, 512, 2, 1)                                                                           \
    X(T, 4, 640, 2, 1)                                                                           \
    X(T, 4, 768, 2, 1)                                                                           \
    X(T, 4, 512, 4, 1)
// Softmax of unit 4: one wave per row holding five, six or eight vectors
// up to 4100 columns.  Teams of 320-512 lanes holding one measured slower
// than the vector kernel, these faster (us, vector or 512 lanes / these):
// 58153 x 2308 119.2 / 90.1, 43633 x 3076 97.2 / 91.6, 32736 x 4100 100.7
// / 90.7, 8192 x 2564 20.5 / 15.8.
#define NF_SHAPES_ODD_U4_BF16_SOFTMAX(X)                                                         \
    NF_SHAPES_NARROW(X, bf16, 8)                                                                 \
    X(bf16, 8, 64, 5, 4)                                                                         \
    X(bf16, 8, 64, 6, 4)                                                                         \
    X(bf16, 8, 64, 8, 4)                                                                         \
    X(bf16, 8, 512, 2, 1)                                                                        \
    X(bf16, 8, 640, 2, 1)                                                                        \
    X(bf16, 8, 768, 2, 1)                                                                        \
    X(bf16, 8, 512, 4, 1)
#define NF_SHAPES_ODD_U2_SOFTMAX(X, T)                                                           \
    NF_SHAPES_NARROW(X, T, 4)                                                                    \
    NF_SHAPES_WIDE_ONE_VEC(X, T, 4)                                                              \
    X(T, 4, 512, 2, 1)                                                                           \
    X(T, 4, 512, 4, 1)
// bf16 rows of unit 2 (8-byte vectors): one wave per row holding six or
// eight vectors, then teams of 128 lanes holding six or eight, where the
// teams above hold 8 or 16 bytes per lane.  Measured on MI355X (us, those
// teams / these): 65472 x 2050 forward 291.7 / 204.4, softmax 139.1 /
// 95.0, backward 230.6 / 152.9; 87267 x 1538 forward 238.7 / 209.2,
// softmax 162.1 / 91.0, backward (on the 4-byte vector kernel) 162.9 /
// 144.4; 8192 x 3074 forward 59.5 / 51.7.  The backward takes two teams of
// 256 lanes holding four past 2050 columns (32752 x 4098: 179.8 -> 154.0
// us against two teams of 512 holding two; teams of 128 lanes lost there:
// 65472 x 2050 213 us), softmax 512 lanes holding two at 4096 (32752 x
// 4098: 91.9 against 94.9 us).
#define NF_SHAPES_ODD_U2_BF16_FWD(X)                                                             \
    NF_SHAPES_NARROW(X, bf16, 4)                                                                 \
    X(bf16, 4, 64, 6, 4)                                                                         \
    X(bf16, 4, 64, 8, 4)                                                                         \
    X(bf16, 4, 128, 6, 2)                                                                        \
    X(bf16, 4, 128, 8, 2)                                                                        \
    X(bf16, 4, 640, 2, 1)                                                                        \
    X(bf16, 4, 768, 2, 1)                                                                        \
    X(bf16, 4, 512, 4, 1)
#define NF_SHAPES_ODD_U2_BF16_SOFTMAX(X)                                                         \
    NF_SHAPES_NARROW(X, bf16, 4)                                                                 \
    X(bf16, 4, 64, 6, 4)                                                                         \
    X(bf16, 4, 64, 8, 4)                                                                         \
    X(bf16, 4, 128, 6, 2)                                                                        \
    X(bf16, 4, 512, 2, 1)                                                                        \
    X(bf16, 4, 512, 4, 1)
#define NF_SHAPES_ODD_U2_BF16_BWD(X)                                                             \
    NF_SHAPES_NARROW(X, bf16, 4)                                                                 \
    X(bf16, 4, 64, 6, 4)                                                                         \
    X(bf16, 4, 64, 8, 4)                                                                         \
    X(bf16, 4, 256, 4, 2)                                                                        \
    X(bf16, 4, 512, 4, 2)
// fp32 rows of unit 2 (16-byte vectors), backward: past 2050 columns two
// teams of 256 lanes holding four or eight vectors (the vector kernel, on
// 8-byte vectors, took the rows past 4098).  Measured on MI355X (us):
// 8190 x 8194 196.3 -> 156.6 (vector kernel before), 16376 x 4098 149.4
// -> 145.1 (two teams of 512 lanes holding two before), 10919 x 6146
// 159.0 -> 155.2.  512 lanes holding four spilled registers with dbias.
#define NF_SHAPES_ODD_U2_F32_BWD(X)                                                              \
    NF_SHAPES_NARROW(X, float, 4)                                                                \
    X(float, 4, 512, 1, 2)                                                                       \
    X(float, 4, 256, 4, 2)                                                                       \
    X(float, 4, 256, 8, 2)
// beyond 8192 columns (bf16 forward, softmax of either dtype)
#define NF_SHAPES_ODD_U2_WIDE(X, T)                                                              \
    X(T, 4, 640, 4, 1)                                                                           \
    X(T, 4, 768, 4, 1)                                                                           \
    X(T, 4, 1024, 4, 1)
// The bf16 backward of unit 4: the narrow layouts, then two teams of 512
// lanes per workgroup (each team keeps one row parity) holding 1 or 2
// vectors; narrower wide teams measured slower than the vector kernel.
#define NF_SHAPES_ODD_U4_BF16_BWD(X)                                                             \
    NF_SHAPES_NARROW(X, bf16, 8)                                                                 \
    X(bf16, 8, 512, 1, 2)                                                                        \
    X(bf16, 8, 512, 2, 2)

// Table entries (FwdEntry / BwdEntry / SoftmaxEntry) of one shape: the unit
// is half the vector width VEC.
#define NF_FWD_ODD(T, VEC, LPR, VPL, TEAMS)                                                        \
    {{LPR, VPL, TEAMS, VEC},                                                                     \
     &launch_fwd_odd<T, VEC / 2, LPR, VPL, TEAMS, false, false>,                                  \
     &launch_fwd_odd<T, VEC / 2, LPR, VPL, TEAMS, true, false>,                                   \
     &launch_fwd_odd<T, VEC / 2, LPR, VPL, TEAMS, false, true>,                                   \
     &launch_fwd_odd<T, VEC / 2, LPR, VPL, TEAMS, true, true>},
#define NF_BWD_ODD(T, VEC, LPR, VPL, TEAMS)                                                        \
    {{LPR, VPL, TEAMS, VEC},                                                                     \
     &launch_bwd_odd<T, VEC / 2, LPR, VPL, TEAMS, false, false>,                                  \
     &launch_bwd_odd<T, VEC / 2, LPR, VPL, TEAMS, true, false>,                                   \
     &launch_bwd_odd<T, VEC / 2, LPR, VPL, TEAMS, false, true>,                                   \
     &launch_bwd_odd<T, VEC / 2, LPR, VPL, TEAMS, true, true>},
#define NF_SOFTMAX_ODD(T, VEC, LPR, VPL, TEAMS)                                                    \
    {{LPR, VPL, TEAMS, VEC}, &launch_softmax_odd<T, VEC / 2, LPR, VPL, TEAMS>},
