// odd_shapes.hpp -- shapes of the odd-row kernels (odd.hpp), as
// X(T, 2, LPR, VPL, TEAMS) lists ordered by capacity LPR * VPL * 2, the
// elements of a row's pairs (N - 1).  Steps of a third to a half: a row
// just past one capacity leaves at most a third of the lanes of the next
// idle (16384 x 6001 bf16 on 512 lanes holding 8 pairs each, 73% of them
// busy: 250 us against 230 us on the single-element kernels).
#pragma once

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
