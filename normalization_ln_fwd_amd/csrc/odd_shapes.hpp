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
