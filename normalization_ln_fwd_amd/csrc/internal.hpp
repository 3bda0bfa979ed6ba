// internal.hpp -- host/device interface between the C-ABI layer (api.cpp)
// and the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf {

// Arguments of one forward call (pointers are device memory; optional ones
// may be null).
// Rows are visited in row groups of `teams` rows; a workgroup takes K row
// groups, interleaved over blocks of A workgroups (see GroupWalk).
struct FwdArgs {
    const void *x, *bias, *res, *gamma, *beta;
    void *y, *res_out;       // y: I/O dtype, or FP8 E4M3 codes (uint8) when y_scale is set
    const float *y_scale;    // FP8 output: one fp32 scale in device memory
    float *mean, *rstd;
    unsigned *amax; // bit pattern of a non-negative float, combined with atomicMax
    // optional: zero before the launch, left zero after it; the cells that
    // combine the workgroups' maxima (amax_arrive)
    unsigned *amax_ws;
    int64_t M;
    int64_t n_groups;
    int N;
    int K, A;
    int64_t wt_group; // row groups from this one on store write-through
    float eps;
    bool zero_centred; // weight = round_T(1 + gamma)
};

// Arguments of one backward stage-1 call.  `ws` holds the per-workgroup
// column partials: dgamma partials [grid][N], then dbeta partials [grid][N].
struct BwdArgs {
    const void *dy, *x, *gamma;
    const float *mean, *rstd; // rstd null (RMSNorm only): recompute from x
    void *dx;
    float *ws;
    int64_t M;
    int64_t n_groups;
    int N;
    int K, A;
    int64_t wt_group; // row groups from this one on store write-through
    float eps;
    bool zero_centred; // weight = round_T(1 + gamma)
    // rows split along N (bwd_split_kernel): `chunks` column chunks per row;
    // rowsums holds the two row sums of every (row, chunk), [M][chunks][2]
    float *rowsums;
    int chunks;
};

typedef hipError_t (*FwdLaunch)(const FwdArgs &, int grid, hipStream_t);
typedef hipError_t (*BwdLaunch)(const BwdArgs &, int grid, hipStream_t);

// One row-kernel shape: a team of `lpr` lanes owns a row; each lane holds
// `vpl` vectors of `vec` elements; a workgroup holds `teams` teams.
// `capacity` = lpr * vpl * vec is the longest row the shape covers.
struct RowShape {
    int lpr, vpl, teams, vec;
    int capacity() const { return lpr * vpl * vec; }
    int threads() const { return lpr * teams; }
};

struct FwdEntry {
    RowShape shape;
    FwdLaunch ln, rms;       // y in the I/O dtype
    FwdLaunch ln_f8, rms_f8; // y as FP8 E4M3 codes
};
struct BwdEntry {
    RowShape shape;
    BwdLaunch ln, rms;       // dgamma, dbeta partials
    BwdLaunch ln_db, rms_db; // also the dbias partials
};

// Arguments of one row-softmax call.
struct SoftmaxArgs {
    const void *x;
    void *y;
    int64_t M;
    int64_t n_groups;
    int N;
    int K, A;
    int64_t wt_group; // row groups from this one on store write-through
};
typedef hipError_t (*SoftmaxLaunch)(const SoftmaxArgs &, int grid, hipStream_t);
struct SoftmaxEntry {
    RowShape shape;
    SoftmaxLaunch run;
};
const SoftmaxEntry *softmax_table_f32(int vec, int *count);
const SoftmaxEntry *softmax_table_bf16(int vec, int *count);

// Tables of instantiated shapes, ordered by capacity, for elements per
// vector access `vec`: 16 / sizeof(T) (16-byte accesses), 4 (bf16, 8-byte),
// 2 (4-byte bf16 pairs, 8-byte fp32 pairs) or 1; an empty table (count 0)
// for other values.  One translation unit per dtype/direction.
const FwdEntry *fwd_table_f32(int vec, int *count);
const FwdEntry *fwd_table_bf16(int vec, int *count);
const BwdEntry *bwd_table_f32(int vec, int *count);
const BwdEntry *bwd_table_bf16(int vec, int *count);

// Kernels for rows whose length is an odd multiple of a unit of U elements
// (U = 1: odd N; 2: N = 2 mod 4; 4: bf16 N = 4 mod 8) and whose [M, N]
// tensors are aligned to 2U elements (odd.hpp): each row read in aligned
// vectors of 2U from its first such element, plus one unit by itself; shape
// capacity = the vectors' elements, N - U.  One table per dtype and unit.
const FwdEntry *fwd_odd_table_bf16_u1(int *count);
const FwdEntry *fwd_odd_table_bf16_u2(int *count);
const FwdEntry *fwd_odd_table_bf16_u4(int *count);
const FwdEntry *fwd_odd_table_f32_u1(int *count);
const FwdEntry *fwd_odd_table_f32_u2(int *count);
const BwdEntry *bwd_odd_table_bf16_u1(int *count);
const BwdEntry *bwd_odd_table_bf16_u2(int *count);
const BwdEntry *bwd_odd_table_bf16_u4(int *count);
const BwdEntry *bwd_odd_table_f32_u1(int *count);
const BwdEntry *bwd_odd_table_f32_u2(int *count);
const SoftmaxEntry *softmax_odd_table_bf16_u1(int *count);
const SoftmaxEntry *softmax_odd_table_bf16_u2(int *count);
const SoftmaxEntry *softmax_odd_table_bf16_u4(int *count);
const SoftmaxEntry *softmax_odd_table_f32_u1(int *count);
const SoftmaxEntry *softmax_odd_table_f32_u2(int *count);

template <class E, size_t n>
const E *table_of(const E (&t)[n], int *count)
{
    *count = int(n);
    return t;
}

// Teams of at least WIDE_LPR lanes (several waves per row) hold few rows per
// CU: their kernels prefetch the next row group, and the host gives their
// workgroups more row groups to walk.
constexpr int WIDE_LPR = 128;

// Small kernels.
hipError_t launch_zero_u32(unsigned *p, hipStream_t s);
// Column sums of the stage-1 partials (nb blocks -- dgamma, dbeta and, when
// nb = 3, dbias -- of `parts` rows of colsum_ld(N) floats at ws); writes the outputs
// given (each optional), divided by `divisor`, in fp32 (out_dtype 0) or
// bf16 (1).  parts = 0 writes zeros.  Up to COLSUM_ONE_LAUNCH parts are
// summed in one launch; more in two: colsum_slices(parts) sums of
// COLSUM_SPAN rows each go to `level2` (nb blocks of that many rows of
// colsum_ld(N) floats), then a final launch adds them.  The short slices give the first
// launch enough workgroups to spread evenly over the CUs.
// Row stride, in floats, of the partial rows in the workspace: N rounded up
// to a multiple of 4, so that the column sums read 16-byte vectors.
__host__ __device__ inline int64_t colsum_ld(int64_t N) { return (N + 3) & ~int64_t(3); }
constexpr int COLSUM_ONE_LAUNCH = 512;
constexpr int COLSUM_SPAN = 128;
inline int colsum_slices(int64_t parts)
{
    return parts <= COLSUM_ONE_LAUNCH ? 1 : int((parts + COLSUM_SPAN - 1) / COLSUM_SPAN);
}
// Backward with the rows split along N (few rows of many columns): the
// columns of one chunk, and the launch of both passes over a grid of
// (chunks, row blocks) workgroups.
int split_chunk_cols(int32_t dtype);
constexpr int SPLIT_ROWS_PER_GROUP = 4; // one row per wave, four waves
hipError_t launch_bwd_split(const BwdArgs &a, int32_t dtype, bool rms, bool dbias, int blocks,
                            hipStream_t s);

hipError_t launch_colsum(const float *ws, int parts, int nb, int N, void *dgamma, void *dbeta,
                         void *dbias, int out_dtype, float divisor, float *level2, hipStream_t s);

} // namespace nf
