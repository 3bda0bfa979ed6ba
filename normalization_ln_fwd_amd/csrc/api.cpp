// api.cpp -- the C ABI declared in include/normfuse.h: argument checks,
// choice of kernel shape, row-group walk sizing and launches on the
// caller's stream.  Nothing here allocates device memory.
#include "normfuse.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <mutex>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "internal.hpp"

// ------------------------------------------- the library's static scratch
// The workspace of ln_bwd_noalloc, for callers that cannot allocate: one
// array per device in the code object's device memory, held until the
// process ends.  Host code never passes `scratch` itself to a kernel (in
// host code the name is a stand-in, not a device address): each device's
// address is taken once, with that device current, by hipGetSymbolAddress
// (static_scratch below), and kept.
static __device__ __align__(256) unsigned char scratch[NORM_STATIC_SCRATCH_BYTES];

namespace {

using namespace nf;

// ---------------------------------------------------------------- device
norm_status_t check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return NORM_ERR_DEVICE;
    return NORM_OK;
}

// ------------------------------------------------ tuning overrides (test build)
// The product library takes every choice below from the call's arguments
// alone.  A separate build of this file with NORMFUSE_TUNING defined
// (libnormfuse_tuning.so, same kernels) also reads these environment
// variables on every call, so that tests can force shapes, walks and the
// split along N and cross-check them against each other, and measurements
// can sweep them:
// NORMFUSE_{FWD,BWD}_SHAPE          : "LPRxVPL" or "LPRxVPLxTEAMS" -- use that
//                                     instantiated shape when it covers the row
//                                     (the FWD one for softmax too)
// NORMFUSE_{FWD,BWD}_GROUPS_PER_WG  : row groups per workgroup (K)
// NORMFUSE_{FWD,BWD}_INTERLEAVE     : workgroups per interleave block (A)
// NORMFUSE_WT_BYTES                 : output bytes, counted from the end,
//                                     stored write-through (see wt_group);
//                                     NORMFUSE_{FWD,BWD}_WT_BYTES for one
//                                     direction (the forward's also applies
//                                     to softmax)
// NORMFUSE_BWD_SPLIT                : 0 never splits backward rows along N,
//                                     1 splits them wherever the kernel can
//                                     (see bwd_plan)
// NORMFUSE_PAIRS                    : 0 turns the odd-row kernels off (rows
//                                     of an odd number of units then take
//                                     the narrower vectors N allows)
constexpr int kFwdGroupsPerWg = 0; // 0: chosen per call (see fwd_common)
constexpr int kBwdGroupsPerWg = 0; // 0: chosen per shape (see bwd_plan)
// Row groups per workgroup.  Teams of several waves (wide rows) have few
// rows in flight per CU; walking several groups per workgroup, with the next
// group's loads in flight, keeps the loads going.  The backward's count also
// sets how many rows one column partial covers, i.e. how finely the column
// reduction is split over the rows (see bwd_groups_per_wg).
constexpr int kFwdGroupsWide = 4;
constexpr int64_t kBwdFewGroups = 64;
// Compute units of the gfx950 parts.  A constant rather than a device query,
// so that the grid (and with it every summation order, and the workspace
// size) follows from the call's arguments alone.
constexpr int64_t kCUs = 256;
constexpr int kFwdInterleave = 1024;
constexpr int kBwdInterleave = 256;
// Output bytes, counted from the end of a call, that its kernel stores
// write-through (device.hpp, BUF_WT).  Measured on MI355X: the gain grows
// with the tail up to about 224 MiB (backward) / 256 MiB (forward) at
// 576000 x 384 -- 5% on both -- and beyond that, near the 256 MiB of the
// last-level cache, the stream turns slower than with no tail at all; short
// calls (8192 x 4096) store write-through throughout and gain 7% (forward)
// and 4% (backward).
constexpr double kWtBytes = 96.0 * 1024 * 1024;

struct Knobs {
    int fwd_lpr = 0, fwd_vpl = 0, bwd_lpr = 0, bwd_vpl = 0, fwd_teams = 0, bwd_teams = 0;
    int fwd_k = kFwdGroupsPerWg, bwd_k = kBwdGroupsPerWg;
    int fwd_a = kFwdInterleave, bwd_a = kBwdInterleave;
    double fwd_wt_bytes = kWtBytes, bwd_wt_bytes = kWtBytes;
    int bwd_split = -1; // -1: chosen per shape
    bool pairs = true;  // rows of an odd multiple of a unit on the odd-row kernels
};

#ifdef NORMFUSE_TUNING
// "LPRxVPL" or "LPRxVPLxTEAMS"
void parse_shape(const char *s, int *lpr, int *vpl, int *teams)
{
    if (!s)
        return;
    const int n = std::sscanf(s, "%dx%dx%d", lpr, vpl, teams);
    if (n < 2) {
        *lpr = 0;
        *vpl = 0;
    }
    if (n < 3)
        *teams = 0;
}

void parse_positive(const char *s, int *out)
{
    if (s) {
        const int v = std::atoi(s);
        if (v > 0)
            *out = v;
    }
}

Knobs knobs()
{
    Knobs r;
    parse_shape(std::getenv("NORMFUSE_FWD_SHAPE"), &r.fwd_lpr, &r.fwd_vpl, &r.fwd_teams);
    parse_shape(std::getenv("NORMFUSE_BWD_SHAPE"), &r.bwd_lpr, &r.bwd_vpl, &r.bwd_teams);
    parse_positive(std::getenv("NORMFUSE_FWD_GROUPS_PER_WG"), &r.fwd_k);
    if (r.fwd_k <= 0)
        r.fwd_k = 0;
    parse_positive(std::getenv("NORMFUSE_BWD_GROUPS_PER_WG"), &r.bwd_k);
    parse_positive(std::getenv("NORMFUSE_FWD_INTERLEAVE"), &r.fwd_a);
    parse_positive(std::getenv("NORMFUSE_BWD_INTERLEAVE"), &r.bwd_a);
    if (const char *v = std::getenv("NORMFUSE_BWD_SPLIT"))
        r.bwd_split = std::atoi(v) != 0 ? 1 : 0;
    if (const char *v = std::getenv("NORMFUSE_PAIRS"))
        r.pairs = std::atoi(v) != 0;
    auto bytes = [](const char *name, double *out) {
        if (const char *v = std::getenv(name)) {
            const double b = std::atof(v);
            if (b >= 0.0)
                *out = b;
        }
    };
    bytes("NORMFUSE_WT_BYTES", &r.fwd_wt_bytes);
    bytes("NORMFUSE_WT_BYTES", &r.bwd_wt_bytes);
    bytes("NORMFUSE_FWD_WT_BYTES", &r.fwd_wt_bytes);
    bytes("NORMFUSE_BWD_WT_BYTES", &r.bwd_wt_bytes);

    return r;
}
#else
Knobs knobs() { return Knobs(); }
#endif

template <class Entry>
const Entry *pick_shape(const Entry *tab, int n, int N, int force_lpr, int force_vpl,
                        int force_teams)
{
    if (force_lpr > 0) {
        for (int i = 0; i < n; ++i)
            if (tab[i].shape.lpr == force_lpr && tab[i].shape.vpl == force_vpl &&
                (force_teams == 0 || tab[i].shape.teams == force_teams) &&
                tab[i].shape.capacity() >= N)
                return &tab[i];
    }
    for (int i = 0; i < n; ++i)
        if (tab[i].shape.capacity() >= N)
            return &tab[i];
    return nullptr;
}

size_t elem_size(int32_t dtype) { return dtype == NORM_F32 ? 4 : 2; }

// Forward workgroups.  The forward's amax combines one atomicMax per
// workgroup on a single address; such atomics serialise, so the launch is
// kept to at most kMaxAmaxWgs workgroups.  Measured on MI355X, 125000 of
// them (4000000 x 384 bf16) still hide behind the rows: an earlier bound of
// 20000 forced longer walks there and cost 3-5% (4000000 x 384: 2320 ->
// 2253 us; 16000000 x 64: 1527 -> 1447 us).  Bigger workgroups (twice the
// teams) are used when they still leave kMinWideGroups workgroups.
constexpr int64_t kMaxAmaxWgs = 131072;
constexpr int64_t kMinWideGroups = 2048;
// Up to this many row groups the forward walks several groups per workgroup
// (about one workgroup per CU, at most kFwdGroupsWide groups each); beyond
// it, one group per workgroup (many workgroups deep) balances best.
constexpr int64_t kFwdFewGroups = 4096;

// Row groups per forward workgroup.  Measured on MI355X: one workgroup per
// CU walking up to kFwdGroupsWide groups suits wide rows and, up to
// kFwdFewGroups groups, narrow ones too (16384 x 1024: 35 -> 25 us);
// narrow rows in larger numbers run one group per workgroup -- two with an
// FP8 y from kFwdF8PairCols columns on (65536 x 2048: 155 -> 152 us,
// 131072 x 1024: 155 -> 153 us; below, one is faster since the first
// group's loads overlap the parameters' staging: 576000 x 384 258 -> 248
// us, 262144 x 768 233 -> 223 us) -- or as many as make kFwdMinGroupBytes
// of each tensor per workgroup: small groups pay their workgroup's set-up
// (staging the parameters, the final amax) too often (524288 x 256 bf16,
// 16 KiB per group: 225 -> 174 us with two; 4-byte vectors at 65536 x 386,
// 3 KiB: 195 -> 54 us with eight).  With amax, at most kMaxAmaxWgs
// workgroups.  The odd-row kernels (`odd`) run narrow rows one group per
// workgroup at any group size (measured on MI355X, 576000 x 385 bf16 445
// -> 366 us, 262144 x 767 376 -> 331 us, 1048576 x 127 500 -> 386 us),
// and the forward's wide bf16 rows up to kFwdOddGroupsWide groups per
// workgroup, their next group's loads in flight
// (8192 x 16383 301 -> 279 us, 8192 x 8191 138 -> 132 us, 16384 x 6001
// 240 -> 233 us; fp32 rows gained nothing from it).  Beyond kFwdFewGroups
// groups, wide rows on the 16-byte path whose lanes hold one or two vectors
// walk two groups per workgroup.  Measured on MI355X against walks of four
// (us): bf16 43690 x 3072 175.6 -> 170.4, 26214 x 5120 188.4 -> 182.9,
// 21845 x 6144 180.8 -> 173.6, 131072 x 4096 725.7 -> 702.1, 32768 x 8192
// 355.0 -> 350.0; fp32 65536 x 4096 730.6 -> 708.0.  (At 8192 x 4096 bf16,
// 4096 groups, walks of two took 48.7 us against 47.0.)  Lanes holding four
// vectors showed no rule: walks of four, eight or one workgroup per CU each
// won somewhere by up to 8%, so they keep walks of four.
constexpr int64_t kFwdOddGroupsWide = 8;
constexpr int64_t kFwdGroupsWideShort = 2;
constexpr double kFwdMinGroupBytes = 24.0 * 1024;
constexpr int64_t kFwdF8PairCols = 1024;
int fwd_groups_per_wg(int64_t M, int64_t N, int32_t dtype, const RowShape &sh, bool amax, bool f8,
                      bool odd = false, bool softmax = false)
{
    const int64_t groups = (M + sh.teams - 1) / sh.teams;
    const double group_bytes = double(sh.teams) * double(N) * double(elem_size(dtype));
    const int64_t kmin = f8 && N >= kFwdF8PairCols && !odd ? 2 : 1;
    int64_t k = odd ? 1 : std::max<int64_t>(kmin, int64_t(std::ceil(kFwdMinGroupBytes / group_bytes)));
    if (sh.lpr >= WIDE_LPR || groups <= kFwdFewGroups) {
        const bool odd_wide = odd && !softmax && dtype == NORM_BF16 && sh.lpr >= WIDE_LPR;
        int64_t kmax = odd_wide ? kFwdOddGroupsWide : kFwdGroupsWide;
        if (!odd && !softmax && sh.lpr >= WIDE_LPR && sh.vec * elem_size(dtype) == 16 &&
            sh.vpl <= 2 && groups > kFwdFewGroups)
            kmax = kFwdGroupsWideShort;
        k = std::min<int64_t>(kmax, std::max<int64_t>(1, (groups + kCUs - 1) / kCUs));
    }
    if (amax)
        k = std::max(k, (groups + kMaxAmaxWgs - 1) / kMaxAmaxWgs);
    return int(std::max<int64_t>(1, k));
}

const FwdEntry *fwd_entry(int dtype, int vec, int64_t M, int N, const Knobs &k)
{
    int n = 0;
    const FwdEntry *tab = dtype == NORM_F32 ? fwd_table_f32(vec, &n) : fwd_table_bf16(vec, &n);
    const FwdEntry *e = pick_shape(tab, n, N, k.fwd_lpr, k.fwd_vpl, k.fwd_teams);
    if (!e || k.fwd_lpr > 0)
        return e;
    // a narrow 16-byte team holding more than four vectors per lane (one
    // wave per row, five vectors: bf16 rows of 2049-2560 columns) only where
    // it leaves kMinWideGroups row groups; otherwise the next shape that
    // holds the row
    if (e->shape.lpr < WIDE_LPR && e->shape.vpl > 4 && e->shape.vec * elem_size(dtype) == 16 &&
        (M + e->shape.teams - 1) / e->shape.teams < kMinWideGroups) {
        for (const FwdEntry *f = e + 1; f < tab + n; ++f)
            if (f->shape.capacity() >= N && f->shape.lpr >= WIDE_LPR) {
                e = f;
                break;
            }
    }
    for (int i = 0; i < n; ++i) {
        const RowShape &w = tab[i].shape;
        if (w.lpr == e->shape.lpr && w.vpl == e->shape.vpl && w.teams == 2 * e->shape.teams &&
            (M + w.teams - 1) / w.teams >= kMinWideGroups)
            return &tab[i];
    }
    return e;
}

const BwdEntry *bwd_entry(int dtype, int vec, int N, const Knobs &k)
{
    int n = 0;
    const BwdEntry *tab = dtype == NORM_F32 ? bwd_table_f32(vec, &n) : bwd_table_bf16(vec, &n);
    return pick_shape(tab, n, N, k.bwd_lpr, k.bwd_vpl, k.bwd_teams);
}

// Grid of a row-group walk: n_groups groups of `teams` rows, K per workgroup.
struct Walk {
    int64_t n_groups = 0, grid = 0;
    int K = 1, A = 1;
    int unit = 0;      // the odd-row kernel's unit (odd.hpp), 0 for the others
};

norm_status_t plan_walk(int64_t M, int teams, int K, int A, Walk *w)
{
    w->n_groups = (M + teams - 1) / teams;
    w->K = K;
    w->A = A;
    w->grid = (w->n_groups + K - 1) / K;
    if (w->grid > INT32_MAX)
        return NORM_ERR_SHAPE;
    return NORM_OK;
}

// First row group of a walk whose stores are write-through: the groups
// from it on write the last the write-through byte count (or more) of the call's output, given
// `out_bytes` bytes written per element of a row.  Row groups are visited in
// about ascending order (the walk's blocks of workgroups are dispatched in
// order and step through their groups together), so these are the last
// stores of the kernel.
int64_t wt_group(const Walk &w, int teams, int64_t N, double out_bytes, double wt_bytes)
{
    const double per_group = double(teams) * double(N) * out_bytes;
    if (per_group <= 0.0)
        return w.n_groups;
    const double g = std::ceil(wt_bytes / per_group);
    return g >= double(w.n_groups) ? 0 : w.n_groups - int64_t(g);
}

// ------------------------------------------------------------- validation

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool dtype_ok(int32_t d) { return d == NORM_F32 || d == NORM_BF16; }

norm_status_t check_shape(int64_t M, int64_t N)
{
    if (M < 0 || N < 1 || N > NORM_N_MAX)
        return NORM_ERR_SHAPE;
    if (M > INT64_MAX / 8 / N) // byte offsets of [M, N] tensors fit int64
        return NORM_ERR_SHAPE;
    return NORM_OK;
}

bool eps_ok(float eps) { return std::isfinite(eps) && eps >= 0.f; }

// Elements per vector access of a call: the widest access of 16, 8 or 4
// bytes (fp32: 16 or 8) that holds whole elements of every row (N a
// multiple of it) and that every pointer is aligned to; else 1.  `f8_y`: an
// FP8 output of one byte per element, aligned to the element count.
int vec_width(int64_t N, int32_t dtype, std::initializer_list<const void *> ptrs,
              const void *f8_y = nullptr)
{
    const int es = int(elem_size(dtype));
    const int min_bytes = dtype == NORM_F32 ? 8 : 4;
    for (int bytes = 16; bytes >= min_bytes; bytes /= 2) {
        const int v = bytes / es;
        if (N % v != 0)
            continue;
        bool ok = f8_y == nullptr || aligned(f8_y, size_t(v));
        for (const void *p : ptrs)
            ok = ok && (p == nullptr || aligned(p, size_t(bytes)));
        if (ok)
            return v;
    }
    return 1;
}

int full_width(int32_t dtype) { return int(16 / elem_size(dtype)); }

// Rows whose length is an odd multiple of a unit U (a power of two, at most
// half a 16-byte vector: U = 1 for odd N) and whose streamed [M, N] tensors
// are all aligned to 2U elements (an FP8 output to 2U bytes) can be read in
// aligned vectors of 2U elements from each row's first such element (the
// odd-row kernels, odd.hpp); the per-column vectors need only their element
// alignment.  Returns U, or 0 where that does not hold.
int odd_unit(int64_t N, int32_t dtype, std::initializer_list<const void *> ptrs,
             const void *f8_y = nullptr)
{
    const int half = full_width(dtype) / 2;
    int u = 1;
    while (u < half && N % (2 * u) == 0)
        u *= 2;
    if (N % (2 * u) != u)
        return 0; // a multiple of a whole vector: the vector layouts
    const size_t vector_bytes = size_t(2 * u) * elem_size(dtype);
    bool ok = f8_y == nullptr || aligned(f8_y, size_t(2 * u));
    for (const void *p : ptrs)
        ok = ok && (p == nullptr || aligned(p, vector_bytes));
    return ok ? u : 0;
}

// The odd-row kernel tables of a dtype and unit (empty where there are
// none).
const FwdEntry *fwd_odd_table(int32_t dtype, int unit, int *count)
{
    *count = 0;
    if (dtype == NORM_F32)
        return unit == 1 ? fwd_odd_table_f32_u1(count)
                         : unit == 2 ? fwd_odd_table_f32_u2(count) : nullptr;
    return unit == 1   ? fwd_odd_table_bf16_u1(count)
           : unit == 2 ? fwd_odd_table_bf16_u2(count)
           : unit == 4 ? fwd_odd_table_bf16_u4(count)
                       : nullptr;
}
const BwdEntry *bwd_odd_table(int32_t dtype, int unit, int *count)
{
    *count = 0;
    if (dtype == NORM_F32)
        return unit == 1 ? bwd_odd_table_f32_u1(count)
                         : unit == 2 ? bwd_odd_table_f32_u2(count) : nullptr;
    return unit == 1   ? bwd_odd_table_bf16_u1(count)
           : unit == 2 ? bwd_odd_table_bf16_u2(count)
           : unit == 4 ? bwd_odd_table_bf16_u4(count)
                       : nullptr;
}
const SoftmaxEntry *softmax_odd_table(int32_t dtype, int unit, int *count)
{
    *count = 0;
    if (dtype == NORM_F32)
        return unit == 1 ? softmax_odd_table_f32_u1(count)
                         : unit == 2 ? softmax_odd_table_f32_u2(count) : nullptr;
    return unit == 1   ? softmax_odd_table_bf16_u1(count)
           : unit == 2 ? softmax_odd_table_bf16_u2(count)
           : unit == 4 ? softmax_odd_table_bf16_u4(count)
                       : nullptr;
}

// The unit a call takes the odd-row kernels with: theirs when their vectors
// are wider than the vector layout's `vec`, else 0.
int odd_unit_for(int unit, int vec) { return unit > 0 && 2 * unit > vec ? unit : 0; }

norm_status_t launched(hipError_t e) { return e == hipSuccess ? NORM_OK : NORM_ERR_LAUNCH; }

// ------------------------------------------------------------------ forward
// Kernel shape and walk of a forward call (shared by the call and by
// norm_describe, so that a description names what a call launches).
// `unit`: the rows may take the odd-row kernels of that unit (odd_unit_for;
// 0: not), used when one of their shapes holds the row's vectors.
norm_status_t fwd_plan(int64_t M, int64_t N, int32_t dtype, int vec, int unit, bool amax,
                       bool f8, const Knobs &kn, const FwdEntry **entry, Walk *w)
{
    const FwdEntry *e = nullptr;
    unit = kn.pairs ? unit : 0;
    if (unit) {
        int n = 0;
        const FwdEntry *tab = fwd_odd_table(dtype, unit, &n);
        e = pick_shape(tab, n, int(N - unit), kn.fwd_lpr, kn.fwd_vpl, kn.fwd_teams);
        unit = e != nullptr ? unit : 0;
    }
    if (!e)
        e = fwd_entry(dtype, vec, M, int(N), kn);
    if (!e)
        return NORM_ERR_SHAPE;
    const int K =
        kn.fwd_k > 0 ? kn.fwd_k : fwd_groups_per_wg(M, N, dtype, e->shape, amax, f8, unit > 0);
    if (norm_status_t st = plan_walk(M, e->shape.teams, K, kn.fwd_a, w))
        return st;
    w->unit = unit;
    *entry = e;
    return NORM_OK;
}

// y_scale == nullptr: y in the I/O dtype; else y holds FP8 E4M3 codes of
// y * (*y_scale) (one byte per element).
norm_status_t fwd_common(bool rms, const void *x, const void *bias, const void *residual,
                         const void *gamma, const void *beta, float eps, int64_t M, int64_t N,
                         int32_t dtype, const float *y_scale, void *y, void *residual_out,
                         float *mean, float *rstd, float *amax, void *amax_ws, bool f8,
                         uint32_t flags, void *stream)
{
    if (!dtype_ok(dtype))
        return NORM_ERR_DTYPE;
    if (norm_status_t st = check_shape(M, N))
        return st;
    // with no rows there is nothing to read or write
    if (M > 0 && (!x || !y || (f8 && !y_scale)))
        return NORM_ERR_NULL;
    if (!eps_ok(eps) || (rms && mean) || (flags & ~uint32_t(NORM_ZERO_CENTERED_GAMMA)))
        return NORM_ERR_ARG;
    const size_t es = elem_size(dtype);
    for (const void *p : {x, bias, residual, gamma, beta, (const void *)(f8 ? nullptr : y),
                          (const void *)residual_out})
        if (p && !aligned(p, es))
            return NORM_ERR_ALIGN;
    for (const void *p : {(const void *)mean, (const void *)rstd, (const void *)amax,
                          (const void *)y_scale, (const void *)amax_ws})
        if (p && !aligned(p, 4))
            return NORM_ERR_ALIGN;

    if (norm_status_t st = check_device())
        return st;
    const Knobs kn = knobs();
    // FP8 codes of a vector of v elements take v bytes
    const int vec = vec_width(N, dtype, {x, bias, residual, gamma, beta, f8 ? nullptr : y,
                                         residual_out},
                              f8 ? y : nullptr);
    const int unit = odd_unit_for(
        odd_unit(N, dtype, {x, residual, f8 ? nullptr : y, residual_out}, f8 ? y : nullptr), vec);
    const FwdEntry *e = nullptr;
    Walk w;
    if (norm_status_t st = fwd_plan(M, N, dtype, vec, unit, amax != nullptr, f8, kn, &e, &w))
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);

    unsigned *amax_bits = reinterpret_cast<unsigned *>(amax);
    // with a workspace the kernel combines and writes amax itself; without
    // one (or with no rows to launch for) a one-thread kernel zeroes it first
    unsigned *ws = amax_bits && M > 0 ? static_cast<unsigned *>(amax_ws) : nullptr;
    if (amax_bits && !ws)
        if (norm_status_t st = launched(launch_zero_u32(amax_bits, s)))
            return st;
    if (M == 0)
        return NORM_OK;

    FwdArgs a;
    a.x = x;
    a.bias = bias;
    a.res = residual;
    a.gamma = gamma;
    a.beta = beta;
    a.y = y;
    a.y_scale = f8 ? y_scale : nullptr;
    a.res_out = residual_out;
    a.mean = mean;
    a.rstd = rstd;
    a.amax = amax_bits;
    a.amax_ws = ws;
    a.M = M;
    a.n_groups = w.n_groups;
    a.N = int(N);
    a.K = w.K;
    a.A = w.A;
    a.wt_group = wt_group(w, e->shape.teams, N,
                          double(y ? (f8 ? 1 : es) : 0) + double(residual_out ? es : 0), kn.fwd_wt_bytes);
    a.eps = eps;
    a.zero_centred = (flags & NORM_ZERO_CENTERED_GAMMA) != 0;
    const FwdLaunch run = f8 ? (rms ? e->rms_f8 : e->ln_f8) : (rms ? e->rms : e->ln);
    return launched(run(a, int(w.grid), s));
}

// ------------------------------------------------------------------ softmax
norm_status_t softmax_plan(int64_t M, int64_t N, int32_t dtype, int vec, int unit,
                           const Knobs &kn, const SoftmaxEntry **entry, Walk *w)
{
    int n = 0;
    const SoftmaxEntry *e = nullptr;
    if (unit && kn.pairs) {
        const SoftmaxEntry *tab = softmax_odd_table(dtype, unit, &n);
        e = pick_shape(tab, n, int(N - unit), kn.fwd_lpr, kn.fwd_vpl, kn.fwd_teams);
        // As in the backward: on a wide team a row of 2- or 4-element units
        // takes the odd-row softmax only where that leaves fewer lanes idle
        // than the vector kernel (measured on MI355X, bf16, us, odd-row /
        // vector: at the same fill 16384 x 2562 41.7 / 33.1, 16384 x 3074
        // 42.2 / 38.2; with fewer idle lanes 16384 x 4100 51.7 / 55.1,
        // 8192 x 12292 67.9 / 78.2).
        if (e && vec > 1 && e->shape.lpr >= WIDE_LPR && kn.fwd_lpr == 0) {
            int nv = 0;
            const SoftmaxEntry *vt =
                dtype == NORM_F32 ? softmax_table_f32(vec, &nv) : softmax_table_bf16(vec, &nv);
            const SoftmaxEntry *v = pick_shape(vt, nv, int(N), 0, 0, 0);
            if (v && (N - unit) * int64_t(v->shape.capacity()) <= N * int64_t(e->shape.capacity()))
                e = nullptr;
        }
        if (e) {
            // rows of odd N (pairs, eight per lane on the wide teams): one row
            // group per workgroup, many workgroups deep.  Measured on MI355X
            // against walks of four (bf16, us): 32760 x 4097 112.3 -> 101.0,
            // 21841 x 6145 118.6 -> 104.9, 16382 x 8193 113.4 -> 104.9.  (Teams
            // holding one or two 8- or 16-byte vectors walk four.)
            const int K = kn.fwd_k > 0 ? kn.fwd_k
                          : unit == 1  ? 1
                                       : fwd_groups_per_wg(M, N, dtype, e->shape, false, false,
                                                           true, true);
            if (norm_status_t st = plan_walk(M, e->shape.teams, K, kn.fwd_a, w))
                return st;
            w->unit = unit;
            *entry = e;
            return NORM_OK;
        }
    }
    const SoftmaxEntry *tab =
        dtype == NORM_F32 ? softmax_table_f32(vec, &n) : softmax_table_bf16(vec, &n);
    e = pick_shape(tab, n, int(N), kn.fwd_lpr, kn.fwd_vpl, kn.fwd_teams);
    if (!e)
        return NORM_ERR_SHAPE;
    // the 512-thread variant of a narrow shape when rows are plentiful
    for (int i = 0; i < n && kn.fwd_lpr == 0; ++i) {
        const RowShape &ws = tab[i].shape;
        if (ws.lpr == e->shape.lpr && ws.vpl == e->shape.vpl && ws.teams == 2 * e->shape.teams &&
            (M + ws.teams - 1) / ws.teams >= kMinWideGroups) {
            e = &tab[i];
            break;
        }
    }
    const int K = kn.fwd_k > 0 ? kn.fwd_k
                               : fwd_groups_per_wg(M, N, dtype, e->shape, false, false, false, true);
    if (norm_status_t st = plan_walk(M, e->shape.teams, K, kn.fwd_a, w))
        return st;
    *entry = e;
    return NORM_OK;
}

norm_status_t softmax_common(const void *x, int64_t M, int64_t N, int32_t dtype, void *y,
                             uint32_t flags, void *stream)
{
    if (!dtype_ok(dtype))
        return NORM_ERR_DTYPE;
    if (norm_status_t st = check_shape(M, N))
        return st;
    if (M > 0 && (!x || !y))
        return NORM_ERR_NULL;
    if (flags != 0)
        return NORM_ERR_ARG;
    const size_t es = elem_size(dtype);
    for (const void *p : {x, (const void *)y})
        if (p && !aligned(p, es))
            return NORM_ERR_ALIGN;
    if (norm_status_t st = check_device())
        return st;
    if (M == 0)
        return NORM_OK;
    const Knobs kn = knobs();
    const int vec = vec_width(N, dtype, {x, y});
    const int unit = odd_unit_for(odd_unit(N, dtype, {x, y}), vec);
    const SoftmaxEntry *e = nullptr;
    Walk w;
    if (norm_status_t st = softmax_plan(M, N, dtype, vec, unit, kn, &e, &w))
        return st;
    SoftmaxArgs a;
    a.x = x;
    a.y = y;
    a.M = M;
    a.n_groups = w.n_groups;
    a.N = int(N);
    a.K = w.K;
    a.A = w.A;
    a.wt_group = wt_group(w, e->shape.teams, N, double(es), kn.fwd_wt_bytes);
    return launched(e->run(a, int(w.grid), static_cast<hipStream_t>(stream)));
}

// ----------------------------------------------------------------- backward
// Stage-1 walk of the backward for the shape used on these pointers, and
// the workspace it needs: the stage-1 partials (nb blocks of `grid` rows of
// colsum_ld(N) floats: dgamma, dbeta, and dbias when asked for), then for many partial
// rows the second summation level (nb blocks of colsum_slices(grid) rows).
struct BwdLayout {
    size_t level2_off = 0, bytes = 0; // in bytes
    bool two_level = false;
    // rows split along N: `chunks` column chunks, `blocks` row blocks of
    // split_k groups of SPLIT_ROWS_PER_GROUP rows; the row sums follow the
    // column partials at rowsums_off
    bool split = false;
    int chunks = 0, blocks = 0, split_k = 0;
    size_t rowsums_off = 0;
};

// Backward workgroups with the rows split along N, for few rows of many
// columns: about two per CU over the grid of (chunk, row block).  Chosen
// where it measured faster on MI355X (graph replays): bf16 rows of
// kSplitMinChunks chunks or more, kSplitMinGroups row groups or more, and a
// whole-row walk that still leaves CUs idle (64 to 384 rows of 16384
// columns: 6-12% less time).  With fewer chunks or rows, and for fp32
// beyond 128 rows, the third launch costs more than the split gains.
constexpr int64_t kSplitTarget = 2 * kCUs;
constexpr int64_t kSplitMinChunks = 8;
constexpr int64_t kSplitMinGroups = 64;

// Row groups per backward workgroup: the split of the column reduction over
// the rows.  Each workgroup's partial row costs N floats per column sum,
// written and read once more, so fewer, longer walks save traffic, but the
// walks must still spread over the CUs.  Measured on MI355X:
//  - wide rows (teams of 320 to 1024 lanes): as many workgroups as the CUs
//    hold at once -- one per CU, two for the fp32 shapes up to 8192
//    columns, whose registers leave room for a second -- each walking at
//    least 2 rows (below 2 rows the partials outweigh the rows themselves)
//    and as many as it takes, so that no second round of workgroups runs
//    behind the first.  A fixed 32-row walk left most CUs idle at small M
//    (64 x 16384 bf16: 102 us, now 18 us) and cut large M into more
//    partials than needed (32768 x 4096 bf16: 141 us, now 129 us; 8192 x
//    4096 fp32: 92 us, now 68 us); walks capped at 128 rows left a partial
//    second round at larger M (52428 x 2560 bf16: 160 us, now 132 us;
//    43690 x 3072: 170 -> 129 us; 131072 x 4096: 556 -> 527 us; 65536 x
//    8192: 549 -> 515 us).  Up to kBwdFewGroups row groups
//    take one workgroup each: their partials are a few MiB at most, the
//    call is latency-bound, and a second row per workgroup adds its memory
//    round trip (4 x 16384 bf16: 11.7 us with two rows per workgroup, 9.0 us
//    with one);
//  - narrow rows (256-thread workgroups of many rows): two workgroups per
//    CU, each walking its share of the groups, at every M.  Exactly two per
//    CU matters: grids of three or four per CU, of one, or many workgroups
//    deep with short walks are all slower.  Against walks of 3 groups many
//    workgroups deep, bf16: 576000 x 384 222.5 -> 218.6 us (with dbias
//    228.7 -> 220.4 us), 262144 x 768 209 -> 194.5 us, 131072 x 1024 143 ->
//    126 us, 65536 x 2048 154 -> 127 us, 1048576 x 256 270 -> 263 us; fp32
//    576000 x 384 460 -> 447 us, 262144 x 1024 571 -> 536 us.  (4 per CU
//    at 524288 x 384: 210 us, 2 per CU: 196 us, 1 per CU: 276 us.)  Row
//    groups under kBwdSmallGroupBytes per tensor take four workgroups per CU
//    instead: two leave too few bytes in flight (262144 x 128 bf16: 47.6 ->
//    40.7 us; 1048576 x 64: 88 -> 73 us; 4-byte vectors at 65536 x 386:
//    53.8 -> 39.8 us).
constexpr double kBwdSmallGroupBytes = 6.0 * 1024;
int bwd_groups_per_wg(int64_t M, int64_t N, const RowShape &sh, int32_t dtype)
{
    const int64_t groups = (M + sh.teams - 1) / sh.teams;
    if (sh.lpr >= WIDE_LPR) {
        int64_t per_cu = dtype == NORM_F32 && sh.capacity() <= 8192 ? 2 : 1;
        // bf16 rows of 8-byte, 4-byte or single-element accesses (and the
        // odd-row pairs) in workgroups of 256 or 512 threads: 1024 threads per
        // CU.  Measured on MI355X, one per CU left them idle: 32768 x 1499
        // odd-row 147 -> 66 us, single-element 209 -> 84 us; 16384 x 4097
        // odd-row 113 -> 82 us; 16384 x 2047 odd-row 88 -> 51 us; 8-byte
        // vectors 43633 x 3076 187.5 -> 164.9 us, 21831 x 6148 186.8 -> 167.1.
        if (dtype == NORM_BF16 && sh.vec * elem_size(dtype) < 16)
            per_cu = std::max<int64_t>(per_cu, 1024 / sh.threads());
        const int64_t kmin = groups <= kBwdFewGroups ? 1 : (2 + sh.teams - 1) / sh.teams;
        const int64_t slots = kCUs * per_cu;
        return int(std::min<int64_t>(INT32_MAX, std::max(kmin, (groups + slots - 1) / slots)));
    }
    const double group_bytes = double(sh.teams) * double(N) * double(elem_size(dtype));
    const int64_t slots = (group_bytes < kBwdSmallGroupBytes ? 4 : 2) * kCUs;
    return int(std::max<int64_t>(1, (groups + slots - 1) / slots));
}

// `unit`: the rows may take the odd-row kernel of that unit (odd_unit_for;
// 0: not), used when one of its shapes holds the row's vectors.
norm_status_t bwd_plan(int64_t M, int64_t N, int32_t dtype, int vec, int unit, int nb,
                       const Knobs &kn, const BwdEntry **entry, Walk *w, BwdLayout *lay)
{
    const BwdEntry *e = nullptr;
    unit = kn.pairs ? unit : 0;
    if (unit) {
        int n = 0;
        const BwdEntry *tab = bwd_odd_table(dtype, unit, &n);
        e = pick_shape(tab, n, int(N - unit), kn.bwd_lpr, kn.bwd_vpl, kn.bwd_teams);
        // Rows of 2- or 4-element units also fit the vector kernel on 4- or
        // 8-byte vectors.  On a wide team (two rows per workgroup, each across
        // several waves) the odd-row backward takes it only where it leaves
        // fewer lanes idle: at the same fill the vector kernel is 4-10% faster
        // on teams of 320-512 lanes (measured on MI355X, 8192 x 6004 bf16:
        // 70.6 against 63.8 us; 16384 x 3076: 79.3 against 75.2 us), and with
        // fewer idle lanes it is slower (16384 x 4100: 92.1 against 99.6 us,
        // 8192 x 8196: 87.4 against 126.8).  Teams of 256 lanes holding four
        // vectors also win at the same fill once 70% of their lanes are busy
        // (43662 x 3074: 159.6 against 164.4 us, 37428 x 3586: 149.1 against
        // 163.5), not below (52387 x 2562: 180.9 against 172.1 us).
        if (e && vec > 1 && e->shape.lpr >= WIDE_LPR && kn.bwd_lpr == 0) {
            const BwdEntry *v = bwd_entry(dtype, vec, int(N), kn);
            const int64_t busy = N - unit, cap = e->shape.capacity();
            const bool fuller = !v || busy * int64_t(v->shape.capacity()) > N * cap;
            const bool busy_team = e->shape.lpr <= 256 && busy * 10 >= 7 * cap;
            if (!fuller && !busy_team)
                e = nullptr;
        }
        unit = e != nullptr ? unit : 0;
    }
    if (!e)
        e = bwd_entry(dtype, vec, int(N), kn);
    if (!e)
        return NORM_ERR_SHAPE;
    const int K = kn.bwd_k > 0 ? kn.bwd_k : bwd_groups_per_wg(M, N, e->shape, dtype);
    if (norm_status_t st = plan_walk(M, e->shape.teams, K, kn.bwd_a, w))
        return st;
    w->unit = unit;
    *entry = e;
    // Split the rows along N where whole-row workgroups of wide rows leave
    // CUs idle (fewer workgroups than CUs) and a row spans two chunks or more.
    const int chunk = split_chunk_cols(dtype);
    const int64_t chunks = (N + chunk - 1) / chunk;
    lay->split = !unit && vec == full_width(dtype) && M > 0 && e->shape.lpr >= WIDE_LPR && chunks >= 2 &&
                 (kn.bwd_split == 1 ||
                  (kn.bwd_split < 0 && dtype == NORM_BF16 && chunks >= kSplitMinChunks &&
                   w->n_groups >= kSplitMinGroups && w->grid < kCUs));
    int64_t parts = w->grid;
    if (lay->split) {
        constexpr int64_t R = SPLIT_ROWS_PER_GROUP;
        const int64_t want = std::max<int64_t>(1, kSplitTarget / chunks);
        const int64_t K = kn.bwd_k > 0 ? kn.bwd_k : std::max<int64_t>(1, (M + R * want - 1) / (R * want));
        const int64_t blocks = (M + R * K - 1) / (R * K);
        if (blocks > 65535 || K > INT32_MAX)
            return NORM_ERR_SHAPE;
        lay->chunks = int(chunks);
        lay->blocks = int(blocks);
        lay->split_k = int(K);
        parts = blocks;
    }
    const int slices = colsum_slices(parts);
    lay->two_level = slices > 1;
    const size_t ld = size_t(colsum_ld(N));
    lay->level2_off = size_t(nb) * size_t(parts) * ld * sizeof(float);
    lay->bytes = lay->level2_off + (lay->two_level ? size_t(nb) * size_t(slices) * ld * sizeof(float) : 0);
    if (lay->split) {
        lay->rowsums_off = lay->bytes;
        lay->bytes += size_t(M) * size_t(lay->chunks) * 2 * sizeof(float);
    }
    return NORM_OK;
}

constexpr int kMaxDevices = 64;

// The address of the current device's scratch.  A stream other than the
// null stream must belong to the current device: hipGetSymbolAddress answers
// for the current device, and the kernels run on the stream's.
norm_status_t static_scratch(hipStream_t stream, void **ptr)
{
    static std::atomic<void *> addr[kMaxDevices];
    static std::mutex mu;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return NORM_ERR_DEVICE;
    if (stream != nullptr) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev)
            return NORM_ERR_DEVICE;
    }
    void *p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(mu);
        p = addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
                return NORM_ERR_DEVICE;
            addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return NORM_OK;
}

// use_static: the workspace is the current device's static scratch (the
// workspace arguments are ignored)
norm_status_t bwd_common(bool rms, const void *dy, const void *x, const void *gamma,
                         const float *mean, const float *rstd, float eps, int64_t M, int64_t N,
                         int32_t dtype, void *dx, void *dgamma, void *dbeta, void *dbias,
                         int32_t dparam_dtype, void *workspace, size_t workspace_bytes,
                         uint32_t flags, void *stream, bool use_static = false)
{
    if (!dtype_ok(dtype) || !dtype_ok(dparam_dtype))
        return NORM_ERR_DTYPE;
    if (norm_status_t st = check_shape(M, N))
        return st;
    if (M > 0 && (!dy || !x || !dx || (!rms && (!mean || !rstd))))
        return NORM_ERR_NULL;
    if (rms && !rstd && !eps_ok(eps))
        return NORM_ERR_ARG;
    if (flags & ~uint32_t(NORM_ZERO_CENTERED_GAMMA | NORM_DPARAM_MEAN))
        return NORM_ERR_ARG;
    const size_t es = elem_size(dtype);
    for (const void *p : {dy, x, gamma, (const void *)dx})
        if (p && !aligned(p, es))
            return NORM_ERR_ALIGN;
    for (const void *p : {(const void *)mean, (const void *)rstd})
        if (p && !aligned(p, 4))
            return NORM_ERR_ALIGN;
    if (workspace && !aligned(workspace, 16)) // the column sums read 16-byte vectors
        return NORM_ERR_ALIGN;
    const size_t ps = elem_size(dparam_dtype);
    for (const void *p : {(const void *)dgamma, (const void *)dbeta, (const void *)dbias})
        if (p && !aligned(p, ps))
            return NORM_ERR_ALIGN;

    if (norm_status_t st = check_device())
        return st;
    const Knobs kn = knobs();
    const int vec = vec_width(N, dtype, {dy, x, gamma, dx});
    const int unit = odd_unit_for(odd_unit(N, dtype, {dy, x, dx}), vec);
    const BwdEntry *e = nullptr;
    Walk w;
    BwdLayout lay;
    const int nb = dbias ? 3 : 2;
    if (norm_status_t st = bwd_plan(M, N, dtype, vec, unit, nb, kn, &e, &w, &lay))
        return st;
    const size_t need = lay.bytes;
    if (use_static) {
        if (need > size_t(NORM_STATIC_SCRATCH_BYTES))
            return NORM_ERR_WORKSPACE;
        workspace = nullptr;
        if (need > 0)
            if (norm_status_t st = static_scratch(static_cast<hipStream_t>(stream), &workspace))
                return st;
    } else if (need > 0 && (!workspace || workspace_bytes < need)) {
        return NORM_ERR_WORKSPACE;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    float *ws = static_cast<float *>(workspace);

    if (M > 0) {
        BwdArgs a;
        a.dy = dy;
        a.x = x;
        a.gamma = gamma;
        a.mean = mean;
        a.rstd = rstd;
        a.dx = dx;
        a.ws = ws;
        a.M = M;
        a.n_groups = w.n_groups;
        a.N = int(N);
        a.K = w.K;
        a.A = w.A;
        a.wt_group = wt_group(w, e->shape.teams, N, double(es), kn.bwd_wt_bytes);
        a.eps = eps;
        a.zero_centred = (flags & NORM_ZERO_CENTERED_GAMMA) != 0;
        a.rowsums = nullptr;
        a.chunks = 0;
        if (lay.split) {
            // rows, not row groups, from which dx is stored write-through
            const double rows_wt = std::ceil(kn.bwd_wt_bytes / (double(N) * double(es)));
            a.wt_group = rows_wt >= double(M) ? 0 : M - int64_t(rows_wt);
            a.K = lay.split_k;
            a.rowsums = reinterpret_cast<float *>(static_cast<char *>(workspace) + lay.rowsums_off);
            a.chunks = lay.chunks;
            if (norm_status_t st =
                    launched(launch_bwd_split(a, dtype, rms, dbias != nullptr, lay.blocks, s)))
                return st;
        } else {
            const BwdLaunch run = dbias ? (rms ? e->rms_db : e->ln_db) : (rms ? e->rms : e->ln);
            if (norm_status_t st = launched(run(a, int(w.grid), s)))
                return st;
        }
    }
    float *level2 =
        lay.two_level ? reinterpret_cast<float *>(static_cast<char *>(workspace) + lay.level2_off)
                      : nullptr;
    // the mean over the rows instead of the sum (no rows: zeros either way)
    const float divisor = (flags & NORM_DPARAM_MEAN) && M > 0 ? float(M) : 1.f;
    const int parts = lay.split ? lay.blocks : int(w.grid);
    return launched(launch_colsum(ws, parts, nb, int(N), dgamma, dbeta, dbias, dparam_dtype,
                                  divisor, level2, s));
}

// Elements per vector access of a call whose pointers are all 16-byte
// aligned: the widest access N is a multiple of.
int vec_of_aligned(int64_t N, int32_t dtype)
{
    const int es = int(elem_size(dtype));
    const int min_bytes = dtype == NORM_F32 ? 8 : 4;
    for (int bytes = 16; bytes >= min_bytes; bytes /= 2)
        if (N % (bytes / es) == 0)
            return bytes / es;
    return 1;
}

const char *dtype_name(int32_t dtype) { return dtype == NORM_F32 ? "fp32" : "bf16"; }

// Appends to buf (the text is truncated to len - 1 characters).
struct Text {
    char *buf;
    size_t len, used = 0;
    void add(const char *fmt, ...) __attribute__((format(printf, 2, 3)))
    {
        if (!buf || len == 0 || used + 1 >= len)
            return;
        va_list ap;
        va_start(ap, fmt);
        const int n = std::vsnprintf(buf + used, len - used, fmt, ap);
        va_end(ap);
        if (n > 0)
            used = std::min(len - 1, used + size_t(n));
    }
};

void describe_shape(Text &t, const char *kernel, int32_t dtype, const RowShape &sh)
{
    t.add("%s<%s, VEC %d, LPR %d, VPL %d, TEAMS %d", kernel, dtype_name(dtype), sh.vec, sh.lpr,
          sh.vpl, sh.teams);
}

// Odd-row kernels: VPL vectors of 2U elements per lane plus the row's
// leftover unit of U.
void describe_odd_shape(Text &t, const char *kernel, int32_t dtype, int unit, const RowShape &sh)
{
    t.add("%s<%s, unit %d, LPR %d, VPL %d, TEAMS %d", kernel, dtype_name(dtype), unit, sh.lpr,
          sh.vpl, sh.teams);
}

} // namespace

extern "C" {

norm_status_t norm_describe(int32_t op, int64_t M, int64_t N, int32_t dtype, uint32_t opts,
                            char *buf, size_t len)
{
    if (!buf || len == 0)
        return NORM_ERR_NULL;
    buf[0] = '\0';
    if (!dtype_ok(dtype))
        return NORM_ERR_DTYPE;
    if (norm_status_t st = check_shape(M, N))
        return st;
    if (op < NORM_OP_LN_FWD || op > NORM_OP_SOFTMAX ||
        (opts & ~uint32_t(NORM_DESCRIBE_AMAX | NORM_DESCRIBE_FP8 | NORM_DESCRIBE_DBIAS |
                          NORM_DESCRIBE_AMAX_WS)))
        return NORM_ERR_ARG;
    const Knobs kn = knobs();
    const int vec = vec_of_aligned(N, dtype);
    Text t{buf, len};
    Walk w;
    if (op == NORM_OP_LN_FWD || op == NORM_OP_RMS_FWD) {
        const bool amax = opts & NORM_DESCRIBE_AMAX, f8 = opts & NORM_DESCRIBE_FP8;
        const FwdEntry *e = nullptr;
        if (norm_status_t st = fwd_plan(M, N, dtype, vec, odd_unit_for(odd_unit(N, dtype, {}), vec),
                                        amax, f8, kn, &e, &w))
            return st;
        if (w.unit)
            describe_odd_shape(t, "fwd_odd_kernel", dtype, w.unit, e->shape);
        else
            describe_shape(t, "fwd_kernel", dtype, e->shape);
        t.add(", %s%s>; grid %lld x %d threads, %d row group(s) of %d rows per workgroup",
              op == NORM_OP_RMS_FWD ? "RMSNorm" : "LayerNorm", f8 ? ", FP8 y" : "",
              (long long)w.grid, e->shape.threads(), w.K, e->shape.teams);
        if (amax && (opts & NORM_DESCRIBE_AMAX_WS) && M > 0)
            t.add("; amax: combined in the caller's workspace, written by the last workgroup");
        else if (amax)
            t.add("; amax: one-thread reset kernel first");
        return NORM_OK;
    }
    if (op == NORM_OP_SOFTMAX) {
        const SoftmaxEntry *e = nullptr;
        if (norm_status_t st = softmax_plan(M, N, dtype, vec,
                                            odd_unit_for(odd_unit(N, dtype, {}), vec), kn, &e, &w))
            return st;
        if (w.unit)
            describe_odd_shape(t, "softmax_odd_kernel", dtype, w.unit, e->shape);
        else
            describe_shape(t, "softmax_kernel", dtype, e->shape);
        t.add(">; grid %lld x %d threads, %d row group(s) of %d rows per workgroup",
              (long long)w.grid, e->shape.threads(), w.K, e->shape.teams);
        return NORM_OK;
    }
    const bool dbias = opts & NORM_DESCRIBE_DBIAS;
    const BwdEntry *e = nullptr;
    BwdLayout lay;
    if (norm_status_t st = bwd_plan(M, N, dtype, vec, odd_unit_for(odd_unit(N, dtype, {}), vec),
                                    dbias ? 3 : 2, kn, &e, &w, &lay))
        return st;
    const char *norm = op == NORM_OP_RMS_BWD ? "RMSNorm" : "LayerNorm";
    if (lay.split) {
        t.add("bwd_split_kernel<%s, VEC %d, %s%s>, two passes; grid %d chunks x %d row blocks "
              "x %d threads", dtype_name(dtype), vec, norm, dbias ? ", dbias" : "", lay.chunks,
              lay.blocks, 64 * SPLIT_ROWS_PER_GROUP);
    } else {
        if (w.unit)
            describe_odd_shape(t, "bwd_odd_kernel", dtype, w.unit, e->shape);
        else
            describe_shape(t, "bwd_kernel", dtype, e->shape);
        t.add(", %s%s>; grid %lld x %d threads, %d row group(s) of %d rows per workgroup", norm,
              dbias ? ", dbias" : "", (long long)w.grid, e->shape.threads(), w.K,
              e->shape.teams);
    }
    const int64_t parts = lay.split ? lay.blocks : w.grid;
    t.add("; then column sums of %lld partial rows in %d launch(es)", (long long)parts,
          lay.two_level ? 2 : 1);
    return NORM_OK;
}

norm_status_t ln_fwd(const void *x, const void *bias, const void *residual, const void *gamma,
                     const void *beta, float eps, int64_t M, int64_t N, int32_t dtype, void *y,
                     void *residual_out, float *mean, float *rstd, float *amax, void *amax_ws,
                     uint32_t flags, void *stream)
{
    return fwd_common(false, x, bias, residual, gamma, beta, eps, M, N, dtype, nullptr, y,
                      residual_out, mean, rstd, amax, amax_ws, false, flags, stream);
}

norm_status_t rms_fwd(const void *x, const void *bias, const void *residual, const void *gamma,
                      const void *beta, float eps, int64_t M, int64_t N, int32_t dtype, void *y,
                      void *residual_out, float *mean, float *rstd, float *amax, void *amax_ws,
                      uint32_t flags, void *stream)
{
    return fwd_common(true, x, bias, residual, gamma, beta, eps, M, N, dtype, nullptr, y,
                      residual_out, mean, rstd, amax, amax_ws, false, flags, stream);
}

norm_status_t ln_fwd_fp8(const void *x, const void *bias, const void *residual,
                         const void *gamma, const void *beta, float eps, int64_t M, int64_t N,
                         int32_t dtype, const float *y_scale, void *y_fp8, void *residual_out,
                         float *mean, float *rstd, float *amax, void *amax_ws, uint32_t flags,
                         void *stream)
{
    return fwd_common(false, x, bias, residual, gamma, beta, eps, M, N, dtype, y_scale, y_fp8,
                      residual_out, mean, rstd, amax, amax_ws, true, flags, stream);
}

norm_status_t rms_fwd_fp8(const void *x, const void *bias, const void *residual,
                          const void *gamma, const void *beta, float eps, int64_t M, int64_t N,
                          int32_t dtype, const float *y_scale, void *y_fp8, void *residual_out,
                          float *mean, float *rstd, float *amax, void *amax_ws, uint32_t flags,
                          void *stream)
{
    return fwd_common(true, x, bias, residual, gamma, beta, eps, M, N, dtype, y_scale, y_fp8,
                      residual_out, mean, rstd, amax, amax_ws, true, flags, stream);
}

norm_status_t softmax_fwd(const void *x, int64_t M, int64_t N, int32_t dtype, void *y,
                          uint32_t flags, void *stream)
{
    return softmax_common(x, M, N, dtype, y, flags, stream);
}

norm_status_t norm_bwd_workspace_size(int64_t M, int64_t N, int32_t dtype, size_t *bytes)
{
    if (!bytes)
        return NORM_ERR_NULL;
    if (!dtype_ok(dtype))
        return NORM_ERR_DTYPE;
    if (norm_status_t st = check_shape(M, N))
        return st;
    if (norm_status_t st = check_device())
        return st;
    // Largest need over the kernels a call of this shape may take (any
    // vector width N allows, the odd-row kernel of N's unit on any such
    // width, with dbias).
    const Knobs kn = knobs();
    size_t best = 0;
    const int unit = odd_unit(N, dtype, {});
    auto need = [&](int v, int u) {
        const BwdEntry *e = nullptr;
        Walk w;
        BwdLayout lay;
        const norm_status_t st = bwd_plan(M, N, dtype, v, u, 3, kn, &e, &w, &lay);
        best = std::max(best, lay.bytes);
        return st;
    };
    for (int v = full_width(dtype); v >= 1; v /= 2) {
        if (N % v != 0)
            continue;
        if (norm_status_t st = need(v, 0))
            return st;
        if (odd_unit_for(unit, v))
            if (norm_status_t st = need(v, unit))
                return st;
    }
    *bytes = best;
    return NORM_OK;
}

norm_status_t ln_bwd(const void *dy, const void *x, const void *gamma, const float *mean,
                     const float *rstd, int64_t M, int64_t N, int32_t dtype, void *dx,
                     void *dgamma, void *dbeta, void *dbias, int32_t dparam_dtype,
                     void *workspace, size_t workspace_bytes, uint32_t flags, void *stream)
{
    return bwd_common(false, dy, x, gamma, mean, rstd, 0.f, M, N, dtype, dx, dgamma, dbeta,
                      dbias, dparam_dtype, workspace, workspace_bytes, flags, stream);
}

norm_status_t rms_bwd(const void *dy, const void *x, const void *gamma, const float *rstd,
                      float eps, int64_t M, int64_t N, int32_t dtype, void *dx, void *dgamma,
                      void *dbeta, void *dbias, int32_t dparam_dtype, void *workspace,
                      size_t workspace_bytes, uint32_t flags, void *stream)
{
    return bwd_common(true, dy, x, gamma, nullptr, rstd, eps, M, N, dtype, dx, dgamma, dbeta,
                      dbias, dparam_dtype, workspace, workspace_bytes, flags, stream);
}

norm_status_t ln_bwd_noalloc(const void *dy, const void *x, const void *gamma, const float *mean,
                             const float *rstd, int64_t M, int64_t N, int32_t dtype, void *dx,
                             void *dgamma, void *dbeta, void *dbias, int32_t dparam_dtype,
                             uint32_t flags, void *stream)
{
    return bwd_common(false, dy, x, gamma, mean, rstd, 0.f, M, N, dtype, dx, dgamma, dbeta,
                      dbias, dparam_dtype, nullptr, 0, flags, stream, true);
}

const char *norm_status_string(norm_status_t st)
{
    switch (st) {
    case NORM_OK: return "ok";
    case NORM_ERR_NULL: return "a required pointer is NULL";
    case NORM_ERR_SHAPE: return "unsupported shape (M < 0, N < 1 or N > NORM_N_MAX)";
    case NORM_ERR_ARG: return "invalid argument (eps negative or not finite, or an argument the op does not take)";
    case NORM_ERR_DTYPE: return "unknown dtype code";
    case NORM_ERR_ALIGN: return "pointer not aligned to its element size";
    case NORM_ERR_WORKSPACE: return "workspace missing or smaller than norm_bwd_workspace_size";
    case NORM_ERR_LAUNCH: return "kernel launch failed";
    case NORM_ERR_DEVICE: return "no usable HIP device";
    default: return "unknown status";
    }
}

} // extern "C"
