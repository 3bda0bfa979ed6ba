// api.cpp -- the C ABI declared in include/normfuse.h: argument checks,
// choice of kernel shape, persistent-grid sizing and launches on the
// caller's stream.  Nothing here allocates device memory.
#include "normfuse.h"

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "internal.hpp"

namespace {

using namespace nf;

// ---------------------------------------------------------------- device
constexpr int kMaxDevices = 64;
std::once_flag g_cu_once[kMaxDevices];
int g_cus[kMaxDevices];

norm_status_t current_device(int *dev, int *cus)
{
    if (hipGetDevice(dev) != hipSuccess || *dev < 0 || *dev >= kMaxDevices)
        return NORM_ERR_DEVICE;
    const int d = *dev;
    std::call_once(g_cu_once[d], [d] {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess)
            n = 0;
        g_cus[d] = n;
    });
    if (g_cus[d] <= 0)
        return NORM_ERR_DEVICE;
    *cus = g_cus[d];
    return NORM_OK;
}

// Resident workgroups per CU of one kernel on one device, cached.
int resident_per_cu(OccFn fn, int dev)
{
    static std::mutex mu;
    static std::map<std::pair<OccFn, int>, int> cache;
    std::lock_guard<std::mutex> lock(mu);
    auto key = std::make_pair(fn, dev);
    auto it = cache.find(key);
    if (it != cache.end())
        return it->second;
    const int n = fn();
    cache[key] = n;
    return n;
}

// ------------------------------------------------------ optional tuning knobs
// NORMFUSE_{FWD,BWD}_WG_PER_CU : cap on workgroups per CU of the persistent grid
// NORMFUSE_{FWD,BWD}_SHAPE     : "LPRxVPL" -- use that instantiated shape when it
//                                covers the row (tests use it to cross-check shapes)
struct Knobs {
    int fwd_wg_per_cu = 0, bwd_wg_per_cu = 0;
    int fwd_lpr = 0, fwd_vpl = 0, bwd_lpr = 0, bwd_vpl = 0;
};

void parse_shape(const char *s, int *lpr, int *vpl)
{
    if (s && std::sscanf(s, "%dx%d", lpr, vpl) != 2) {
        *lpr = 0;
        *vpl = 0;
    }
}

const Knobs &knobs()
{
    static Knobs k = [] {
        Knobs r;
        if (const char *s = std::getenv("NORMFUSE_FWD_WG_PER_CU"))
            r.fwd_wg_per_cu = std::atoi(s);
        if (const char *s = std::getenv("NORMFUSE_BWD_WG_PER_CU"))
            r.bwd_wg_per_cu = std::atoi(s);
        parse_shape(std::getenv("NORMFUSE_FWD_SHAPE"), &r.fwd_lpr, &r.fwd_vpl);
        parse_shape(std::getenv("NORMFUSE_BWD_SHAPE"), &r.bwd_lpr, &r.bwd_vpl);
        return r;
    }();
    return k;
}

template <class Entry>
const Entry *pick_shape(const Entry *tab, int n, int N, int force_lpr, int force_vpl)
{
    if (force_lpr > 0) {
        for (int i = 0; i < n; ++i)
            if (tab[i].shape.lpr == force_lpr && tab[i].shape.vpl == force_vpl &&
                tab[i].shape.capacity() >= N)
                return &tab[i];
    }
    for (int i = 0; i < n; ++i)
        if (tab[i].shape.capacity() >= N)
            return &tab[i];
    return nullptr;
}

const FwdEntry *fwd_entry(int dtype, bool vec, int N)
{
    int n = 0;
    const FwdEntry *tab = dtype == NORM_F32 ? fwd_table_f32(vec, &n) : fwd_table_bf16(vec, &n);
    return pick_shape(tab, n, N, knobs().fwd_lpr, knobs().fwd_vpl);
}

const BwdEntry *bwd_entry(int dtype, bool vec, int N)
{
    int n = 0;
    const BwdEntry *tab = dtype == NORM_F32 ? bwd_table_f32(vec, &n) : bwd_table_bf16(vec, &n);
    return pick_shape(tab, n, N, knobs().bwd_lpr, knobs().bwd_vpl);
}

// Persistent grid: as many workgroups as are resident at once, but no more
// than there are row groups.
int64_t persistent_grid(int64_t M, int teams, int cus, int per_cu, int cap_per_cu)
{
    if (cap_per_cu > 0 && cap_per_cu < per_cu)
        per_cu = cap_per_cu;
    const int64_t want = (M + teams - 1) / teams;
    const int64_t have = int64_t(cus) * per_cu;
    return want < have ? want : have;
}

// ------------------------------------------------------------- validation
size_t elem_size(int32_t dtype) { return dtype == NORM_F32 ? 4 : 2; }

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

// 16-byte path: whole 16-byte vectors per row and 16-byte aligned tensors.
bool vectorisable(int64_t N, int32_t dtype, std::initializer_list<const void *> ptrs)
{
    const int vec = int(16 / elem_size(dtype));
    if (N % vec != 0)
        return false;
    for (const void *p : ptrs)
        if (p && !aligned(p, 16))
            return false;
    return true;
}

norm_status_t launched(hipError_t e) { return e == hipSuccess ? NORM_OK : NORM_ERR_LAUNCH; }

// ------------------------------------------------------------------ forward
norm_status_t fwd_common(bool rms, const void *x, const void *bias, const void *residual,
                         const void *gamma, const void *beta, float eps, int64_t M, int64_t N,
                         int32_t dtype, void *y, void *residual_out, float *mean, float *rstd,
                         float *amax, void *stream)
{
    if (!dtype_ok(dtype))
        return NORM_ERR_DTYPE;
    if (norm_status_t st = check_shape(M, N))
        return st;
    if (M > 0 && (!x || !y)) // with no rows there is nothing to read or write
        return NORM_ERR_NULL;
    if (!eps_ok(eps) || (rms && mean))
        return NORM_ERR_ARG;
    const size_t es = elem_size(dtype);
    for (const void *p : {x, bias, residual, gamma, beta, (const void *)y, (const void *)residual_out})
        if (p && !aligned(p, es))
            return NORM_ERR_ALIGN;
    for (const void *p : {(const void *)mean, (const void *)rstd, (const void *)amax})
        if (p && !aligned(p, 4))
            return NORM_ERR_ALIGN;

    int dev = 0, cus = 0;
    if (norm_status_t st = current_device(&dev, &cus))
        return st;
    const bool vec = vectorisable(N, dtype, {x, bias, residual, gamma, beta, y, residual_out});
    const FwdEntry *e = fwd_entry(dtype, vec, int(N));
    if (!e)
        return NORM_ERR_SHAPE;
    hipStream_t s = static_cast<hipStream_t>(stream);

    unsigned *amax_bits = reinterpret_cast<unsigned *>(amax);
    if (amax_bits)
        if (norm_status_t st = launched(launch_zero_u32(amax_bits, s)))
            return st;
    if (M == 0)
        return NORM_OK;

    const int per_cu = resident_per_cu(rms ? e->occ_rms : e->occ_ln, dev);
    const int64_t grid = persistent_grid(M, e->shape.teams, cus, per_cu, knobs().fwd_wg_per_cu);
    FwdArgs a;
    a.x = x;
    a.bias = bias;
    a.res = residual;
    a.gamma = gamma;
    a.beta = beta;
    a.y = y;
    a.res_out = residual_out;
    a.mean = mean;
    a.rstd = rstd;
    a.amax = amax_bits;
    a.M = M;
    a.N = int(N);
    a.eps = eps;
    return launched((rms ? e->rms : e->ln)(a, int(grid), s));
}

// ----------------------------------------------------------------- backward
// Stage-1 grid of the backward for the shape used on these pointers.
norm_status_t bwd_plan(bool rms, int64_t M, int64_t N, int32_t dtype, bool vec, int dev, int cus,
                       const BwdEntry **entry, int64_t *grid)
{
    const BwdEntry *e = bwd_entry(dtype, vec, int(N));
    if (!e)
        return NORM_ERR_SHAPE;
    const int per_cu = resident_per_cu(rms ? e->occ_rms : e->occ_ln, dev);
    *entry = e;
    *grid = M == 0 ? 0 : persistent_grid(M, e->shape.teams, cus, per_cu, knobs().bwd_wg_per_cu);
    return NORM_OK;
}

size_t ws_bytes_for(int64_t grid, int64_t N) { return size_t(2) * size_t(grid) * size_t(N) * 4; }

norm_status_t bwd_common(bool rms, const void *dy, const void *x, const void *gamma,
                         const float *mean, const float *rstd, float eps, int64_t M, int64_t N,
                         int32_t dtype, void *dx, void *dgamma, void *dbeta, int32_t dparam_dtype,
                         void *workspace, size_t workspace_bytes, void *stream)
{
    if (!dtype_ok(dtype) || !dtype_ok(dparam_dtype))
        return NORM_ERR_DTYPE;
    if (norm_status_t st = check_shape(M, N))
        return st;
    if (M > 0 && (!dy || !x || !dx || (!rms && (!mean || !rstd))))
        return NORM_ERR_NULL;
    if (rms && !rstd && !eps_ok(eps))
        return NORM_ERR_ARG;
    const size_t es = elem_size(dtype);
    for (const void *p : {dy, x, gamma, (const void *)dx})
        if (p && !aligned(p, es))
            return NORM_ERR_ALIGN;
    for (const void *p : {(const void *)mean, (const void *)rstd, (const void *)workspace})
        if (p && !aligned(p, 4))
            return NORM_ERR_ALIGN;
    const size_t ps = elem_size(dparam_dtype);
    for (const void *p : {(const void *)dgamma, (const void *)dbeta})
        if (p && !aligned(p, ps))
            return NORM_ERR_ALIGN;

    int dev = 0, cus = 0;
    if (norm_status_t st = current_device(&dev, &cus))
        return st;
    const bool vec = vectorisable(N, dtype, {dy, x, gamma, dx});
    const BwdEntry *e = nullptr;
    int64_t grid = 0;
    if (norm_status_t st = bwd_plan(rms, M, N, dtype, vec, dev, cus, &e, &grid))
        return st;
    const size_t need = ws_bytes_for(grid, N);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return NORM_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);

    if (M > 0) {
        BwdArgs a;
        a.dy = dy;
        a.x = x;
        a.gamma = gamma;
        a.mean = mean;
        a.rstd = rstd;
        a.dx = dx;
        a.ws = static_cast<float *>(workspace);
        a.M = M;
        a.N = int(N);
        a.eps = eps;
        if (norm_status_t st = launched((rms ? e->rms : e->ln)(a, int(grid), s)))
            return st;
    }
    return launched(launch_colsum(static_cast<const float *>(workspace), int(grid), int(N), dgamma,
                                  dbeta, dparam_dtype, s));
}

} // namespace

extern "C" {

norm_status_t ln_fwd(const void *x, const void *bias, const void *residual, const void *gamma,
                     const void *beta, float eps, int64_t M, int64_t N, int32_t dtype, void *y,
                     void *residual_out, float *mean, float *rstd, float *amax, void *stream)
{
    return fwd_common(false, x, bias, residual, gamma, beta, eps, M, N, dtype, y, residual_out,
                      mean, rstd, amax, stream);
}

norm_status_t rms_fwd(const void *x, const void *bias, const void *residual, const void *gamma,
                      const void *beta, float eps, int64_t M, int64_t N, int32_t dtype, void *y,
                      void *residual_out, float *mean, float *rstd, float *amax, void *stream)
{
    return fwd_common(true, x, bias, residual, gamma, beta, eps, M, N, dtype, y, residual_out,
                      mean, rstd, amax, stream);
}

norm_status_t norm_bwd_workspace_size(int64_t M, int64_t N, int32_t dtype, size_t *bytes)
{
    if (!bytes)
        return NORM_ERR_NULL;
    if (!dtype_ok(dtype))
        return NORM_ERR_DTYPE;
    if (norm_status_t st = check_shape(M, N))
        return st;
    int dev = 0, cus = 0;
    if (norm_status_t st = current_device(&dev, &cus))
        return st;
    // Largest need over the kernels a call of this shape may take (the
    // 16-byte path or the element-wise one, LayerNorm or RMSNorm).
    size_t best = 0;
    const int vec = int(16 / elem_size(dtype));
    for (int v = 0; v < 2; ++v) {
        if (v == 1 && N % vec != 0)
            continue;
        for (int rms = 0; rms < 2; ++rms) {
            const BwdEntry *e = nullptr;
            int64_t grid = 0;
            if (norm_status_t st = bwd_plan(rms != 0, M, N, dtype, v == 1, dev, cus, &e, &grid))
                return st;
            const size_t b = ws_bytes_for(grid, N);
            if (b > best)
                best = b;
        }
    }
    *bytes = best;
    return NORM_OK;
}

norm_status_t ln_bwd(const void *dy, const void *x, const void *gamma, const float *mean,
                     const float *rstd, int64_t M, int64_t N, int32_t dtype, void *dx,
                     void *dgamma, void *dbeta, int32_t dparam_dtype, void *workspace,
                     size_t workspace_bytes, void *stream)
{
    return bwd_common(false, dy, x, gamma, mean, rstd, 0.f, M, N, dtype, dx, dgamma, dbeta,
                      dparam_dtype, workspace, workspace_bytes, stream);
}

norm_status_t rms_bwd(const void *dy, const void *x, const void *gamma, const float *rstd,
                      float eps, int64_t M, int64_t N, int32_t dtype, void *dx, void *dgamma,
                      void *dbeta, int32_t dparam_dtype, void *workspace,
                      size_t workspace_bytes, void *stream)
{
    return bwd_common(true, dy, x, gamma, nullptr, rstd, eps, M, N, dtype, dx, dgamma, dbeta,
                      dparam_dtype, workspace, workspace_bytes, stream);
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
