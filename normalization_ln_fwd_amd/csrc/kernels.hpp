// kernels.hpp -- fused LayerNorm / RMSNorm kernels for gfx950.
//
// Row ownership.  A "team" of LPR lanes owns one row; lane `tl` of the team
// holds VPL vectors of VEC consecutive elements, vector k covering columns
// [(k*LPR + tl)*VEC, +VEC).  For one k the team's lanes touch one contiguous
// span of LPR*VEC elements, so every access instruction is fully coalesced.
// LPR <= 64 packs 64/LPR teams (rows) into a wave and reduces with DPP /
// permlane inside the wave; LPR > 64 spans LPR/64 waves and finishes its
// reductions through LDS.  A workgroup holds TEAMS teams, i.e. it covers a
// "row group" of TEAMS consecutive rows at a time.
//
// The whole row stays in registers between the statistics and the
// normalisation (or between the two reductions of the backward): every
// [M, N] tensor crosses HBM exactly once, with nontemporal loads and stores.
//
// Grid.  Streaming on this GPU is fastest when each workgroup covers a small
// contiguous piece and exits, so that the workgroups in flight always sweep
// one compact window of memory: the forward gives each workgroup one row
// group.  The backward gives each workgroup K row groups (GroupWalk) so that
// its dgamma / dbeta column partials are written once per K groups.
#pragma once

#include <type_traits>

#include "device.hpp"
#include "internal.hpp"

// Whether a workgroup walking several row groups issues the next group's
// loads before working on the current one (two groups in flight per wave, at
// the cost of the registers that hold them).
#ifndef NORMFUSE_PREFETCH
#define NORMFUSE_PREFETCH 0
#endif

namespace nf {

// Row groups of workgroup b = q*A + r (A_q = min(A, grid - q*A) workgroups in
// its block of A): groups q*A*K + k*A_q + r for k < K.  The workgroups of one
// block sweep K contiguous windows of A_q groups, one window per k, and with
// grid = ceil(n_groups / K) every group is visited exactly once.
struct GroupWalk {
    int64_t base, step;
    __device__ __forceinline__ GroupWalk(int K, int A)
    {
        // grid and A fit 31 bits: 32-bit division (uniform, scalar unit)
        const uint32_t b = blockIdx.x, q = b / uint32_t(A), r = b - q * uint32_t(A);
        const uint32_t left = gridDim.x - q * uint32_t(A);
        step = left < uint32_t(A) ? left : uint32_t(A);
        base = int64_t(q) * A * K + r;
    }
    __device__ __forceinline__ int64_t group(int k) const { return base + k * step; }
};

// Sum over a team.  LPR <= 64: inside the wave.  LPR > 64: wave partials
// meet in LDS (double-buffered by `parity`, so one barrier per reduction
// suffices) and are added in wave order.  NV values are reduced together.
template <int LPR, int TEAMS, int NV>
__device__ __forceinline__ void team_sum(float (&v)[NV], float *lds, int &parity, int team,
                                         int wave_in_team, int lane)
{
    if constexpr (LPR <= 64) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            v[i] = group_reduce<LPR, OpSum>(v[i]);
    } else {
        constexpr int WPT = LPR / 64;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            v[i] = group_reduce<64, OpSum>(v[i]);
        float *b = lds + parity * (TEAMS * WPT * NV);
        if (lane == 0) {
#pragma unroll
            for (int i = 0; i < NV; ++i)
                b[(team * WPT + wave_in_team) * NV + i] = v[i];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float s = b[(team * WPT) * NV + i];
#pragma unroll
            for (int w = 1; w < WPT; ++w)
                s += b[(team * WPT + w) * NV + i];
            v[i] = s;
        }
        parity ^= 1;
    }
}

template <int LPR, int TEAMS, int NV>
struct TeamLds {
    static constexpr int size = LPR > 64 ? 2 * TEAMS * (LPR / 64) * NV : 1;
};

// fp64 sum over a team (same scheme as team_sum, one value).
template <int LPR, int TEAMS>
__device__ __forceinline__ double team_sum_f64(double v, double *lds, int &parity, int team,
                                               int wave_in_team, int lane)
{
    if constexpr (LPR <= 64) {
        return group_sum_f64<LPR>(v);
    } else {
        constexpr int WPT = LPR / 64;
        v = group_sum_f64<64>(v);
        double *b = lds + parity * (TEAMS * WPT);
        if (lane == 0)
            b[team * WPT + wave_in_team] = v;
        __syncthreads();
        double s = b[team * WPT];
#pragma unroll
        for (int w = 1; w < WPT; ++w)
            s += b[team * WPT + w];
        parity ^= 1;
        return s;
    }
}

// ---------------------------------------------------------------------------
// Forward: t = (x + bias) + residual (fp32), u = round(t) -> residual_out,
// statistics of u, y = normalise(u) * gamma + beta -> y, running max |y|.
// ---------------------------------------------------------------------------
template <typename T, int VEC, int LPR, int VPL, int TEAMS, bool RMS>
__global__ void __launch_bounds__(LPR *TEAMS) fwd_kernel(const FwdArgs a)
{
    using IO = VecIO<T, VEC>;
    using Raw = typename IO::Raw;
    constexpr int E = VPL * VEC;
    constexpr int WG = LPR * TEAMS;
    static_assert(WG % 64 == 0, "workgroup of whole waves");

    __shared__ float red_lds[TeamLds<LPR, TEAMS, 1>::size];
    __shared__ double red_lds_f64[TeamLds<LPR, TEAMS, 1>::size];
    __shared__ float max_lds[WG / 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int team = tid / LPR;
    const int tl = tid % LPR;
    const int wave_in_team = LPR > 64 ? tl / 64 : 0;
    const int N = a.N;

    const bool has_bias = a.bias != nullptr, has_res = a.res != nullptr;
    const bool has_gamma = a.gamma != nullptr, has_beta = a.beta != nullptr;
    const bool fused_add = has_bias || has_res;

    bool cvalid[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k)
        cvalid[k] = (k * LPR + tl) * VEC < N; // VEC > 1: N % VEC == 0, whole vector valid

    float lane_max = 0.f;
    int parity = 0;
    const GroupWalk walk(a.K, a.A);

    // x and residual of a row group, nontemporal; zeros outside the matrix.
    // With NORMFUSE_PREFETCH the next group's loads are issued before the
    // current group is worked on.
    Raw xn[VPL], rn[VPL];
    auto issue = [&](int64_t g) {
        const int64_t row = g * TEAMS + team;
        const bool rv = g < a.n_groups && row < a.M;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int64_t idx = row * (int64_t)N + (k * LPR + tl) * VEC;
            const bool ok = rv && cvalid[k];
            xn[k] = ok ? IO::load_stream(a.x, idx) : IO::zero();
            rn[k] = (ok && has_res) ? IO::load_stream(a.res, idx) : IO::zero();
        }
    };
    if (NORMFUSE_PREFETCH)
        issue(walk.group(0));

    for (int kk = 0; kk < a.K; ++kk) {
        const int64_t grp = walk.group(kk);
        if (grp >= a.n_groups)
            break; // uniform over the workgroup; later groups are larger
        const int64_t row = grp * TEAMS + team;
        const bool rv = row < a.M;
        const int64_t roff = row * (int64_t)N;
        if (!NORMFUSE_PREFETCH)
            issue(grp);

        // Fused add.  ur holds u, the value actually normalised, in its
        // packed I/O form (exact: u is rounded to T); every later pass
        // unpacks it again rather than keeping a float copy live.
        Raw ur[VPL], rr[VPL], br[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            ur[k] = xn[k];
            rr[k] = rn[k];
            br[k] = (cvalid[k] && has_bias) ? IO::load(a.bias, (k * LPR + tl) * VEC) : IO::zero();
        }
        if (NORMFUSE_PREFETCH && kk + 1 < a.K)
            issue(walk.group(kk + 1));
        // fused add; u = round_T((x + bias) + residual), and the row sum of
        // u for LayerNorm (fp32 for bf16 rows, whose sums of values of
        // similar magnitude are exact in fp32; fp64 for fp32 rows).
        using Acc = typename std::conditional<std::is_same<T, float>::value, double, float>::type;
        Acc sum = Acc(0);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float t[VEC];
            IO::unpack(ur[k], t);
            if (fused_add) {
                float bv[VEC], rv_[VEC];
                IO::unpack(br[k], bv);
                IO::unpack(rr[k], rv_);
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    t[e] = (t[e] + bv[e]) + rv_[e];
                ur[k] = IO::pack(t);
                IO::unpack(ur[k], t);
            }
            if constexpr (!RMS) {
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    sum += Acc(t[e]); // invalid columns hold 0
            }
        }
        if (a.res_out) {
#pragma unroll
            for (int k = 0; k < VPL; ++k)
                if (rv && cvalid[k])
                    IO::store_stream(a.res_out, roff + (k * LPR + tl) * VEC, ur[k]);
        }
        // per-column scale and shift, in flight during the reductions
        Raw gr[VPL], betar[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int c0 = (k * LPR + tl) * VEC;
            gr[k] = (cvalid[k] && has_gamma) ? IO::load(a.gamma, c0) : IO::zero();
            betar[k] = (cvalid[k] && has_beta) ? IO::load(a.beta, c0) : IO::zero();
        }

        // Statistics.  LayerNorm keeps its mean as an fp32 pair mean + lo
        // (lo = the rounding error of the fp32 mean), so that centring stays
        // accurate when the mean is large next to the spread: d = u - mean is
        // exact near the mean, sum(d^2) = N var + N lo^2, and the normalised
        // value is d * rstd - lo * rstd.
        float mean = 0.f, lo = 0.f, rstd;
        if constexpr (!RMS) {
            if constexpr (std::is_same<T, float>::value) {
                const double sd =
                    team_sum_f64<LPR, TEAMS>(sum, red_lds_f64, parity, team, wave_in_team, lane);
                const double mean_d = sd / double(N);
                mean = float(mean_d);
                lo = float(mean_d - double(mean));
            } else {
                float sv[1] = {sum};
                team_sum<LPR, TEAMS, 1>(sv, red_lds, parity, team, wave_in_team, lane);
                mean = sv[0] / float(N);
                lo = fmaf(-mean, float(N), sv[0]) / float(N);
            }
#pragma unroll
            for (int k = 0; k < VPL; ++k)
                reload_barrier(ur[k]);
            float d2[1] = {0.f};
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                if (cvalid[k]) {
                    float u[VEC];
                    IO::unpack(ur[k], u);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const float d = u[e] - mean;
                        d2[0] = fmaf(d, d, d2[0]);
                    }
                }
            }
            team_sum<LPR, TEAMS, 1>(d2, red_lds, parity, team, wave_in_team, lane);
            const float var = fmaxf(d2[0] / float(N) - lo * lo, 0.f);
            rstd = rsqrtf(var + a.eps);
        } else {
            float s2[1] = {0.f};
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                float u[VEC];
                IO::unpack(ur[k], u);
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    s2[0] = fmaf(u[e], u[e], s2[0]);
            }
            team_sum<LPR, TEAMS, 1>(s2, red_lds, parity, team, wave_in_team, lane);
            rstd = rsqrtf(s2[0] / float(N) + a.eps);
        }
        const float lo_r = -lo * rstd;

        // normalise, affine, store; amax over |y| before rounding (rounding
        // to nearest is monotone, so max |round(y)| = round(max |y|))
#pragma unroll
        for (int k = 0; k < VPL; ++k)
            reload_barrier(ur[k]);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int c0 = (k * LPR + tl) * VEC;
            const bool ok = rv && cvalid[k];
            float u[VEC], gv[VEC], bv[VEC], yv[VEC];
            IO::unpack(ur[k], u);
            IO::unpack(gr[k], gv);
            IO::unpack(betar[k], bv);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                float n = fmaf(u[e] - mean, rstd, lo_r);
                if (has_gamma)
                    n = has_beta ? fmaf(n, gv[e], bv[e]) : n * gv[e];
                else if (has_beta)
                    n += bv[e];
                yv[e] = n;
            }
            if (ok) {
                IO::store_stream(a.y, roff + c0, IO::pack(yv));
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    lane_max = fmaxf(lane_max, fabsf(yv[e]));
            }
        }
        if (tl == 0 && rv) {
            if (a.mean)
                a.mean[row] = mean;
            if (a.rstd)
                a.rstd[row] = rstd;
        }
    }

    // amax, first stage: wave max through DPP / permlane, then the
    // workgroup's waves through LDS; second stage: one atomicMax per
    // workgroup on the float's bit pattern (non-negative floats order like
    // their unsigned patterns).  Atomics on one address serialise, which is
    // one reason a workgroup covers several row groups.
    if (a.amax) {
        const float m = group_reduce<64, OpMax>(lane_max);
        if (lane == 0)
            max_lds[tid >> 6] = m;
        __syncthreads();
        if (tid == 0) {
            float mm = max_lds[0];
#pragma unroll
            for (int w = 1; w < WG / 64; ++w)
                mm = fmaxf(mm, max_lds[w]);
            float r[1] = {mm};
            VecIO<T, 1>::unpack(VecIO<T, 1>::pack(r), r); // max of the stored y
            atomicMax(a.amax, __float_as_uint(r[0]));
        }
    }
}

// ---------------------------------------------------------------------------
// Backward stage 1 (mix-order): per row, one load of dy and x; the row
// reduction gives dx; the column reduction is accumulated in registers over
// the workgroup's rows, folded over the workgroup in a fixed order and
// written as this workgroup's partial row of the workspace.
// ---------------------------------------------------------------------------
template <typename T, int VEC, int LPR, int VPL, int TEAMS, bool RMS>
__global__ void __launch_bounds__(LPR *TEAMS) bwd_kernel(const BwdArgs a)
{
    using IO = VecIO<T, VEC>;
    using Raw = typename IO::Raw;
    constexpr int E = VPL * VEC;
    constexpr int WG = LPR * TEAMS;
    constexpr int NW = WG / 64;
    constexpr int CAP = LPR * VPL * VEC;
    // partial slots to fold in LDS: waves (LPR <= 64) or teams (LPR > 64)
    constexpr int SLOTS = LPR <= 64 ? NW : TEAMS;
    static_assert(WG % 64 == 0, "workgroup of whole waves");

    __shared__ float red_lds[TeamLds<LPR, TEAMS, 2>::size];
    __shared__ float col_lds[SLOTS > 1 ? 2 * CAP : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int team = tid / LPR;
    const int tl = tid % LPR;
    const int wave_in_team = LPR > 64 ? tl / 64 : 0;
    const int N = a.N;
    const bool has_gamma = a.gamma != nullptr;
    const bool recompute = RMS && a.rstd == nullptr;

    bool cvalid[VPL];
    Raw gamma_r[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int c0 = (k * LPR + tl) * VEC;
        cvalid[k] = c0 < N;
        gamma_r[k] = (has_gamma && cvalid[k]) ? IO::load(a.gamma, c0) : IO::zero();
    }

    float acc_g[E], acc_b[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        acc_g[e] = 0.f;
        acc_b[e] = 0.f;
    }

    int parity = 0;
    const GroupWalk walk(a.K, a.A);

    // x, dy and the row statistics of a row group (with NORMFUSE_PREFETCH the
    // next group's loads are issued before the current group is worked on).
    Raw xn[VPL], dn[VPL];
    float mean_n = 0.f, rstd_n = 0.f;
    auto issue = [&](int64_t g) {
        const int64_t row = g * TEAMS + team;
        const bool rv = g < a.n_groups && row < a.M;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int64_t idx = row * (int64_t)N + (k * LPR + tl) * VEC;
            const bool ok = rv && cvalid[k];
            xn[k] = ok ? IO::load_stream(a.x, idx) : IO::zero();
            dn[k] = ok ? IO::load_stream(a.dy, idx) : IO::zero();
        }
        mean_n = (rv && !RMS) ? a.mean[row] : 0.f;
        rstd_n = (rv && !recompute) ? a.rstd[row] : 0.f;
    };
    if (NORMFUSE_PREFETCH)
        issue(walk.group(0));

    for (int kk = 0; kk < a.K; ++kk) {
        const int64_t grp = walk.group(kk);
        if (grp >= a.n_groups)
            break; // uniform over the workgroup; later groups are larger
        const int64_t row = grp * TEAMS + team;
        const bool rv = row < a.M;
        const int64_t roff = row * (int64_t)N;
        if (!NORMFUSE_PREFETCH)
            issue(grp);

        Raw xr[VPL], dr[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            xr[k] = xn[k];
            dr[k] = dn[k];
            reload_barrier(gamma_r[k]); // unpack gamma here, not once outside the loop
        }
        float mean = mean_n, rstd = rstd_n;
        if (NORMFUSE_PREFETCH && kk + 1 < a.K)
            issue(walk.group(kk + 1));

        // g = dy * gamma; the rows stay packed and are unpacked per pass
        float c1, c2 = 0.f;
        {
            float s[2] = {0.f, 0.f};
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                float xv[VEC], dv[VEC], gv[VEC];
                IO::unpack(xr[k], xv);
                IO::unpack(dr[k], dv);
                IO::unpack(gamma_r[k], gv);
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float g = has_gamma ? dv[e] * gv[e] : dv[e]; // invalid: 0
                    if constexpr (!RMS) {
                        s[0] += g * ((xv[e] - mean) * rstd);
                        s[1] += g;
                    } else {
                        if (recompute) {
                            // rstd from the same load: sum x^2 and sum g*x
                            // reduce together; mean(g*xhat) = rstd * mean(g*x)
                            s[0] += xv[e] * xv[e];
                            s[1] += g * xv[e];
                        } else {
                            s[0] += g * (xv[e] * rstd);
                        }
                    }
                }
            }
            team_sum<LPR, TEAMS, 2>(s, red_lds, parity, team, wave_in_team, lane);
            if constexpr (!RMS) {
                c1 = s[0] / float(N);
                c2 = s[1] / float(N);
            } else if (recompute) {
                rstd = rsqrtf(s[0] / float(N) + a.eps);
                c1 = rstd * (s[1] / float(N));
            } else {
                c1 = s[0] / float(N);
            }
        }

#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            reload_barrier(xr[k]);
            reload_barrier(dr[k]);
        }
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int c0 = (k * LPR + tl) * VEC;
            const bool ok = rv && cvalid[k];
            float xv[VEC], dv[VEC], gv[VEC], dxv[VEC];
            IO::unpack(xr[k], xv);
            IO::unpack(dr[k], dv);
            IO::unpack(gamma_r[k], gv);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int i = k * VEC + e;
                const float g = has_gamma ? dv[e] * gv[e] : dv[e];
                const float xh = RMS ? xv[e] * rstd : (xv[e] - mean) * rstd;
                dxv[e] = rstd * (g - c2 - xh * c1);
                if (ok) {
                    acc_g[i] += dv[e] * xh;
                    acc_b[i] += dv[e];
                }
            }
            if (ok)
                IO::store_stream(a.dx, roff + c0, IO::pack(dxv));
        }
    }

    // ---- fold the column partials of this workgroup, in a fixed order ----
    float *pg = a.ws + (int64_t)blockIdx.x * N;
    float *pb = a.ws + (int64_t)gridDim.x * N + (int64_t)blockIdx.x * N;
    if constexpr (LPR < 64) {
        // teams of one wave cover the same columns: fold them first
#pragma unroll
        for (int e = 0; e < E; ++e) {
            acc_g[e] = fold_teams_sum<LPR>(acc_g[e]);
            acc_b[e] = fold_teams_sum<LPR>(acc_b[e]);
        }
    }
    if constexpr (SLOTS == 1) {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int c0 = (k * LPR + tl) * VEC;
            if (cvalid[k] && (LPR >= 64 || lane < LPR)) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    if (VEC > 1 || c0 + e < N) {
                        pg[c0 + e] = acc_g[k * VEC + e];
                        pb[c0 + e] = acc_b[k * VEC + e];
                    }
                }
            }
        }
    } else {
        const int slot = LPR <= 64 ? (tid >> 6) : team;
        const bool holder = LPR < 64 ? lane < LPR : true;
        for (int s = 0; s < SLOTS; ++s) {
            if (slot == s && holder) {
#pragma unroll
                for (int k = 0; k < VPL; ++k) {
                    const int c0 = (k * LPR + tl) * VEC;
                    if (cvalid[k]) {
#pragma unroll
                        for (int e = 0; e < VEC; ++e) {
                            const int c = c0 + e;
                            col_lds[c] = (s == 0 ? 0.f : col_lds[c]) + acc_g[k * VEC + e];
                            col_lds[CAP + c] = (s == 0 ? 0.f : col_lds[CAP + c]) + acc_b[k * VEC + e];
                        }
                    }
                }
            }
            __syncthreads();
        }
        for (int c = tid; c < N; c += WG) {
            pg[c] = col_lds[c];
            pb[c] = col_lds[CAP + c];
        }
    }
}

// ---------------------------------------------------------------------------
// Backward stage 2: column sums of the partial rows.  src holds two blocks
// (dgamma, dbeta) of `rows` rows of N floats.  Workgroup (column tile, slice
// s, block) adds rows [s*span, min(rows, (s+1)*span)): thread (c, t) takes
// rows t, t + 4, ... of the slice in ascending order, and the four threads of
// a column are added in order t = 0..3.  FINAL: one slice, the down-cast and
// the store to dgamma / dbeta; otherwise slice s writes row s of dst (two
// blocks of `gridDim.y` rows), the input of the next level.
// ---------------------------------------------------------------------------
constexpr int COLSUM_COLS = 64;
constexpr int COLSUM_SUB = 4;

template <bool FINAL, bool BF16_OUT>
__global__ void __launch_bounds__(COLSUM_COLS *COLSUM_SUB)
    colsum_kernel(const float *src, int rows, int N, int span, float *dst, void *dgamma,
                  void *dbeta)
{
    const int tx = threadIdx.x % COLSUM_COLS;
    const int ty = threadIdx.x / COLSUM_COLS;
    const int which = blockIdx.z;
    if (FINAL && (which == 0 ? dgamma : dbeta) == nullptr)
        return; // uniform over the block
    const int j = blockIdx.x * COLSUM_COLS + tx;
    const int s = blockIdx.y;
    const int r0 = s * span;
    const int r1 = min(rows, r0 + span);
    const float *part = src + (int64_t)which * rows * N;
    float acc = 0.f;
    if (j < N) {
#pragma unroll 8
        for (int r = r0 + ty; r < r1; r += COLSUM_SUB)
            acc += part[(int64_t)r * N + j];
    }
    __shared__ float sl[COLSUM_SUB][COLSUM_COLS];
    sl[ty][tx] = acc;
    __syncthreads();
    if (ty == 0 && j < N) {
        float t = sl[0][tx];
#pragma unroll
        for (int q = 1; q < COLSUM_SUB; ++q)
            t += sl[q][tx];
        if constexpr (!FINAL) {
            dst[((int64_t)which * gridDim.y + s) * N + j] = t;
        } else if constexpr (BF16_OUT) {
            static_cast<uint16_t *>(which == 0 ? dgamma : dbeta)[j] =
                uint16_t(pack_bf16x2(t, 0.f) & 0xffffu);
        } else {
            static_cast<float *>(which == 0 ? dgamma : dbeta)[j] = t;
        }
    }
}

template <typename T, int VEC, int LPR, int VPL, int TEAMS, bool RMS>
hipError_t launch_fwd(const FwdArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((fwd_kernel<T, VEC, LPR, VPL, TEAMS, RMS>), dim3(grid), dim3(LPR * TEAMS),
                       0, s, a);
    return hipGetLastError();
}

template <typename T, int VEC, int LPR, int VPL, int TEAMS, bool RMS>
hipError_t launch_bwd(const BwdArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((bwd_kernel<T, VEC, LPR, VPL, TEAMS, RMS>), dim3(grid), dim3(LPR * TEAMS),
                       0, s, a);
    return hipGetLastError();
}

} // namespace nf
