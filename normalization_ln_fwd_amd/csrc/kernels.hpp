// kernels.hpp -- fused LayerNorm / RMSNorm kernels for gfx950.
//
// Row ownership.  A "team" of LPR lanes owns one row at a time; lane `tl` of
// the team holds VPL vectors of VEC consecutive elements, vector k covering
// columns [(k*LPR + tl)*VEC, +VEC).  For one k the team's lanes therefore
// touch one contiguous span of LPR*VEC elements: every access instruction is
// fully coalesced.  LPR <= 64 packs 64/LPR teams (rows) into a wave and
// reduces with DPP / permlane inside the wave; LPR > 64 spans LPR/64 waves
// and finishes its reductions through LDS.  A workgroup holds TEAMS teams
// and walks rows with a grid-stride loop over a persistent grid, so the
// per-column vectors (bias, gamma, beta) are loaded once per team and stay
// in registers.
//
// The whole row stays in registers between the statistics and the
// normalisation (or between the two reductions of the backward): every
// [M, N] tensor crosses HBM exactly once.
#pragma once

#include "device.hpp"
#include "internal.hpp"

namespace nf {

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
    constexpr int NW = WG / 64;
    static_assert(WG % 64 == 0, "workgroup of whole waves");

    __shared__ float red_lds[TeamLds<LPR, TEAMS, 1>::size];
    __shared__ float max_lds[NW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int team = tid / LPR;
    const int tl = tid % LPR;
    const int wave_in_team = LPR > 64 ? tl / 64 : 0;
    const int N = a.N;

    const bool has_bias = a.bias != nullptr, has_res = a.res != nullptr;
    const bool has_gamma = a.gamma != nullptr, has_beta = a.beta != nullptr;
    const bool fused_add = has_bias || has_res;

    // Column validity and the per-column vectors, once per team.
    bool cvalid[VPL];
    Raw bias_r[VPL], gamma_r[VPL], beta_r[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int c0 = (k * LPR + tl) * VEC;
        cvalid[k] = c0 < N; // VEC > 1 implies N % VEC == 0: whole vector valid
        float zero[VEC] = {};
        bias_r[k] = (has_bias && cvalid[k]) ? IO::load_raw(a.bias, c0) : IO::pack(zero);
        gamma_r[k] = (has_gamma && cvalid[k]) ? IO::load_raw(a.gamma, c0) : IO::pack(zero);
        beta_r[k] = (has_beta && cvalid[k]) ? IO::load_raw(a.beta, c0) : IO::pack(zero);
    }

    float lane_max = 0.f;
    int parity = 0;
    const int64_t stride = (int64_t)gridDim.x * TEAMS;
    for (int64_t base = (int64_t)blockIdx.x * TEAMS; base < a.M; base += stride) {
        const int64_t row = base + team;
        const bool rv = row < a.M;
        const int64_t roff = row * (int64_t)N;

        // fused add; u = value actually normalised (rounded to the I/O dtype)
        float u[E];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int c0 = (k * LPR + tl) * VEC;
            const bool ok = rv && cvalid[k];
            float *uk = &u[k * VEC];
            Raw xr;
            if (ok) {
                xr = IO::load_raw(a.x, roff + c0);
            } else {
                float zero[VEC] = {};
                xr = IO::pack(zero);
            }
            IO::unpack(xr, uk);
            if (fused_add) {
                if (has_bias) {
                    float bv[VEC];
                    IO::unpack(bias_r[k], bv);
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        uk[e] += bv[e];
                }
                if (has_res) {
                    float rvv[VEC] = {};
                    if (ok)
                        IO::unpack(IO::load_raw(a.res, roff + c0), rvv);
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        uk[e] += rvv[e];
                }
                xr = IO::pack(uk);
                IO::unpack(xr, uk);
            }
            if (a.res_out && ok)
                IO::store_raw(a.res_out, roff + c0, xr);
        }

        // statistics (two passes over registers for LayerNorm)
        float mean = 0.f, rstd;
        if constexpr (!RMS) {
            float s[1] = {0.f};
#pragma unroll
            for (int e = 0; e < E; ++e)
                s[0] += u[e]; // invalid columns hold 0
            team_sum<LPR, TEAMS, 1>(s, red_lds, parity, team, wave_in_team, lane);
            mean = s[0] / float(N);
            float d[1] = {0.f};
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                if (cvalid[k]) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const float z = u[k * VEC + e] - mean;
                        d[0] += z * z;
                    }
                }
            }
            team_sum<LPR, TEAMS, 1>(d, red_lds, parity, team, wave_in_team, lane);
            rstd = rsqrtf(d[0] / float(N) + a.eps);
        } else {
            float s[1] = {0.f};
#pragma unroll
            for (int e = 0; e < E; ++e)
                s[0] += u[e] * u[e];
            team_sum<LPR, TEAMS, 1>(s, red_lds, parity, team, wave_in_team, lane);
            rstd = rsqrtf(s[0] / float(N) + a.eps);
        }

        // normalise, affine, store, amax
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int c0 = (k * LPR + tl) * VEC;
            const bool ok = rv && cvalid[k];
            float gv[VEC], bv[VEC], yv[VEC];
            IO::unpack(gamma_r[k], gv);
            IO::unpack(beta_r[k], bv);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                float n = (u[k * VEC + e] - mean) * rstd;
                if (has_gamma)
                    n *= gv[e];
                if (has_beta)
                    n += bv[e];
                yv[e] = n;
            }
            const Raw yr = IO::pack(yv);
            if (ok) {
                IO::store_raw(a.y, roff + c0, yr);
                float ys[VEC];
                IO::unpack(yr, ys);
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    lane_max = fmaxf(lane_max, fabsf(ys[e]));
            }
        }
        if (tl == 0 && rv) {
            if (a.mean)
                a.mean[row] = mean;
            if (a.rstd)
                a.rstd[row] = rstd;
        }
    }

    // amax, first stage: wave max, then the workgroup's waves through LDS;
    // second stage: one atomicMax per workgroup on the float's bit pattern
    // (non-negative floats order like their unsigned patterns).
    if (a.amax) {
        const float m = group_reduce<64, OpMax>(lane_max);
        if (lane == 0)
            max_lds[tid >> 6] = m;
        __syncthreads();
        if (tid == 0) {
            float mm = max_lds[0];
#pragma unroll
            for (int w = 1; w < NW; ++w)
                mm = fmaxf(mm, max_lds[w]);
            atomicMax(a.amax, __float_as_uint(mm));
        }
    }
}

// ---------------------------------------------------------------------------
// Backward stage 1 (mix-order): per row, one load of dy and x; the row
// reduction gives dx; the column reduction is accumulated in registers across
// the team's rows, folded over the workgroup in a fixed order and written as
// this workgroup's partial row of the workspace.
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
        float zero[VEC] = {};
        gamma_r[k] = (has_gamma && cvalid[k]) ? IO::load_raw(a.gamma, c0) : IO::pack(zero);
    }

    float acc_g[E], acc_b[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        acc_g[e] = 0.f;
        acc_b[e] = 0.f;
    }

    int parity = 0;
    const int64_t stride = (int64_t)gridDim.x * TEAMS;
    for (int64_t base = (int64_t)blockIdx.x * TEAMS; base < a.M; base += stride) {
        const int64_t row = base + team;
        const bool rv = row < a.M;
        const int64_t roff = row * (int64_t)N;

        float xv[E], dyv[E], g[E];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int c0 = (k * LPR + tl) * VEC;
            const bool ok = rv && cvalid[k];
            float *xk = &xv[k * VEC], *dk = &dyv[k * VEC];
            if (ok) {
                IO::unpack(IO::load_raw(a.x, roff + c0), xk);
                IO::unpack(IO::load_raw(a.dy, roff + c0), dk);
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    xk[e] = 0.f;
                    dk[e] = 0.f;
                }
            }
            float gv[VEC];
            IO::unpack(gamma_r[k], gv);
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                g[k * VEC + e] = has_gamma ? dk[e] * gv[e] : dk[e];
        }

        float mean = 0.f, rstd = 0.f, c1, c2 = 0.f;
        if constexpr (!RMS) {
            if (rv) {
                mean = a.mean[row];
                rstd = a.rstd[row];
            }
            float s[2] = {0.f, 0.f};
#pragma unroll
            for (int e = 0; e < E; ++e) {
                s[0] += g[e] * ((xv[e] - mean) * rstd); // invalid: g = 0
                s[1] += g[e];
            }
            team_sum<LPR, TEAMS, 2>(s, red_lds, parity, team, wave_in_team, lane);
            c1 = s[0] / float(N);
            c2 = s[1] / float(N);
        } else if (!recompute) {
            if (rv)
                rstd = a.rstd[row];
            float s[2] = {0.f, 0.f};
#pragma unroll
            for (int e = 0; e < E; ++e)
                s[0] += g[e] * (xv[e] * rstd);
            team_sum<LPR, TEAMS, 2>(s, red_lds, parity, team, wave_in_team, lane);
            c1 = s[0] / float(N);
        } else {
            // rstd from the same load: sum x^2 and sum g*x reduce together,
            // and mean(g*xhat) = rstd * mean(g*x)
            float s[2] = {0.f, 0.f};
#pragma unroll
            for (int e = 0; e < E; ++e) {
                s[0] += xv[e] * xv[e];
                s[1] += g[e] * xv[e];
            }
            team_sum<LPR, TEAMS, 2>(s, red_lds, parity, team, wave_in_team, lane);
            rstd = rsqrtf(s[0] / float(N) + a.eps);
            c1 = rstd * (s[1] / float(N));
        }

#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int c0 = (k * LPR + tl) * VEC;
            const bool ok = rv && cvalid[k];
            float dxv[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int i = k * VEC + e;
                const float xh = RMS ? xv[i] * rstd : (xv[i] - mean) * rstd;
                dxv[e] = rstd * (g[i] - c2 - xh * c1);
                if (ok) {
                    acc_g[i] += dyv[i] * xh;
                    acc_b[i] += dyv[i];
                }
            }
            if (ok)
                IO::store_raw(a.dx, roff + c0, IO::pack(dxv));
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
// Backward stage 2: dgamma_j = sum_g partial[g][j] (g ascending within each of
// 32 interleaved slices, slices added in order), then the down-cast.
// ---------------------------------------------------------------------------
constexpr int COLSUM_COLS = 32;
constexpr int COLSUM_SLICES = 32;

template <bool BF16_OUT>
__global__ void __launch_bounds__(COLSUM_COLS *COLSUM_SLICES)
    colsum_kernel(const float *ws, int G, int N, void *dgamma, void *dbeta)
{
    const int tx = threadIdx.x % COLSUM_COLS;
    const int ty = threadIdx.x / COLSUM_COLS;
    const int which = blockIdx.y;
    void *out = which == 0 ? dgamma : dbeta;
    if (out == nullptr)
        return; // uniform over the block
    const int j = blockIdx.x * COLSUM_COLS + tx;
    const float *part = ws + (int64_t)which * G * N;
    float s = 0.f;
    if (j < N) {
#pragma unroll 8
        for (int g = ty; g < G; g += COLSUM_SLICES)
            s += part[(int64_t)g * N + j];
    }
    __shared__ float sl[COLSUM_SLICES][COLSUM_COLS];
    sl[ty][tx] = s;
    __syncthreads();
    if (ty == 0 && j < N) {
        float t = sl[0][tx];
#pragma unroll
        for (int q = 1; q < COLSUM_SLICES; ++q)
            t += sl[q][tx];
        if constexpr (BF16_OUT)
            static_cast<uint16_t *>(out)[j] = uint16_t(pack_bf16x2(t, 0.f) & 0xffffu);
        else
            static_cast<float *>(out)[j] = t;
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

template <typename T, int VEC, int LPR, int VPL, int TEAMS, bool RMS>
int occupancy_fwd()
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void *>(&fwd_kernel<T, VEC, LPR, VPL, TEAMS, RMS>),
            LPR * TEAMS, 0) != hipSuccess)
        return 1;
    return n > 0 ? n : 1;
}

template <typename T, int VEC, int LPR, int VPL, int TEAMS, bool RMS>
int occupancy_bwd()
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void *>(&bwd_kernel<T, VEC, LPR, VPL, TEAMS, RMS>),
            LPR * TEAMS, 0) != hipSuccess)
        return 1;
    return n > 0 ? n : 1;
}

} // namespace nf
