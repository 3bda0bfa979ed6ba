// odd.hpp -- forward, softmax and backward kernels for rows whose length is
// an odd multiple of a unit of U elements (U = 1: odd N; U = 2: N = 2 mod 4;
// U = 4: N = 4 mod 8), read in aligned vectors of 2U elements.
//
// Row r of such an N starts at element r*N, a multiple of 2U for even r and
// an odd multiple of U for odd r.  With the tensors aligned to 2U elements,
// a row's elements from its first 2U-aligned one on group into aligned
// vectors of 2U: columns 0..N-U-1 of an even row, U..N-1 of an odd one,
// (N - U) / (2U) vectors either way.  The unit left over -- columns N-U..N-1
// of an even row, 0..U-1 of an odd one -- is read and written by itself, by
// the team's first lane.  The vectors are twice the width the row's length
// alone allows (bf16: 4, 8 or 16 bytes for U = 1, 2, 4; fp32: 8 or 16 for
// U = 1, 2).  A team of LPR lanes owns a row as in kernels.hpp: lane tl holds
// vectors j = k*LPR + tl, k < VPL, from the row's first aligned element on,
// so every access instruction of a wave covers one contiguous span.  Every
// access lies inside its row: no range check is relied on beyond the
// matrix's end.
//
// The columns a lane holds move by U with the row's parity, so the
// per-column vectors are staged in LDS per column and read U columns at a
// time (one aligned LDS read each: the columns of a unit start on a multiple
// of U).
#pragma once

#include "kernels.hpp"

namespace nf {

// Columns staged as fp32 up to this many (12 bytes a column for the three
// vectors); bf16 vectors past it, and those of the U = 1 kernels, as their
// 16-bit patterns (6 bytes a column).
constexpr int ODD_F32_STAGE_MAX = 4096;

template <typename T, int U, int PE>
using odd_stage_t =
    typename std::conditional<sizeof(T) == 2 && (U == 1 || PE > ODD_F32_STAGE_MAX + U), uint16_t,
                              float>::type;

// One per-column vector staged in LDS as S, one entry per column (neutral
// past N or where absent).  fetch() issues this thread's loads, put()
// converts and stores them (two phases, so that the first rows' loads go
// out between).
template <typename T, typename S, int PE, int WG>
struct OddStage {
    static constexpr int SI = (PE + WG - 1) / WG;
    typename VecIO<T, 1>::Raw r[SI];

    __device__ __forceinline__ void fetch(const void *src, int N, int tid)
    {
        const rsrc_t rs = make_rsrc(src, src ? uint32_t(N) * uint32_t(sizeof(T)) : 0u);
#pragma unroll
        for (int i = 0; i < SI; ++i) {
            const int c = tid + i * WG;
            r[i] = BufIO<T, 1>::load_cached(rs, c < N ? uint32_t(c) * uint32_t(sizeof(T)) : BUF_OOB);
        }
    }
    // zero_centred: the weight round_T(1 + v) of a zero-centred gamma
    __device__ __forceinline__ void put(S *dst, const void *src, int N, float neutral, int tid,
                                        bool zero_centred = false) const
    {
#pragma unroll
        for (int i = 0; i < SI; ++i) {
            const int c = tid + i * WG;
            if (c < PE) {
                float v;
                VecIO<T, 1>::unpack(r[i], &v);
                if (zero_centred)
                    VecIO<T, 1>::unpack(plus_one<T, 1>(&v), &v);
                v = src != nullptr && c < N ? v : neutral;
                if constexpr (sizeof(S) == 2)
                    dst[c] = uint16_t(__float_as_uint(v) >> 16); // exact: v is a bf16 value
                else
                    dst[c] = v;
            }
        }
    }
};

// The staged values of columns c .. c+U-1 (c a multiple of U), in one LDS
// read.
template <int U, typename S>
__device__ __forceinline__ void odd_params(const S *base, int c, float *out)
{
    if constexpr (sizeof(S) == 4) {
        if constexpr (U == 4) {
            const float4 v = *reinterpret_cast<const float4 *>(base + c);
            out[0] = v.x;
            out[1] = v.y;
            out[2] = v.z;
            out[3] = v.w;
        } else if constexpr (U == 2) {
            const float2 v = *reinterpret_cast<const float2 *>(base + c);
            out[0] = v.x;
            out[1] = v.y;
        } else {
            out[0] = base[c];
        }
    } else {
        if constexpr (U == 4) {
            const uint2 w = *reinterpret_cast<const uint2 *>(base + c);
            out[0] = bf16_lo(w.x);
            out[1] = bf16_hi(w.x);
            out[2] = bf16_lo(w.y);
            out[3] = bf16_hi(w.y);
        } else if constexpr (U == 2) {
            const uint32_t w = *reinterpret_cast<const uint32_t *>(base + c);
            out[0] = bf16_lo(w);
            out[1] = bf16_hi(w);
        } else {
            out[0] = __uint_as_float(uint32_t(base[c]) << 16);
        }
    }
}

// Whether the forward keeps the next row group's loads in flight (wide
// teams, as fwd_prefetch; the per-column vectors are always in LDS).
template <typename T, int U, int LPR, int VPL, int TEAMS>
constexpr bool odd_prefetch()
{
    constexpr int raw = 2 * U * int(sizeof(T)) / 4;
    constexpr int waves_per_simd = (LPR * TEAMS / 64 + 3) / 4;
    constexpr int share = 512 / waves_per_simd;
    return LPR >= WIDE_LPR && 4 * VPL * raw + 28 <= share;
}

// Where a lane's accesses of one row group go: the byte offsets of its
// vectors and of the leftover unit (lane 0 of the team only; BUF_OOB
// elsewhere) inside the group, and the first column of its vector k = 0
// and of the leftover.
template <typename T, int U, int LPR, int VPL>
struct OddRow {
    uint32_t off[VPL], off1;
    int c0, c1;
    __device__ __forceinline__ OddRow(int team, int tl, int N, int64_t row)
    {
        const int par = int(row & 1);
        const int nv = (N - U) / (2 * U);
        c0 = par * U + 2 * U * tl;
        c1 = par ? 0 : N - U;
        const uint32_t base = uint32_t(team) * uint32_t(N);
#pragma unroll
        for (int k = 0; k < VPL; ++k)
            off[k] = k * LPR + tl < nv
                         ? (base + uint32_t(c0 + 2 * U * k * LPR)) * uint32_t(sizeof(T))
                         : BUF_OOB;
        off1 = tl == 0 ? (base + uint32_t(c1)) * uint32_t(sizeof(T)) : BUF_OOB;
    }
};

// LDS rows of the three staged per-column vectors, each on a 16-byte
// boundary (the U = 4 reads of fp32 are 16 bytes).
template <typename S, int PE>
struct OddRows {
    static constexpr int STRIDE = (PE + 7) & ~7;
    static constexpr int SIZE = 3 * STRIDE;
};

// ---------------------------------------------------------------------------
// Forward: as fwd_kernel -- t = (x + bias) + residual, u = round(t) ->
// residual_out, two-pass statistics of u from registers (the mean as an
// fp32 pair), y = normalise(u) * gamma + beta -> y (or FP8 codes), running
// max |y| -- on the row's vectors plus its leftover unit.
// ---------------------------------------------------------------------------
template <typename T, int U, int LPR, int VPL, int TEAMS, bool RMS, bool F8>
__global__ void __launch_bounds__(LPR *TEAMS) fwd_odd_kernel(const FwdArgs a)
{
    constexpr int VE = 2 * U; // elements per vector
    using IO = VecIO<T, VE>;
    using BIO = BufIO<T, VE>;
    using IO1 = VecIO<T, U>;
    using BIO1 = BufIO<T, U>;
    using Raw = typename IO::Raw;
    using Raw1 = typename IO1::Raw;
    using Acc = typename std::conditional<std::is_same<T, float>::value, double, float>::type;
    constexpr int WG = LPR * TEAMS;
    constexpr int PE = VE * LPR * VPL + U; // columns staged: the longest row
    constexpr bool PREFETCH = odd_prefetch<T, U, LPR, VPL, TEAMS>();
    using S = odd_stage_t<T, U, PE>;
    using Stage = OddStage<T, S, PE, WG>;
    using Rows = OddRows<S, PE>;
    static_assert(WG % 64 == 0, "workgroup of whole waves");

    __shared__ float red_lds[TeamLds<LPR, TEAMS, 1>::size];
    __shared__ double red_lds_f64[TeamLds<LPR, TEAMS, 1>::size];
    __shared__ float max_lds[WG / 64];
    __shared__ __attribute__((aligned(16))) S par[Rows::SIZE];
    S *const pb = par, *const pg = par + Rows::STRIDE, *const pe = par + 2 * Rows::STRIDE;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int team = tid / LPR;
    const int tl = tid % LPR;
    const int wave_in_team = LPR > 64 ? tl / 64 : 0;
    const int N = a.N;
    const bool has_res = a.res != nullptr;
    const bool fused_add = a.bias != nullptr || has_res;
    const float y_scale = F8 ? *a.y_scale : 1.f;

    Raw xn[VPL], rn[VPL];
    Raw1 xn1, rn1;
    auto issue = [&](int64_t g) {
        const RowGroup rg(g, TEAMS, a.M, N, sizeof(T));
        const OddRow<T, U, LPR, VPL> o(team, tl, N, rg.r0 + team);
        const rsrc_t xs = make_rsrc(static_cast<const char *>(a.x) + rg.byte0, rg.bytes);
        const rsrc_t rs = make_rsrc(has_res ? static_cast<const char *>(a.res) + rg.byte0 : nullptr,
                                    has_res ? rg.bytes : 0u);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            xn[k] = BIO::load(xs, o.off[k]);
            rn[k] = has_res ? BIO::load(rs, o.off[k]) : IO::zero();
        }
        xn1 = BIO1::load(xs, o.off1);
        rn1 = has_res ? BIO1::load(rs, o.off1) : IO1::zero();
    };
    const GroupWalk walk(a.K, a.A);
    {
        Stage sb, sg, se;
        sb.fetch(a.bias, N, tid);
        sg.fetch(a.gamma, N, tid);
        se.fetch(a.beta, N, tid);
        issue(walk.group(0));
        sb.put(pb, a.bias, N, 0.f, tid);
        sg.put(pg, a.gamma, N, 1.f, tid, a.zero_centred);
        se.put(pe, a.beta, N, 0.f, tid);
        __syncthreads();
    }
    const int nv = (N - U) / (2 * U);

    float lane_max = 0.f;
    int parity = 0;
    for (int kk = 0; kk < a.K; ++kk) {
        const int64_t grp = walk.group(kk);
        if (grp >= a.n_groups)
            break; // uniform over the workgroup
        const RowGroup rg(grp, TEAMS, a.M, N, sizeof(T));
        const int64_t row = rg.r0 + team;
        const bool rv = row < a.M;
        const bool wt = grp >= a.wt_group;
        if (!PREFETCH && kk > 0)
            issue(grp);
        Raw ur[VPL], rr[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            ur[k] = xn[k];
            rr[k] = rn[k];
        }
        Raw1 ur1 = xn1;
        const Raw1 rr1 = rn1;
        const int64_t next = walk.group(kk + 1);
        if (PREFETCH && kk + 1 < a.K && next < a.n_groups)
            issue(next);
        const OddRow<T, U, LPR, VPL> o(team, tl, N, row);

        // fused add and the row sum (fp64 for fp32 rows, as fwd_kernel);
        // vectors past the row and the leftover outside lane 0 take no part
        // (their x and residual read as zeros, but not the bias)
        Acc sum = Acc(0);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float t[VE];
            IO::unpack(ur[k], t);
            if (fused_add) {
                const int c = o.c0 + VE * k * LPR;
                float r[VE], bv[VE];
                IO::unpack(rr[k], r);
                odd_params<U>(pb, c, bv);
                odd_params<U>(pb, c + U, bv + U);
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    t[e] = (t[e] + bv[e]) + r[e];
                ur[k] = IO::pack(t);
                IO::unpack(ur[k], t);
            }
            if constexpr (!RMS) {
                if (k * LPR + tl < nv) {
#pragma unroll
                    for (int e = 0; e < VE; ++e)
                        sum += Acc(t[e]);
                }
            }
        }
        {
            float t[U];
            IO1::unpack(ur1, t);
            if (fused_add) {
                float r[U], bv[U];
                IO1::unpack(rr1, r);
                odd_params<U>(pb, o.c1, bv);
#pragma unroll
                for (int e = 0; e < U; ++e)
                    t[e] = (t[e] + bv[e]) + r[e];
                ur1 = IO1::pack(t);
                IO1::unpack(ur1, t);
            }
            if constexpr (!RMS) {
                if (tl == 0) {
#pragma unroll
                    for (int e = 0; e < U; ++e)
                        sum += Acc(t[e]);
                }
            }
        }
        if (a.res_out) {
            const rsrc_t os = make_rsrc(static_cast<char *>(a.res_out) + rg.byte0, rg.bytes);
#pragma unroll
            for (int k = 0; k < VPL; ++k)
                BIO::store(os, o.off[k], ur[k], wt);
            BIO1::store(os, o.off1, ur1, wt);
        }

        // statistics (as fwd_kernel: LayerNorm keeps the mean as an fp32
        // pair mean + lo)
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
        }
#pragma unroll
        for (int k = 0; k < VPL; ++k)
            reload_barrier(ur[k]);
        float d2[1] = {0.f};
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            if (k * LPR + tl < nv) {
                float u[VE];
                IO::unpack(ur[k], u);
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    const float d = u[e] - mean;
                    d2[0] = fmaf(d, d, d2[0]);
                }
            }
        }
        if (tl == 0) {
            float u[U];
            IO1::unpack(ur1, u);
#pragma unroll
            for (int e = 0; e < U; ++e) {
                const float d = u[e] - mean;
                d2[0] = fmaf(d, d, d2[0]);
            }
        }
        team_sum<LPR, TEAMS, 1>(d2, red_lds, parity, team, wave_in_team, lane);
        if constexpr (RMS)
            rstd = rsqrtf(d2[0] / float(N) + a.eps);
        else
            rstd = rsqrtf(fmaxf(d2[0] / float(N) - lo * lo, 0.f) + a.eps);
        const float lo_r = -lo * rstd;

        // normalise, affine, store; amax over |y| before rounding (as
        // fwd_kernel: rounding is monotone)
#pragma unroll
        for (int k = 0; k < VPL; ++k)
            reload_barrier(ur[k]);
        const rsrc_t ys = F8 ? make_rsrc(static_cast<char *>(a.y) + rg.byte0 / int64_t(sizeof(T)),
                                         rg.bytes / uint32_t(sizeof(T)))
                             : make_rsrc(static_cast<char *>(a.y) + rg.byte0, rg.bytes);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int c = o.c0 + VE * k * LPR;
            float u[VE], gv[VE], bv[VE], yv[VE];
            IO::unpack(ur[k], u);
            odd_params<U>(pg, c, gv);
            odd_params<U>(pg, c + U, gv + U);
            odd_params<U>(pe, c, bv);
            odd_params<U>(pe, c + U, bv + U);
#pragma unroll
            for (int e = 0; e < VE; ++e)
                yv[e] = fmaf(fmaf(u[e] - mean, rstd, lo_r), gv[e], bv[e]);
            if constexpr (F8) {
                float q[VE];
                IO::unpack(IO::pack(yv), q);
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    q[e] *= y_scale;
                store_e4m3<VE>(ys, o.off[k] == BUF_OOB ? BUF_OOB : o.off[k] / uint32_t(sizeof(T)),
                               q, wt);
            } else {
                BIO::store(ys, o.off[k], IO::pack(yv), wt);
            }
            if (rv && k * LPR + tl < nv) {
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    lane_max = fmaxf(lane_max, fabsf(yv[e]));
            }
        }
        if (tl == 0) {
            float u[U], gv[U], bv[U], yv[U];
            IO1::unpack(ur1, u);
            odd_params<U>(pg, o.c1, gv);
            odd_params<U>(pe, o.c1, bv);
#pragma unroll
            for (int e = 0; e < U; ++e)
                yv[e] = fmaf(fmaf(u[e] - mean, rstd, lo_r), gv[e], bv[e]);
            if constexpr (F8) {
                float q[U];
                IO1::unpack(IO1::pack(yv), q);
#pragma unroll
                for (int e = 0; e < U; ++e)
                    q[e] *= y_scale;
                store_e4m3<U>(ys, o.off1 / uint32_t(sizeof(T)), q, wt);
            } else {
                BIO1::store(ys, o.off1, IO1::pack(yv), wt);
            }
            if (rv) {
#pragma unroll
                for (int e = 0; e < U; ++e)
                    lane_max = fmaxf(lane_max, fabsf(yv[e]));
                if (a.mean)
                    a.mean[row] = mean;
                if (a.rstd)
                    a.rstd[row] = rstd;
            }
        }
    }

    // amax, as fwd_kernel
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
            const unsigned bits = __float_as_uint(r[0]);
            if (a.amax_ws == nullptr)
                atomicMax(a.amax, bits); // *amax was zeroed by a kernel before this one
            else
                amax_arrive(a.amax, a.amax_ws, bits);
        }
    }
}

template <typename T, int U, int LPR, int VPL, int TEAMS, bool RMS, bool F8>
hipError_t launch_fwd_odd(const FwdArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((fwd_odd_kernel<T, U, LPR, VPL, TEAMS, RMS, F8>), dim3(grid),
                       dim3(LPR * TEAMS), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row softmax: as softmax_kernel, on the row's vectors plus its leftover
// unit.
// ---------------------------------------------------------------------------
template <typename T, int U, int LPR, int VPL, int TEAMS>
__global__ void __launch_bounds__(LPR *TEAMS) softmax_odd_kernel(const SoftmaxArgs a)
{
    constexpr int VE = 2 * U;
    using IO = VecIO<T, VE>;
    using BIO = BufIO<T, VE>;
    using IO1 = VecIO<T, U>;
    using BIO1 = BufIO<T, U>;
    using Raw = typename IO::Raw;
    constexpr int WG = LPR * TEAMS;
    static_assert(WG % 64 == 0, "workgroup of whole waves");

    __shared__ float red_lds[TeamLds<LPR, TEAMS, 1>::size];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int team = tid / LPR;
    const int tl = tid % LPR;
    const int wave_in_team = LPR > 64 ? tl / 64 : 0;
    const int N = a.N;
    const int nv = (N - U) / (2 * U);

    int parity = 0;
    const GroupWalk walk(a.K, a.A);
    for (int kk = 0; kk < a.K; ++kk) {
        const int64_t grp = walk.group(kk);
        if (grp >= a.n_groups)
            break; // uniform over the workgroup
        const RowGroup rg(grp, TEAMS, a.M, N, sizeof(T));
        const OddRow<T, U, LPR, VPL> o(team, tl, N, rg.r0 + team);
        const bool wt = grp >= a.wt_group;
        const rsrc_t xs = make_rsrc(static_cast<const char *>(a.x) + rg.byte0, rg.bytes);
        Raw xr[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k)
            xr[k] = BIO::load(xs, o.off[k]);
        float x1[U];
        IO1::unpack(BIO1::load(xs, o.off1), x1);

        // row max (vectors past the row and the leftover outside lane 0
        // take no part)
        float m[1] = {-INFINITY};
        if (tl == 0) {
#pragma unroll
            for (int e = 0; e < U; ++e)
                m[0] = fmaxf(m[0], x1[e]);
        }
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            if (k * LPR + tl < nv) {
                float v[VE];
                IO::unpack(xr[k], v);
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    m[0] = fmaxf(m[0], v[e]);
            }
        }
        team_reduce<LPR, TEAMS, 1, OpMax>(m, red_lds, parity, team, wave_in_team, lane);

        float ev[VPL][VE], e1[U];
        float sum[1] = {0.f};
#pragma unroll
        for (int e = 0; e < U; ++e) {
            e1[e] = tl == 0 ? __expf(x1[e] - m[0]) : 0.f;
            sum[0] += e1[e];
        }
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float v[VE];
            IO::unpack(xr[k], v);
            const bool ok = k * LPR + tl < nv;
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                ev[k][e] = ok ? __expf(v[e] - m[0]) : 0.f;
                sum[0] += ev[k][e];
            }
        }
        team_sum<LPR, TEAMS, 1>(sum, red_lds, parity, team, wave_in_team, lane);
        const float inv = 1.f / sum[0];

        const rsrc_t ys = make_rsrc(static_cast<char *>(a.y) + rg.byte0, rg.bytes);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
#pragma unroll
            for (int e = 0; e < VE; ++e)
                ev[k][e] *= inv;
            BIO::store(ys, o.off[k], IO::pack(ev[k]), wt);
        }
#pragma unroll
        for (int e = 0; e < U; ++e)
            e1[e] *= inv;
        BIO1::store(ys, o.off1, IO1::pack(e1), wt);
    }
}

template <typename T, int U, int LPR, int VPL, int TEAMS>
hipError_t launch_softmax_odd(const SoftmaxArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((softmax_odd_kernel<T, U, LPR, VPL, TEAMS>), dim3(grid), dim3(LPR * TEAMS),
                       0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Backward stage 1: as bwd_kernel (one load of dy and x per row, the row
// sums give dx, the column sums are accumulated over the workgroup's rows
// and written as its partial row), on the row's vectors plus its leftover
// unit.  Workgroups hold an even number of teams and row groups start on
// even rows, so each team keeps one row parity and with it one set of
// columns for its whole walk: its column sums stay in registers, one per
// element as in bwd_kernel (plus the leftover's on the team's first lane).
// The teams' sums meet in LDS by column, added in team order, and the
// workgroup stores the partial row from there.
// ---------------------------------------------------------------------------
template <typename T, int U, int LPR, int VPL, int TEAMS, bool RMS, bool DB>
__global__ void __launch_bounds__(LPR *TEAMS) bwd_odd_kernel(const BwdArgs a)
{
    constexpr int VE = 2 * U;
    using IO = VecIO<T, VE>;
    using BIO = BufIO<T, VE>;
    using IO1 = VecIO<T, U>;
    using BIO1 = BufIO<T, U>;
    using Raw = typename IO::Raw;
    using Raw1 = typename IO1::Raw;
    constexpr int WG = LPR * TEAMS;
    constexpr int PE = VE * LPR * VPL + U; // columns staged: the longest row
    constexpr int NB = DB ? 3 : 2;         // column sums: dgamma, dbeta (, dbias)
    using S = odd_stage_t<T, U, PE>;
    using Stage = OddStage<T, S, PE, WG>;
    static_assert(TEAMS % 2 == 0, "each team keeps one row parity");
    static_assert(WG % 64 == 0, "workgroup of whole waves");

    __shared__ float red_lds[TeamLds<LPR, TEAMS, 2>::size];
    __shared__ __attribute__((aligned(16))) S par[(PE + 7) & ~7];
    __shared__ float col_lds[NB * PE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int team = tid / LPR;
    const int tl = tid % LPR;
    const int wave_in_team = LPR > 64 ? tl / 64 : 0;
    const int N = a.N;
    const int nv = (N - U) / (2 * U);
    const bool recompute = RMS && a.rstd == nullptr;
    // rows r0 + team with r0 even: the team's parity is its own
    const OddRow<T, U, LPR, VPL> o(team, tl, N, team);

    Raw xr[VPL], dr[VPL];
    Raw1 x1, d1;
    float mean = 0.f, rstd = 0.f;
    auto issue = [&](int64_t g) {
        const RowGroup rg(g, TEAMS, a.M, N, sizeof(T));
        const rsrc_t xs = make_rsrc(static_cast<const char *>(a.x) + rg.byte0, rg.bytes);
        const rsrc_t ds = make_rsrc(static_cast<const char *>(a.dy) + rg.byte0, rg.bytes);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            xr[k] = BIO::load(xs, o.off[k]);
            dr[k] = BIO::load(ds, o.off[k]);
        }
        x1 = BIO1::load(xs, o.off1);
        d1 = BIO1::load(ds, o.off1);
        mean = RMS ? 0.f : row_stat(a.mean, rg, team);
        rstd = recompute ? 0.f : row_stat(a.rstd, rg, team);
    };
    const GroupWalk walk(a.K, a.A);
    {
        Stage sg;
        sg.fetch(a.gamma, N, tid);
        issue(walk.group(0));
        sg.put(par, a.gamma, N, 1.f, tid, a.zero_centred);
        __syncthreads();
    }

    float ag[VPL][VE], ab[VPL][VE], ad[DB ? VPL : 1][VE];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            ag[k][e] = 0.f;
            ab[k][e] = 0.f;
            if constexpr (DB)
                ad[k][e] = 0.f;
        }
    }
    float a1g[U], a1b[U], a1d[U]; // the leftover's columns (team's first lane)
#pragma unroll
    for (int e = 0; e < U; ++e)
        a1g[e] = a1b[e] = a1d[e] = 0.f;
    int parity = 0;

    for (int kk = 0; kk < a.K; ++kk) {
        const int64_t grp = walk.group(kk);
        if (grp >= a.n_groups)
            break; // uniform over the workgroup; later groups are larger
        if (kk > 0)
            issue(grp); // group 0 was issued before gamma was staged
        const RowGroup rg(grp, TEAMS, a.M, N, sizeof(T));
        const bool rv = rg.r0 + team < a.M;
        // this lane's columns, opaque to the compiler on each group: gamma
        // is read from LDS where it is used, not hoisted out of the walk
        // into registers (32 more for 16 pairs per lane)
        int cb = o.c0, cl = o.c1;
        reload_barrier(cb);
        reload_barrier(cl);

        // Row sums, g = dy * gamma (vectors past the row and the leftover
        // outside the first lane read dy = 0, so g = 0):
        //   LN : s0 = sum g (x - mean), s1 = sum g
        //   RMS: s0 = sum g x; without rstd also s1 = sum x^2
        float s[2] = {0.f, 0.f};
        auto row_sums = [&](float xv, float dv, float gm) {
            const float g = dv * gm;
            if constexpr (!RMS) {
                s[0] = fmaf(g, xv - mean, s[0]);
                s[1] += g;
            } else {
                s[0] = fmaf(g, xv, s[0]);
                if (recompute)
                    s[1] = fmaf(xv, xv, s[1]);
            }
        };
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int c = cb + VE * k * LPR;
            float xv[VE], dv[VE], gv[VE];
            IO::unpack(xr[k], xv);
            IO::unpack(dr[k], dv);
            odd_params<U>(par, c, gv);
            odd_params<U>(par, c + U, gv + U);
#pragma unroll
            for (int e = 0; e < VE; ++e)
                row_sums(xv[e], dv[e], gv[e]);
        }
        {
            float xv[U], dv[U], gv[U];
            IO1::unpack(x1, xv);
            IO1::unpack(d1, dv);
            odd_params<U>(par, cl, gv);
#pragma unroll
            for (int e = 0; e < U; ++e)
                row_sums(xv[e], dv[e], gv[e]);
        }
        team_sum<LPR, TEAMS, 2>(s, red_lds, parity, team, wave_in_team, lane);
        if (recompute)
            rstd = rsqrtf(s[1] / float(N) + a.eps);
        // dx = rstd (g - c2 - xhat c1) = fma(xhat, -rstd c1, fma(g, rstd, -rstd c2))
        const float c1 = rstd * (s[0] / float(N));
        const float c2 = RMS ? 0.f : s[1] / float(N);
        const float k1 = -rstd * c1, k2 = -rstd * c2;
        // dx of one element; its column sums when the row is valid (the
        // sums of vectors past the row are never stored)
        auto grad = [&](float xv, float dv, float gm, float &sg, float &sb, float &sd) {
            const float xh = RMS ? xv * rstd : (xv - mean) * rstd;
            const float dxv = fmaf(xh, k1, fmaf(dv * gm, rstd, k2));
            if (rv) {
                sg = fmaf(dv, xh, sg);
                sb += dv;
                if constexpr (DB)
                    sd += dxv;
            }
            return dxv;
        };

#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            reload_barrier(xr[k]);
            reload_barrier(dr[k]);
        }
        const rsrc_t dxs = make_rsrc(static_cast<char *>(a.dx) + rg.byte0, rg.bytes);
        const bool wt = grp >= a.wt_group;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int c = cb + VE * k * LPR;
            float xv[VE], dv[VE], gv[VE], dxv[VE], unused = 0.f;
            IO::unpack(xr[k], xv);
            IO::unpack(dr[k], dv);
            odd_params<U>(par, c, gv);
            odd_params<U>(par, c + U, gv + U);
#pragma unroll
            for (int e = 0; e < VE; ++e)
                dxv[e] = grad(xv[e], dv[e], gv[e], ag[k][e], ab[k][e],
                              DB ? ad[DB ? k : 0][e] : unused);
            BIO::store(dxs, o.off[k], IO::pack(dxv), wt);
        }
        {
            float xv[U], dv[U], gv[U], dxv[U];
            IO1::unpack(x1, xv);
            IO1::unpack(d1, dv);
            odd_params<U>(par, cl, gv);
#pragma unroll
            for (int e = 0; e < U; ++e)
                dxv[e] = grad(xv[e], dv[e], gv[e], a1g[e], a1b[e], a1d[e]);
            BIO1::store(dxs, o.off1, IO1::pack(dxv), wt);
        }
    }

    // ---- fold the teams' column sums in LDS by column, in team order ----
    // Every team covers every column (its vectors and its leftover), so
    // team 0 writes each column and the others add to it.
    for (int t = 0; t < TEAMS; ++t) {
        if (team == t) {
            auto put = [&](int b, int c, float v) {
                float &dst = col_lds[b * PE + c];
                dst = t == 0 ? v : dst + v;
            };
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                if (k * LPR + tl < nv) {
                    const int c = o.c0 + VE * k * LPR;
#pragma unroll
                    for (int e = 0; e < VE; ++e) {
                        put(0, c + e, ag[k][e]);
                        put(1, c + e, ab[k][e]);
                        if constexpr (DB)
                            put(2, c + e, ad[k][e]);
                    }
                }
            }
            if (tl == 0) {
#pragma unroll
                for (int e = 0; e < U; ++e) {
                    put(0, o.c1 + e, a1g[e]);
                    put(1, o.c1 + e, a1b[e]);
                    if constexpr (DB)
                        put(2, o.c1 + e, a1d[e]);
                }
            }
        }
        __syncthreads();
    }
    // Block b of the workspace (dgamma, dbeta, dbias) holds row blockIdx.x.
    const int64_t ld = colsum_ld(N);
    for (int c = tid; c < N; c += WG) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
            a.ws[((int64_t)b * gridDim.x + blockIdx.x) * ld + c] = col_lds[b * PE + c];
    }
}

template <typename T, int U, int LPR, int VPL, int TEAMS, bool RMS, bool DB>
hipError_t launch_bwd_odd(const BwdArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((bwd_odd_kernel<T, U, LPR, VPL, TEAMS, RMS, DB>), dim3(grid),
                       dim3(LPR * TEAMS), 0, s, a);
    return hipGetLastError();
}

} // namespace nf
