// odd.hpp -- forward, softmax and backward kernels for rows of an odd
// number of elements, read in aligned pairs.
//
// Row r of an odd length N starts at element r*N, which is even for even r
// and odd for odd r.  With the tensors aligned to two elements, a row's
// elements from its first even one on pair up into aligned two-element
// accesses (4 bytes for bf16, 8 for fp32): columns 0..N-2 of an even row and
// columns 1..N-1 of an odd one, (N - 1) / 2 pairs either way.  The one
// element left over -- column N-1 of an even row, column 0 of an odd one --
// is read and written by itself, by the team's first lane.  A team of LPR
// lanes owns a row as in kernels.hpp: lane tl holds pairs j = k*LPR + tl,
// k < VPL, starting at the row's parity (its first even element), so every
// access instruction of a wave covers one contiguous span.  Every access
// lies inside its row: no range check is relied on beyond the matrix's end.
//
// Against the single-element kernels this halves the access instructions
// and keeps the per-element work of the paired (4-byte) kernels; the price
// is the per-row parity of the columns a lane holds, so the per-column
// vectors are staged in LDS, read per column (two 16-bit or 32-bit LDS
// reads per pair, the pair's first column being odd in odd rows).
#pragma once

#include "kernels.hpp"

namespace nf {

// One per-column vector staged in LDS, one entry per column (neutral past N
// or where absent): bf16 vectors as their 16-bit patterns, fp32 ones as
// floats.  fetch() issues this thread's loads, put() converts and stores
// them (two phases, so that the first rows' loads go out between).
template <typename T, int PE, int WG>
struct OddStage {
    using S = typename std::conditional<sizeof(T) == 2, uint16_t, float>::type;
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
                if constexpr (sizeof(T) == 2)
                    dst[c] = uint16_t(__float_as_uint(v) >> 16); // exact: v is a bf16 value
                else
                    dst[c] = v;
            }
        }
    }
};

// The staged value of column c.
template <typename S>
__device__ __forceinline__ float odd_param(const S *base, int c)
{
    if constexpr (sizeof(S) == 2)
        return __uint_as_float(uint32_t(base[c]) << 16);
    else
        return base[c];
}

// Whether the odd-row forward keeps the next row group's loads in flight
// (wide teams, as fwd_prefetch; the per-column vectors are always in LDS).
template <typename T, int LPR, int VPL, int TEAMS>
constexpr bool odd_prefetch()
{
    constexpr int raw = 2 * int(sizeof(T)) / 4;
    constexpr int waves_per_simd = (LPR * TEAMS / 64 + 3) / 4;
    constexpr int share = 512 / waves_per_simd;
    return LPR >= WIDE_LPR && 4 * VPL * raw + 28 <= share;
}

// Where a lane's accesses of one row group go: the byte offsets of its pairs
// and of the leftover element (lane 0 of the team only; BUF_OOB elsewhere)
// inside the group, and the column of its pair k = 0 and of the leftover.
template <typename T, int LPR, int VPL>
struct OddRow {
    uint32_t off[VPL], off1;
    int c0, c1;
    __device__ __forceinline__ OddRow(int team, int tl, int N, int64_t row)
    {
        const int par = int(row & 1);
        const int np = (N - 1) / 2;
        c0 = par + 2 * tl;
        c1 = par ? 0 : N - 1;
        const uint32_t base = uint32_t(team) * uint32_t(N);
#pragma unroll
        for (int k = 0; k < VPL; ++k)
            off[k] = k * LPR + tl < np ? (base + uint32_t(c0 + 2 * k * LPR)) * uint32_t(sizeof(T))
                                       : BUF_OOB;
        off1 = tl == 0 ? (base + uint32_t(c1)) * uint32_t(sizeof(T)) : BUF_OOB;
    }
};

// ---------------------------------------------------------------------------
// Forward on rows of an odd length: as fwd_kernel -- t = (x + bias) +
// residual, u = round(t) -> residual_out, two-pass statistics of u from
// registers (the mean as an fp32 pair), y = normalise(u) * gamma + beta -> y
// (or FP8 codes), running max |y| -- on pairs plus the leftover element.
// ---------------------------------------------------------------------------
template <typename T, int LPR, int VPL, int TEAMS, bool RMS, bool F8>
__global__ void __launch_bounds__(LPR *TEAMS) fwd_odd_kernel(const FwdArgs a)
{
    using IO = VecIO<T, 2>;
    using BIO = BufIO<T, 2>;
    using IO1 = VecIO<T, 1>;
    using BIO1 = BufIO<T, 1>;
    using Raw = typename IO::Raw;
    using Raw1 = typename IO1::Raw;
    using Acc = typename std::conditional<std::is_same<T, float>::value, double, float>::type;
    constexpr int WG = LPR * TEAMS;
    constexpr int PE = 2 * LPR * VPL + 1; // columns staged: the longest row
    constexpr bool PREFETCH = odd_prefetch<T, LPR, VPL, TEAMS>();
    using Stage = OddStage<T, PE, WG>;
    using S = typename Stage::S;
    static_assert(WG % 64 == 0, "workgroup of whole waves");

    __shared__ float red_lds[TeamLds<LPR, TEAMS, 1>::size];
    __shared__ double red_lds_f64[TeamLds<LPR, TEAMS, 1>::size];
    __shared__ float max_lds[WG / 64];
    __shared__ __attribute__((aligned(16))) S par[3 * PE];

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
        const OddRow<T, LPR, VPL> o(team, tl, N, rg.r0 + team);
        const rsrc_t xs = make_rsrc(static_cast<const char *>(a.x) + rg.byte0, rg.bytes);
        const rsrc_t rs = make_rsrc(has_res ? static_cast<const char *>(a.res) + rg.byte0 : nullptr,
                                    has_res ? rg.bytes : 0u);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            xn[k] = BIO::load(xs, o.off[k]);
            rn[k] = has_res ? BIO::load(rs, o.off[k]) : IO::zero();
        }
        xn1 = BIO1::load(xs, o.off1);
        rn1 = has_res ? BIO1::load(rs, o.off1) : Raw1(0);
    };
    const GroupWalk walk(a.K, a.A);
    {
        Stage sb, sg, se;
        sb.fetch(a.bias, N, tid);
        sg.fetch(a.gamma, N, tid);
        se.fetch(a.beta, N, tid);
        issue(walk.group(0));
        sb.put(par, a.bias, N, 0.f, tid);
        sg.put(par + PE, a.gamma, N, 1.f, tid, a.zero_centred);
        se.put(par + 2 * PE, a.beta, N, 0.f, tid);
        __syncthreads();
    }
    const int np = (N - 1) / 2;

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
        const OddRow<T, LPR, VPL> o(team, tl, N, row);

        // fused add and the row sum (fp64 for fp32 rows, as fwd_kernel);
        // pairs past the row and the leftover outside lane 0 take no part
        // (their x and residual read as zeros, but not the bias)
        Acc sum = Acc(0);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float t[2];
            IO::unpack(ur[k], t);
            if (fused_add) {
                const int c = o.c0 + 2 * k * LPR;
                float r[2];
                IO::unpack(rr[k], r);
                t[0] = (t[0] + odd_param(par, c)) + r[0];
                t[1] = (t[1] + odd_param(par, c + 1)) + r[1];
                ur[k] = IO::pack(t);
                IO::unpack(ur[k], t);
            }
            if constexpr (!RMS)
                if (k * LPR + tl < np)
                    sum += Acc(t[0]) + Acc(t[1]);
        }
        {
            float t[1];
            IO1::unpack(ur1, t);
            if (fused_add) {
                float r[1];
                IO1::unpack(rr1, r);
                t[0] = (t[0] + odd_param(par, o.c1)) + r[0];
                ur1 = IO1::pack(t);
                IO1::unpack(ur1, t);
            }
            if constexpr (!RMS)
                if (tl == 0)
                    sum += Acc(t[0]);
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
            if (k * LPR + tl < np) {
                float u[2];
                IO::unpack(ur[k], u);
                const float e0 = u[0] - mean, e1 = u[1] - mean;
                d2[0] = fmaf(e0, e0, fmaf(e1, e1, d2[0]));
            }
        }
        if (tl == 0) {
            float u[1];
            IO1::unpack(ur1, u);
            const float e = u[0] - mean;
            d2[0] = fmaf(e, e, d2[0]);
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
            const int c = o.c0 + 2 * k * LPR;
            float u[2], yv[2];
            IO::unpack(ur[k], u);
#pragma unroll
            for (int e = 0; e < 2; ++e)
                yv[e] = fmaf(fmaf(u[e] - mean, rstd, lo_r), odd_param(par + PE, c + e),
                             odd_param(par + 2 * PE, c + e));
            if constexpr (F8) {
                float q[2];
                IO::unpack(IO::pack(yv), q);
                q[0] *= y_scale;
                q[1] *= y_scale;
                store_e4m3<2>(ys, o.off[k] == BUF_OOB ? BUF_OOB : o.off[k] / uint32_t(sizeof(T)), q,
                              wt);
            } else {
                BIO::store(ys, o.off[k], IO::pack(yv), wt);
            }
            if (rv && k * LPR + tl < np)
                lane_max = fmaxf(lane_max, fmaxf(fabsf(yv[0]), fabsf(yv[1])));
        }
        if (tl == 0) {
            float u[1], yv[1];
            IO1::unpack(ur1, u);
            yv[0] = fmaf(fmaf(u[0] - mean, rstd, lo_r), odd_param(par + PE, o.c1),
                         odd_param(par + 2 * PE, o.c1));
            if constexpr (F8) {
                float q[1];
                IO1::unpack(IO1::pack(yv), q);
                q[0] *= y_scale;
                store_e4m3<1>(ys, o.off1 / uint32_t(sizeof(T)), q, wt);
            } else {
                BIO1::store(ys, o.off1, IO1::pack(yv), wt);
            }
            if (rv)
                lane_max = fmaxf(lane_max, fabsf(yv[0]));
            if (rv) {
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
            IO1::unpack(IO1::pack(r), r); // max of the stored y
            const unsigned bits = __float_as_uint(r[0]);
            if (a.amax_ws == nullptr)
                atomicMax(a.amax, bits); // *amax was zeroed by a kernel before this one
            else
                amax_arrive(a.amax, a.amax_ws, bits);
        }
    }
}

template <typename T, int LPR, int VPL, int TEAMS, bool RMS, bool F8>
hipError_t launch_fwd_odd(const FwdArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((fwd_odd_kernel<T, LPR, VPL, TEAMS, RMS, F8>), dim3(grid),
                       dim3(LPR * TEAMS), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row softmax on rows of an odd length: as softmax_kernel, on pairs plus the
// leftover element.
// ---------------------------------------------------------------------------
template <typename T, int LPR, int VPL, int TEAMS>
__global__ void __launch_bounds__(LPR *TEAMS) softmax_odd_kernel(const SoftmaxArgs a)
{
    using IO = VecIO<T, 2>;
    using BIO = BufIO<T, 2>;
    using IO1 = VecIO<T, 1>;
    using BIO1 = BufIO<T, 1>;
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
    const int np = (N - 1) / 2;

    int parity = 0;
    const GroupWalk walk(a.K, a.A);
    for (int kk = 0; kk < a.K; ++kk) {
        const int64_t grp = walk.group(kk);
        if (grp >= a.n_groups)
            break; // uniform over the workgroup
        const RowGroup rg(grp, TEAMS, a.M, N, sizeof(T));
        const OddRow<T, LPR, VPL> o(team, tl, N, rg.r0 + team);
        const bool wt = grp >= a.wt_group;
        const rsrc_t xs = make_rsrc(static_cast<const char *>(a.x) + rg.byte0, rg.bytes);
        Raw xr[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k)
            xr[k] = BIO::load(xs, o.off[k]);
        float x1[1];
        IO1::unpack(BIO1::load(xs, o.off1), x1);

        // row max (pairs past the row and the leftover outside lane 0 take
        // no part)
        float m[1] = {tl == 0 ? x1[0] : -INFINITY};
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            if (k * LPR + tl < np) {
                float v[2];
                IO::unpack(xr[k], v);
                m[0] = fmaxf(m[0], fmaxf(v[0], v[1]));
            }
        }
        team_reduce<LPR, TEAMS, 1, OpMax>(m, red_lds, parity, team, wave_in_team, lane);

        float ev[VPL][2];
        float e1 = tl == 0 ? __expf(x1[0] - m[0]) : 0.f;
        float sum[1] = {e1};
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float v[2];
            IO::unpack(xr[k], v);
            const bool ok = k * LPR + tl < np;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                ev[k][e] = ok ? __expf(v[e] - m[0]) : 0.f;
                sum[0] += ev[k][e];
            }
        }
        team_sum<LPR, TEAMS, 1>(sum, red_lds, parity, team, wave_in_team, lane);
        const float inv = 1.f / sum[0];

        const rsrc_t ys = make_rsrc(static_cast<char *>(a.y) + rg.byte0, rg.bytes);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            ev[k][0] *= inv;
            ev[k][1] *= inv;
            BIO::store(ys, o.off[k], IO::pack(ev[k]), wt);
        }
        e1 *= inv;
        BIO1::store(ys, o.off1, IO1::pack(&e1), wt);
    }
}

template <typename T, int LPR, int VPL, int TEAMS>
hipError_t launch_softmax_odd(const SoftmaxArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((softmax_odd_kernel<T, LPR, VPL, TEAMS>), dim3(grid), dim3(LPR * TEAMS),
                       0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Backward stage 1 on rows of an odd length: as bwd_kernel (one load of dy
// and x per row, the row sums give dx, the column sums are accumulated over
// the workgroup's rows and written as its partial row), on pairs plus the
// leftover element.  Workgroups hold an even number of teams and row groups
// start on even rows, so each team keeps one row parity and with it one set
// of columns for its whole walk: its column sums stay in registers, one per
// element as in bwd_kernel (plus the leftover's on the team's first lane).
// The teams' sums meet in LDS by column, added in team order, and the
// workgroup stores the partial row from there.
// ---------------------------------------------------------------------------
template <typename T, int LPR, int VPL, int TEAMS, bool RMS, bool DB>
__global__ void __launch_bounds__(LPR *TEAMS) bwd_odd_kernel(const BwdArgs a)
{
    using IO = VecIO<T, 2>;
    using BIO = BufIO<T, 2>;
    using IO1 = VecIO<T, 1>;
    using BIO1 = BufIO<T, 1>;
    using Raw = typename IO::Raw;
    using Raw1 = typename IO1::Raw;
    constexpr int WG = LPR * TEAMS;
    constexpr int PE = 2 * LPR * VPL + 1; // columns staged: the longest row
    constexpr int NB = DB ? 3 : 2;        // column sums: dgamma, dbeta (, dbias)
    using Stage = OddStage<T, PE, WG>;
    using S = typename Stage::S;
    static_assert(TEAMS % 2 == 0, "each team keeps one row parity");
    static_assert(LPR % 64 == 0, "teams of whole waves");

    __shared__ float red_lds[TeamLds<LPR, TEAMS, 2>::size];
    __shared__ __attribute__((aligned(16))) S par[PE];
    __shared__ float col_lds[NB * PE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int team = tid / LPR;
    const int tl = tid % LPR;
    const int wave_in_team = LPR > 64 ? tl / 64 : 0;
    const int N = a.N;
    const int np = (N - 1) / 2;
    const bool recompute = RMS && a.rstd == nullptr;
    // rows r0 + team with r0 even: the team's parity is its own
    const OddRow<T, LPR, VPL> o(team, tl, N, team);

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

    float ag[VPL][2], ab[VPL][2], ad[DB ? VPL : 1][2];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            ag[k][e] = 0.f;
            ab[k][e] = 0.f;
            if constexpr (DB)
                ad[k][e] = 0.f;
        }
    }
    float a1g = 0.f, a1b = 0.f, a1d = 0.f; // the leftover's column (team's first lane)
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

        // Row sums, g = dy * gamma (pairs past the row and the leftover
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
            const int c = cb + 2 * k * LPR;
            float xv[2], dv[2];
            IO::unpack(xr[k], xv);
            IO::unpack(dr[k], dv);
            row_sums(xv[0], dv[0], odd_param(par, c));
            row_sums(xv[1], dv[1], odd_param(par, c + 1));
        }
        {
            float xv[1], dv[1];
            IO1::unpack(x1, xv);
            IO1::unpack(d1, dv);
            row_sums(xv[0], dv[0], odd_param(par, cl));
        }
        team_sum<LPR, TEAMS, 2>(s, red_lds, parity, team, wave_in_team, lane);
        if (recompute)
            rstd = rsqrtf(s[1] / float(N) + a.eps);
        // dx = rstd (g - c2 - xhat c1) = fma(xhat, -rstd c1, fma(g, rstd, -rstd c2))
        const float c1 = rstd * (s[0] / float(N));
        const float c2 = RMS ? 0.f : s[1] / float(N);
        const float k1 = -rstd * c1, k2 = -rstd * c2;
        // dx of one element; its column sums when the row is valid (the
        // sums of pairs past the row are never stored)
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
            const int c = cb + 2 * k * LPR;
            float xv[2], dv[2], dxv[2], unused = 0.f;
            IO::unpack(xr[k], xv);
            IO::unpack(dr[k], dv);
#pragma unroll
            for (int e = 0; e < 2; ++e)
                dxv[e] = grad(xv[e], dv[e], odd_param(par, c + e), ag[k][e], ab[k][e],
                              DB ? ad[DB ? k : 0][e] : unused);
            BIO::store(dxs, o.off[k], IO::pack(dxv), wt);
        }
        {
            float xv[1], dv[1], dxv[1];
            IO1::unpack(x1, xv);
            IO1::unpack(d1, dv);
            dxv[0] = grad(xv[0], dv[0], odd_param(par, cl), a1g, a1b, a1d);
            BIO1::store(dxs, o.off1, IO1::pack(dxv), wt);
        }
    }

    // ---- fold the teams' column sums in LDS by column, in team order ----
    // Every team covers every column (its pairs and its leftover), so team
    // 0 writes each column and the others add to it.
    for (int t = 0; t < TEAMS; ++t) {
        if (team == t) {
            auto put = [&](int b, int c, float v) {
                float &dst = col_lds[b * PE + c];
                dst = t == 0 ? v : dst + v;
            };
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                if (k * LPR + tl < np) {
                    const int c = o.c0 + 2 * k * LPR;
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        put(0, c + e, ag[k][e]);
                        put(1, c + e, ab[k][e]);
                        if constexpr (DB)
                            put(2, c + e, ad[k][e]);
                    }
                }
            }
            if (tl == 0) {
                put(0, o.c1, a1g);
                put(1, o.c1, a1b);
                if constexpr (DB)
                    put(2, o.c1, a1d);
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

template <typename T, int LPR, int VPL, int TEAMS, bool RMS, bool DB>
hipError_t launch_bwd_odd(const BwdArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((bwd_odd_kernel<T, LPR, VPL, TEAMS, RMS, DB>), dim3(grid),
                       dim3(LPR * TEAMS), 0, s, a);
    return hipGetLastError();
}

} // namespace nf
