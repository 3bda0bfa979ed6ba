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
// [M, N] tensor crosses HBM exactly once, with nontemporal loads and stores
// (the stores of a call's last output bytes write through, see BUF_WT).
//
// Grid.  Streaming on this GPU is fastest when each workgroup covers a small
// contiguous piece and exits, so that the workgroups in flight always sweep
// one compact window of memory: the forward gives each workgroup one row
// group when there are many (a few when wide rows or few groups would leave
// CUs idle).  The backward gives each workgroup K row groups (GroupWalk), so
// that its dgamma / dbeta column partials are written once per K groups.
#pragma once

#include <type_traits>

#include "device.hpp"
#include "internal.hpp"

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

// Bytes of row group g: it starts byte0 bytes into an [M, N] tensor and holds
// `bytes` valid bytes (fewer rows in the last group).
struct RowGroup {
    int64_t r0 = 0, byte0 = 0;
    uint32_t rows = 0, bytes = 0;
    RowGroup() = default;
    __device__ __forceinline__ RowGroup(int64_t g, int teams, int64_t M, int N, int elem)
    {
        r0 = g * teams;
        const int64_t left = M - r0;
        rows = uint32_t(left < teams ? (left > 0 ? left : 0) : teams);
        byte0 = r0 * int64_t(N) * elem;
        bytes = rows * uint32_t(N) * uint32_t(elem);
    }
};

// Element `team` of a per-row fp32 vector over row group rg (0 past M or
// when v is absent).  A buffer load: no branch, so the compiler can count
// it exactly among the loads in flight.
__device__ __forceinline__ float row_stat(const float *v, const RowGroup &rg, int team)
{
    const rsrc_t r = make_rsrc(v ? v + rg.r0 : nullptr, v ? rg.rows * 4u : 0u);
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, team * 4, 0, 0));
}

// Reduction (Op: sum or max) over a team.  LPR <= 64: inside the wave.
// LPR > 64: wave partials meet in LDS (double-buffered by `parity`, so one
// barrier per reduction suffices) and are combined in wave order.  NV values
// are reduced together.
template <int LPR, int TEAMS, int NV, class Op>
__device__ __forceinline__ void team_reduce(float (&v)[NV], float *lds, int &parity, int team,
                                            int wave_in_team, int lane)
{
    if constexpr (LPR <= 64) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            v[i] = group_reduce<LPR, Op>(v[i]);
    } else {
        constexpr int WPT = LPR / 64;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            v[i] = group_reduce<64, Op>(v[i]);
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
                s = Op::apply(s, b[(team * WPT + w) * NV + i]);
            v[i] = s;
        }
        parity ^= 1;
    }
}

template <int LPR, int TEAMS, int NV>
__device__ __forceinline__ void team_sum(float (&v)[NV], float *lds, int &parity, int team,
                                         int wave_in_team, int lane)
{
    team_reduce<LPR, TEAMS, NV, OpSum>(v, lds, parity, team, wave_in_team, lane);
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
// Per-column vectors (bias, gamma, beta).  For rows up to PARAMS_LDS_MAX
// elements a workgroup converts them once to fp32 in LDS, with the neutral
// value (0, 1, 0) where a vector is absent or beyond N, so the row loops read
// them with LDS loads and no unpacking or selects.  For wider rows each lane
// keeps its own columns in registers in the packed I/O form, loaded once per
// workgroup (zeros beyond N or where absent, ones for an absent gamma), so
// the row walk issues no memory reads besides its rows -- except the
// backward's 1024-thread workgroups of the widest rows, which are short of
// registers and stage gamma in LDS up to 16384 elements (see bwd_kernel).
// ---------------------------------------------------------------------------
constexpr int PARAMS_LDS_MAX = 4096;

// The weight of a zero-centred gamma, w = 1 + gamma, formed in fp32 and
// rounded to the I/O dtype (as a weight tensor holding it would be).
template <typename T, int VEC>
__device__ __forceinline__ typename VecIO<T, VEC>::Raw plus_one(const float *g)
{
    float w[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        w[e] = 1.f + g[e];
    return VecIO<T, VEC>::pack(w);
}

// Staging of one per-column vector into LDS (fp32, `neutral` beyond N or
// where absent) in two phases, so that the workgroup's first row loads go out
// between them: fetch() issues this thread's loads, put() converts and
// stores.  VEC > 1 kernels have 16-byte aligned vectors and N % VEC == 0.
template <typename T, int VEC, int CAP, int WG>
struct ParamStage {
    using Raw = typename VecIO<T, VEC>::Raw;
    static constexpr int SI = (CAP + WG * VEC - 1) / (WG * VEC);
    Raw r[SI];

    __device__ __forceinline__ void fetch(const void *src, int N, int tid)
    {
        const rsrc_t rs = make_rsrc(src, src ? uint32_t(N) * uint32_t(sizeof(T)) : 0u);
#pragma unroll
        for (int i = 0; i < SI; ++i) {
            const int c = (tid + i * WG) * VEC;
            r[i] = BufIO<T, VEC>::load_cached(rs, c < CAP ? uint32_t(c) * uint32_t(sizeof(T))
                                                          : BUF_OOB);
        }
    }
    // bf16 rows: the same values as put() in their 16-bit patterns (bf16
    // values convert to fp32 and back exactly)
    __device__ __forceinline__ void put_raw(uint16_t *dst, const void *src, int N, float neutral,
                                            int tid, bool zero_centred = false) const
    {
        static_assert(sizeof(T) == 2, "16-bit elements");
#pragma unroll
        for (int i = 0; i < SI; ++i) {
            const int c = (tid + i * WG) * VEC;
            if (c < CAP) {
                float v[VEC];
                VecIO<T, VEC>::unpack(r[i], v);
                if (zero_centred)
                    VecIO<T, VEC>::unpack(plus_one<T, VEC>(v), v);
                const bool ok = src != nullptr && c < N;
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    dst[c + e] = uint16_t(__float_as_uint(ok ? v[e] : neutral) >> 16);
            }
        }
    }
    // zero_centred: store round_T(1 + v) (the weight of a zero-centred
    // gamma; 1 where absent)
    __device__ __forceinline__ void put(float *dst, const void *src, int N, float neutral,
                                        int tid, bool zero_centred = false) const
    {
#pragma unroll
        for (int i = 0; i < SI; ++i) {
            const int c = (tid + i * WG) * VEC;
            if (c < CAP) {
                float v[VEC];
                VecIO<T, VEC>::unpack(r[i], v);
                if (zero_centred)
                    VecIO<T, VEC>::unpack(plus_one<T, VEC>(v), v);
                const bool ok = src != nullptr && c < N;
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    dst[c + e] = ok ? v[e] : neutral;
            }
        }
    }
};

// This lane's VPL vectors of a per-column vector (registers, packed);
// zero_centred: the weight round_T(1 + gamma) instead (1 where absent).
template <typename T, int VEC, int VPL>
__device__ __forceinline__ void load_param_regs(typename VecIO<T, VEC>::Raw (&dst)[VPL],
                                                const void *src, int N, const uint32_t (&poff)[VPL],
                                                bool ones_if_absent, bool zero_centred = false)
{
    using IO = VecIO<T, VEC>;
    if (src == nullptr && ones_if_absent) {
        float one[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            one[e] = 1.f;
#pragma unroll
        for (int k = 0; k < VPL; ++k)
            dst[k] = IO::pack(one);
        return;
    }
    const rsrc_t r = make_rsrc(src, src ? uint32_t(N) * uint32_t(sizeof(T)) : 0u);
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        dst[k] = BufIO<T, VEC>::load_cached(r, poff[k]);
        if (zero_centred) {
            float v[VEC];
            IO::unpack(dst[k], v);
            dst[k] = plus_one<T, VEC>(v); // columns past N are never used
        }
    }
}

// VEC values of a per-column vector at column c0: from LDS when staged, else
// unpacked from this lane's registers.
template <typename T, int VEC, bool IN_LDS, typename Raw>
__device__ __forceinline__ void param_vec(const float *lds, const Raw &reg, int c0, float *out)
{
    if constexpr (IN_LDS)
        lds_read<VEC>(lds + c0, out);
    else
        VecIO<T, VEC>::unpack(reg, out);
}

// Whether the forward walk keeps the next row group's loads in flight (wide
// teams): the rows of two groups, packed, and the parameters held in
// registers when they are not staged in LDS (3 VPL vectors) must fit the
// wave's share of the 512 VGPRs of a SIMD with about 24 to spare.  The
// widest fp32 rows (1024 lanes x 4 vectors) and the element-wise rows of
// 1024 lanes x 16 do not fit: with the prefetch they spilled about 200
// registers to scratch and ran at 16% of the HBM peak.
template <typename T, int VEC, int LPR, int VPL, int TEAMS>
constexpr bool fwd_prefetch()
{
    constexpr int raw = VEC * int(sizeof(T)) >= 4 ? VEC * int(sizeof(T)) / 4 : 1;
    constexpr int waves_per_simd = (LPR * TEAMS / 64 + 3) / 4;
    constexpr int share = 512 / waves_per_simd;
    constexpr bool plds = LPR * VPL * VEC <= PARAMS_LDS_MAX;
    constexpr int need = 4 * VPL * raw + (plds ? 0 : 3 * VPL * raw) + 24;
    return LPR >= WIDE_LPR && need <= share;
}

// ---------------------------------------------------------------------------
// The second stage of amax in one launch, through a caller workspace that is
// zero when the launch starts.  A cell of two words -- [0] the maxima
// combined so far (atomicMax on the bit pattern), [1] how many of its
// members have added theirs -- counts the arrivals of a set of members.
// Workgroup b is a member of subgroup cell b % AMAX_SUBGROUPS; the last
// member to arrive at a subgroup cell takes its maximum (swapping in 0),
// zeroes its count and arrives with it at the top cell, whose last arrival
// writes amax.  (With one cell for all workgroups, their returning atomics
// on one address serialise: 18000 workgroups took 150 us longer.)
// Every atomic here is a device-scope read-modify-write whose result returns
// from the memory-side point where all atomics on that address are
// performed, so a returned value means the operation has been applied
// there.  An arrival's count addend depends on the value its max returned,
// so the count is issued only after the max has been applied; the arrival
// that raises a cell's count to its number of members therefore finds every
// member's maximum in the cell when it takes it.  Every cell is left zero
// for the next call on the same stream.
// ---------------------------------------------------------------------------
constexpr unsigned AMAX_SUBGROUPS = 64;
constexpr unsigned AMAX_CELL_WORDS = 16; // one 64-byte line per cell

// Arrive at `cell` with `bits`; true for the last of `members` arrivals,
// which receives the combined maximum in `all`.
__device__ __forceinline__ bool amax_cell_arrive(unsigned *cell, unsigned bits, unsigned members,
                                                 unsigned &all)
{
    const unsigned prev =
        __hip_atomic_fetch_max(cell, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // prev is the bit pattern of a non-negative float: bit 31 is clear, so the
    // addend is 1, but only known once prev has returned
    const unsigned one = 1u + (prev >> 31);
    const unsigned arrived =
        __hip_atomic_fetch_add(cell + 1, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (arrived != members - 1)
        return false;
    all = __hip_atomic_exchange(cell, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(cell + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

__device__ __forceinline__ void amax_arrive(unsigned *amax, unsigned *ws, unsigned bits)
{
    const unsigned G = gridDim.x, b = blockIdx.x;
    const unsigned sg = b % AMAX_SUBGROUPS;
    const unsigned members = (G - 1 - sg) / AMAX_SUBGROUPS + 1; // b' < G with b' % 64 == sg
    const unsigned cells = G < AMAX_SUBGROUPS ? G : AMAX_SUBGROUPS;
    unsigned all = 0;
    if (!amax_cell_arrive(ws + sg * AMAX_CELL_WORDS, bits, members, all))
        return;
    if (amax_cell_arrive(ws + AMAX_SUBGROUPS * AMAX_CELL_WORDS, all, cells, all))
        *amax = all;
}

// ---------------------------------------------------------------------------
// Forward: t = (x + bias) + residual (fp32), u = round(t) -> residual_out,
// statistics of u, y = normalise(u) * gamma + beta -> y, running max |y|.
// ---------------------------------------------------------------------------
template <typename T, int VEC, int LPR, int VPL, int TEAMS, bool RMS, bool F8>
__global__ void __launch_bounds__(LPR *TEAMS) fwd_kernel(const FwdArgs a)
{
    using IO = VecIO<T, VEC>;
    using BIO = BufIO<T, VEC>;
    using Raw = typename IO::Raw;
    constexpr int WG = LPR * TEAMS;
    constexpr int CAP = LPR * VPL * VEC;
    // 1024-thread workgroups of 8 or more elements per lane in 4-byte or
    // single-element accesses (128 registers, one per element or pair)
    // stage bias, gamma and beta in LDS: as fp32 up to 8192 columns (96 KiB),
    // beyond that bf16 rows as their 16-bit patterns, unpacked at each use
    // (fp32 rows that wide keep them in registers).  Held in registers they
    // spilled to scratch; measured on MI355X: 8192 x 16383 bf16 474 -> 295
    // us, 16384 x 8191 fp32 471 -> 432 us.  (8-byte vectors hold them packed
    // in few registers: in LDS, 8192 x 16380 bf16 took 211 against 206 us.)
    constexpr bool TIGHT = WG >= 1024 && VPL * VEC >= 8 && VEC * int(sizeof(T)) <= 4;
    constexpr bool PLDS = CAP <= PARAMS_LDS_MAX || (TIGHT && CAP <= 2 * PARAMS_LDS_MAX);
    constexpr bool PRAW = !PLDS && TIGHT && sizeof(T) == 2;
    constexpr bool PREFETCH = fwd_prefetch<T, VEC, LPR, VPL, TEAMS>();
    static_assert(WG % 64 == 0, "workgroup of whole waves");

    __shared__ float red_lds[TeamLds<LPR, TEAMS, 1>::size];
    __shared__ double red_lds_f64[TeamLds<LPR, TEAMS, 1>::size];
    __shared__ float max_lds[WG / 64];
    __shared__ __attribute__((aligned(16))) float par[PLDS ? 3 * CAP : 4];
    __shared__ __attribute__((aligned(16))) uint16_t praw[PRAW ? 3 * CAP : 8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int team = tid / LPR;
    const int tl = tid % LPR;
    const int wave_in_team = LPR > 64 ? tl / 64 : 0;
    const int N = a.N;
    const bool has_res = a.res != nullptr;
    const bool fused_add = a.bias != nullptr || has_res;

    bool cvalid[VPL];
    uint32_t off[VPL]; // this lane's byte offset of vector k inside a row group
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        cvalid[k] = (k * LPR + tl) * VEC < N; // VEC > 1: N % VEC == 0, whole vector valid
        off[k] = cvalid[k] ? uint32_t(team * N + (k * LPR + tl) * VEC) * uint32_t(sizeof(T))
                           : BUF_OOB;
    }
    // FP8 output: one byte per element, and the scale every value takes
    const float y_scale = F8 ? *a.y_scale : 1.f;

    // x and residual of row group g (zeros outside the matrix).  Wide teams
    // walk their row groups with the next group's loads in flight while the
    // current one is worked on (PREFETCH).
    Raw xn[VPL], rn[VPL];
    auto issue = [&](int64_t g) {
        const RowGroup rg(g, TEAMS, a.M, N, sizeof(T));
        const rsrc_t xs = make_rsrc(static_cast<const char *>(a.x) + rg.byte0, rg.bytes);
        const rsrc_t rs = make_rsrc(has_res ? static_cast<const char *>(a.res) + rg.byte0 : nullptr,
                                    has_res ? rg.bytes : 0u);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            xn[k] = BIO::load(xs, off[k]);
            rn[k] = has_res ? BIO::load(rs, off[k]) : IO::zero();
        }
    };
    const GroupWalk walk(a.K, a.A);

    // Parameters: their loads first, then the first row group's (every
    // kernel: the rows' latency then overlaps the parameters' staging), so
    // that the wait for the parameters does not include the rows.
    constexpr int PR = PLDS || PRAW ? 1 : VPL;
    Raw pbias[PR], pgam[PR], pbeta[PR];
    if constexpr (PLDS) {
        ParamStage<T, VEC, CAP, WG> sb, sg, se;
        sb.fetch(a.bias, N, tid);
        sg.fetch(a.gamma, N, tid);
        se.fetch(a.beta, N, tid);
        issue(walk.group(0));
        sb.put(par, a.bias, N, 0.f, tid);
        sg.put(par + CAP, a.gamma, N, 1.f, tid, a.zero_centred);
        se.put(par + 2 * CAP, a.beta, N, 0.f, tid);
        __syncthreads();
    } else if constexpr (PRAW) {
        ParamStage<T, VEC, CAP, WG> sb, sg, se;
        sb.fetch(a.bias, N, tid);
        sg.fetch(a.gamma, N, tid);
        se.fetch(a.beta, N, tid);
        issue(walk.group(0));
        sb.put_raw(praw, a.bias, N, 0.f, tid);
        sg.put_raw(praw + CAP, a.gamma, N, 1.f, tid, a.zero_centred);
        se.put_raw(praw + 2 * CAP, a.beta, N, 0.f, tid);
        __syncthreads();
    } else {
        uint32_t poff[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k)
            poff[k] = cvalid[k] ? uint32_t((k * LPR + tl) * VEC) * uint32_t(sizeof(T)) : BUF_OOB;
        load_param_regs<T, VEC, VPL>(pbias, a.bias, N, poff, false);
        load_param_regs<T, VEC, VPL>(pgam, a.gamma, N, poff, true, a.zero_centred);
        load_param_regs<T, VEC, VPL>(pbeta, a.beta, N, poff, false);
        issue(walk.group(0));
    }

    // VEC values of per-column vector `which` (0 bias, 1 gamma, 2 beta) at
    // column c0; `reg`: this lane's packed registers when not staged
    auto pvec = [&](int which, const Raw &reg, int c0, float *out) {
        if constexpr (PRAW)
            IO::unpack(*reinterpret_cast<const Raw *>(praw + which * CAP + c0), out);
        else
            param_vec<T, VEC, PLDS>(par + which * CAP, reg, c0, out);
    };

    float lane_max = 0.f;
    int parity = 0;

    for (int kk = 0; kk < a.K; ++kk) {
        const int64_t grp = walk.group(kk);
        if (grp >= a.n_groups)
            break; // uniform over the workgroup; later groups are larger
        const int64_t row = grp * TEAMS + team;
        const bool rv = row < a.M;
        const RowGroup rgp(grp, TEAMS, a.M, N, sizeof(T));
        const uint32_t bytes = rgp.bytes;
        const int64_t gbyte = rgp.byte0;
        const bool wt = grp >= a.wt_group; // store policy (see BUF_WT)
        if (!PREFETCH && kk > 0)
            issue(grp); // group 0 was issued before the parameters were staged
        if constexpr (!PLDS && !PRAW) {
            // keep the parameters packed: unpacking them once for the whole
            // walk would cost more registers than the unpacking per group
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                reload_barrier(pbias[k]);
                reload_barrier(pgam[k]);
                reload_barrier(pbeta[k]);
            }
        }

        // ur holds u, the value actually normalised, in its packed I/O form
        // (exact: u is rounded to T); every later pass unpacks it again.
        Raw ur[VPL], rr[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            ur[k] = xn[k];
            rr[k] = rn[k];
        }
        const int64_t next = walk.group(kk + 1);
        const bool has_next = kk + 1 < a.K && next < a.n_groups;
        if (PREFETCH && has_next)
            issue(next); // early: in flight during this group's work

        // fused add; u = round_T((x + bias) + residual), and the row sum of
        // u for LayerNorm (fp32 for bf16 rows, whose sums of values of
        // similar magnitude are exact in fp32; fp64 for fp32 rows).  Narrow
        // RMSNorm teams take their sum of squares here too, in the order of
        // the later pass, so that residual_out is stored only after every
        // load has been used: a store issued while loads are pending makes
        // the next wait for a load wait for the store as well.  Measured on
        // MI355X (bf16, bias and residual): 576000 x 384 288.2 -> 286.6 us,
        // 131072 x 1024 174.0 -> 170.5 us; on 512-lane teams (32768 x 4096)
        // the early sum measured 1.7% slower, so wide teams keep the pass.
        using Acc = typename std::conditional<std::is_same<T, float>::value, double, float>::type;
        constexpr bool SQ_EARLY = RMS && LPR < WIDE_LPR;
        Acc sum = Acc(0);
        float sq = 0.f;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int c0 = (k * LPR + tl) * VEC;
            float t[VEC];
            IO::unpack(ur[k], t);
            if (fused_add) {
                float bv[VEC], rv_[VEC];
                pvec(0, pbias[PR == 1 ? 0 : k], c0, bv);
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
            } else if constexpr (SQ_EARLY) {
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    sq = fmaf(t[e], t[e], sq);
            }
        }
        if (a.res_out) {
            const rsrc_t os = make_rsrc(static_cast<char *>(a.res_out) + gbyte, bytes);
#pragma unroll
            for (int k = 0; k < VPL; ++k)
                BIO::store(os, off[k], ur[k], wt);
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
            float s2[1] = {sq};
            if constexpr (!SQ_EARLY) {
#pragma unroll
                for (int k = 0; k < VPL; ++k) {
                    float u[VEC];
                    IO::unpack(ur[k], u);
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        s2[0] = fmaf(u[e], u[e], s2[0]);
                }
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
        // FP8: y rounded to the I/O dtype (the values amax is taken over),
        // times the scale, to E4M3 codes, one byte per element
        const rsrc_t ys = F8 ? make_rsrc(static_cast<char *>(a.y) + gbyte / int64_t(sizeof(T)),
                                         bytes / uint32_t(sizeof(T)))
                             : make_rsrc(static_cast<char *>(a.y) + gbyte, bytes);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int c0 = (k * LPR + tl) * VEC;
            float u[VEC], gv[VEC], bv[VEC], yv[VEC];
            IO::unpack(ur[k], u);
            pvec(1, pgam[PR == 1 ? 0 : k], c0, gv);
            pvec(2, pbeta[PR == 1 ? 0 : k], c0, bv);
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                yv[e] = fmaf(fmaf(u[e] - mean, rstd, lo_r), gv[e], bv[e]);
            if constexpr (F8) {
                float q[VEC];
                IO::unpack(IO::pack(yv), q);
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    q[e] *= y_scale;
                const uint32_t off8 = cvalid[k] ? off[k] / uint32_t(sizeof(T)) : BUF_OOB;
                if constexpr (VEC == 8 && LPR >= 2) {
                    // lane pairs store 16 codes at once
                    const bool pvalid = ((k * LPR + (tl ^ 1)) * VEC) < N;
                    store_e4m3_pair(ys, off8, q, (tl & 1) == 0, pvalid, wt);
                } else {
                    store_e4m3<VEC>(ys, off8, q, wt);
                }
            } else {
                BIO::store(ys, off[k], IO::pack(yv), wt);
            }
            if (rv && cvalid[k]) {
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
    // their unsigned patterns).  Atomics on one address serialise: the host
    // keeps the number of workgroups that issue them bounded.
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
            if (a.amax_ws == nullptr) {
                atomicMax(a.amax, bits); // *amax was zeroed by a kernel before this one
            } else {
                amax_arrive(a.amax, a.amax_ws, bits);
            }
        }
    }
}

// Whether the backward pipelines its row walk (wide teams of bf16 in 16- or
// 8-byte vectors, see bwd_kernel): two groups' packed rows, one group's
// packed dx, the column accumulators and the unpacked working values (about
// 4E + 24 registers) must fit the wave's share of the 512 VGPRs of a SIMD,
// less 16.  Narrow teams hold several rows per wave and keep enough loads in
// flight without it; fp32 rows (twice the registers per element) and the
// 4-byte and single-element paths do not pipeline (in 1024-thread
// workgroups, capped at 128 registers, they spilled).  The 8-byte bf16 rows
// gained from it, measured on MI355X: 16384 x 4100 122.2 -> 99.5 us,
// 16384 x 6140 150.7 -> 118.7 us, 32768 x 1500 97.5 -> 69.5 us,
// 16384 x 8188 186.1 -> 160.2 us.
template <typename T, int VEC, int LPR, int VPL, int TEAMS>
constexpr bool bwd_pipelined()
{
    constexpr int raw = VEC * int(sizeof(T)) >= 4 ? VEC * int(sizeof(T)) / 4 : 1;
    constexpr int slot = 2 * VPL * raw; // x and dy of one group, packed
    constexpr int E = VPL * VEC;
    constexpr int waves_per_simd = (LPR * TEAMS / 64 + 3) / 4;
    constexpr int share = 512 / waves_per_simd;
    constexpr int budget = share - 16;
    return sizeof(T) == 2 && VEC * int(sizeof(T)) >= 8 && LPR >= WIDE_LPR &&
           2 * slot + VPL * raw + 4 * E + 24 <= budget;
}

// ---------------------------------------------------------------------------
// Backward stage 1 (mix-order): per row, one load of dy and x; the row
// reduction gives dx; the column reduction is accumulated in registers over
// the workgroup's rows, folded over the workgroup in a fixed order and
// written as this workgroup's partial row of the workspace.
// ---------------------------------------------------------------------------
// One lane's VEC consecutive columns, from c0, of the partial rows pg / pb
// (/ pd): 16-byte stores when VEC is a multiple of 4 (the rows start on
// 16-byte boundaries and vectorised kernels have N a multiple of VEC).  The
// partials keep the default write-back policy: the column sums read them
// next, and measured, write-through or nontemporal partials were slower.
template <int VEC, bool DB>
__device__ __forceinline__ void store_partial(float *pg, float *pb, float *pd, int c0, int N,
                                              const float *vg, const float *vb, const float *vd)
{
    if constexpr (VEC % 4 == 0) {
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
            *reinterpret_cast<float4 *>(pg + c0 + e) = float4{vg[e], vg[e + 1], vg[e + 2], vg[e + 3]};
            *reinterpret_cast<float4 *>(pb + c0 + e) = float4{vb[e], vb[e + 1], vb[e + 2], vb[e + 3]};
            if constexpr (DB)
                *reinterpret_cast<float4 *>(pd + c0 + e) =
                    float4{vd[e], vd[e + 1], vd[e + 2], vd[e + 3]};
        }
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            if (c0 + e < N) {
                pg[c0 + e] = vg[e];
                pb[c0 + e] = vb[e];
                if constexpr (DB)
                    pd[c0 + e] = vd[e];
            }
        }
    }
}

template <typename T, int VEC, int LPR, int VPL, int TEAMS, bool RMS, bool DB>
__global__ void __launch_bounds__(LPR *TEAMS) bwd_kernel(const BwdArgs a)
{
    using IO = VecIO<T, VEC>;
    using BIO = BufIO<T, VEC>;
    using Raw = typename IO::Raw;
    constexpr int E = VPL * VEC;
    constexpr int WG = LPR * TEAMS;
    constexpr int NW = WG / 64;
    constexpr int CAP = LPR * VPL * VEC;
    // 1024-thread workgroups of 16 or more elements per lane (the widest
    // rows) get 128 registers per lane: they stage gamma in LDS, like the
    // narrower rows, and keep the dbias sums in LDS too (each lane its own
    // slots, so no barrier).  Held in registers these spilled to scratch;
    // measured on MI355X, backward with dbias: 8192 x 16384 fp32 312 ->
    // 284 us, 8192 x 16380 bf16 233 -> 188 us, 8192 x 16383 bf16 711 ->
    // 235 us (without dbias 345 -> 217 us).
    constexpr bool TIGHT = WG >= 1024 && E >= 16;
    constexpr bool PLDS = CAP <= PARAMS_LDS_MAX || TIGHT;
    constexpr bool DLDS = DB && TIGHT;
    constexpr bool PIPE = bwd_pipelined<T, VEC, LPR, VPL, TEAMS>();
    // partial slots to fold in LDS: waves (LPR <= 64) or teams (LPR > 64)
    constexpr int SLOTS = LPR <= 64 ? NW : TEAMS;
    static_assert(WG % 64 == 0, "workgroup of whole waves");

    __shared__ float red_lds[TeamLds<LPR, TEAMS, 2>::size];
    constexpr int NB = DB ? 3 : 2; // column sums: dgamma, dbeta (, dbias)
    __shared__ float col_lds[SLOTS > 1 ? NB * CAP : 1];
    __shared__ __attribute__((aligned(16))) float par[PLDS ? CAP : 4];
    __shared__ float dacc[DLDS ? E * WG : 1];
    static_assert(!DLDS || SLOTS == 1, "LDS dbias sums only for one-team workgroups");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int team = tid / LPR;
    const int tl = tid % LPR;
    const int wave_in_team = LPR > 64 ? tl / 64 : 0;
    const int N = a.N;
    const bool recompute = RMS && a.rstd == nullptr;

    bool cvalid[VPL];
    uint32_t off[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        cvalid[k] = (k * LPR + tl) * VEC < N;
        off[k] = cvalid[k] ? uint32_t(team * N + (k * LPR + tl) * VEC) * uint32_t(sizeof(T))
                           : BUF_OOB;
    }

    // x, dy and the row statistics of one row group, as loaded.
    struct Slot {
        Raw x[VPL], d[VPL];
        float mean, rstd;
    };
    auto issue = [&](int64_t g, Slot &sl) {
        const RowGroup rg(g, TEAMS, a.M, N, sizeof(T));
        const rsrc_t xs = make_rsrc(static_cast<const char *>(a.x) + rg.byte0, rg.bytes);
        const rsrc_t ds = make_rsrc(static_cast<const char *>(a.dy) + rg.byte0, rg.bytes);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            sl.x[k] = BIO::load(xs, off[k]);
            sl.d[k] = BIO::load(ds, off[k]);
        }
        if constexpr (PIPE) {
            sl.mean = RMS ? 0.f : row_stat(a.mean, rg, team);
            sl.rstd = recompute ? 0.f : row_stat(a.rstd, rg, team);
        } else {
            const int64_t row = g * TEAMS + team;
            const bool rv = row < a.M;
            sl.mean = (rv && !RMS) ? a.mean[row] : 0.f;
            sl.rstd = (rv && !recompute) ? a.rstd[row] : 0.f;
        }
    };
    const GroupWalk walk(a.K, a.A);
    auto valid = [&](int kk) { return kk < a.K && walk.group(kk) < a.n_groups; };

    // Slot A holds the group being worked on; pipelined walks load the next
    // group into slot B meanwhile (the two alternate).
    Slot A, B;

    // gamma's loads first, then the first row group's (see the forward)
    constexpr int PR = PLDS ? 1 : VPL;
    Raw pgam[PR];
    if constexpr (PLDS) {
        ParamStage<T, VEC, CAP, WG> sg;
        sg.fetch(a.gamma, N, tid);
        issue(walk.group(0), A);
        sg.put(par, a.gamma, N, 1.f, tid, a.zero_centred);
        __syncthreads();
    } else {
        uint32_t poff[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k)
            poff[k] = cvalid[k] ? uint32_t((k * LPR + tl) * VEC) * uint32_t(sizeof(T)) : BUF_OOB;
        load_param_regs<T, VEC, VPL>(pgam, a.gamma, N, poff, true, a.zero_centred);
        issue(walk.group(0), A);
    }

    float acc_g[E], acc_b[E], acc_d[DB && !DLDS ? E : 1];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        acc_g[e] = 0.f;
        acc_b[e] = 0.f;
        if constexpr (DLDS)
            dacc[e * WG + tid] = 0.f;
        else if constexpr (DB)
            acc_d[e] = 0.f;
    }
    int parity = 0;

    // dx of the last group worked on, held back by pipelined walks
    Raw dxh[VPL];
    RowGroup hrg;
    bool held = false, hwt = false; // hwt: store policy of the held dx (see BUF_WT)

    // The work on row group grp, whose rows and statistics are in sl; dx is
    // stored, or held in dxh when `hold`.
    auto work = [&](int64_t grp, Slot &sl, bool hold) {
        const int64_t row = grp * TEAMS + team;
        const bool rv = row < a.M;
        const RowGroup rgp(grp, TEAMS, a.M, N, sizeof(T));
        if constexpr (!PLDS) {
#pragma unroll
            for (int k = 0; k < VPL; ++k)
                reload_barrier(pgam[k]); // unpacked per group, not held unpacked
        }
        const float mean = sl.mean;
        float rstd = sl.rstd;

        // Row sums, g = dy * gamma (invalid elements hold 0):
        //   LN : s0 = sum g (x - mean), s1 = sum g  ->  mean(g xhat) = rstd s0 / N
        //   RMS: s0 = sum g x                      ->  mean(g xhat) = rstd s0 / N
        //   RMS without rstd: s1 = sum x^2 gives rstd from the same load.
        float s[2] = {0.f, 0.f};
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int c0 = (k * LPR + tl) * VEC;
            float xv[VEC], dv[VEC], gv[VEC];
            IO::unpack(sl.x[k], xv);
            IO::unpack(sl.d[k], dv);
            param_vec<T, VEC, PLDS>(par, pgam[PLDS ? 0 : k], c0, gv);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float g = dv[e] * gv[e];
                if constexpr (!RMS) {
                    s[0] = fmaf(g, xv[e] - mean, s[0]);
                    s[1] += g;
                } else {
                    s[0] = fmaf(g, xv[e], s[0]);
                    if (recompute)
                        s[1] = fmaf(xv[e], xv[e], s[1]);
                }
            }
        }
        team_sum<LPR, TEAMS, 2>(s, red_lds, parity, team, wave_in_team, lane);
        if (recompute)
            rstd = rsqrtf(s[1] / float(N) + a.eps);
        // dx = rstd (g - c2 - xhat c1) = fma(xhat, -rstd c1, fma(g, rstd, -rstd c2))
        const float c1 = rstd * (s[0] / float(N));
        const float c2 = RMS ? 0.f : s[1] / float(N);
        const float k1 = -rstd * c1, k2 = -rstd * c2;

#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            reload_barrier(sl.x[k]);
            reload_barrier(sl.d[k]);
        }
        const rsrc_t dxs = make_rsrc(static_cast<char *>(a.dx) + rgp.byte0, rgp.bytes);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int c0 = (k * LPR + tl) * VEC;
            float xv[VEC], dv[VEC], gv[VEC], dxv[VEC];
            IO::unpack(sl.x[k], xv);
            IO::unpack(sl.d[k], dv);
            param_vec<T, VEC, PLDS>(par, pgam[PLDS ? 0 : k], c0, gv);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int i = k * VEC + e;
                const float xh = RMS ? xv[e] * rstd : (xv[e] - mean) * rstd;
                dxv[e] = fmaf(xh, k1, fmaf(dv[e] * gv[e], rstd, k2));
                if (rv) { // rows past M read zeros; columns past N too
                    acc_g[i] = fmaf(dv[e], xh, acc_g[i]);
                    acc_b[i] += dv[e];
                    if constexpr (DB)
                        if constexpr (DLDS)
                            dacc[i * WG + tid] += dxv[e]; // this lane's own slots
                        else
                            acc_d[i] += dxv[e]; // dbias: column sums of dx
                }
            }
            if (hold)
                dxh[k] = IO::pack(dxv);
            else
                BIO::store(dxs, off[k], IO::pack(dxv), grp >= a.wt_group);
        }
        if (hold) {
            hrg = rgp;
            hwt = grp >= a.wt_group;
            held = true;
        }
    };

    if constexpr (PIPE) {
        // Two-stage pipeline.  As soon as a group's rows have arrived, the
        // next group's loads and the previous group's dx stores are issued;
        // then the group is worked on and its dx held.  Each wait thus finds
        // only loads and stores issued a whole group earlier.  (A wait for a
        // load while any store is outstanding waits for all of them, so a
        // store issued just before the wait would put its latency on every
        // group's path.)
        auto arrive = [&](Slot &sl) {
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                order_after_arrival(sl.x[k]);
                order_after_arrival(sl.d[k]);
            }
            order_after_arrival(sl.mean);
            order_after_arrival(sl.rstd);
        };
        auto flush = [&]() {
            if (held) {
                const rsrc_t dxs = make_rsrc(static_cast<char *>(a.dx) + hrg.byte0, hrg.bytes);
#pragma unroll
                for (int k = 0; k < VPL; ++k)
                    BIO::store(dxs, off[k], dxh[k], hwt);
            }
        };
        for (int kk = 0; kk < a.K; kk += 2) {
            if (!valid(kk))
                break;
            arrive(A);
            if (valid(kk + 1))
                issue(walk.group(kk + 1), B);
            flush();
            work(walk.group(kk), A, true);
            if (!valid(kk + 1))
                break;
            arrive(B);
            if (valid(kk + 2))
                issue(walk.group(kk + 2), A);
            flush();
            work(walk.group(kk + 1), B, true);
        }
        flush();
    } else {
        for (int kk = 0; kk < a.K; ++kk) {
            const int64_t grp = walk.group(kk);
            if (grp >= a.n_groups)
                break; // uniform over the workgroup; later groups are larger
            if (kk > 0)
                issue(grp, A); // group 0 was issued before gamma was staged
            work(grp, A, false);
        }
    }

    // ---- fold the column partials of this workgroup, in a fixed order ----
    // Block b of the workspace (dgamma, dbeta, dbias) holds row blockIdx.x.
    const int64_t ld = colsum_ld(N);
    float *pg = a.ws + (int64_t)blockIdx.x * ld;
    float *pb = a.ws + (int64_t)gridDim.x * ld + (int64_t)blockIdx.x * ld;
    float *pd = a.ws + 2 * (int64_t)gridDim.x * ld + (int64_t)blockIdx.x * ld;
    if constexpr (LPR < 64) {
        // teams of one wave cover the same columns: fold them first
#pragma unroll
        for (int e = 0; e < E; ++e) {
            acc_g[e] = fold_teams_sum<LPR>(acc_g[e]);
            acc_b[e] = fold_teams_sum<LPR>(acc_b[e]);
            if constexpr (DB && !DLDS)
                acc_d[e] = fold_teams_sum<LPR>(acc_d[e]);
        }
    }
    if constexpr (SLOTS == 1) {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int c0 = (k * LPR + tl) * VEC;
            if (cvalid[k] && (LPR >= 64 || lane < LPR)) {
                if constexpr (DLDS) {
                    float vd[VEC];
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        vd[e] = dacc[(k * VEC + e) * WG + tid];
                    store_partial<VEC, DB>(pg, pb, pd, c0, N, acc_g + k * VEC, acc_b + k * VEC, vd);
                } else {
                    store_partial<VEC, DB>(pg, pb, pd, c0, N, acc_g + k * VEC, acc_b + k * VEC,
                                           acc_d + (DB ? k * VEC : 0));
                }
            }
        }
    } else {
        // slots 0 .. SLOTS-2 add their sums into LDS in slot order; the last
        // slot adds its own and stores the row from registers
        const int slot = LPR <= 64 ? (tid >> 6) : team;
        const bool holder = LPR < 64 ? lane < LPR : true;
        for (int sl = 0; sl < SLOTS - 1; ++sl) {
            if (slot == sl && holder) {
#pragma unroll
                for (int k = 0; k < VPL; ++k) {
                    const int c0 = (k * LPR + tl) * VEC;
                    if (cvalid[k]) {
#pragma unroll
                        for (int e = 0; e < VEC; ++e) {
                            const int c = c0 + e;
                            const int i = k * VEC + e;
                            col_lds[c] = sl == 0 ? acc_g[i] : col_lds[c] + acc_g[i];
                            col_lds[CAP + c] = sl == 0 ? acc_b[i] : col_lds[CAP + c] + acc_b[i];
                            if constexpr (DB)
                                col_lds[2 * CAP + c] =
                                    sl == 0 ? acc_d[i] : col_lds[2 * CAP + c] + acc_d[i];
                        }
                    }
                }
            }
            __syncthreads();
        }
        if (slot == SLOTS - 1 && holder) {
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                const int c0 = (k * LPR + tl) * VEC;
                if (!cvalid[k])
                    continue;
                float vg[VEC], vb[VEC], vd[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const int i = k * VEC + e;
                    vg[e] = col_lds[c0 + e] + acc_g[i];
                    vb[e] = col_lds[CAP + c0 + e] + acc_b[i];
                    if constexpr (DB)
                        vd[e] = col_lds[2 * CAP + c0 + e] + acc_d[i];
                    else
                        vd[e] = 0.f;
                }
                store_partial<VEC, DB>(pg, pb, pd, c0, N, vg, vb, vd);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Backward with the rows split along N, for few rows of many columns, where
// whole-row workgroups cannot fill the GPU.  Row sums need the whole row, so
// the work takes two passes over a grid of (chunk s, row block b)
// workgroups: chunk s is SPLIT_VPL * 64 * VEC columns, and a row block is K
// groups of SPLIT_ROWS_PER_GROUP rows (one row per wave).
//  pass 0: each wave's two row sums over its chunk go to rowsums[row][s];
//          with mean and rstd given, the chunk's dgamma / dbeta column
//          partials are added as well;
//  pass 1: the row sums of all chunks are added in chunk order, giving the
//          row's c1, c2 (and rstd when it is recomputed); dx of the chunk is
//          stored, and the dbias partials (and dgamma / dbeta when rstd is
//          recomputed) are added.
// Each pass folds its partials over the four waves in wave order into row b
// of the workspace blocks, at the chunk's columns, for the usual column sums.
// The second pass reads x and dy again; at these sizes they come from the
// last-level cache.
// ---------------------------------------------------------------------------
constexpr int SPLIT_VPL = 4;
template <typename T, int VEC>
constexpr int split_cols()
{
    return 64 * SPLIT_VPL * VEC;
}

template <typename T, int VEC, bool RMS, bool DB, int PASS>
__global__ void __launch_bounds__(64 * SPLIT_ROWS_PER_GROUP) bwd_split_kernel(const BwdArgs a)
{
    using IO = VecIO<T, VEC>;
    using BIO = BufIO<T, VEC>;
    using Raw = typename IO::Raw;
    constexpr int E = SPLIT_VPL * VEC;
    constexpr int C = split_cols<T, VEC>();
    constexpr int W = SPLIT_ROWS_PER_GROUP;
    __shared__ float fold[W][C];

    const int s = blockIdx.x, b = blockIdx.y;
    const int wave = threadIdx.x / 64, lane = threadIdx.x & 63;
    const int N = a.N, S = a.chunks;
    const bool recompute = RMS && a.rstd == nullptr;
    // which column partials this pass adds
    const bool add_gb = PASS == 0 ? !recompute : recompute;
    const bool add_d = PASS == 1 && DB;

    bool cvalid[SPLIT_VPL];
    uint32_t off[SPLIT_VPL];
#pragma unroll
    for (int k = 0; k < SPLIT_VPL; ++k) {
        const int col = s * C + (k * 64 + lane) * VEC;
        cvalid[k] = col < N;
        off[k] = cvalid[k] ? uint32_t(col) * uint32_t(sizeof(T)) : BUF_OOB;
    }
    Raw pg[SPLIT_VPL];
    load_param_regs<T, VEC, SPLIT_VPL>(pg, a.gamma, N, off, true, a.zero_centred);

    float acc_g[E], acc_b[E], acc_d[DB ? E : 1];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        acc_g[e] = 0.f;
        acc_b[e] = 0.f;
        if constexpr (DB)
            acc_d[e] = 0.f;
    }
    const uint32_t row_bytes = uint32_t(N) * uint32_t(sizeof(T));
    for (int kk = 0; kk < a.K; ++kk) {
        const int64_t row = (int64_t(b) * a.K + kk) * W + wave;
        if (row >= a.M)
            break; // uniform over the wave; no barrier in this loop
        const int64_t byte0 = row * int64_t(row_bytes);
        const rsrc_t xs = make_rsrc(static_cast<const char *>(a.x) + byte0, row_bytes);
        const rsrc_t ds = make_rsrc(static_cast<const char *>(a.dy) + byte0, row_bytes);
        Raw xr[SPLIT_VPL], dr[SPLIT_VPL];
#pragma unroll
        for (int k = 0; k < SPLIT_VPL; ++k) {
            xr[k] = BIO::load(xs, off[k]);
            dr[k] = BIO::load(ds, off[k]);
        }
        const float mean = RMS ? 0.f : a.mean[row];
        float rstd = recompute ? 0.f : a.rstd[row];
        float c1 = 0.f, c2 = 0.f;
        if constexpr (PASS == 0) {
            // row sums over the chunk, g = dy * gamma (invalid columns hold 0):
            //   LN: sum g (x - mean), sum g;  RMS: sum g x (, sum x^2)
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int k = 0; k < SPLIT_VPL; ++k) {
                float xv[VEC], dv[VEC], gv[VEC];
                IO::unpack(xr[k], xv);
                IO::unpack(dr[k], dv);
                IO::unpack(pg[k], gv);
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float g = dv[e] * gv[e];
                    if constexpr (!RMS) {
                        s0 = fmaf(g, xv[e] - mean, s0);
                        s1 += g;
                    } else {
                        s0 = fmaf(g, xv[e], s0);
                        if (recompute)
                            s1 = fmaf(xv[e], xv[e], s1);
                    }
                }
            }
            s0 = group_reduce<64, OpSum>(s0);
            s1 = group_reduce<64, OpSum>(s1);
            if (lane == 0) {
                a.rowsums[(row * S + s) * 2] = s0;
                a.rowsums[(row * S + s) * 2 + 1] = s1;
            }
        } else {
            // the row's sums: the chunks' sums added in chunk order
            float s0 = 0.f, s1 = 0.f;
            for (int q = 0; q < S; ++q) {
                s0 += a.rowsums[(row * S + q) * 2];
                s1 += a.rowsums[(row * S + q) * 2 + 1];
            }
            if (recompute)
                rstd = rsqrtf(s1 / float(N) + a.eps);
            c1 = rstd * (s0 / float(N));
            c2 = RMS ? 0.f : s1 / float(N);
        }
        const float k1 = -rstd * c1, k2 = -rstd * c2;
        const rsrc_t dxs = make_rsrc(static_cast<char *>(a.dx) + byte0, row_bytes);
#pragma unroll
        for (int k = 0; k < SPLIT_VPL; ++k) {
            float xv[VEC], dv[VEC], gv[VEC], dxv[VEC];
            IO::unpack(xr[k], xv);
            IO::unpack(dr[k], dv);
            IO::unpack(pg[k], gv);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int i = k * VEC + e;
                const float xh = RMS ? xv[e] * rstd : (xv[e] - mean) * rstd;
                if (add_gb && cvalid[k]) {
                    acc_g[i] = fmaf(dv[e], xh, acc_g[i]);
                    acc_b[i] += dv[e];
                }
                if constexpr (PASS == 1) {
                    dxv[e] = fmaf(xh, k1, fmaf(dv[e] * gv[e], rstd, k2));
                    if constexpr (DB)
                        if (cvalid[k])
                            acc_d[i] += dxv[e];
                }
            }
            if constexpr (PASS == 1)
                BIO::store(dxs, off[k], IO::pack(dxv), row >= a.wt_group);
        }
    }

    // ---- fold the four waves' partials (wave order) into row b ----
    const int64_t ld = colsum_ld(N);
    auto fold_store = [&](const float *acc, float *dst) {
#pragma unroll
        for (int k = 0; k < SPLIT_VPL; ++k) {
            const int c = (k * 64 + lane) * VEC;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                fold[wave][c + e] = acc[k * VEC + e];
        }
        __syncthreads();
        for (int c = threadIdx.x; c < C; c += 64 * W) {
            const int col = s * C + c;
            float v = fold[0][c];
#pragma unroll
            for (int w = 1; w < W; ++w)
                v += fold[w][c];
            if (col < N)
                dst[col] = v;
        }
        __syncthreads();
    };
    if (add_gb) { // uniform
        fold_store(acc_g, a.ws + (int64_t)b * ld);
        fold_store(acc_b, a.ws + (int64_t)gridDim.y * ld + (int64_t)b * ld);
    }
    if (add_d)
        fold_store(acc_d, a.ws + 2 * (int64_t)gridDim.y * ld + (int64_t)b * ld);
}

// ---------------------------------------------------------------------------
// Row softmax in one pass over HBM: per row group the rows are loaded once,
// the team takes the row max, then sum_j exp(x_j - max) with the exponentials
// kept in registers, and stores exp(x_j - max) / sum.
// ---------------------------------------------------------------------------
// Whether the softmax walk keeps the next row group's loads in flight: on
// wide teams whose lanes hold at most 16 bytes of a row, whose one load per
// lane otherwise leaves the memory system idle through the two team
// reductions.  Measured on MI355X (bf16, us, without / with): 26214 x 2560
// 55.9 / 51.9, 21845 x 3072 51.4 / 46.6, 16384 x 4096 46.9 / 45.1, fp32
// 16384 x 2048 44.7 / 43.3; lanes holding more lost up to 3% with it
// (8192 x 12288: 66.3 / 68.2).
template <typename T, int VEC, int LPR, int VPL, int TEAMS>
constexpr bool softmax_prefetch()
{
    return LPR >= WIDE_LPR && VPL * VEC * int(sizeof(T)) <= 16;
}

template <typename T, int VEC, int LPR, int VPL, int TEAMS>
__global__ void __launch_bounds__(LPR *TEAMS) softmax_kernel(const SoftmaxArgs a)
{
    using IO = VecIO<T, VEC>;
    using BIO = BufIO<T, VEC>;
    using Raw = typename IO::Raw;
    constexpr int WG = LPR * TEAMS;
    constexpr bool PREFETCH = softmax_prefetch<T, VEC, LPR, VPL, TEAMS>();
    static_assert(WG % 64 == 0, "workgroup of whole waves");

    __shared__ float red_lds[TeamLds<LPR, TEAMS, 1>::size];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int team = tid / LPR;
    const int tl = tid % LPR;
    const int wave_in_team = LPR > 64 ? tl / 64 : 0;
    const int N = a.N;

    bool cvalid[VPL];
    uint32_t off[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        cvalid[k] = (k * LPR + tl) * VEC < N;
        off[k] = cvalid[k] ? uint32_t(team * N + (k * LPR + tl) * VEC) * uint32_t(sizeof(T))
                           : BUF_OOB;
    }

    // x of row group g (zeros outside the matrix)
    Raw xn[VPL];
    auto issue = [&](int64_t g) {
        const RowGroup rg(g, TEAMS, a.M, N, sizeof(T));
        const rsrc_t xs = make_rsrc(static_cast<const char *>(a.x) + rg.byte0, rg.bytes);
#pragma unroll
        for (int k = 0; k < VPL; ++k)
            xn[k] = BIO::load(xs, off[k]);
    };

    int parity = 0;
    const GroupWalk walk(a.K, a.A);
    if (PREFETCH)
        issue(walk.group(0));
    for (int kk = 0; kk < a.K; ++kk) {
        const int64_t grp = walk.group(kk);
        if (grp >= a.n_groups)
            break; // uniform over the workgroup; later groups are larger
        const RowGroup rg(grp, TEAMS, a.M, N, sizeof(T));
        if (!PREFETCH)
            issue(grp);
        Raw xr[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k)
            xr[k] = xn[k];
        const int64_t next = walk.group(kk + 1);
        if (PREFETCH && kk + 1 < a.K && next < a.n_groups)
            issue(next); // in flight during this group's work

        // row max (columns past N do not take part)
        float m[1] = {-INFINITY};
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            if (cvalid[k]) {
                float v[VEC];
                IO::unpack(xr[k], v);
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    m[0] = fmaxf(m[0], v[e]);
            }
        }
        team_reduce<LPR, TEAMS, 1, OpMax>(m, red_lds, parity, team, wave_in_team, lane);

        // exponentials and their sum
        float ev[VPL][VEC];
        float sum[1] = {0.f};
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float v[VEC];
            IO::unpack(xr[k], v);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                ev[k][e] = cvalid[k] ? __expf(v[e] - m[0]) : 0.f;
                sum[0] += ev[k][e];
            }
        }
        team_sum<LPR, TEAMS, 1>(sum, red_lds, parity, team, wave_in_team, lane);
        const float inv = 1.f / sum[0];

        const rsrc_t ys = make_rsrc(static_cast<char *>(a.y) + rg.byte0, rg.bytes);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float yv[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                yv[e] = ev[k][e] * inv;
            BIO::store(ys, off[k], IO::pack(yv), grp >= a.wt_group);
        }
    }
}

template <typename T, int VEC, int LPR, int VPL, int TEAMS>
hipError_t launch_softmax(const SoftmaxArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((softmax_kernel<T, VEC, LPR, VPL, TEAMS>), dim3(grid), dim3(LPR * TEAMS),
                       0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Backward stage 2: column sums of the partial rows.  src holds gridDim.z
// blocks (dgamma, dbeta, dbias) of `rows` rows of N floats, each row padded
// to colsum_ld(N) floats so that a thread reads 16-byte vectors of 4 columns.
// Workgroup (column tile, slice s, block) adds rows [s*span, min(rows,
// (s+1)*span)) of its 4*QUADS columns with QUADS x SUB threads: thread
// (q, t) takes rows t, t + SUB, t + 2 SUB, ... of the slice in ascending
// order, RPT of them per pass with all RPT loads in flight at once (one
// memory round trip per pass; the launches size SUB * RPT to cover a slice
// in one pass).  The SUB row subsets of a column are then added in a fixed
// tree: within a wave by xor-shuffles over the subsets it holds (64 / QUADS
// of them), then the waves' sums in wave order.  FINAL: one slice; divide
// by `divisor` (1, or M for the mean over the rows), down-cast and store to
// dgamma / dbeta / dbias.  Otherwise slice s stores its sums as row s of dst
// (blocks of gridDim.y rows), which a FINAL launch then adds.  Every
// addition happens in a fixed order.
// ---------------------------------------------------------------------------
template <bool FINAL, bool BF16_OUT, int QUADS, int SUB, int RPT>
__global__ void __launch_bounds__(QUADS *SUB)
    colsum_kernel(const float *src, int rows, int N, int span, float *dst, void *dgamma,
                  void *dbeta, void *dbias, float divisor)
{
    static_assert(QUADS <= 64 && 64 % QUADS == 0 && (QUADS * SUB) % 64 == 0, "layout");
    constexpr int NWAVE = QUADS * SUB / 64;
    const int tq = threadIdx.x % QUADS;
    const int ty = threadIdx.x / QUADS;
    const int wave = threadIdx.x / 64;
    const int which = blockIdx.z;
    void *out = which == 0 ? dgamma : (which == 1 ? dbeta : dbias);
    if (FINAL && out == nullptr)
        return; // uniform over the block
    const int64_t ld = colsum_ld(N);
    const int j0 = blockIdx.x * (4 * QUADS) + tq * 4;
    const int s = blockIdx.y;
    const int r0 = s * span;
    const int nr = max(0, min(rows, r0 + span) - r0); // rows of this slice
    // the slice's rows, and nothing else, in range of the descriptor: loads
    // of rows past the slice (and of columns past N) return zeros
    const float *part = src + ((int64_t)which * rows + r0) * ld;
    const rsrc_t rs = make_rsrc(part, uint32_t(nr) * uint32_t(ld) * 4u);
    const bool cv = j0 < N; // columns j0 .. j0+3 lie within the padded row
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int rb = 0; rb < nr; rb += SUB * RPT) { // uniform
        f32x4_t v[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const uint32_t r = uint32_t(rb + ty + i * SUB);
            const uint32_t off = cv ? (r * uint32_t(ld) + uint32_t(j0)) * 4u : BUF_OOB;
            v[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, int(off), 0, 0));
        }
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            acc.x += v[i].x;
            acc.y += v[i].y;
            acc.z += v[i].z;
            acc.w += v[i].w;
        }
    }
#pragma unroll
    for (int m = QUADS; m < 64; m <<= 1) {
        acc.x += __shfl_xor(acc.x, m);
        acc.y += __shfl_xor(acc.y, m);
        acc.z += __shfl_xor(acc.z, m);
        acc.w += __shfl_xor(acc.w, m);
    }
    __shared__ f32x4_t sl[NWAVE][QUADS];
    if ((threadIdx.x & 63) < QUADS)
        sl[wave][tq] = acc;
    __syncthreads();
    if (threadIdx.x < QUADS && cv) {
        f32x4_t t = sl[0][tq];
#pragma unroll
        for (int w = 1; w < NWAVE; ++w) {
            const f32x4_t u = sl[w][tq];
            t.x += u.x;
            t.y += u.y;
            t.z += u.z;
            t.w += u.w;
        }
        const float tv[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = j0 + e;
            if (j >= N)
                break;
            float v = tv[e];
            if constexpr (FINAL)
                v = v / divisor; // 1, or M for the row mean
            if constexpr (!FINAL) {
                dst[((int64_t)which * gridDim.y + s) * ld + j] = v;
            } else if constexpr (BF16_OUT) {
                static_cast<uint16_t *>(out)[j] = uint16_t(pack_bf16x2(v, 0.f) & 0xffffu);
            } else {
                static_cast<float *>(out)[j] = v;
            }
        }
    }
}

template <typename T, int VEC, int LPR, int VPL, int TEAMS, bool RMS, bool F8>
hipError_t launch_fwd(const FwdArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((fwd_kernel<T, VEC, LPR, VPL, TEAMS, RMS, F8>), dim3(grid),
                       dim3(LPR * TEAMS), 0, s, a);
    return hipGetLastError();
}

template <typename T, int VEC, int LPR, int VPL, int TEAMS, bool RMS, bool DB>
hipError_t launch_bwd(const BwdArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((bwd_kernel<T, VEC, LPR, VPL, TEAMS, RMS, DB>), dim3(grid),
                       dim3(LPR * TEAMS), 0, s, a);
    return hipGetLastError();
}

} // namespace nf
