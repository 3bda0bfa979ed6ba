// device.hpp -- gfx950 device helpers shared by the normalisation kernels:
// 16-byte vector I/O of fp32 / bf16 rows with fp32 compute, bf16 rounding to
// nearest-even through the hardware converter, and wave64 group reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf {

// bf16 storage tag: the upper half of a binary32 pattern.
struct bf16 {
    uint16_t bits;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (round to nearest, ties to even; v_cvt_pk_bf16_f32),
// element `a` in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------------------
// Register forms.  VecIO<T, VEC> converts VEC consecutive elements of type T
// between their packed register form `Raw` (what one 16-, 8- or 4-byte
// access per lane, or one element, VEC = 1, brings in; see BufIO below) and
// floats.  pack() rounds to T (nearest, ties to even); unpack() widens
// exactly.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename T, int VEC>
struct VecIO;

template <>
struct VecIO<bf16, 8> {
    using Raw = u32x4_t;
    static __device__ __forceinline__ void unpack(const Raw &r, float *f)
    {
        f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x);
        f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
        f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z);
        f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
    }
    static __device__ __forceinline__ Raw pack(const float *f)
    {
        return Raw{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                   pack_bf16x2(f[6], f[7])};
    }
    static __device__ __forceinline__ Raw zero() { return Raw{0u, 0u, 0u, 0u}; }
};

template <>
struct VecIO<bf16, 4> {
    using Raw = u32x2_t;
    static __device__ __forceinline__ void unpack(const Raw &r, float *f)
    {
        f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x);
        f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
    }
    static __device__ __forceinline__ Raw pack(const float *f)
    {
        return Raw{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])};
    }
    static __device__ __forceinline__ Raw zero() { return Raw{0u, 0u}; }
};

template <>
struct VecIO<bf16, 2> {
    using Raw = uint32_t;
    static __device__ __forceinline__ void unpack(const Raw &r, float *f)
    {
        f[0] = bf16_lo(r); f[1] = bf16_hi(r);
    }
    static __device__ __forceinline__ Raw pack(const float *f) { return pack_bf16x2(f[0], f[1]); }
    static __device__ __forceinline__ Raw zero() { return 0u; }
};

template <>
struct VecIO<bf16, 1> {
    using Raw = uint16_t;
    static __device__ __forceinline__ void unpack(const Raw &r, float *f)
    {
        f[0] = __uint_as_float(uint32_t(r) << 16);
    }
    static __device__ __forceinline__ Raw pack(const float *f)
    {
        return uint16_t(pack_bf16x2(f[0], 0.f) & 0xffffu);
    }
    static __device__ __forceinline__ Raw zero() { return 0; }
};

template <>
struct VecIO<float, 4> {
    using Raw = f32x4_t;
    static __device__ __forceinline__ void unpack(const Raw &r, float *f)
    {
        f[0] = r.x; f[1] = r.y; f[2] = r.z; f[3] = r.w;
    }
    static __device__ __forceinline__ Raw pack(const float *f) { return Raw{f[0], f[1], f[2], f[3]}; }
    static __device__ __forceinline__ Raw zero() { return Raw{0.f, 0.f, 0.f, 0.f}; }
};

template <>
struct VecIO<float, 2> {
    using Raw = f32x2_t;
    static __device__ __forceinline__ void unpack(const Raw &r, float *f)
    {
        f[0] = r.x; f[1] = r.y;
    }
    static __device__ __forceinline__ Raw pack(const float *f) { return Raw{f[0], f[1]}; }
    static __device__ __forceinline__ Raw zero() { return Raw{0.f, 0.f}; }
};

template <>
struct VecIO<float, 1> {
    using Raw = float;
    static __device__ __forceinline__ void unpack(const Raw &r, float *f) { f[0] = r; }
    static __device__ __forceinline__ Raw pack(const float *f) { return f[0]; }
    static __device__ __forceinline__ Raw zero() { return 0.f; }
};

// ---------------------------------------------------------------------------
// Buffer I/O for streamed [M, N] tensors.  A buffer descriptor covers the
// valid bytes of one row group (uniform, scalar registers); each lane adds a
// 32-bit byte offset.  Accesses beyond the descriptor's range read 0 and
// write nothing, so rows past M and columns past N need no predication: such
// lanes use an offset past the range (BUF_OOB).  Loads carry the
// nontemporal hint; stores too, or the write-through policy (BUF_WT).
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t BUF_OOB = 0x80000000u; // above any row group's byte range
constexpr int BUF_NT = 2;                 // cache policy: nontemporal
// Stores marked with system-scope coherence (sc0 sc1) are written through
// the L2 instead of being held there dirty.  Streams store this way from
// their last row groups on: what the L2 still holds dirty when a kernel ends
// is written back before the kernel counts as complete, a few microseconds
// that short kernels feel.  Earlier row groups keep the nontemporal policy,
// which streams slightly faster.
constexpr int BUF_WT = 17;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    // raw buffer: stride 0, num_records in bytes, gfx9 word-3 format bits
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, int(bytes), 0x00020000);
}

template <typename T, int VEC>
struct BufIO;

template <>
struct BufIO<bf16, 8> {
    using Raw = u32x4_t;
    static __device__ __forceinline__ Raw load(rsrc_t r, uint32_t off)
    {
        return __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, BUF_NT);
    }
    static __device__ __forceinline__ Raw load_cached(rsrc_t r, uint32_t off)
    {
        return __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0);
    }
    static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, Raw v, bool wt)
    {
        if (wt)
            __builtin_amdgcn_raw_buffer_store_b128(v, r, int(off), 0, BUF_WT);
        else
            __builtin_amdgcn_raw_buffer_store_b128(v, r, int(off), 0, BUF_NT);
    }
};
template <>
struct BufIO<float, 4> {
    using Raw = f32x4_t;
    static __device__ __forceinline__ Raw load(rsrc_t r, uint32_t off)
    {
        return __builtin_bit_cast(Raw, __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, BUF_NT));
    }
    static __device__ __forceinline__ Raw load_cached(rsrc_t r, uint32_t off)
    {
        return __builtin_bit_cast(Raw, __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0));
    }
    static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, Raw v, bool wt)
    {
        if (wt)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, int(off), 0, BUF_WT);
        else
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, int(off), 0, BUF_NT);
    }
};
template <>
struct BufIO<bf16, 4> {
    using Raw = u32x2_t;
    static __device__ __forceinline__ Raw load(rsrc_t r, uint32_t off)
    {
        return __builtin_amdgcn_raw_buffer_load_b64(r, int(off), 0, BUF_NT);
    }
    static __device__ __forceinline__ Raw load_cached(rsrc_t r, uint32_t off)
    {
        return __builtin_amdgcn_raw_buffer_load_b64(r, int(off), 0, 0);
    }
    static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, Raw v, bool wt)
    {
        if (wt)
            __builtin_amdgcn_raw_buffer_store_b64(v, r, int(off), 0, BUF_WT);
        else
            __builtin_amdgcn_raw_buffer_store_b64(v, r, int(off), 0, BUF_NT);
    }
};
template <>
struct BufIO<bf16, 2> {
    using Raw = uint32_t;
    static __device__ __forceinline__ Raw load(rsrc_t r, uint32_t off)
    {
        return __builtin_amdgcn_raw_buffer_load_b32(r, int(off), 0, BUF_NT);
    }
    static __device__ __forceinline__ Raw load_cached(rsrc_t r, uint32_t off)
    {
        return __builtin_amdgcn_raw_buffer_load_b32(r, int(off), 0, 0);
    }
    static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, Raw v, bool wt)
    {
        if (wt)
            __builtin_amdgcn_raw_buffer_store_b32(v, r, int(off), 0, BUF_WT);
        else
            __builtin_amdgcn_raw_buffer_store_b32(v, r, int(off), 0, BUF_NT);
    }
};
template <>
struct BufIO<float, 2> {
    using Raw = f32x2_t;
    static __device__ __forceinline__ Raw load(rsrc_t r, uint32_t off)
    {
        return __builtin_bit_cast(Raw, __builtin_amdgcn_raw_buffer_load_b64(r, int(off), 0, BUF_NT));
    }
    static __device__ __forceinline__ Raw load_cached(rsrc_t r, uint32_t off)
    {
        return __builtin_bit_cast(Raw, __builtin_amdgcn_raw_buffer_load_b64(r, int(off), 0, 0));
    }
    static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, Raw v, bool wt)
    {
        if (wt)
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), r, int(off), 0, BUF_WT);
        else
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), r, int(off), 0, BUF_NT);
    }
};
template <>
struct BufIO<bf16, 1> {
    using Raw = uint16_t;
    static __device__ __forceinline__ Raw load(rsrc_t r, uint32_t off)
    {
        return __builtin_amdgcn_raw_buffer_load_b16(r, int(off), 0, BUF_NT);
    }
    static __device__ __forceinline__ Raw load_cached(rsrc_t r, uint32_t off)
    {
        return __builtin_amdgcn_raw_buffer_load_b16(r, int(off), 0, 0);
    }
    static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, Raw v, bool wt)
    {
        if (wt)
            __builtin_amdgcn_raw_buffer_store_b16(v, r, int(off), 0, BUF_WT);
        else
            __builtin_amdgcn_raw_buffer_store_b16(v, r, int(off), 0, BUF_NT);
    }
};
template <>
struct BufIO<float, 1> {
    using Raw = float;
    static __device__ __forceinline__ Raw load(rsrc_t r, uint32_t off)
    {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, int(off), 0, BUF_NT));
    }
    static __device__ __forceinline__ Raw load_cached(rsrc_t r, uint32_t off)
    {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, int(off), 0, 0));
    }
    static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, Raw v, bool wt)
    {
        if (wt)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, int(off), 0, BUF_WT);
        else
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, int(off), 0, BUF_NT);
    }
};

// ---------------------------------------------------------------------------
// FP8 output: VEC fp32 values, each already scaled, to OCP FP8 E4M3 codes
// (round to nearest even by the hardware convert, which turns magnitudes
// beyond the format into NaN, so they are first clamped to +-448, the
// largest finite E4M3 value) stored as VEC bytes at byte offset `off`.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sat_e4m3(float v)
{
    return __builtin_amdgcn_fmed3f(v, -448.f, 448.f);
}

template <int VEC>
__device__ __forceinline__ void store_e4m3(rsrc_t r, uint32_t off, const float *v, bool wt)
{
    if constexpr (VEC == 8) {
        int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(v[0]), sat_e4m3(v[1]), 0, false);
        w0 = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(v[2]), sat_e4m3(v[3]), w0, true);
        int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(v[4]), sat_e4m3(v[5]), 0, false);
        w1 = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(v[6]), sat_e4m3(v[7]), w1, true);
        const u32x2_t w{unsigned(w0), unsigned(w1)};
        if (wt)
            __builtin_amdgcn_raw_buffer_store_b64(w, r, int(off), 0, BUF_WT);
        else
            __builtin_amdgcn_raw_buffer_store_b64(w, r, int(off), 0, BUF_NT);
    } else if constexpr (VEC == 4) {
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(v[0]), sat_e4m3(v[1]), 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(v[2]), sat_e4m3(v[3]), w, true);
        if (wt)
            __builtin_amdgcn_raw_buffer_store_b32(unsigned(w), r, int(off), 0, BUF_WT);
        else
            __builtin_amdgcn_raw_buffer_store_b32(unsigned(w), r, int(off), 0, BUF_NT);
    } else if constexpr (VEC == 2) {
        const int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(v[0]), sat_e4m3(v[1]), 0, false);
        const unsigned short h = static_cast<unsigned short>(w & 0xffff);
        if (wt)
            __builtin_amdgcn_raw_buffer_store_b16(h, r, int(off), 0, BUF_WT);
        else
            __builtin_amdgcn_raw_buffer_store_b16(h, r, int(off), 0, BUF_NT);
    } else {
        static_assert(VEC == 1, "FP8 store of 1, 2, 4 or 8 values");
        const int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(v[0]), 0.f, 0, false);
        const unsigned char b = static_cast<unsigned char>(w & 0xff);
        if (wt)
            __builtin_amdgcn_raw_buffer_store_b8(b, r, int(off), 0, BUF_WT);
        else
            __builtin_amdgcn_raw_buffer_store_b8(b, r, int(off), 0, BUF_NT);
    }
}

// FP8 codes of the 8 values of this lane and of its partner lane (lane ^ 1),
// whose 8 columns directly follow (even lane) or precede (odd lane) this
// lane's: the even lane stores both as one 16-byte vector when the partner's
// columns are valid, else its own 8 bytes; odd lanes store nothing.  Every
// lane of the wave must call it (the codes move across lanes).
__device__ __forceinline__ void store_e4m3_pair(rsrc_t r, uint32_t off, const float *v,
                                                bool even, bool partner_valid, bool wt)
{
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(v[0]), sat_e4m3(v[1]), 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(v[2]), sat_e4m3(v[3]), w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(v[4]), sat_e4m3(v[5]), 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(v[6]), sat_e4m3(v[7]), w1, true);
    const int p0 = __shfl_xor(w0, 1), p1 = __shfl_xor(w1, 1);
    if (!even)
        return;
    if (partner_valid) {
        const u32x4_t w{unsigned(w0), unsigned(w1), unsigned(p0), unsigned(p1)};
        if (wt)
            __builtin_amdgcn_raw_buffer_store_b128(w, r, int(off), 0, BUF_WT);
        else
            __builtin_amdgcn_raw_buffer_store_b128(w, r, int(off), 0, BUF_NT);
    } else {
        const u32x2_t w{unsigned(w0), unsigned(w1)};
        if (wt)
            __builtin_amdgcn_raw_buffer_store_b64(w, r, int(off), 0, BUF_WT);
        else
            __builtin_amdgcn_raw_buffer_store_b64(w, r, int(off), 0, BUF_NT);
    }
}

// VEC floats from LDS (16-byte reads when VEC is a multiple of 4).
template <int VEC>
__device__ __forceinline__ void lds_read(const float *p, float *out)
{
    if constexpr (VEC % 4 == 0) {
#pragma unroll
        for (int i = 0; i < VEC; i += 4) {
            const float4 v = *reinterpret_cast<const float4 *>(p + i);
            out[i] = v.x;
            out[i + 1] = v.y;
            out[i + 2] = v.z;
            out[i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            out[i] = p[i];
    }
}

// Opaque to the optimiser: after this the compiler must assume `r` changed,
// so values computed from it before (e.g. unpacked floats) are recomputed
// afterwards instead of being kept live.  Emits no instruction.
template <typename R>
__device__ __forceinline__ void reload_barrier(R &r)
{
    asm volatile("" : "+v"(r));
}

// Uses `r` (so the compiler first waits for the load that writes it) and
// keeps every memory access after this point from moving above it.  Emits no
// instruction.
template <typename R>
__device__ __forceinline__ void order_after_arrival(R &r)
{
    asm volatile("" : "+v"(r) : : "memory");
}

// ---------------------------------------------------------------------------
// Group reductions over aligned groups of W lanes of a wave64 (W a power of
// two, 1..64).  Every lane of a group receives the same bits: each step
// combines a lane with its partner by a commutative operation.
//   W <= 16 : DPP within a row of 16 lanes (quad_perm xor 1 / xor 2,
//             row_half_mirror, row_mirror)
//   W  = 32 : + v_permlane16_swap (rows 0<->1, 2<->3)
//   W  = 64 : + v_permlane32_swap (lanes 0-31 <-> 32-63)
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

struct OpSum {
    static __device__ __forceinline__ float apply(float a, float b) { return a + b; }
};
struct OpMax {
    static __device__ __forceinline__ float apply(float a, float b) { return fmaxf(a, b); }
};

template <class Op>
__device__ __forceinline__ float xor16_combine(float v)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return Op::apply(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <class Op>
__device__ __forceinline__ float xor32_combine(float v)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return Op::apply(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int W, class Op>
__device__ __forceinline__ float group_reduce(float v)
{
    static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "group width");
    if constexpr (W >= 2) v = Op::apply(v, dpp<0xB1>(v));  // quad_perm [1,0,3,2]
    if constexpr (W >= 4) v = Op::apply(v, dpp<0x4E>(v));  // quad_perm [2,3,0,1]
    if constexpr (W >= 8) v = Op::apply(v, dpp<0x141>(v)); // row_half_mirror
    if constexpr (W >= 16) v = Op::apply(v, dpp<0x140>(v)); // row_mirror
    if constexpr (W >= 32) v = xor16_combine<Op>(v);
    if constexpr (W >= 64) v = xor32_combine<Op>(v);
    return v;
}

// fp64 group sum over aligned groups of W lanes: the same exchange pattern
// applied to both 32-bit halves of each value.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_update_dpp(0, int(uint32_t(b)), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, int(uint32_t(b >> 32)), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo));
}

__device__ __forceinline__ double join_f64(uint32_t lo, uint32_t hi)
{
    return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
}

template <int W>
__device__ __forceinline__ double group_sum_f64(double v)
{
    static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "group width");
    if constexpr (W >= 2) v += dpp_f64<0xB1>(v);
    if constexpr (W >= 4) v += dpp_f64<0x4E>(v);
    if constexpr (W >= 8) v += dpp_f64<0x141>(v);
    if constexpr (W >= 16) v += dpp_f64<0x140>(v);
    if constexpr (W >= 32) {
        const uint64_t b = __builtin_bit_cast(uint64_t, v);
        auto lo = __builtin_amdgcn_permlane16_swap(uint32_t(b), uint32_t(b), false, false);
        auto hi = __builtin_amdgcn_permlane16_swap(uint32_t(b >> 32), uint32_t(b >> 32), false, false);
        v = join_f64(lo[0], hi[0]) + join_f64(lo[1], hi[1]);
    }
    if constexpr (W >= 64) {
        const uint64_t b = __builtin_bit_cast(uint64_t, v);
        auto lo = __builtin_amdgcn_permlane32_swap(uint32_t(b), uint32_t(b), false, false);
        auto hi = __builtin_amdgcn_permlane32_swap(uint32_t(b >> 32), uint32_t(b >> 32), false, false);
        v = join_f64(lo[0], hi[0]) + join_f64(lo[1], hi[1]);
    }
    return v;
}

// Combine the values of lanes l, l + W, l + 2W, ... (W < 64) so that every
// lane holds the sum over the lanes of the wave that share (lane mod W).
// Used to fold teams of W lanes that cover the same columns.
template <int W>
__device__ __forceinline__ float fold_teams_sum(float v)
{
    static_assert(W >= 1 && W <= 64, "team width");
    if constexpr (W <= 8) v += __shfl_xor(v, 8);
    if constexpr (W <= 4) v += __shfl_xor(v, 4);
    if constexpr (W <= 2) v += __shfl_xor(v, 2);
    if constexpr (W <= 1) v += __shfl_xor(v, 1);
    if constexpr (W <= 16) v = xor16_combine<OpSum>(v);
    if constexpr (W <= 32) v = xor32_combine<OpSum>(v);
    return v;
}

} // namespace nf
