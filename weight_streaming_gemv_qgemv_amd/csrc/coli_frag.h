// coli_frag.h -- device helpers of the matrix-core kernels (gfx950): weight
// codes, the activation fragment order, loads and the bf16 MFMA step.
//
// The products are the pages' dequant-on-use matrix-vector products
// [glm.c@98759bf -- matmul_q, matmul_i4, matmul_i2; metal@93cde63 -- mm_gemv,
// moe_gemv] arranged for v_mfma_f32_16x16x32_bf16:
//   * each int8 / int4 / int2 weight value v becomes an exact bf16 "code"
//     v + OFF; OFF * sum(x) is removed per output after the sum;
//   * activations are bf16 (once rounded, or an exact-to-2^-16 hi + lo pair);
//   * inside each group of 8 (int4, int8) or 16 (int2) elements the k order is
//     the order the unpacking produces, and activations are stored in that
//     order ("fragment order"), so no shuffle is needed in the product loop.
#ifndef COLI_FRAG_H
#define COLI_FRAG_H

#include "coli_device.h"

namespace coli {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <int FMT> struct MF;
// A k-block of one weight row is SEGS x 64 bytes: lane group q (= lane / 16)
// reads 16-byte segment sg at byte 64 sg + 16 q, so one load instruction
// covers 64 contiguous bytes of each of its 16 rows and the SEGS = 2 loads of
// a k-block consume whole 128-byte lines.  SPS: 8-element MFMA steps per
// segment; STEPS = SEGS * SPS; KB: elements per k-block; OFF: code - value.
template <> struct MF<kI8> { static constexpr int BITS = 8, SEGS = 2, SPS = 2, STEPS = 4, KB = 128; static constexpr float OFF = 128.f; };
template <> struct MF<kI4> { static constexpr int BITS = 4, SEGS = 2, SPS = 4, STEPS = 8, KB = 256; static constexpr float OFF = 136.f; };
template <> struct MF<kI2> { static constexpr int BITS = 2, SEGS = 1, SPS = 8, STEPS = 8, KB = 256; static constexpr float OFF = 130.f; };

__device__ __forceinline__ uint32_t wsel(const uint4 &v, int d)
{
    return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

// Constants hidden from constant folding (an empty asm statement emits no
// instruction): with the mask in a scalar register and the exponent pattern
// in a vector register, (a & m) | o becomes one v_and_or_b32 -- with literal
// operands it would be an AND and an OR.
__device__ __forceinline__ uint32_t opaque_s(uint32_t v)
{
    asm("" : "+s"(v));
    return v;
}
__device__ __forceinline__ uint32_t opaque_v(uint32_t v)
{
    asm("" : "+v"(v));
    return v;
}

// bf16 codes for MFMA step s (8 elements) of a 16-byte segment.
template <int FMT> __device__ __forceinline__ uint4 codes(const uint4 &w, int s);

// int4: word s holds nibbles n0..n7; the pairs (n_i, n_i+4) sit at bits
// 4i and 4i+16, so (word >> 4i) & 0x000F000F | 0x43004300 is the bf16 pair
// (128 + n_i, 128 + n_i+4).  Slot order [0,4,1,5,2,6,3,7].
template <> __device__ __forceinline__ uint4 codes<kI4>(const uint4 &w, int s)
{
    const uint32_t u = wsel(w, s);
    const uint32_t m = opaque_s(0x000F000Fu), e = opaque_v(0x43004300u);
    return make_uint4((u & m) | e, ((u >> 4) & m) | e, ((u >> 8) & m) | e, ((u >> 12) & m) | e);
}

// int2: word s/2 holds crumbs c0..c15; (word >> 2k) & 0x00030003 | 0x43004300
// is the pair (128 + c_k, 128 + c_k+8).  Step s covers k = 4(s&1) .. +3.
// Slot order [0,8,1,9,2,10,3,11 | 4,12,5,13,6,14,7,15].
template <> __device__ __forceinline__ uint4 codes<kI2>(const uint4 &w, int s)
{
    const uint32_t u = wsel(w, s >> 1);
    const int k0 = 4 * (s & 1);
    const uint32_t m = opaque_s(0x00030003u), e = opaque_v(0x43004300u);
    return make_uint4(((u >> (2 * k0)) & m) | e, ((u >> (2 * k0 + 2)) & m) | e,
                      ((u >> (2 * k0 + 4)) & m) | e, ((u >> (2 * k0 + 6)) & m) | e);
}

// int8: bytes 8s..8s+7, sign bit flipped (code = v + 128 in 0..255, exact
// in bf16: the fp32 value's low half is zero), natural order.
__device__ __forceinline__ uint32_t bf_pair_of_bytes(uint32_t b, int k)
{
    const uint32_t f0 = __float_as_uint((float)((b >> (8 * k)) & 0xFFu));
    const uint32_t f1 = __float_as_uint((float)((b >> (8 * k + 8)) & 0xFFu));
    return __builtin_amdgcn_perm(f1, f0, 0x07060302u);
}
template <> __device__ __forceinline__ uint4 codes<kI8>(const uint4 &w, int s)
{
    const uint32_t b0 = wsel(w, 2 * s) ^ 0x80808080u, b1 = wsel(w, 2 * s + 1) ^ 0x80808080u;
    return make_uint4(bf_pair_of_bytes(b0, 0), bf_pair_of_bytes(b0, 2), bf_pair_of_bytes(b1, 0),
                      bf_pair_of_bytes(b1, 2));
}

// codes<FMT>(w, s) with the word(s) step s reads first passed through an
// empty asm statement: the compiler can then neither compute them ahead of
// that point nor merge them with an identical computation on another path.
template <int FMT> __device__ __forceinline__ uint4 codes_late(const uint4 &w, int s)
{
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if constexpr (FMT == kI8) {
        uint32_t a = wsel(w, 2 * s), b = wsel(w, 2 * s + 1);
        asm volatile("" : "+v"(a), "+v"(b));
        if (s == 0) { v.x = a; v.y = b; }
        else { v.z = a; v.w = b; }
        return codes<FMT>(v, s);
    } else {
        const int d = FMT == kI4 ? s : s >> 1;
        uint32_t a = wsel(w, d);
        asm volatile("" : "+v"(a));
        v.x = a;
        return codes<FMT>(v, FMT == kI4 ? 0 : (s & 1));
    }
}

__device__ __forceinline__ uint16_t bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Loads through the global address space: a flat load counts on both the
// vector-memory and the LDS counters and may return out of order, which makes
// the compiler wait for every outstanding load before the first use.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 g_u32x4;
typedef __attribute__((address_space(1))) const float g_float;
__device__ __forceinline__ uint4 gload16(const void *p)
{
    const u32x4 v = *(g_u32x4 *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float gloadf(const float *p) { return *(g_float *)p; }
// A streaming load (non-temporal hint): data read once, kept out of the way
// of the small tables that are reused from L2.
__device__ __forceinline__ uint4 gload16_nt(const void *p)
{
    const u32x4 v = __builtin_nontemporal_load((g_u32x4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const f32x4 g_f32x4;
__device__ __forceinline__ float4 gload4f(const float *p)
{
    const f32x4 v = *(g_f32x4 *)p;
    return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ floatx4 mfma(const uint4 &a, const uint4 &b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int FMT> __device__ __forceinline__ int elem_of(int kbi, int s, int q, int j)
{
    using T = MF<FMT>;
    const int sg = s / T::SPS, sub = s % T::SPS;
    const int first = kbi * T::KB + (64 * sg + 16 * q) * 8 / T::BITS;
    if constexpr (FMT == kI4) return first + 8 * sub + (j >> 1) + 4 * (j & 1);
    if constexpr (FMT == kI8) return first + 8 * sub + j;
    return first + 16 * (sub >> 1) + 4 * (sub & 1) + (j >> 1) + 8 * (j & 1);
}

template <int FMT> __device__ __forceinline__ void pos_of(int e, int &c, int &j)
{
    using T = MF<FMT>;
    const int kbi = e / T::KB, r = e % T::KB;
    const int byte = r * T::BITS / 8;
    const int sg = byte / 64, q = (byte % 64) / 16;
    const int u = r - (64 * sg + 16 * q) * 8 / T::BITS;   // element inside the 16-byte segment
    int sub;
    if constexpr (FMT == kI4) {
        sub = u >> 3;
        const int v = u & 7;
        j = 2 * (v & 3) + (v >> 2);
    } else if constexpr (FMT == kI8) {
        sub = u >> 3;
        j = u & 7;
    } else {
        const int uu = u & 15, k = uu & 7;
        sub = 2 * (u >> 4) + (k >> 2);
        j = 2 * (k & 3) + (uu >> 3);
    }
    c = (kbi * T::STEPS + sg * T::SPS + sub) * 4 + q;
}

// Tiled weight layout (coli_pack_tiled): a matrix is cut into 1 KB units of
// 16 rows x 64 bytes, each unit in the A-operand lane order (lane 16 q + c
// holds row c's bytes 16 q .. 16 q + 15 of the segment), so a wave loads a
// row tile's segment with one contiguous 1 KB load and needs no transpose.
// Units are ordered by groups of kTileGroup row tiles (128 rows), inside a
// group by segment, then by row tile: the units of one group and one k-block
// are one contiguous run.  ns = segments per row (ceil(rb / 64)), mt16 = row
// tiles (ceil(O / 16)).
constexpr int kTileGroup = 8;
// byte offset of unit (m, 0)
__device__ __forceinline__ uint32_t tiled_base(int m, int ns)
{
    const int T = m / kTileGroup, mm = m - T * kTileGroup;
    return (uint32_t)(T * kTileGroup * ns + mm) * 1024u;
}
// bytes from unit (m, g) to unit (m, g + 1)
__device__ __forceinline__ uint32_t tiled_gstride(int m, int mt16)
{
    const int T = m / kTileGroup;
    return (uint32_t)min(kTileGroup, mt16 - T * kTileGroup) * 1024u;
}

// Work-list and group-offset reads: written by an earlier kernel and never
// written here, so they are read through the constant address space (scalar
// loads) when the index is uniform.
__device__ __forceinline__ int cload(const int *p)
{
    return *(__attribute__((address_space(4))) const int *)p;
}

}  // namespace
}  // namespace coli

#endif
