// coli_device.h -- device helpers shared by libcoli's kernels (gfx950, wave64).
#ifndef COLI_DEVICE_H
#define COLI_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coli {

constexpr int kWave = 64;

// Row formats (same codes as the public enum coli_fmt).
enum : int { kF32 = 0, kI8 = 1, kI4 = 2, kI2 = 3 };

// Per-format facts for a 16-byte load of one packed row:
//   EPS  elements carried by 16 bytes;
//   OFF  constant the unpacked "code" exceeds the true value by. The kernels
//        multiply codes (not values) by x and subtract OFF * sum(x) once per
//        row, which saves one subtract per element: the int8 byte is read as
//        an unsigned byte after flipping its sign bit (code = v + 128), a
//        nibble as 0..15 (code = v + 8), a crumb as 0..3 (code = v + 2).
template <int FMT> struct Fmt;
template <> struct Fmt<kF32> { static constexpr int EPS = 4;  static constexpr float OFF = 0.f; };
template <> struct Fmt<kI8>  { static constexpr int EPS = 16; static constexpr float OFF = 128.f; };
template <> struct Fmt<kI4>  { static constexpr int EPS = 32; static constexpr float OFF = 8.f; };
template <> struct Fmt<kI2>  { static constexpr int EPS = 64; static constexpr float OFF = 2.f; };

// Unpack one 32-bit word of a packed row into its EPS/4 codes, in element
// order.  Element order inside a byte follows the pages' layouts:
//   int4: element 2k = low nibble of byte k, 2k+1 = high nibble;
//   int2: element 4k+j = bits 2j..2j+1 of byte k.
// Each byte-to-float conversion is one v_cvt_f32_ubyte{0..3}.
__device__ __forceinline__ float ubyte_f(uint32_t u, int k)
{
    return (float)((u >> (8 * k)) & 0xFFu);
}

template <int FMT> __device__ __forceinline__ void unpack_word(uint32_t u, float *c);

template <> __device__ __forceinline__ void unpack_word<kF32>(uint32_t u, float *c)
{
    c[0] = __uint_as_float(u);
}

template <> __device__ __forceinline__ void unpack_word<kI8>(uint32_t u, float *c)
{
    uint32_t b = u ^ 0x80808080u;  // signed byte v -> unsigned v + 128
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = ubyte_f(b, k);
}

template <> __device__ __forceinline__ void unpack_word<kI4>(uint32_t u, float *c)
{
    uint32_t lo = u & 0x0F0F0F0Fu;
    uint32_t hi = (u >> 4) & 0x0F0F0F0Fu;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        c[2 * k] = ubyte_f(lo, k);
        c[2 * k + 1] = ubyte_f(hi, k);
    }
}

template <> __device__ __forceinline__ void unpack_word<kI2>(uint32_t u, float *c)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t m = (u >> (2 * j)) & 0x03030303u;
#pragma unroll
        for (int k = 0; k < 4; ++k) c[4 * k + j] = ubyte_f(m, k);
    }
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64);
// every lane of a group ends with the group's total.
__device__ __forceinline__ float group_sum(float v, int width)
{
    for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ double wave_sum_d(double v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

}  // namespace coli

#endif
