// coli_xrows.h -- one run of an activation row table (device code shared by
// the decode row-table kernel and the one-launch grouping kernel).
#ifndef COLI_XROWS_H
#define COLI_XROWS_H

#include "coli_device.h"
#include "coli_frag.h"

namespace coli {

// Elements per run: 8 (one chunk), int2 16 (the chunks of an even/odd step
// pair).
template <int FMT> constexpr int xrows_run_len() { return FMT == kI2 ? 16 : 8; }

// Run r of row xr (I elements, zeros past I): split into bf16 hi/lo and
// stored in the row's table dst (2 kpad bf16) as the run's chunks' 16-byte
// hi and lo units, slot pairs in the order the weight unpacking produces
// the codes.  vec: xr is 16-byte aligned.
template <int FMT>
__device__ __forceinline__ void xrows_run(const float *__restrict__ xr, int I, int r,
                                          uint16_t *__restrict__ dst, int vec)
{
    constexpr int RUN = xrows_run_len<FMT>();
    const int e0 = r * RUN;
    float v[RUN];
    if (vec && e0 + RUN <= I) {
#pragma unroll
        for (int i = 0; i < RUN / 4; ++i) {
            const float4 f = *reinterpret_cast<const float4 *>(xr + e0 + 4 * i);
            v[4 * i] = f.x;
            v[4 * i + 1] = f.y;
            v[4 * i + 2] = f.z;
            v[4 * i + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < RUN; ++i) v[i] = e0 + i < I ? xr[e0 + i] : 0.f;
    }
    uint16_t hv[RUN], lv[RUN];
#pragma unroll
    for (int i = 0; i < RUN; ++i) {
        hv[i] = bf16_rne(v[i]);
        lv[i] = bf16_rne(v[i] - bf16_f(hv[i]));
    }
    // slot pairs (2m, 2m+1) of each chunk, in the order the unpacking
    // produces the weight codes
    int c, j;
    pos_of<FMT>(e0, c, j);
    uint32_t hw[RUN / 2], lw[RUN / 2];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        int k0, k1;
        if constexpr (FMT == kI8) { k0 = 2 * m; k1 = 2 * m + 1; }
        else if constexpr (FMT == kI4) { k0 = m; k1 = m + 4; }
        else { k0 = m; k1 = m + 8; }
        hw[m] = (uint32_t)hv[k0] | ((uint32_t)hv[k1] << 16);
        lw[m] = (uint32_t)lv[k0] | ((uint32_t)lv[k1] << 16);
        if constexpr (FMT == kI2) {
            hw[4 + m] = (uint32_t)hv[m + 4] | ((uint32_t)hv[m + 12] << 16);
            lw[4 + m] = (uint32_t)lv[m + 4] | ((uint32_t)lv[m + 12] << 16);
        }
    }
#pragma unroll
    for (int h = 0; h < RUN / 8; ++h) {
        uint16_t *u = dst + (int64_t)(c + 4 * h) * 16;   // chunk c + 4h: next MFMA step
        *reinterpret_cast<uint4 *>(u) = make_uint4(hw[4 * h], hw[4 * h + 1], hw[4 * h + 2], hw[4 * h + 3]);
        *reinterpret_cast<uint4 *>(u + 8) = make_uint4(lw[4 * h], lw[4 * h + 1], lw[4 * h + 2], lw[4 * h + 3]);
    }
}

}  // namespace coli

#endif
