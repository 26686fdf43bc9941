// coli_gemv.hip -- grouped dequant-on-use GEMV on the vector ALUs (gfx950).
//
// One kernel serves three products of the path:
//   * the plain qgemv  y[s,o] = scale[o] * sum_i v(o,i) x[s,i]
//     [glm.c@98759bf -- matmul_q, matmul_i4, matmul_i2; metal@93cde63 -- mm_gemv]
//   * the fused expert gate/up pass with SwiGLU applied before h is stored
//     [glm.c@97c756a -- matmul_i4_pair, expert_gate_up; glm.c@98759bf -- moe,
//      phase D; metal@93cde63 -- moe_gemv, moe_silu]
//   * the expert down pass [glm.c@98759bf -- moe, phase D].
// A "group" is one expert (or the shared expert, or the single matrix of a
// plain qgemv) together with the activation rows routed to it; every group's
// weight rows are streamed from HBM once per token pass.
//
// Mapping (wave64):
//   - a row is cut into 16-byte segments; a "row group" of `lpr` lanes walks
//     the segments of RPW rows at once (one global_load_dwordx4 per lane per
//     row), so each x value read from LDS is reused RPW (x M) times;
//   - a wave holds 64/lpr row groups; a 256-thread block holds 4 waves;
//   - x for up to NT tokens is staged in LDS (zero padded past I, 16-byte
//     chunks XOR-swizzled so the 64 lanes of a wave hit distinct banks);
//   - codes (value + OFF) multiply x in fp32 FMAs; OFF * sum(x) is removed
//     once per row; the per-row scale multiplies the finished sum;
//   - lanes of a row group reduce with xor-shuffles; lane 0 of the group
//     writes.
#include "coli_device.h"
#include "coli_gemv.h"

namespace coli {

namespace {

__device__ __forceinline__ uint4 load_seg(const uint8_t *row, int64_t seg, int64_t rb,
                                          bool aligned)
{
    if (aligned) return *reinterpret_cast<const uint4 *>(row + 16 * seg);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    for (int b = 0; b < 16; ++b) {
        int64_t off = 16 * seg + b;
        if (off < rb) w[b >> 2] |= (uint32_t)row[off] << (8 * (b & 3));
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint32_t word_of(const uint4 &v, int d)
{
    return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

template <int FMT, int M, int RPW, int NT, bool ALIGNED>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a)
{
    constexpr int EPS = Fmt<FMT>::EPS;   // elements per 16-byte segment
    constexpr int CPS = EPS / 4;         // 16-byte x chunks per segment
    constexpr int EPD = EPS / 4;         // elements per 32-bit word
    constexpr int SWM = (CPS < 8 ? CPS : 8) - 1;
    constexpr float OFF = Fmt<FMT>::OFF;

    extern __shared__ float4 xs4[];      // [NT][ich / 4]
    __shared__ float red[NT][4];
    __shared__ float xsum[NT];

    const int g = blockIdx.x / a.tiles;
    const int tile = blockIdx.x % a.tiles;
    const bool extra = a.has_extra && g == a.ngroups;

    int r0, cnt, Og;
    const uint8_t *W[M];
    const float *SC[M];
    if (extra) {
        r0 = a.x_row0;
        cnt = a.x_rows;
        Og = a.xO;
#pragma unroll
        for (int m = 0; m < M; ++m) { W[m] = a.xw[m]; SC[m] = a.xs[m]; }
    } else {
        if (a.offsets) {
            r0 = a.offsets[g];
            cnt = a.offsets[g + 1] - r0;
        } else {
            r0 = 0;
            cnt = a.x_rows;
        }
        Og = a.O;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            W[m] = a.w[m] + (int64_t)g * a.w_gstride;
            SC[m] = a.s[m] ? a.s[m] + (int64_t)g * a.s_gstride : nullptr;
        }
    }
    const int lpr = a.lpr;
    const int nrg = kWave / lpr;
    const int rows_per_block = 4 * nrg * RPW;
    if (cnt <= 0 || tile * rows_per_block >= Og) return;   // uniform per block

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int rg = lane / lpr, lig = lane % lpr;
    const int obase = tile * rows_per_block + (wave * nrg + rg) * RPW;
    const int64_t rb = a.rb;
    const int nseg = (int)((rb + 15) / 16);
    const int nq = a.ich / 4;            // 16-byte chunks per staged token row

    for (int t0 = 0; t0 < cnt; t0 += NT) {
        const int nt = min(NT, cnt - t0);
        float acc[M][RPW][NT];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int r = 0; r < RPW; ++r)
#pragma unroll
                for (int s = 0; s < NT; ++s) acc[m][r][s] = 0.f;
        float sx[NT];
#pragma unroll
        for (int s = 0; s < NT; ++s) sx[s] = 0.f;

        for (int e0 = 0; e0 < a.I; e0 += a.ich) {
            __syncthreads();   // the previous window is no longer read
            // ---- stage x[t0 .. t0+nt) x [e0, e0+ich) into LDS
#pragma unroll
            for (int s = 0; s < NT; ++s) {
                const bool live = s < nt;
                const float *xp = nullptr;
                if (live) {
                    const int tok = t0 + s;
                    int xr;
                    if (!a.xrow_token) xr = r0 + tok;
                    else if (extra) xr = tok;
                    else xr = a.row_pair[r0 + tok] / a.K;
                    xp = a.x + (int64_t)xr * a.ldx;
                }
                for (int q = tid; q < nq; q += 256) {
                    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                    const int e = e0 + 4 * q;
                    if (live) {
                        if (a.x_vec4 && e + 3 < a.I) {
                            v = *reinterpret_cast<const float4 *>(xp + e);
                        } else {
                            if (e + 0 < a.I) v.x = xp[e + 0];
                            if (e + 1 < a.I) v.y = xp[e + 1];
                            if (e + 2 < a.I) v.z = xp[e + 2];
                            if (e + 3 < a.I) v.w = xp[e + 3];
                        }
                        sx[s] += (v.x + v.y) + (v.z + v.w);
                    }
                    const int gl = q / CPS, c = q % CPS;
                    xs4[s * nq + gl * CPS + (c ^ (gl & SWM))] = v;
                }
            }
            __syncthreads();
            // ---- stream the weight segments of this window
            const int gw0 = e0 / EPS;
            const int nsw = min(nq / CPS, nseg - gw0);
            for (int gl = lig; gl < nsw; gl += lpr) {
                const int64_t gseg = gw0 + gl;
                uint4 wv[M][RPW];
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int r = 0; r < RPW; ++r) {
                        const int o = obase + r;
                        wv[m][r] = (o < Og) ? load_seg(W[m] + (int64_t)o * rb, gseg, rb, ALIGNED)
                                            : make_uint4(0u, 0u, 0u, 0u);
                    }
                const int sw = gl & SWM;
                if constexpr (FMT == kF32) {
#pragma unroll
                    for (int s = 0; s < NT; ++s) {
                        if (s < nt) {
                            const float4 xv = xs4[s * nq + gl];
#pragma unroll
                            for (int m = 0; m < M; ++m)
#pragma unroll
                                for (int r = 0; r < RPW; ++r) {
                                    float t = acc[m][r][s];
                                    t = fmaf(__uint_as_float(wv[m][r].x), xv.x, t);
                                    t = fmaf(__uint_as_float(wv[m][r].y), xv.y, t);
                                    t = fmaf(__uint_as_float(wv[m][r].z), xv.z, t);
                                    t = fmaf(__uint_as_float(wv[m][r].w), xv.w, t);
                                    acc[m][r][s] = t;
                                }
                        }
                    }
                } else {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        float cw[M][RPW][EPD];
#pragma unroll
                        for (int m = 0; m < M; ++m)
#pragma unroll
                            for (int r = 0; r < RPW; ++r) unpack_word<FMT>(word_of(wv[m][r], d), cw[m][r]);
#pragma unroll
                        for (int s = 0; s < NT; ++s) {
                            if (s < nt) {
                                float xv[EPD];
#pragma unroll
                                for (int c4 = 0; c4 < EPD / 4; ++c4) {
                                    const int c = d * (EPD / 4) + c4;
                                    const float4 q4 = xs4[s * nq + gl * CPS + (c ^ sw)];
                                    xv[4 * c4 + 0] = q4.x;
                                    xv[4 * c4 + 1] = q4.y;
                                    xv[4 * c4 + 2] = q4.z;
                                    xv[4 * c4 + 3] = q4.w;
                                }
#pragma unroll
                                for (int m = 0; m < M; ++m)
#pragma unroll
                                    for (int r = 0; r < RPW; ++r) {
                                        float t = acc[m][r][s];
#pragma unroll
                                        for (int e = 0; e < EPD; ++e) t = fmaf(cw[m][r][e], xv[e], t);
                                        acc[m][r][s] = t;
                                    }
                            }
                        }
                    }
                }
            }
        }
        // ---- sum(x) per token over the whole block (fixed order)
        if constexpr (OFF != 0.f) {
#pragma unroll
            for (int s = 0; s < NT; ++s) {
                const float v = wave_sum(sx[s]);
                if (lane == 0) red[s][wave] = v;
            }
            __syncthreads();
            if (tid < NT) xsum[tid] = (red[tid][0] + red[tid][1]) + (red[tid][2] + red[tid][3]);
            __syncthreads();
        }
        // ---- reduce each row group and write
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int r = 0; r < RPW; ++r)
#pragma unroll
                for (int s = 0; s < NT; ++s) acc[m][r][s] = group_sum(acc[m][r][s], lpr);
        if (lig == 0) {
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                const int o = obase + r;
                if (o >= Og) continue;
                const float sc0 = SC[0] ? SC[0][o] : 1.f;
                float sc1 = 1.f;
                if constexpr (M == 2) sc1 = SC[1] ? SC[1][o] : 1.f;
#pragma unroll
                for (int s = 0; s < NT; ++s) {
                    if (s >= nt) continue;
                    const float corr = (OFF != 0.f) ? OFF * xsum[s] : 0.f;
                    float v = sc0 * (acc[0][r][s] - corr);
                    if constexpr (M == 2) {
                        const float u = sc1 * (acc[1][r][s] - corr);
                        v = silu_f(v) * u;
                    }
                    a.out[(int64_t)(r0 + t0 + s) * a.ldo + o] = v;
                }
            }
        }
    }
}

template <int FMT, int M, int NT, bool AL>
hipError_t launch_t(const GemvArgs &a, int grid, size_t lds, hipStream_t st)
{
    constexpr int RPW = (M == 1) ? 4 : 2;
    auto kern = k_gemv<FMT, M, RPW, NT, AL>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, st, a);
    return hipGetLastError();
}

template <int FMT, int M, int NT>
hipError_t launch_al(const GemvArgs &a, int grid, size_t lds, hipStream_t st)
{
    return a.aligned ? launch_t<FMT, M, NT, true>(a, grid, lds, st)
                     : launch_t<FMT, M, NT, false>(a, grid, lds, st);
}

template <int FMT, int M>
hipError_t launch_nt(const GemvArgs &a, int nt, int grid, size_t lds, hipStream_t st)
{
    switch (nt) {
    case 1: return launch_al<FMT, M, 1>(a, grid, lds, st);
    case 2: return launch_al<FMT, M, 2>(a, grid, lds, st);
    case 4: return launch_al<FMT, M, 4>(a, grid, lds, st);
    default: return launch_al<FMT, M, 8>(a, grid, lds, st);
    }
}

int eps_of(int fmt) { return fmt == kF32 ? 4 : fmt == kI8 ? 16 : fmt == kI4 ? 32 : 64; }

}  // namespace

// Host-side planning: lanes per row group, x window, token pass width.
hipError_t gemv_launch(GemvArgs a, int fmt, int M, int max_rows_per_group, hipStream_t st)
{
    const int EPS = eps_of(fmt);
    int nt = 1;
    while (nt < max_rows_per_group && nt < 8) nt <<= 1;
    const int64_t nseg = (a.rb + 15) / 16;
    int lpr = 64;
    while (lpr > 1 && ((nseg % lpr) != 0 || (int64_t)lpr > nseg)) lpr >>= 1;
    // x window: whole (segment-padded) row when it fits 64 KB of LDS, else
    // a multiple of lpr * EPS elements.
    const size_t budget = 64 * 1024;
    int64_t full = ((int64_t)a.I + EPS - 1) / EPS * EPS;
    if (full < EPS) full = EPS;
    int64_t ich = full;
    if ((size_t)nt * (size_t)full * 4 > budget) {
        const int64_t unit = (int64_t)lpr * EPS;
        int64_t n = (int64_t)(budget / ((size_t)nt * 4)) / unit;
        if (n < 1) n = 1;
        ich = n * unit;
        if (ich > full) ich = full;
    }
    a.ich = (int)ich;
    a.lpr = lpr;
    const int RPW = (M == 1) ? 4 : 2;
    const int rows_per_block = 4 * (64 / lpr) * RPW;
    const int Omax = a.has_extra && a.xO > a.O ? a.xO : a.O;
    a.tiles = (Omax + rows_per_block - 1) / rows_per_block;
    const int groups = a.ngroups + (a.has_extra ? 1 : 0);
    const int64_t grid64 = (int64_t)groups * a.tiles;
    if (grid64 <= 0) return hipSuccess;
    if (grid64 > 0x7FFFFFFF) return hipErrorInvalidValue;
    const size_t lds = (size_t)nt * (size_t)ich * 4;
    const int grid = (int)grid64;
    if (M == 1) {
        switch (fmt) {
        case kF32: return launch_nt<kF32, 1>(a, nt, grid, lds, st);
        case kI8:  return launch_nt<kI8, 1>(a, nt, grid, lds, st);
        case kI4:  return launch_nt<kI4, 1>(a, nt, grid, lds, st);
        default:   return launch_nt<kI2, 1>(a, nt, grid, lds, st);
        }
    }
    switch (fmt) {
    case kI8: return launch_nt<kI8, 2>(a, nt, grid, lds, st);
    case kI4: return launch_nt<kI4, 2>(a, nt, grid, lds, st);
    case kI2: return launch_nt<kI2, 2>(a, nt, grid, lds, st);
    default:  return hipErrorInvalidValue;
    }
}

}  // namespace coli
