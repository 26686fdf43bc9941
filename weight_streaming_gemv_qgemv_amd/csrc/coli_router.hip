// coli_router.hip -- sigmoid noaux_tc router (one group) on gfx950.
//
// [glm.c@98759bf -- moe, phase A; metal@93cde63 -- r_router, r_top8,
//  r_top8_par]
//
//   logit[s,e] = sum_d Wr[e,d] x[s,d]   fp64 products and sums (exact widening
//                                        of the fp32 inputs), on the fp64
//                                        matrix cores, split over d into
//                                        slices that are summed in a fixed
//                                        order afterwards
//   sig[s,e]   = fp32(1 / (1 + exp(-logit)))   (fp64, rounded once)
//   choice     = sig + bias                    (fp32 add)
//   K picks by largest choice, lower index on ties; w = sig[pick]; optional
//   top-p truncation; optional normalisation; times routed_scale (fp32, in
//   the pages' order).
//
// Taking the logit in fp64 makes the rounded fp32 score independent of the
// summation order (up to a rounding-boundary case of probability ~1e-8 per
// score), so the picks match a sequential fp64 reference bit for bit.
#include "coli_device.h"
#include "coli_router.h"

namespace coli {

namespace {

typedef double double4_t __attribute__((ext_vector_type(4)));

constexpr int kRouterMaxE = 1024;   // the experts a wave holds: 16 per lane

// Partial logits over one d-slice for a tile of 16 TSUB tokens x 64 experts
// (4 waves, 16 experts each; a wave multiplies its expert fragment into
// TSUB token sub-tiles, so larger batches re-read the router rows less).
// v_mfma_f64_16x16x4f64 operand layout:
//   A (16 x 4):  lane l holds A[l % 16][l / 16]
//   B (4 x 16):  lane l holds B[l / 16][l % 16]
//   D (16 x 16): lane l, element r holds D[4 * r + l / 16][l % 16]
//                (the fp64 variant interleaves rows across the lane groups)
// A = router rows (experts), B = x rows (tokens) transposed.  Each lane
// reads 4 consecutive d of its expert row and of its token rows, and feeds
// them to 4 consecutive MFMAs per sub-tile, so MFMA k-slot l/16 at step j
// is d = d0 + 4 * (l / 16) + j: every product Wr[e,d] * x[s,d] is formed
// once, and each sub-tile's sum runs over d in the same order.
// VEC: rows are 16-byte aligned and D % 4 == 0, so the 4 values are one
// 16-byte load; the loads of kSteps 16-d steps are issued together and the
// next ones are in flight while the current ones are multiplied.
template <bool VEC, int TSUB>
__global__ __launch_bounds__(256) void k_router_partial(const float *__restrict__ Wr,
                                                        const float *__restrict__ x, int S,
                                                        int E, int D, int slice,
                                                        double *__restrict__ part)
{
    constexpr int kSteps = TSUB == 1 ? 6 : 1;   // 16-d steps per chunk
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * 16 * TSUB;
    const int e0 = blockIdx.y * 64 + wave * 16;
    const int split = blockIdx.z;
    const int dbeg = split * slice;
    const int dend = min(D, dbeg + slice);
    const int row = lane & 15, kg = lane >> 4;
    const int e = e0 + row;
    const float *wp = (e < E) ? Wr + (int64_t)e * D : nullptr;
    const float *xp[TSUB];
#pragma unroll
    for (int u = 0; u < TSUB; ++u) {
        const int t = t0 + 16 * u + row;
        xp[u] = (t < S) ? x + (int64_t)t * D : nullptr;
    }
    double4_t acc[TSUB];
#pragma unroll
    for (int u = 0; u < TSUB; ++u) acc[u] = double4_t{0.0, 0.0, 0.0, 0.0};
    auto ld4 = [&](const float *p, int d) {
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
        if (VEC) {
            // d and dend are multiples of 4: the 4 values are all in or all out
            if (p && d < dend) a = *reinterpret_cast<const float4 *>(p + d);
        } else {
            float av[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) av[j] = (p && d + j < dend) ? p[d + j] : 0.f;
            a = make_float4(av[0], av[1], av[2], av[3]);
        }
        return a;
    };
    auto load = [&](int d0, float4 (&wa)[kSteps], float4 (&xb)[kSteps][TSUB]) {
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
            const int d = d0 + 16 * st + 4 * kg;
            if constexpr (TSUB == 1 && VEC) {
                float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
                if (d < dend) {
                    if (wp) a = *reinterpret_cast<const float4 *>(wp + d);
                    if (xp[0]) b = *reinterpret_cast<const float4 *>(xp[0] + d);
                }
                wa[st] = a;
                xb[st][0] = b;
                continue;
            }
            wa[st] = ld4(wp, d);
#pragma unroll
            for (int u = 0; u < TSUB; ++u) xb[st][u] = ld4(xp[u], d);
        }
    };
    auto product = [&](const float4 (&wa)[kSteps], const float4 (&xb)[kSteps][TSUB]) {
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
            if constexpr (TSUB == 1) {
                acc[0] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)wa[st].x, (double)xb[st][0].x, acc[0], 0, 0, 0);
                acc[0] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)wa[st].y, (double)xb[st][0].y, acc[0], 0, 0, 0);
                acc[0] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)wa[st].z, (double)xb[st][0].z, acc[0], 0, 0, 0);
                acc[0] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)wa[st].w, (double)xb[st][0].w, acc[0], 0, 0, 0);
                continue;
            }
            const double a[4] = {(double)wa[st].x, (double)wa[st].y, (double)wa[st].z, (double)wa[st].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int u = 0; u < TSUB; ++u) {
                    const float4 b = xb[st][u];
                    const float bj = j == 0 ? b.x : j == 1 ? b.y : j == 2 ? b.z : b.w;
                    acc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[j], (double)bj, acc[u], 0, 0, 0);
                }
            }
        }
    };
    constexpr int CH = 16 * kSteps;   // d per chunk
    float4 wa0[kSteps], wa1[kSteps];
    float4 xb0[kSteps][TSUB], xb1[kSteps][TSUB];
    load(dbeg, wa0, xb0);
    if constexpr (TSUB == 1) {
        for (int d0 = dbeg; d0 < dend; d0 += 2 * CH) {
            load(d0 + CH, wa1, xb1);   // past dend: all zeros, no access
            product(wa0, xb0);
            if (d0 + CH >= dend) break;
            load(d0 + 2 * CH, wa0, xb0);
            product(wa1, xb1);
        }
    } else {
        // one 16-d step per chunk, two chunks ahead (the registers of a
        // 32-d chunk kept two ahead would lower the occupancy)
        float4 wa2[kSteps], xb2[kSteps][TSUB];
        load(dbeg + CH, wa1, xb1);
        for (int d0 = dbeg; d0 < dend; d0 += 3 * CH) {
            load(d0 + 2 * CH, wa2, xb2);
            product(wa0, xb0);
            if (d0 + CH >= dend) break;
            load(d0 + 3 * CH, wa0, xb0);
            product(wa1, xb1);
            if (d0 + 2 * CH >= dend) break;
            load(d0 + 4 * CH, wa1, xb1);
            product(wa2, xb2);
        }
    }
    // D[i][j]: i = expert row 4*r + kg, j = token column `row` of sub-tile u
#pragma unroll
    for (int u = 0; u < TSUB; ++u) {
        const int tt = t0 + 16 * u + row;
        if (tt < S) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ee = e0 + 4 * r + kg;
                if (ee < E) part[((int64_t)split * S + tt) * E + ee] = acc[u][r];
            }
        }
    }
}

// Order-preserving key of a finite float: a > b  <=>  key(a) > key(b) (-0
// is first made +0, so equal values get equal keys); every key is > 0.
__device__ __forceinline__ uint32_t order_key(float f)
{
    const uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave-wide max of a 64-bit value on the DPP network (registers only):
// pairs within quads, half rows and rows, then rows 0-1 into 1 and 3, rows
// 0-2 into 3; lane 63 ends with the whole wave's result.  Each step moves
// both halves and keeps the larger (all values here are >= 0, so the 0 a
// lane of a disabled row reads is never the larger).
template <int CTRL, int RM>
__device__ __forceinline__ uint64_t dpp_max64(uint64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, RM, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, RM, 0xF, false);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    return o > v ? o : v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
    v = dpp_max64<0xB1, 0xF>(v);    // quad_perm 1,0,3,2
    v = dpp_max64<0x4E, 0xF>(v);    // quad_perm 2,3,0,1
    v = dpp_max64<0x141, 0xF>(v);   // row_half_mirror
    v = dpp_max64<0x140, 0xF>(v);   // row_mirror
    v = dpp_max64<0x142, 0xA>(v);   // row_bcast:15
    v = dpp_max64<0x143, 0xC>(v);   // row_bcast:31
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// One token per block.  First the block sums each score's slices in slice
// order and takes the sigmoid in fp64, rounded once (scores go to `sig` and
// to LDS).  Then the first wave runs the greedy top-K over
// choice = sig + bias:
//  - expert e (held by lane e % 64, slot e / 64; PER >= ceil(E / 64) slots)
//    gets the unique 64-bit value (order key of its choice, ~e): the largest
//    value is the largest choice and, among equal choices, the lowest e --
//    the sequential scan's first maximum;
//  - each lane sorts its values once (Batcher's odd-even merge network), so
//    its best untaken expert is always its list head;
//  - per pick one wave-wide max of the heads names the expert; its lane
//    drops its head; lane 0 then reads the picks' scores from LDS and runs
//    the pages' tail (top-p, normalisation, routed_scale) sequentially in
//    fp32.
template <int PER>
__global__ __launch_bounds__(256) void k_router_topk(const double *__restrict__ part, int splits,
                                                     const float *__restrict__ bias, int S,
                                                     int E, int K, int norm_topk,
                                                     float routed_scale, float topp,
                                                     float *__restrict__ sig,
                                                     int32_t *__restrict__ idx,
                                                     float *__restrict__ w,
                                                     int32_t *__restrict__ keff)
{
    __shared__ int pick_s[64];
    __shared__ float pw_s[64];
    __shared__ float sig_s[kRouterMaxE];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int s0 = blockIdx.x;
    const int nt = 1;
    // the selecting wave's biases, requested before anything else
    float bz[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = lane + 64 * j;
        bz[j] = (wave == 0 && e < E) ? bias[e] : 0.f;
    }
    {
        const int64_t n = (int64_t)S * E;
        for (int i = threadIdx.x; i < nt * E; i += 256) {
            const int64_t g = (int64_t)s0 * E + i;
            // the loads of up to 32 slices are issued before the first add
            constexpr int kChunk = 32;
            double l = 0.0;
            for (int k0 = 0; k0 < splits; k0 += kChunk) {
                double pv[kChunk];
#pragma unroll
                for (int k = 0; k < kChunk; ++k)
                    pv[k] = k0 + k < splits ? part[(int64_t)(k0 + k) * n + g] : 0.0;
#pragma unroll
                for (int k = 0; k < kChunk; ++k)
                    if (k0 + k < splits) l += pv[k];
            }
            const float sv = (float)(1.0 / (1.0 + exp(-l)));
            sig[g] = sv;
            sig_s[i] = sv;
        }
    }
    __syncthreads();
    const int s = s0;
    if (wave != 0) return;   // whole waves leave; no block barrier below
    // (key, ~e); slots past E hold 0, below every real value (keys are > 0)
    uint64_t ck[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = lane + 64 * j;
        ck[j] = e < E ? ((uint64_t)order_key(sig_s[e] + bz[j]) << 32) | (uint32_t)~(uint32_t)e : 0ull;
    }
    // descending sort, Batcher's odd-even merge network on PER values
#pragma unroll
    for (int p = 1; p < PER; p <<= 1)
#pragma unroll
        for (int k = p; k >= 1; k >>= 1)
#pragma unroll
            for (int j = k % p; j + k < PER; j += 2 * k)
#pragma unroll
                for (int i = 0; i < k; ++i)
                    if ((i + j) / (2 * p) == (i + j + k) / (2 * p)) {
                        const uint64_t a = ck[i + j], b = ck[i + j + k];
                        ck[i + j] = a > b ? a : b;
                        ck[i + j + k] = a > b ? b : a;
                    }
    int *pick = pick_s;
    float *pw = pw_s;
    for (int kk = 0; kk < K; ++kk) {
        const uint64_t m = wave_max_u64(ck[0]);
        const int e = (int)~(uint32_t)m;   // K <= E: m is a real expert's value
        if ((e & 63) == lane) {
#pragma unroll
            for (int j = 0; j + 1 < PER; ++j) ck[j] = ck[j + 1];
            ck[PER - 1] = 0ull;
        }
        if (lane == 0) pick[kk] = e;
    }
    if (lane != 0) return;
    for (int kk = 0; kk < K; ++kk) pw[kk] = sig_s[pick[kk]];
    int ke = K;
    if (topp > 0.f && topp < 1.f) {
        for (int a2 = 1; a2 < K; ++a2) {
            const int ii = pick[a2];
            const float wv = pw[a2];
            int b = a2 - 1;
            while (b >= 0 && pw[b] < wv) {
                pw[b + 1] = pw[b];
                pick[b + 1] = pick[b];
                --b;
            }
            pw[b + 1] = wv;
            pick[b + 1] = ii;
        }
        float tot = 1e-20f;
        for (int kk = 0; kk < K; ++kk) tot += pw[kk];
        float cum = 0.f;
        for (int kk = 0; kk < K; ++kk) {
            cum += pw[kk];
            if (cum >= topp * tot) { ke = kk + 1; break; }
        }
    }
    if (norm_topk) {
        float sm = 0.f;
        for (int kk = 0; kk < ke; ++kk) sm += pw[kk];
        sm += 1e-20f;
        for (int kk = 0; kk < ke; ++kk) pw[kk] /= sm;
    }
    for (int kk = 0; kk < K; ++kk) {
        const bool in = kk < ke;
        idx[(int64_t)s * K + kk] = in ? pick[kk] : -1;
        w[(int64_t)s * K + kk] = in ? pw[kk] * routed_scale : 0.f;
    }
    if (keff) keff[s] = ke;
}

}  // namespace

hipError_t router_launch(const float *Wr, const float *bias, const float *x, int S, int E,
                         int D, int K, int norm_topk, float routed_scale, float topp,
                         int32_t *idx, float *w, int32_t *keff, float *sig, double *part,
                         hipStream_t st)
{
    if (S <= 0) return hipSuccess;
    int slice = 0;
    const int splits = coli__router_splits(S, E, D, &slice);
    const int tt = coli__router_token_tile(S);
    dim3 grid((S + tt - 1) / tt, (E + 63) / 64, splits);
    const bool vec = D % 4 == 0 && ((uintptr_t)Wr & 15u) == 0 && ((uintptr_t)x & 15u) == 0;
    if (tt == 64) {
        if (vec)
            hipLaunchKernelGGL((k_router_partial<true, 4>), grid, dim3(256), 0, st, Wr, x, S, E, D, slice, part);
        else
            hipLaunchKernelGGL((k_router_partial<false, 4>), grid, dim3(256), 0, st, Wr, x, S, E, D, slice, part);
    } else {
        if (vec)
            hipLaunchKernelGGL((k_router_partial<true, 1>), grid, dim3(256), 0, st, Wr, x, S, E, D, slice, part);
        else
            hipLaunchKernelGGL((k_router_partial<false, 1>), grid, dim3(256), 0, st, Wr, x, S, E, D, slice, part);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (E > kRouterMaxE || K > E || K > 64) return hipErrorInvalidValue;
    // slots per lane: the sort network's size
#define COLI_TOPK(P) hipLaunchKernelGGL(k_router_topk<P>, dim3(S), dim3(256), 0, st, part, splits, bias, S, \
                                        E, K, norm_topk, routed_scale, topp, sig, idx, w, keff)
    if (E <= 64) COLI_TOPK(1);
    else if (E <= 128) COLI_TOPK(2);
    else if (E <= 256) COLI_TOPK(4);
    else if (E <= 512) COLI_TOPK(8);
    else COLI_TOPK(16);
#undef COLI_TOPK
    return hipGetLastError();
}

}  // namespace coli
