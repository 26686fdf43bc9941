// coli_api.hip -- libcoli entry points, expert grouping and the combine.
//
// Expert grouping is the pages' batch-union [glm.c@98759bf -- moe, phase B
// and the per-expert row lists of phase D; metal@93cde63 -- moe_submit's
// erow table]: every routed slot (s, kk) of an expert becomes one row of that
// expert's group, groups are laid out expert by expert, and inside a group
// rows keep slot order s*K + kk, so each active expert streams its weights
// once per call and the whole result is independent of thread timing.  Here
// the grouping runs on the device (no host round trip).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "coli.h"
#include "coli_dec.h"
#include "coli_device.h"
#include "coli_gemv.h"
#include "coli_pre.h"
#include "coli_qmv.h"
#include "coli_idot.h"
#include "coli_xrows.h"

#include "coli_internal.h"
#include "coli_router.h"
#include "coli_stages.h"

static_assert(COLI_MM_TPP_FP32 == coli::kDecTpp, "decode pass size");
static_assert(COLI_MM_TPP_BF16 == coli::kPreTpp, "prefill pass size");

namespace coli {

namespace {

constexpr int kGroupWaves = 16;          // experts per block in the grouping kernels
constexpr int kWorkClasses = 4;          // classes of a class-sorted work list

// Passes of a group of `rows` rows, counted by class into n[]: unsorted
// (cls == 0) every pass is class 0; class-sorted, class c holds the passes
// with tpp / 16 - c live 16-row tiles: the full passes in class 0 and the
// last, partial pass in the class of its live tiles (tpp / 16 <= 4).
__device__ __forceinline__ void add_passes(int rows, int tpp, int cls, int *n)
{
    if (!cls) {
        n[0] += (rows + tpp - 1) / tpp;
        return;
    }
    const int full = rows / tpp, rem = rows - full * tpp;
    n[0] += full;
    if (rem > 0) n[tpp / 16 - (rem + 15) / 16] += 1;
}

// Work-list entries of group g (rows rows): pass p goes to the slot of its
// class, start[c] + pre[c] (+ p in class 0, which holds passes 0, 1, ...);
// passes p0, p0 + step, ...
__device__ __forceinline__ void write_passes(int32_t *work, int g, int rows, int tpp, int cls,
                                             const int *start, const int *pre, int p0, int step)
{
    const int np = (rows + tpp - 1) / tpp;
    for (int p = p0; p < np; p += step) {
        const int live = min(tpp, rows - p * tpp);
        const int c = cls ? tpp / 16 - (live + 15) / 16 : 0;
        work[start[c] + pre[c] + (c == 0 ? p : 0)] = g | (p << 11);
    }
}

// n_work[0] = the number of entries; class-sorted, n_work[1 + c] = the end
// of class c.
__device__ __forceinline__ void write_ends(int32_t *n_work, int cls, const int *start, const int *tot)
{
    n_work[0] = start[kWorkClasses - 1] + tot[kWorkClasses - 1];
    if (cls)
        for (int c = 0; c < kWorkClasses; ++c) n_work[1 + c] = start[c] + tot[c];
}

// Flags written by the grouping kernel (plain stores from block 0).
constexpr uint32_t kFlagBadId = 1u;
constexpr uint32_t kFlagDup = 2u;

// Grouping of at most COLI_GROUP_CHUNK slots, one launch.  Every block
// stages all slots in LDS and counts the slots of every expert there (LDS
// atomics: integer counts, so the order of the adds does not matter), which
// gives each of its experts the exclusive prefix of the counts without an
// earlier launch.  Block 0 also writes the counts and validates every slot.
// Each expert's wave then writes its offset and, when `work` is given, the
// matrix-core work list entries of its group (passes of `tpp` rows, entry
// g | pass << 11, in group order within each class, cls: sorted by class;
// the wave of the last expert adds those of the extra group g = E
// (extra_rows rows) and the ends), and scatters the expert's slots into its
// group in slot order (stable).
// XF >= 0: blocks gblocks .. gblocks + rows - 1 instead write the activation
// row tables of the rows of x for weight format XF (coli_xrows.h), work
// that does not depend on the routing and so shares the launch.
struct XrowsJob {
    const float *x;
    int64_t ldx;
    int I, kpad, vec;
    uint16_t *table;
};
template <int XF>
__global__ __launch_bounds__(1024) void k_group_one(const int32_t *__restrict__ idx, int P, int K,
                                                    int E, int32_t *__restrict__ counts,
                                                    int32_t *__restrict__ offsets,
                                                    int32_t *__restrict__ row_pair,
                                                    int32_t *__restrict__ pair_row, int extra_rows,
                                                    int tpp, int cls, int32_t *__restrict__ work,
                                                    int32_t *__restrict__ n_work,
                                                    uint32_t *__restrict__ flags, int gblocks,
                                                    XrowsJob xj)
{
    __shared__ int32_t sidx[COLI_GROUP_CHUNK];
    __shared__ int32_t cnt[COLI_MAX_E];
    __shared__ uint32_t sflag;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    if constexpr (XF >= 0) {
        if ((int)blockIdx.x >= gblocks) {   // whole block, before any barrier
            const int row = (int)blockIdx.x - gblocks;
            const float *xr = xj.x + (int64_t)row * xj.ldx;
            uint16_t *dst = xj.table + (int64_t)row * 2 * xj.kpad;
            const int nruns = xj.kpad / xrows_run_len<XF>();
            for (int r = t; r < nruns; r += 1024) xrows_run<XF>(xr, xj.I, r, dst, xj.vec);
            return;
        }
    }
    const int e = blockIdx.x * kGroupWaves + wave;
    for (int i = t; i < E; i += 1024) cnt[i] = 0;
    if (t == 0) sflag = 0u;
    __syncthreads();
    for (int i = t; i < P; i += 1024) {
        const int v = idx[i];
        sidx[i] = v;
        if (v >= 0 && v < E) atomicAdd(&cnt[v], 1);
    }
    __syncthreads();
    if (blockIdx.x == 0) {
        // ids in [-1, E), and no expert twice among one token's K slots
        uint32_t f = 0u;
        for (int i = t; i < P; i += 1024) {
            const int v = sidx[i];
            if (v < -1 || v >= E) f |= kFlagBadId;
            if (v >= 0) {
                const int s0 = (i / K) * K;
                for (int q = s0; q < i; ++q)
                    if (sidx[q] == v) { f |= kFlagDup; break; }
            }
            if (v < 0 || v >= E) pair_row[i] = -1;
        }
        if (f) atomicOr(&sflag, f);
        for (int i = t; i < E; i += 1024) counts[i] = cnt[i];
        __syncthreads();
        if (t == 0) flags[0] = sflag;
    }
    if (e >= E) return;   // whole waves; no barrier below
    // rows and passes per class of the experts before e (pre) and of all
    // experts (tot)
    int part = 0, pre[kWorkClasses] = {0, 0, 0, 0}, tot[kWorkClasses] = {0, 0, 0, 0};
    for (int j = lane; j < E; j += 64) {
        const int c = cnt[j];
        if (j < e) {
            part += c;
            add_passes(c, tpp, cls, pre);
        }
        add_passes(c, tpp, cls, tot);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        part += __shfl_xor(part, o, kWave);
#pragma unroll
        for (int c = 0; c < kWorkClasses; ++c) {
            pre[c] += __shfl_xor(pre[c], o, kWave);
            tot[c] += __shfl_xor(tot[c], o, kWave);
        }
    }
    const int off = part;
    const int ce = cnt[e];
    if (lane == 0) {
        offsets[e] = off;
        if (e == E - 1) offsets[E] = off + ce;
    }
    if (work) {
        int xpre[kWorkClasses], start[kWorkClasses];
#pragma unroll
        for (int c = 0; c < kWorkClasses; ++c) xpre[c] = tot[c];   // the extra group follows every expert
        add_passes(extra_rows, tpp, cls, tot);
        start[0] = 0;
#pragma unroll
        for (int c = 1; c < kWorkClasses; ++c) start[c] = start[c - 1] + tot[c - 1];
        write_passes(work, e, ce, tpp, cls, start, pre, lane, 64);
        if (e == E - 1) {
            write_passes(work, E, extra_rows, tpp, cls, start, xpre, lane, 64);
            if (lane == 0) write_ends(n_work, cls, start, tot);
        }
    }
    int run = 0;
    for (int c = 0; c < P; c += 64) {
        const int i = c + lane;
        const bool hit = i < P && sidx[i] == e;
        const uint64_t m = __ballot(hit);
        if (hit) {
            const uint64_t below = lane ? (m & ((~0ull) >> (64 - lane))) : 0ull;
            const int pos = off + run + __popcll(below);
            row_pair[pos] = i;
            pair_row[i] = pos;
        }
        run += __popcll(m);
    }
}

// Chunked grouping for large batches (P > COLI_GROUP_CHUNK slots): the same
// outputs as k_group_one, with the slots cut into chunks
// so that a wave scans one expert over one chunk only.
//   k_group_hist:  block (expert group, chunk) -> hist[c][e] = the chunk's
//                  slots of expert e; block (0, c) validates the chunk
//                  (flags word C E + c);
//   k_group_prefix: one block: counts, offsets (exclusive prefix over e),
//                  the work list and n_work, the flags, and hist[c][e]
//                  turned into the chunk's first position for expert e
//                  (offsets[e] + the earlier chunks' counts);
//   k_group_place: block (expert group, chunk): the stable scatter of the
//                  chunk's slots from those first positions.
constexpr int kChunk = COLI_GROUP_CHUNK;

__global__ __launch_bounds__(1024) void k_group_hist(const int32_t *__restrict__ idx, int P, int K,
                                                     int E, int32_t *__restrict__ gpart)
{
    __shared__ int32_t sidx[kChunk];
    __shared__ uint32_t sflag;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.x * kGroupWaves + wave, c = blockIdx.y, C = gridDim.y;
    const int base = c * kChunk, n = min(kChunk, P - base);
    if (threadIdx.x == 0) sflag = 0u;
    for (int i = threadIdx.x; i < n; i += blockDim.x) sidx[i] = idx[base + i];
    __syncthreads();
    if (e < E) {
        int count = 0;
        for (int k = 0; k < n; k += 64) {
            const int i = k + lane;
            count += __popcll(__ballot(i < n && sidx[i] == e));
        }
        if (lane == 0) gpart[(int64_t)c * E + e] = count;
    }
    if (blockIdx.x == 0) {
        uint32_t f = 0u;
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
            const int p = base + i, v = sidx[i];
            if (v < -1 || v >= E) f |= kFlagBadId;
            if (v >= 0) {
                const int s0 = (p / K) * K;
                for (int q = s0; q < p; ++q)
                    if (idx[q] == v) { f |= kFlagDup; break; }
            }
        }
        if (f) atomicOr(&sflag, f);
        __syncthreads();
        if (threadIdx.x == 0) gpart[(int64_t)C * E + c] = (int32_t)sflag;
    }
}

__global__ __launch_bounds__(1024) void k_group_prefix(int E, int C, int32_t *__restrict__ gpart,
                                                       int32_t *__restrict__ counts,
                                                       int32_t *__restrict__ offsets, int extra_rows,
                                                       int tpp, int cls, int32_t *__restrict__ work,
                                                       int32_t *__restrict__ n_work,
                                                       uint32_t *__restrict__ flags)
{
    // the per-chunk counts are read once, coalesced, into LDS when they fit
    // (C E <= 8192), so the per-expert loops below run on LDS
    __shared__ int32_t hs[8192];
    __shared__ int32_t wsum[16][1 + kWorkClasses];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const bool in_lds = (int64_t)C * E <= 8192;
    if (in_lds)
        for (int i = t; i < C * E; i += 1024) hs[i] = gpart[i];
    __syncthreads();
    int ce = 0;
    if (t < E)
        for (int c = 0; c < C; ++c) ce += in_lds ? hs[c * E + t] : gpart[(int64_t)c * E + t];
    // exclusive prefix over experts of the counts and of the passes per
    // class; tot: the passes per class of all experts
    int own[kWorkClasses] = {0, 0, 0, 0};
    if (t < E) add_passes(ce, tpp, cls, own);
    int v = ce, pv[kWorkClasses];
#pragma unroll
    for (int c = 0; c < kWorkClasses; ++c) pv[c] = own[c];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int a = __shfl_up(v, o, kWave);
        if (lane >= o) v += a;
#pragma unroll
        for (int c = 0; c < kWorkClasses; ++c) {
            const int b = __shfl_up(pv[c], o, kWave);
            if (lane >= o) pv[c] += b;
        }
    }
    if (lane == 63) {
        wsum[wave][0] = v;
#pragma unroll
        for (int c = 0; c < kWorkClasses; ++c) wsum[wave][1 + c] = pv[c];
    }
    __syncthreads();
    int wo = 0, pre[kWorkClasses], tot[kWorkClasses];
#pragma unroll
    for (int c = 0; c < kWorkClasses; ++c) { pre[c] = pv[c] - own[c]; tot[c] = 0; }
    for (int ww = 0; ww < 16; ++ww) {
        if (ww < wave) wo += wsum[ww][0];
#pragma unroll
        for (int c = 0; c < kWorkClasses; ++c) {
            if (ww < wave) pre[c] += wsum[ww][1 + c];
            tot[c] += wsum[ww][1 + c];
        }
    }
    const int off = wo + v - ce;                                  // exclusive
    if (t < E) {
        counts[t] = ce;
        offsets[t] = off;
        if (t == E - 1) offsets[E] = off + ce;
        if (work) {
            int xpre[kWorkClasses], start[kWorkClasses];
#pragma unroll
            for (int c = 0; c < kWorkClasses; ++c) xpre[c] = tot[c];
            add_passes(extra_rows, tpp, cls, tot);
            start[0] = 0;
#pragma unroll
            for (int c = 1; c < kWorkClasses; ++c) start[c] = start[c - 1] + tot[c - 1];
            write_passes(work, t, ce, tpp, cls, start, pre, 0, 1);
            if (t == E - 1) {
                write_passes(work, E, extra_rows, tpp, cls, start, xpre, 0, 1);
                write_ends(n_work, cls, start, tot);
            }
        }
        // the chunks' first positions for expert t
        int run = off;
        for (int c = 0; c < C; ++c) {
            const int h = in_lds ? hs[c * E + t] : gpart[(int64_t)c * E + t];
            gpart[(int64_t)c * E + t] = run;
            run += h;
        }
    }
    if (t == 0) {
        uint32_t f = 0u;
        for (int c = 0; c < C; ++c) f |= (uint32_t)gpart[(int64_t)C * E + c];
        flags[0] = f;
    }
}

__global__ __launch_bounds__(1024) void k_group_place(const int32_t *__restrict__ idx, int P, int E,
                                                      const int32_t *__restrict__ gpart,
                                                      int32_t *__restrict__ row_pair,
                                                      int32_t *__restrict__ pair_row)
{
    __shared__ int32_t sidx[kChunk];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.x * kGroupWaves + wave, c = blockIdx.y;
    const int base = c * kChunk, n = min(kChunk, P - base);
    for (int i = threadIdx.x; i < n; i += blockDim.x) sidx[i] = idx[base + i];
    __syncthreads();
    if (e < E) {
        int pos0 = gpart[(int64_t)c * E + e];
        for (int k = 0; k < n; k += 64) {
            const int i = k + lane;
            const bool hit = i < n && sidx[i] == e;
            const uint64_t m = __ballot(hit);
            if (hit) {
                const uint64_t below = lane ? (m & ((~0ull) >> (64 - lane))) : 0ull;
                const int pos = pos0 + __popcll(below);
                row_pair[pos] = base + i;
                pair_row[base + i] = pos;
            }
            pos0 += __popcll(m);
        }
    }
    if (blockIdx.x == 0) {
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
            const int v = sidx[i];
            if (v < 0 || v >= E) pair_row[base + i] = -1;
        }
    }
}

// out[s, :] = sum_{kk: slot kept} w[s,kk] * y[row(s,kk), :]  (+ y[shared row]),
// slots in order kk = 0..K-1, then the shared expert: a fixed order; with a
// residual, out[s, :] = resid[s, :] + that sum (resid may be out itself: each
// element is read and written by the same thread).
// Block (s, c) covers columns [c * kCombineCols, +kCombineCols) of token s:
// one float4 (vec4) or one float per thread, all K rows read together.
constexpr int kCombineThreads = 256;
// y rows in fp32, or (bf16-precision layers) rounded to bf16
__device__ __forceinline__ float4 yload4(const float *y, int64_t i) { return *reinterpret_cast<const float4 *>(y + i); }
__device__ __forceinline__ float4 yload4(const uint16_t *y, int64_t i)
{
    const uint2 u = *reinterpret_cast<const uint2 *>(y + i);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
}
// 8 bf16 (16 bytes) -> two float4
__device__ __forceinline__ void yload8(const uint16_t *y, int64_t i, float4 &lo, float4 &hi)
{
    const uint4 u = *reinterpret_cast<const uint4 *>(y + i);
    lo = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
    hi = make_float4(__uint_as_float(u.z << 16), __uint_as_float(u.z & 0xFFFF0000u),
                     __uint_as_float(u.w << 16), __uint_as_float(u.w & 0xFFFF0000u));
}
__device__ __forceinline__ float yload1(const float *y, int64_t i) { return y[i]; }
__device__ __forceinline__ float yload1(const uint16_t *y, int64_t i) { return __uint_as_float((uint32_t)y[i] << 16); }

template <typename YT>
__global__ __launch_bounds__(kCombineThreads) void k_combine(const YT *__restrict__ y, int D, int K,
                                                 const int32_t *__restrict__ pair_row,
                                                 const float *__restrict__ w, int has_shared,
                                                 int64_t shared_row0, const float *resid, float *out,
                                                 int vec4)
{
    const int s = blockIdx.x;
    const int32_t *pr = pair_row + (int64_t)s * K;
    const float *ws = w + (int64_t)s * K;
    // slots in runs of kCombineRun: the run's rows are all requested before
    // the first is added, the additions stay in slot order
    constexpr int kCombineRun = 8;
    if constexpr (sizeof(YT) == 2) {
        if (vec4 == 2) {   // bf16 rows, 8 elements (one 16-byte load per row) per thread
            const int d = (blockIdx.y * kCombineThreads + threadIdx.x) * 8;
            if (d >= D) return;
            float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
            auto fma4 = [](float wk, const float4 &v, float4 &acc) {
                acc.x = fmaf(wk, v.x, acc.x);
                acc.y = fmaf(wk, v.y, acc.y);
                acc.z = fmaf(wk, v.z, acc.z);
                acc.w = fmaf(wk, v.w, acc.w);
            };
            for (int k0 = 0; k0 < K; k0 += kCombineRun) {
                int r[kCombineRun];
                float wk[kCombineRun];
                float4 v0[kCombineRun], v1[kCombineRun];
#pragma unroll
                for (int j = 0; j < kCombineRun; ++j) {
                    r[j] = k0 + j < K ? pr[k0 + j] : -1;
                    wk[j] = k0 + j < K ? ws[k0 + j] : 0.f;
                }
#pragma unroll
                for (int j = 0; j < kCombineRun; ++j) {
                    v0[j] = v1[j] = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (r[j] >= 0) yload8(y, (int64_t)r[j] * D + d, v0[j], v1[j]);
                }
#pragma unroll
                for (int j = 0; j < kCombineRun; ++j) {
                    if (r[j] < 0) continue;
                    fma4(wk[j], v0[j], a0);
                    fma4(wk[j], v1[j], a1);
                }
            }
            if (has_shared) {
                float4 v0, v1;
                yload8(y, (shared_row0 + s) * (int64_t)D + d, v0, v1);
                a0.x += v0.x; a0.y += v0.y; a0.z += v0.z; a0.w += v0.w;
                a1.x += v1.x; a1.y += v1.y; a1.z += v1.z; a1.w += v1.w;
            }
            if (resid) {
                const float4 r0 = *reinterpret_cast<const float4 *>(resid + (int64_t)s * D + d);
                const float4 r1 = *reinterpret_cast<const float4 *>(resid + (int64_t)s * D + d + 4);
                a0 = make_float4(r0.x + a0.x, r0.y + a0.y, r0.z + a0.z, r0.w + a0.w);
                a1 = make_float4(r1.x + a1.x, r1.y + a1.y, r1.z + a1.z, r1.w + a1.w);
            }
            float4 *o = reinterpret_cast<float4 *>(out + (int64_t)s * D + d);
            o[0] = a0;
            o[1] = a1;
            return;
        }
    }
    if (vec4) {
        const int d = (blockIdx.y * kCombineThreads + threadIdx.x) * 4;
        if (d >= D) return;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int k0 = 0; k0 < K; k0 += kCombineRun) {
            int r[kCombineRun];
            float wk[kCombineRun];
            float4 v[kCombineRun];
#pragma unroll
            for (int j = 0; j < kCombineRun; ++j) {
                r[j] = k0 + j < K ? pr[k0 + j] : -1;
                wk[j] = k0 + j < K ? ws[k0 + j] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < kCombineRun; ++j)
                v[j] = r[j] >= 0 ? yload4(y, (int64_t)r[j] * D + d) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int j = 0; j < kCombineRun; ++j) {
                if (r[j] < 0) continue;
                acc.x = fmaf(wk[j], v[j].x, acc.x);
                acc.y = fmaf(wk[j], v[j].y, acc.y);
                acc.z = fmaf(wk[j], v[j].z, acc.z);
                acc.w = fmaf(wk[j], v[j].w, acc.w);
            }
        }
        if (has_shared) {
            const float4 v = yload4(y, (shared_row0 + s) * (int64_t)D + d);
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        if (resid) {
            const float4 r = *reinterpret_cast<const float4 *>(resid + (int64_t)s * D + d);
            acc.x = r.x + acc.x;
            acc.y = r.y + acc.y;
            acc.z = r.z + acc.z;
            acc.w = r.w + acc.w;
        }
        *reinterpret_cast<float4 *>(out + (int64_t)s * D + d) = acc;
    } else {
        const int d = blockIdx.y * kCombineThreads + threadIdx.x;
        if (d >= D) return;
        float acc = 0.f;
        for (int k0 = 0; k0 < K; k0 += kCombineRun) {
            int r[kCombineRun];
            float v[kCombineRun];
#pragma unroll
            for (int j = 0; j < kCombineRun; ++j) r[j] = k0 + j < K ? pr[k0 + j] : -1;
#pragma unroll
            for (int j = 0; j < kCombineRun; ++j) v[j] = r[j] >= 0 ? yload1(y, (int64_t)r[j] * D + d) : 0.f;
#pragma unroll
            for (int j = 0; j < kCombineRun; ++j)
                if (r[j] >= 0) acc = fmaf(ws[k0 + j], v[j], acc);
        }
        if (has_shared) acc += yload1(y, (shared_row0 + s) * (int64_t)D + d);
        if (resid) acc = resid[(int64_t)s * D + d] + acc;
        out[(int64_t)s * D + d] = acc;
    }
}

// y_bf16: the y rows are bf16 (uint16_t elements, same row stride D)
hipError_t combine_launch(const float *y, int S, int D, int K, const int32_t *pair_row,
                          const float *w, int has_shared, int64_t shared_row0, float *out,
                          int vec4, hipStream_t st, const float *resid, int y_bf16 = 0)
{
    // bf16 rows: 8 elements per thread when whole 16-byte runs (vec4 = 2)
    if (y_bf16 && vec4 && D % 8 == 0 && ((uintptr_t)y & 15u) == 0) vec4 = 2;
    const int per = vec4 ? 4 * vec4 * kCombineThreads : kCombineThreads;
    const dim3 grid((unsigned)S, (unsigned)((D + per - 1) / per));
    if (y_bf16)
        hipLaunchKernelGGL(k_combine<uint16_t>, grid, dim3(kCombineThreads), 0, st,
                           reinterpret_cast<const uint16_t *>(y), D, K, pair_row, w, has_shared, shared_row0,
                           resid, out, vec4);
    else
        hipLaunchKernelGGL(k_combine<float>, grid, dim3(kCombineThreads), 0, st, y, D, K, pair_row, w,
                           has_shared, shared_row0, resid, out, vec4);
    return hipGetLastError();
}

// Post-attention RMSNorm of one row per block [glm.c@98759bf -- rmsnorm]:
// the mean square in fp64 (each square exact; per-thread sums over a fixed
// stride, then a fixed-order tree), converted once to fp32, eps added in
// fp32, r = 1 / sqrtf(.) (correctly rounded division and root), and each
// output (x * r) * w rounded in fp32 after each product.
constexpr int kNormThreads = 256;
__global__ __launch_bounds__(kNormThreads) void k_rmsnorm(const float *__restrict__ x,
                                                  const float *__restrict__ nw, int D, float eps,
                                                  float *__restrict__ out, int vec4)
{
    __shared__ double red[kNormThreads / kWave];
    const int s = blockIdx.x, tid = threadIdx.x;
    const float *xs = x + (int64_t)s * D;
    float *os = out + (int64_t)s * D;
    double acc = 0.0;
    if (vec4) {
        for (int i = 4 * tid; i < D; i += 4 * kNormThreads) {
            const float4 v = *reinterpret_cast<const float4 *>(xs + i);
            acc += (double)v.x * (double)v.x;
            acc += (double)v.y * (double)v.y;
            acc += (double)v.z * (double)v.z;
            acc += (double)v.w * (double)v.w;
        }
    } else {
        for (int i = tid; i < D; i += kNormThreads) acc += (double)xs[i] * (double)xs[i];
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kWave);
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = acc;
    __syncthreads();
    const double ms = (red[0] + red[1]) + (red[2] + red[3]);
    const float mean = (float)(ms / (double)D);
    const float r = 1.0f / sqrtf(mean + eps);
    if (vec4) {
        for (int i = 4 * tid; i < D; i += 4 * kNormThreads) {
            const float4 v = *reinterpret_cast<const float4 *>(xs + i);
            const float4 g = *reinterpret_cast<const float4 *>(nw + i);
            *reinterpret_cast<float4 *>(os + i) =
                make_float4((v.x * r) * g.x, (v.y * r) * g.y, (v.z * r) * g.z, (v.w * r) * g.w);
        }
    } else {
        for (int i = tid; i < D; i += kNormThreads) os[i] = (xs[i] * r) * nw[i];
    }
}
static_assert(kNormThreads / kWave == 4, "fixed-order tree over 4 waves");

inline bool al16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int to_status(hipError_t e) { return e == hipSuccess ? COLI_OK : COLI_EDEVICE; }

// The shared expert alone on the vector ALUs (used when its format or width
// differs from the routed experts'): h rows and y rows start at shared_row0.
int run_shared_valu(const coli_mlp *sh, const float *x, int S, int D, float *h, int64_t h_ld,
                    float *y, int64_t shared_row0, int hint, hipStream_t st)
{
    const int64_t rbs = coli_row_bytes(sh->fmt, D), rbf = coli_row_bytes(sh->fmt, sh->F);
    GemvArgs b = {};
    b.ngroups = 0;
    b.has_extra = 1;
    b.xw[0] = (const uint8_t *)sh->w_gate;
    b.xw[1] = (const uint8_t *)sh->w_up;
    b.xs[0] = sh->s_gate;
    b.xs[1] = sh->s_up;
    b.xO = sh->F;
    b.O = sh->F;
    b.x_rows = S;
    b.x_row0 = (int)shared_row0;
    b.I = D;
    b.rb = rbs;
    b.K = 1;
    b.xrow_token = 1;
    b.x = x;
    b.ldx = D;
    b.x_vec4 = al16(x) && (D % 4 == 0);
    b.out = h;
    b.ldo = h_ld;
    b.aligned = (rbs % 16 == 0) && al16(sh->w_gate) && al16(sh->w_up);
    if (gemv_launch(b, sh->fmt, 2, hint, st) != hipSuccess) return COLI_EDEVICE;
    GemvArgs d = {};
    d.ngroups = 0;
    d.has_extra = 1;
    d.xw[0] = (const uint8_t *)sh->w_down;
    d.xs[0] = sh->s_down;
    d.xO = D;
    d.O = D;
    d.x_rows = S;
    d.x_row0 = (int)shared_row0;
    d.I = sh->F;
    d.rb = rbf;
    d.K = 1;
    d.xrow_token = 0;
    d.x = h;
    d.ldx = h_ld;
    d.x_vec4 = (h_ld % 4 == 0);
    d.out = y;
    d.ldo = D;
    d.aligned = (rbf % 16 == 0) && al16(sh->w_down);
    if (gemv_launch(d, sh->fmt, 1, hint, st) != hipSuccess) return COLI_EDEVICE;
    return COLI_OK;
}

// Grouped expert products: routed experts (+ shared) -> h -> y -> out.
int run_experts(const coli_experts *ex, const coli_mlp *sh, const float *x, int S, int K,
                const int32_t *idx, const float *w, float *out, int prec, uint8_t *ws,
                const coli_ws_layout &L, hipStream_t st, const float *resid = nullptr)
{
    const int E = ex->E, D = ex->D, F = ex->F;
    const int P = S * K;
    uint32_t *flags = reinterpret_cast<uint32_t *>(ws + L.flags);
    int32_t *counts = reinterpret_cast<int32_t *>(ws + L.counts);
    int32_t *offsets = reinterpret_cast<int32_t *>(ws + L.offsets);
    int32_t *row_pair = reinterpret_cast<int32_t *>(ws + L.row_pair);
    int32_t *pair_row = reinterpret_cast<int32_t *>(ws + L.pair_row);
    float *h = reinterpret_cast<float *>(ws + L.h);
    float *y = reinterpret_cast<float *>(ws + L.y);
    const int gblocks = (E + kGroupWaves - 1) / kGroupWaves;
    hipError_t err;
    const int64_t rbD = coli_row_bytes(ex->fmt, D), rbF = coli_row_bytes(ex->fmt, F);
    const int64_t shared_row0 = (int64_t)P;
    const int hint = 8;
    // matrix-core path: whole 16-byte row segments, 16-byte aligned tensors
    const bool mm = rbD % 16 == 0 && rbF % 16 == 0 && al16(ex->w_gate) && al16(ex->w_up) &&
                    al16(ex->w_down) && (ex->fmt == COLI_I8 || ex->fmt == COLI_I4 || ex->fmt == COLI_I2);
    const bool sh_mm = mm && sh && sh->fmt == ex->fmt && sh->F == F && sh->layout == ex->layout &&
                       al16(sh->w_gate) && al16(sh->w_up) && al16(sh->w_down);
    // tiled weights: matrix cores only (the host checks guarantee mm)
    const int tiled = ex->layout != COLI_LAYOUT_ROWS ? 1 : 0;
    if (tiled && !mm) return COLI_EALIGN;
    // grouped-scale int4 (fp32 precision, grouped tiled layout): group
    // scales packed [row tile][group][16 rows], kpad / gs groups per row
    const int gs = ex->gs;
    if (gs && (prec == COLI_PREC_IDOT || ex->layout != COLI_LAYOUT_TILED_GROUPED || !mm)) return COLI_EINVAL;
    const int64_t gstrD = tiled ? coli_tiled_bytes(ex->fmt, 1, F, D) : (int64_t)F * rbD;   // gate, up
    const int64_t gstrF = tiled ? coli_tiled_bytes(ex->fmt, 1, D, F) : (int64_t)D * rbF;   // down
    // matrix-core passes: 16 rows as bf16 hi/lo column pairs (fp32-level
    // accuracy) or 64 rows rounded once to bf16
    const int bf16 = prec == COLI_PREC_BF16 ? 1 : 0, idot = prec == COLI_PREC_IDOT ? 1 : 0;
    if (idot && !(mm && tiled && (!sh || sh_mm))) return COLI_EINVAL;   // the host checks rule these out
    const int tpp = bf16 || idot ? COLI_MM_TPP_BF16 : COLI_MM_TPP_FP32;
    int32_t *work = reinterpret_cast<int32_t *>(ws + L.work);
    int32_t *n_work = reinterpret_cast<int32_t *>(ws + L.n_work);
    // fp32 matrix-core path with one grouping launch: that launch also
    // writes x's row tables
    const bool x_fused = mm && prec == COLI_PREC_FP32 && P <= kChunk;
    {
    StageTimer tg(kStGroup, st);
    if (P > kChunk) {
        const int C = (P + kChunk - 1) / kChunk;
        int32_t *gpart = reinterpret_cast<int32_t *>(ws + L.gpart);
        hipLaunchKernelGGL(k_group_hist, dim3(gblocks, C), dim3(1024), 0, st, idx, P, K, E, gpart);
        err = hipGetLastError();
        if (err != hipSuccess) return COLI_EDEVICE;
        hipLaunchKernelGGL(k_group_prefix, dim3(1), dim3(1024), 0, st, E, C, gpart, counts, offsets,
                           sh_mm ? S : 0, tpp, bf16 | idot, mm ? work : nullptr, n_work, flags);
        err = hipGetLastError();
        if (err != hipSuccess) return COLI_EDEVICE;
        hipLaunchKernelGGL(k_group_place, dim3(gblocks, C), dim3(1024), 0, st, idx, P, E, gpart,
                           row_pair, pair_row);
    } else {
        // the fp32 matrix-core path's row tables of x ride along
        XrowsJob xj = {x, D, D, (int)coli__kpad(D), (int)(D % 4 == 0 && al16(x)),
                       reinterpret_cast<uint16_t *>(ws + L.xf)};
        const int xg = x_fused ? S : 0;
#define COLI_GROUP_ONE(XF)                                                                         \
    hipLaunchKernelGGL(k_group_one<XF>, dim3(gblocks + xg), dim3(1024), 0, st, idx, P, K, E, counts, \
                       offsets, row_pair, pair_row, sh_mm ? S : 0, tpp, bf16 | idot, mm ? work : nullptr, n_work, \
                       flags, gblocks, xj)
        if (!x_fused) COLI_GROUP_ONE(-1);
        else if (ex->fmt == kI8) COLI_GROUP_ONE(kI8);
        else if (ex->fmt == kI4) COLI_GROUP_ONE(kI4);
        else COLI_GROUP_ONE(kI2);
#undef COLI_GROUP_ONE
    }
    err = hipGetLastError();
    if (err != hipSuccess) return COLI_EDEVICE;
    }

    if (mm && prec == COLI_PREC_FP32) {
        // fp32 precision: x as one row table per token, the SwiGLU output as
        // one per grouped row
        uint16_t *xt = reinterpret_cast<uint16_t *>(ws + L.xf);
        uint16_t *ht = reinterpret_cast<uint16_t *>(ws + L.hf);
        const int64_t max_gp = L.n_pass_max;
        const int kpD = (int)coli__kpad(D), kpF = (int)coli__kpad(F);
        if (!x_fused) {   // else the grouping launch wrote them
            StageTimer tp(kStPrep, st);
            if (xrows_launch(ex->fmt, x, D, S, D, kpD, xt, st) != hipSuccess) return COLI_EDEVICE;
        }
        {
            StageTimer tgu(kStGateUp, st, true);
            DecArgs a = {};
            a.w[0] = (const uint8_t *)ex->w_gate;
            a.w[1] = (const uint8_t *)ex->w_up;
            a.s[0] = ex->s_gate;
            a.s[1] = ex->s_up;
            a.w_gstride = gstrD;
            a.tiled = tiled;
            a.s_gstride = gs ? (int64_t)((F + 15) / 16) * (kpD / gs) * 16 : F;
            a.gs_spg = gs / 32;
            a.gs_ngp = gs ? kpD / gs : 0;
            a.ngroups = E;
            a.O = F;
            if (sh_mm) {
                a.has_extra = 1;
                a.xw[0] = (const uint8_t *)sh->w_gate;
                a.xw[1] = (const uint8_t *)sh->w_up;
                a.xs[0] = sh->s_gate;
                a.xs[1] = sh->s_up;
                a.xO = F;
                a.x_rows = S;
                a.x_row0 = (int)shared_row0;
            }
            a.I = D;
            a.kpad = kpD;
            a.rb = rbD;
            a.offsets = offsets;
            a.row_pair = row_pair;
            a.K = K;
            a.act_by_token = 1;
            a.act = xt;
            a.work = work;
            a.n_work = n_work;
            a.out = h;
            a.ldo = L.h_ld;
            a.out_vec4 = L.h_ld % 4 == 0 && al16(h);
            a.hf = ht;
            a.hf_kpad = kpF;
            if (dec_launch(a, ex->fmt, 2, max_gp, st) != hipSuccess) return COLI_EDEVICE;
        }
        {
            StageTimer tdn(kStDown, st, true);
            DecArgs d = {};
            d.w[0] = (const uint8_t *)ex->w_down;
            d.s[0] = ex->s_down;
            d.w_gstride = gstrF;
            d.tiled = tiled;
            d.s_gstride = gs ? (int64_t)((D + 15) / 16) * (kpF / gs) * 16 : D;
            d.gs_spg = gs / 32;
            d.gs_ngp = gs ? kpF / gs : 0;
            d.ngroups = E;
            d.O = D;
            if (sh_mm) {
                d.has_extra = 1;
                d.xw[0] = (const uint8_t *)sh->w_down;
                d.xs[0] = sh->s_down;
                d.xO = D;
                d.x_rows = S;
                d.x_row0 = (int)shared_row0;
            }
            d.I = F;
            d.kpad = kpF;
            d.rb = rbF;
            d.offsets = offsets;
            d.row_pair = row_pair;
            d.K = K;
            d.act_by_token = 0;
            d.act = ht;
            d.work = work;
            d.n_work = n_work;
            d.out = y;
            d.ldo = D;
            d.out_vec4 = D % 4 == 0 && al16(y);
            if (dec_launch(d, ex->fmt, 1, max_gp, st) != hipSuccess) return COLI_EDEVICE;
        }
        if (sh && !sh_mm) {
            int rc = run_shared_valu(sh, x, S, D, h, L.h_ld, y, shared_row0, hint, st);
            if (rc != COLI_OK) return rc;
        }
        StageTimer tcb(kStCombine, st);
        return to_status(combine_launch(y, S, D, K, pair_row, w, sh ? 1 : 0, shared_row0, out,
                                        (int)(al16(out) && al16(y) && D % 4 == 0 && (!resid || al16(resid))), st, resid));
    }
    if (idot) {
        // integer dots: x quantised once per token, the SwiGLU output once
        // per grouped row (int8 tables, scales and sums of the int8 values)
        const int64_t rows = (int64_t)P + (sh ? S : 0);   // grouped rows (the workspace has no shared rows without one)
        const int64_t kqD = coli__kpad(D), kqF = coli__kpad(F);
        int8_t *xt = reinterpret_cast<int8_t *>(ws + L.xf);
        float *tok_sx = reinterpret_cast<float *>(ws + L.xsum);
        int *tok_sq = reinterpret_cast<int *>(ws + L.xsum + (int64_t)S * 4);
        int32_t *act_row = reinterpret_cast<int32_t *>(ws + L.xsum + (int64_t)5 * S * 4);
        float *row_sx = reinterpret_cast<float *>(ws + L.xsum + ((int64_t)5 * S + rows) * 4);
        int *row_sq = reinterpret_cast<int *>(ws + L.xsum + ((int64_t)5 * S + 2 * rows) * 4);
        int8_t *ht = reinterpret_cast<int8_t *>(ws + L.hf);
        float *h_sx = reinterpret_cast<float *>(ws + L.hsum);
        int *h_sq = reinterpret_cast<int *>(ws + L.hsum + rows * 4);
        float *hrow_sx = reinterpret_cast<float *>(ws + L.hsum + rows * 5 * 4);
        int *hrow_sq = reinterpret_cast<int *>(ws + L.hsum + rows * 6 * 4);
        const int64_t max_gp = L.n_pass_max;
        {
            StageTimer tp(kStPrep, st);
            if (qrow_launch(ex->fmt, x, S, D, kqD, xt, tok_sx, tok_sq, st) != hipSuccess) return COLI_EDEVICE;
            if (idrows_launch(row_pair, P, K, S, (int)rows, tok_sx, tok_sq, act_row, row_sx, row_sq, st) !=
                hipSuccess)
                return COLI_EDEVICE;
        }
        {
            StageTimer tgu(kStGateUp, st, true);
            PreIdArgs a = {};
            a.w[0] = (const uint8_t *)ex->w_gate;
            a.w[1] = (const uint8_t *)ex->w_up;
            a.s[0] = ex->s_gate;
            a.s[1] = ex->s_up;
            a.w_gstride = gstrD;
            a.s_gstride = F;
            a.ngroups = E;
            a.O = F;
            if (sh) {
                a.has_extra = 1;
                a.xw[0] = (const uint8_t *)sh->w_gate;
                a.xw[1] = (const uint8_t *)sh->w_up;
                a.xs[0] = sh->s_gate;
                a.xs[1] = sh->s_up;
                a.xO = F;
                a.x_rows = S;
                a.x_row0 = (int)shared_row0;
            }
            a.I = D;
            a.rb = rbD;
            a.kq = kqD;
            a.offsets = offsets;
            a.work = work;
            a.n_work = n_work;
            a.act_row = act_row;
            a.row_sx = row_sx;
            a.row_sq = row_sq;
            a.act = xt;
            a.out = h;
            a.ldo = L.h_ld;
            a.out_vec4 = L.h_ld % 4 == 0 && al16(h);
            if (preid_launch(a, ex->fmt, 2, max_gp, st) != hipSuccess) return COLI_EDEVICE;
        }
        {
            StageTimer tdn(kStDown, st);
            // h rows are F wide (a shared expert has the same F here)
            if (qrow_launch(ex->fmt, h, (int)rows, F, kqF, ht, h_sx, h_sq, st) != hipSuccess ||
                idrows_launch(nullptr, 0, K, (int)rows, (int)rows, h_sx, h_sq, nullptr, hrow_sx, hrow_sq, st) !=
                    hipSuccess)
                return COLI_EDEVICE;
            PreIdArgs d = {};
            d.w[0] = (const uint8_t *)ex->w_down;
            d.s[0] = ex->s_down;
            d.w_gstride = gstrF;
            d.s_gstride = D;
            d.ngroups = E;
            d.O = D;
            if (sh) {
                d.has_extra = 1;
                d.xw[0] = (const uint8_t *)sh->w_down;
                d.xs[0] = sh->s_down;
                d.xO = D;
                d.x_rows = S;
                d.x_row0 = (int)shared_row0;
            }
            d.I = F;
            d.rb = rbF;
            d.kq = kqF;
            d.offsets = offsets;
            d.work = work;
            d.n_work = n_work;
            d.act_row = nullptr;
            d.row_sx = hrow_sx;
            d.row_sq = hrow_sq;
            d.act = ht;
            d.out = y;
            d.ldo = D;
            d.out_vec4 = D % 4 == 0 && al16(y);
            if (preid_launch(d, ex->fmt, 1, max_gp, st) != hipSuccess) return COLI_EDEVICE;
        }
        StageTimer tcb(kStCombine, st);
        return to_status(combine_launch(y, S, D, K, pair_row, w, sh ? 1 : 0, shared_row0, out,
                                        (int)(al16(out) && al16(y) && D % 4 == 0 && (!resid || al16(resid))), st, resid));
    }
    if (mm) {
        // bf16 precision: x as one bf16 row table per token, the SwiGLU
        // output as one per grouped row; per-row activation sums
        const int64_t rows = (int64_t)P + (sh ? S : 0);   // grouped rows (the workspace has no shared rows without one)
        const int kpD = (int)coli__kpad(D), kpF = (int)coli__kpad(F);
        const int nparts = pre_parts(kpF, gs != 0);   // h's partial sums per grouped row
        uint16_t *xt = reinterpret_cast<uint16_t *>(ws + L.xf);
        float *tok_sum = reinterpret_cast<float *>(ws + L.xsum);
        int32_t *act_row = reinterpret_cast<int32_t *>(ws + L.xsum + (int64_t)S * 4);
        float *row_sum = reinterpret_cast<float *>(ws + L.xsum + ((int64_t)S + rows) * 4);
        uint16_t *ht = reinterpret_cast<uint16_t *>(ws + L.hf);
        float *hpart = reinterpret_cast<float *>(ws + L.hsum);
        float *hsum = reinterpret_cast<float *>(ws + L.hsum + rows * nparts * 4);
        const int64_t max_gp = L.n_pass_max;
        const int ybf = sh && !sh_mm ? 0 : 1;
        {
            StageTimer tp(kStPrep, st);
            if (xrows_bf16_launch(ex->fmt, x, D, S, D, kpD, xt, tok_sum, st) != hipSuccess) return COLI_EDEVICE;
            if (pre_rows_launch(row_pair, P, K, S, (int)(rows - P), tok_sum, act_row, row_sum, st) != hipSuccess)
                return COLI_EDEVICE;
        }
        {
            StageTimer tgu(kStGateUp, st, true);
            PreArgs a = {};
            a.w[0] = (const uint8_t *)ex->w_gate;
            a.w[1] = (const uint8_t *)ex->w_up;
            a.s[0] = ex->s_gate;
            a.s[1] = ex->s_up;
            a.w_gstride = gstrD;
            a.tiled = tiled;
            a.s_gstride = gs ? (int64_t)((F + 15) / 16) * (kpD / gs) * 16 : F;
            a.gs_spg = gs / 32;
            a.gs_ngp = gs ? kpD / gs : 0;
            a.ngroups = E;
            a.O = F;
            if (sh_mm) {
                a.has_extra = 1;
                a.xw[0] = (const uint8_t *)sh->w_gate;
                a.xw[1] = (const uint8_t *)sh->w_up;
                a.xs[0] = sh->s_gate;
                a.xs[1] = sh->s_up;
                a.xO = F;
                a.x_rows = S;
                a.x_row0 = (int)shared_row0;
            }
            a.kpad = kpD;
            a.rb = rbD;
            a.offsets = offsets;
            a.work = work;
            a.n_work = n_work;
            a.act_row = act_row;
            a.row_sum = row_sum;
            a.act = xt;
            a.out = nullptr;   // h only as the down product's bf16 row table
            a.hf = ht;
            a.hf_kpad = kpF;
            a.hpart = hpart;
            a.nparts = nparts;
            if (pre_launch(a, ex->fmt, 2, max_gp, st) != hipSuccess) return COLI_EDEVICE;
        }
        {
            StageTimer tdn(kStDown, st);
            if (pre_sum_launch(hpart, nparts, (int)rows, hsum, st) != hipSuccess) return COLI_EDEVICE;
            PreArgs d = {};
            d.w[0] = (const uint8_t *)ex->w_down;
            d.s[0] = ex->s_down;
            d.w_gstride = gstrF;
            d.tiled = tiled;
            d.s_gstride = gs ? (int64_t)((D + 15) / 16) * (kpF / gs) * 16 : D;
            d.gs_spg = gs / 32;
            d.gs_ngp = gs ? kpF / gs : 0;
            d.ngroups = E;
            d.O = D;
            if (sh_mm) {
                d.has_extra = 1;
                d.xw[0] = (const uint8_t *)sh->w_down;
                d.xs[0] = sh->s_down;
                d.xO = D;
                d.x_rows = S;
                d.x_row0 = (int)shared_row0;
            }
            d.kpad = kpF;
            d.rb = rbF;
            d.offsets = offsets;
            d.work = work;
            d.n_work = n_work;
            d.act_row = nullptr;
            d.row_sum = hsum;
            d.act = ht;
            d.out = y;
            d.ldo = D;
            // y rounded to bf16 (half the bytes written here and read by the
            // combine), unless a vector-ALU shared expert writes fp32 rows
            d.out_bf16 = ybf;
            d.out_vec4 = D % 4 == 0 && al16(y);
            if (pre_launch(d, ex->fmt, 1, max_gp, st) != hipSuccess) return COLI_EDEVICE;
        }
        if (sh && !sh_mm) {
            int rc = run_shared_valu(sh, x, S, D, h, L.h_ld, y, shared_row0, hint, st);
            if (rc != COLI_OK) return rc;
        }
        StageTimer tcb(kStCombine, st);
        return to_status(combine_launch(y, S, D, K, pair_row, w, sh ? 1 : 0, shared_row0, out,
                                        (int)(al16(out) && al16(y) && D % 4 == 0 && (!resid || al16(resid))), st, resid,
                                        ybf));
    }
    const bool sh_same_up = sh && sh->fmt == ex->fmt;
    const bool sh_same_down = sh && sh->fmt == ex->fmt && sh->F == F;

    // ---- gate/up + SwiGLU -> h
    {
    StageTimer tgu(kStGateUp, st);
    GemvArgs a = {};
    a.w[0] = (const uint8_t *)ex->w_gate;
    a.w[1] = (const uint8_t *)ex->w_up;
    a.s[0] = ex->s_gate;
    a.s[1] = ex->s_up;
    a.w_gstride = (int64_t)F * rbD;
    a.s_gstride = F;
    a.ngroups = E;
    a.O = F;
    a.I = D;
    a.rb = rbD;
    a.offsets = offsets;
    a.row_pair = row_pair;
    a.K = K;
    a.xrow_token = 1;
    a.x = x;
    a.ldx = D;
    a.x_vec4 = al16(x) && (D % 4 == 0);
    a.out = h;
    a.ldo = L.h_ld;
    a.aligned = (rbD % 16 == 0) && al16(ex->w_gate) && al16(ex->w_up);
    if (sh_same_up) {
        a.has_extra = 1;
        a.xw[0] = (const uint8_t *)sh->w_gate;
        a.xw[1] = (const uint8_t *)sh->w_up;
        a.xs[0] = sh->s_gate;
        a.xs[1] = sh->s_up;
        a.xO = sh->F;
        a.x_rows = S;
        a.x_row0 = (int)shared_row0;
        a.aligned = a.aligned && al16(sh->w_gate) && al16(sh->w_up);
    }
    err = gemv_launch(a, ex->fmt, 2, hint, st);
    if (err != hipSuccess) return COLI_EDEVICE;
    if (sh && !sh_same_up) {
        GemvArgs b = a;
        const int64_t rbs = coli_row_bytes(sh->fmt, D);
        b.ngroups = 0;
        b.has_extra = 1;
        b.xw[0] = (const uint8_t *)sh->w_gate;
        b.xw[1] = (const uint8_t *)sh->w_up;
        b.xs[0] = sh->s_gate;
        b.xs[1] = sh->s_up;
        b.xO = sh->F;
        b.O = sh->F;
        b.x_rows = S;
        b.x_row0 = (int)shared_row0;
        b.rb = rbs;
        b.aligned = (rbs % 16 == 0) && al16(sh->w_gate) && al16(sh->w_up);
        err = gemv_launch(b, sh->fmt, 2, hint, st);
        if (err != hipSuccess) return COLI_EDEVICE;
    }
    }

    // ---- down -> y
    {
    StageTimer tdn(kStDown, st);
    GemvArgs d = {};
    d.w[0] = (const uint8_t *)ex->w_down;
    d.s[0] = ex->s_down;
    d.w_gstride = (int64_t)D * rbF;
    d.s_gstride = D;
    d.ngroups = E;
    d.O = D;
    d.I = F;
    d.rb = rbF;
    d.offsets = offsets;
    d.row_pair = row_pair;
    d.K = K;
    d.xrow_token = 0;
    d.x = h;
    d.ldx = L.h_ld;
    d.x_vec4 = (L.h_ld % 4 == 0);
    d.out = y;
    d.ldo = D;
    d.aligned = (rbF % 16 == 0) && al16(ex->w_down);
    if (sh_same_down) {
        d.has_extra = 1;
        d.xw[0] = (const uint8_t *)sh->w_down;
        d.xs[0] = sh->s_down;
        d.xO = D;
        d.x_rows = S;
        d.x_row0 = (int)shared_row0;
        d.aligned = d.aligned && al16(sh->w_down);
    }
    err = gemv_launch(d, ex->fmt, 1, hint, st);
    if (err != hipSuccess) return COLI_EDEVICE;
    if (sh && !sh_same_down) {
        GemvArgs b = d;
        const int64_t rbs = coli_row_bytes(sh->fmt, sh->F);
        b.ngroups = 0;
        b.has_extra = 1;
        b.xw[0] = (const uint8_t *)sh->w_down;
        b.xs[0] = sh->s_down;
        b.xO = D;
        b.x_rows = S;
        b.x_row0 = (int)shared_row0;
        b.I = sh->F;
        b.rb = rbs;
        b.aligned = (rbs % 16 == 0) && al16(sh->w_down);
        err = gemv_launch(b, sh->fmt, 1, hint, st);
        if (err != hipSuccess) return COLI_EDEVICE;
    }
    }

    // ---- weighted combine, fixed order
    StageTimer tcb(kStCombine, st);
    return to_status(combine_launch(y, S, D, K, pair_row, w, sh ? 1 : 0, shared_row0, out,
                                    (int)(al16(out) && al16(y) && D % 4 == 0 && (!resid || al16(resid))), st, resid));
}

}  // namespace
}  // namespace coli

using namespace coli;

extern "C" int coli_qgemv(int fmt, const void *W, const float *scale, const float *x, float *y,
                          int S, int I, int O, void *stream)
{
    int rc = coli__check_qgemv(fmt, W, scale, x, y, S, I, O);
    if (rc != COLI_OK) return rc;
    if (S == 0 || O == 0) return COLI_OK;
    const int64_t rb = coli_row_bytes(fmt, I);
    if (fmt == COLI_F32 && qmv_f32_supported(I, W, x)) {
        // fp32 matrix cores: whole 16-byte runs, aligned operands
        QmvArgs q = {};
        q.W = (const uint8_t *)W;
        q.scale = scale;
        q.x = x;
        q.y = y;
        q.S = S;
        q.I = I;
        q.O = O;
        q.rb = rb;
        StageTimer t(kStQgemv, (hipStream_t)stream);
        return to_status(qmv_f32_launch(q, (hipStream_t)stream));
    }
    if (qmv_supported(fmt, rb, I, O, W, x)) {
        // matrix cores: whole 16-byte row segments, aligned operands
        QmvArgs q = {};
        q.W = (const uint8_t *)W;
        q.scale = scale;
        q.x = x;
        q.y = y;
        q.S = S;
        q.I = I;
        q.O = O;
        q.rb = rb;
        StageTimer t(kStQgemv, (hipStream_t)stream);
        return to_status(qmv_launch(q, fmt, (hipStream_t)stream));
    }
    GemvArgs a = {};
    a.w[0] = (const uint8_t *)W;
    a.s[0] = scale;
    a.ngroups = 1;
    a.O = O;
    a.x_rows = S;
    a.I = I;
    a.rb = rb;
    a.K = 1;
    a.x = x;
    a.ldx = I;
    a.x_vec4 = al16(x) && (I % 4 == 0);
    a.out = y;
    a.ldo = O;
    a.aligned = (rb % 16 == 0) && al16(W);
    StageTimer t(kStQgemv, (hipStream_t)stream);
    return to_status(gemv_launch(a, fmt, 1, S, (hipStream_t)stream));
}

extern "C" int coli_qgemv_grouped(const void *W, const float *scale, int gs, const float *x, float *y,
                                  int S, int I, int O, void *stream)
{
    if (S < 0 || I < 0 || O < 0) return COLI_ESHAPE;
    if (gs < 1) return COLI_ERANGE;
    int rc = coli__check_qgemv(COLI_I4, W, scale, x, y, S, I, O);
    if (rc != COLI_OK) return rc;
    if (S == 0 || O == 0) return COLI_OK;
    if (I < 1) return COLI_ESHAPE;
    const int64_t rb = coli_row_bytes(COLI_I4, I);
    if (!(gs == 32 || gs == 64 || (gs >= 128 && gs % 128 == 0))) return COLI_ERANGE;
    if (I > 12288) return COLI_ERANGE;
    if ((int64_t)O * rb >= ((int64_t)1 << 32) - 4096) return COLI_ERANGE;
    if (!qmv_grouped_supported(rb, I, gs, W, scale, x)) return COLI_EALIGN;
    QmvArgs q = {};
    q.W = (const uint8_t *)W;
    q.scale = scale;
    q.x = x;
    q.y = y;
    q.S = S;
    q.I = I;
    q.O = O;
    q.rb = rb;
    q.gs = gs;
    StageTimer t(kStQgemv, (hipStream_t)stream);
    return to_status(qmv_grouped_launch(q, (hipStream_t)stream));
}

extern "C" size_t coli_qgemv_idot_workspace_bytes(int S, int I)
{
    if (S < 0 || I < 1) return 0;
    return (size_t)idot_workspace_bytes(S, I);
}

extern "C" int coli_qgemv_idot(int fmt, const void *W, const float *scale, const float *x, float *y,
                               int S, int I, int O, void *ws, size_t ws_bytes, void *stream)
{
    if (fmt != COLI_I8 && fmt != COLI_I4) return COLI_EFMT;
    int rc = coli__check_qgemv(fmt, W, scale, x, y, S, I, O);
    if (rc != COLI_OK) return rc;
    if (S == 0 || O == 0) return COLI_OK;
    if (I < 1) return COLI_ESHAPE;
    const int64_t rb = coli_row_bytes(fmt, I);
    if (rb % 16 != 0 || ((uintptr_t)W & 15u)) return COLI_EALIGN;
    const int KB = idot_kblock(fmt);
    if ((I + KB - 1) / KB > 8 * idot_max_kblocks_per_wave()) return COLI_ERANGE;
    if ((int64_t)O * rb >= ((int64_t)1 << 32) - 4096) return COLI_ERANGE;
    if (!ws || ws_bytes < (size_t)idot_workspace_bytes(S, I)) return COLI_EWORKSPACE;
    if ((uintptr_t)ws & 255u) return COLI_EALIGN;
    IdotArgs a = {};
    a.W = (const uint8_t *)W;
    a.scale = scale;
    a.x = x;
    a.y = y;
    a.S = S;
    a.I = I;
    a.O = O;
    a.rb = rb;
    const int64_t tb = ((int64_t)S * idot_row_bytes(I) + 255) / 256 * 256;
    a.table = (int8_t *)ws;
    a.sx = reinterpret_cast<float *>((uint8_t *)ws + tb);
    a.sq = reinterpret_cast<int *>((uint8_t *)ws + tb + (int64_t)S * 4);
    StageTimer t(kStQgemv, (hipStream_t)stream);
    return to_status(idot_launch(a, fmt, (hipStream_t)stream));
}

extern "C" int coli_router(const float *Wr, const float *bias, const float *x, int S, int E,
                           int D, int K, int norm_topk, float routed_scale, float topp,
                           int32_t *idx, float *w, int32_t *keff, float *sig, void *ws,
                           size_t ws_bytes, void *stream)
{
    int rc = coli__check_router(Wr, bias, x, S, E, D, K, norm_topk, idx, w, sig, ws, ws_bytes);
    if (rc != COLI_OK) return rc;
    if (S == 0) return COLI_OK;
    StageTimer t(kStRouter, (hipStream_t)stream);
    return to_status(router_launch(Wr, bias, x, S, E, D, K, norm_topk, routed_scale, topp, idx,
                                   w, keff, sig, (double *)ws, (hipStream_t)stream));
}

extern "C" int coli_moe_gemv(const coli_experts *ex, const float *x, int S, int K,
                             const int32_t *idx, const float *w, float *out, int prec, void *ws,
                             size_t ws_bytes, void *stream)
{
    int rc = coli__check_moe(ex, nullptr, x, S, K, idx, w, out, prec, ws, ws_bytes, 1);
    if (rc != COLI_OK) return rc;
    if (S == 0) return COLI_OK;
    coli_ws_layout L;
    rc = coli_moe_workspace_layout(S, K, ex->E, ex->D, ex->F, 0, prec, &L);
    if (rc != COLI_OK) return rc;
    return run_experts(ex, nullptr, x, S, K, idx, w, out, prec, (uint8_t *)ws, L, (hipStream_t)stream);
}

// The MoE block on x; with resid, out = resid + block (the layer tail).
static int moe_layer_impl(const coli_router_params *r, const coli_experts *ex,
                          const coli_mlp *shared, const float *x, int S,
                          const int32_t *pre_idx, const float *pre_w, float *out,
                          int32_t *idx_out, float *w_out, int prec, void *ws,
                          size_t ws_bytes, void *stream, const float *norm_w, float eps)
{
    if (!r) return COLI_EINVAL;
    if ((pre_idx == nullptr) != (pre_w == nullptr)) return COLI_EINVAL;
    const int K = r->K;
    int rc = coli__check_moe(ex, shared, x, S, K, pre_idx, pre_w, out, prec, ws, ws_bytes, 0);
    if (rc != COLI_OK) return rc;
    if ((idx_out && ((uintptr_t)idx_out & 3)) || (w_out && ((uintptr_t)w_out & 3)))
        return COLI_EALIGN;
    const bool run_router = pre_idx == nullptr;
    if (run_router) {
        if (!r->w || !r->bias) return COLI_EINVAL;
        if (K > ex->E) return COLI_ERANGE;
        if (r->norm_topk != 0 && r->norm_topk != 1) return COLI_EINVAL;
        if (((uintptr_t)r->w & 3) || ((uintptr_t)r->bias & 3)) return COLI_EALIGN;
    }
    if (norm_w) {
        if (!(eps >= 0.f)) return COLI_EINVAL;   // also rejects NaN
        if ((uintptr_t)norm_w & 3) return COLI_EALIGN;
    }
    if (S == 0) return COLI_OK;
    coli_ws_layout L;
    rc = coli_moe_workspace_layout(S, K, ex->E, ex->D, ex->F, shared ? shared->F : 0, prec, &L);
    if (rc != COLI_OK) return rc;
    uint8_t *wsb = (uint8_t *)ws;
    hipStream_t st = (hipStream_t)stream;
    const int32_t *idx = pre_idx;
    const float *w = pre_w;
    const float *resid = nullptr;
    if (norm_w) {
        // the block runs on the normalised rows; x stays the residual
        float *xn = reinterpret_cast<float *>(wsb + L.xn);
        StageTimer tn(kStNorm, st);
        const int D = ex->D;
        const int vec4 = D % 4 == 0 && al16(x) && al16(norm_w) && al16(xn);
        hipLaunchKernelGGL(k_rmsnorm, dim3((unsigned)S), dim3(kNormThreads), 0, st, x, norm_w, D, eps, xn,
                           vec4);
        if (hipGetLastError() != hipSuccess) return COLI_EDEVICE;
        resid = x;
        x = xn;
    }
    if (run_router) {
        int32_t *ri = idx_out ? idx_out : reinterpret_cast<int32_t *>(wsb + L.idx);
        float *rw = w_out ? w_out : reinterpret_cast<float *>(wsb + L.w);
        StageTimer tr(kStRouter, st);
        hipError_t e = router_launch(r->w, r->bias, x, S, ex->E, ex->D, K, r->norm_topk,
                                     r->routed_scale, r->topp, ri, rw, nullptr,
                                     reinterpret_cast<float *>(wsb + L.sig),
                                     reinterpret_cast<double *>(wsb + L.router_part), st);
        if (e != hipSuccess) return COLI_EDEVICE;
        idx = ri;
        w = rw;
    } else {
        const size_t n = (size_t)S * K;
        if (idx_out && hipMemcpyAsync(idx_out, pre_idx, n * 4, hipMemcpyDeviceToDevice, st) != hipSuccess)
            return COLI_EDEVICE;
        if (w_out && hipMemcpyAsync(w_out, pre_w, n * 4, hipMemcpyDeviceToDevice, st) != hipSuccess)
            return COLI_EDEVICE;
    }
    return run_experts(ex, shared, x, S, K, idx, w, out, prec, wsb, L, st, resid);
}

extern "C" int coli_moe_layer(const coli_router_params *r, const coli_experts *ex,
                              const coli_mlp *shared, const float *x, int S,
                              const int32_t *pre_idx, const float *pre_w, float *out,
                              int32_t *idx_out, float *w_out, int prec, void *ws,
                              size_t ws_bytes, void *stream)
{
    return moe_layer_impl(r, ex, shared, x, S, pre_idx, pre_w, out, idx_out, w_out, prec, ws, ws_bytes,
                          stream, nullptr, 0.f);
}

// ---------------------------------------------------------------- no allocation
// The MoE layer for callers that cannot allocate: its scratch is one static
// device array, which every GPU the library runs on holds (at its own
// address) until the process ends.  Host code never passes the array's name
// to a kernel (on the host it is only a stand-in for the symbol): the device
// address is looked up once per device with hipGetSymbolAddress and kept.
static __device__ __align__(256) uint8_t scratch[COLI_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<uintptr_t> g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (looked up on the first call made
// with that device current).
int scratch_ptr(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return COLI_EDEVICE;
    if (dev < 0 || dev >= kMaxDevices) return COLI_EDEVICE;
    uintptr_t p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return COLI_EDEVICE;
        p = (uintptr_t)ptr;
        g_scratch_ptr[dev].store(p, std::memory_order_release);   // same value from any racing caller
    }
    *out = (void *)p;
    return COLI_OK;
}
}  // namespace

extern "C" int coli_moe_layer_noalloc(const coli_router_params *r, const coli_experts *ex,
                                      const coli_mlp *shared, const float *x, int S,
                                      const int32_t *pre_idx, const float *pre_w, float *out,
                                      int32_t *idx_out, float *w_out, int prec, void *stream)
{
    if (!r || !ex) return COLI_EINVAL;
    const size_t need = coli_moe_workspace_bytes(S, r->K, ex->E, ex->D, ex->F, shared ? shared->F : 0, prec);
    if (need > (size_t)COLI_NOALLOC_SCRATCH_BYTES) return COLI_ERANGE;   // before any device call
    if (need == 0 || S == 0)   // invalid sizes or an empty batch: the ordinary checks answer
        return moe_layer_impl(r, ex, shared, x, S, pre_idx, pre_w, out, idx_out, w_out, prec, nullptr, 0,
                              stream, nullptr, 0.f);
    void *ws = nullptr;
    const int rc = scratch_ptr(&ws);
    if (rc != COLI_OK) return rc;
    return moe_layer_impl(r, ex, shared, x, S, pre_idx, pre_w, out, idx_out, w_out, prec, ws, need, stream,
                          nullptr, 0.f);
}

extern "C" int coli_moe_layer_tail(const coli_router_params *r, const coli_experts *ex,
                                   const coli_mlp *shared, const float *x, const float *norm_w,
                                   float eps, int S, const int32_t *pre_idx, const float *pre_w,
                                   float *out, int32_t *idx_out, float *w_out, int prec, void *ws,
                                   size_t ws_bytes, void *stream)
{
    if (!norm_w) return COLI_EINVAL;
    return moe_layer_impl(r, ex, shared, x, S, pre_idx, pre_w, out, idx_out, w_out, prec, ws, ws_bytes,
                          stream, norm_w, eps);
}

extern "C" int coli_check_device_flags(const void *ws, void *stream, uint32_t *flags_out)
{
    if (!ws) return COLI_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    uint32_t f = 0;
    if (hipMemcpyAsync(&f, ws, sizeof f, hipMemcpyDeviceToHost, st) != hipSuccess)
        return COLI_EDEVICE;
    if (hipStreamSynchronize(st) != hipSuccess) return COLI_EDEVICE;
    if (flags_out) *flags_out = f;
    return f ? COLI_EIDX : COLI_OK;
}
