// coli_mfma.hip -- grouped dequant-on-use products on the bf16 matrix cores
// (gfx950 v_mfma_f32_16x16x32_bf16), fp32-equivalent accuracy.
//
// Same products as coli_gemv.hip [glm.c@98759bf -- matmul_q, matmul_i4,
// matmul_i2, moe phase D; glm.c@97c756a -- matmul_i4_pair, expert_gate_up;
// metal@93cde63 -- moe_gemv, moe_silu], arranged for the matrix cores:
//
//   * weights: each int8 / int4 / int2 value v is turned into an exact bf16
//     "code" v + OFF with a mask-and-or against a bf16 exponent pattern
//     (0x4300 = 128.0: 128 + nibble, 128 + crumb) or, for int8, a byte
//     conversion; OFF * sum(x) is removed per output after the sum.
//   * activations: x = hi + lo with hi = bf16(x), lo = bf16(x - hi), both
//     rounded to nearest even; |x - hi - lo| <= 2^-16 |x|, so the product
//     keeps fp32-level accuracy (the bound of the per-row tolerance is
//     1e-4).  Token t of a pass occupies MFMA columns 2t (hi) and 2t+1 (lo):
//     16 columns = 8 tokens; the two columns are added in the epilogue.
//   * the k order inside each group of 8 (int4) or 16 (int2) elements is the
//     order the unpacking produces; activations are stored in that order, so
//     no shuffle is needed in the loop.
//   * work: a list of (group, token pass) built on the device; each item is
//     one (group, pass, 128-row tile); persistent blocks walk the items of
//     their XCD, and all tiles of one group-pass run on the same XCD so its
//     activation rows are fetched into one L2.
#include "coli_device.h"
#include "coli_mfma.h"

namespace coli {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kRowsPerWave = 32;   // two 16-row MFMA tiles
constexpr int kRowsPerBlock = 128; // four waves
constexpr int kXcds = 8;

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

// bf16 codes for MFMA step s (8 elements) of a 16-byte segment.
template <int FMT> __device__ __forceinline__ uint4 codes(const uint4 &w, int s);

// int4: word s holds nibbles n0..n7; the pairs (n_i, n_i+4) sit at bits
// 4i and 4i+16, so (word >> 4i) & 0x000F000F | 0x43004300 is the bf16 pair
// (128 + n_i, 128 + n_i+4).  Slot order [0,4,1,5,2,6,3,7].
template <> __device__ __forceinline__ uint4 codes<kI4>(const uint4 &w, int s)
{
    const uint32_t u = wsel(w, s);
    const uint32_t m = 0x000F000Fu, e = 0x43004300u;
    return make_uint4((u & m) | e, ((u >> 4) & m) | e, ((u >> 8) & m) | e, ((u >> 12) & m) | e);
}

// int2: word s/2 holds crumbs c0..c15; (word >> 2k) & 0x00030003 | 0x43004300
// is the pair (128 + c_k, 128 + c_k+8).  Step s covers k = 4(s&1) .. +3.
// Slot order [0,8,1,9,2,10,3,11 | 4,12,5,13,6,14,7,15].
template <> __device__ __forceinline__ uint4 codes<kI2>(const uint4 &w, int s)
{
    const uint32_t u = wsel(w, s >> 1);
    const int k0 = 4 * (s & 1);
    const uint32_t m = 0x00030003u, e = 0x43004300u;
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

__device__ __forceinline__ floatx4 mfma(const uint4 &a, const uint4 &b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- layout
// Work is cut into passes of up to kTPP = 16 activation rows ("tokens") of
// one group.  A pass's activations are stored "fragment-major": for k-block
// kbi, MFMA step s and lane group q, chunk c = (kbi*STEPS + s)*4 + q holds,
// for each of the kCols = 32 columns (token t: column 2t = hi, 2t+1 = lo;
// N-tile n = columns 16n..16n+15), the 8 bf16 values of the slots that lane
// (col, q) feeds to that step.  A k-block's activations are one contiguous
// STEPS*2 KB run, and the live tokens' columns are a prefix of every chunk.
// Element e of the product's input sits in chunk c, slot j = pos_of(e).
constexpr int kTPP = 16;
constexpr int kCols = 2 * kTPP;

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

__device__ __forceinline__ void pos_any(int fmt, int e, int &c, int &j)
{
    if (fmt == kI4) pos_of<kI4>(e, c, j);
    else if (fmt == kI2) pos_of<kI2>(e, c, j);
    else pos_of<kI8>(e, c, j);
}

// Group-pass decode shared by the prep and the product kernels.
struct GP {
    int g, pass, r0, cnt, t0, nt;
    bool extra;
};
__device__ __forceinline__ GP decode_gp(const MmArgs &a, int gp)
{
    GP d;
    if (a.work) {
        const int wv = a.work[gp];
        d.g = wv & 0x7FF;
        d.pass = wv >> 11;
    } else {
        d.g = 0;
        d.pass = gp;
    }
    d.extra = a.has_extra && d.g == a.ngroups;
    if (d.extra) {
        d.r0 = a.x_row0;
        d.cnt = a.x_rows;
    } else if (a.offsets) {
        d.r0 = a.offsets[d.g];
        d.cnt = a.offsets[d.g + 1] - d.r0;
    } else {
        d.r0 = 0;
        d.cnt = a.x_rows;
    }
    d.t0 = d.pass * kTPP;
    d.nt = min(kTPP, d.cnt - d.t0);
    return d;
}

__device__ __forceinline__ int n_group_passes(const MmArgs &a)
{
    return a.work ? *a.n_work : (a.x_rows + kTPP - 1) / kTPP;
}

// ---------------------------------------------------------------- x prep
// One block per group-pass: gathers the pass's activation rows (dead ones
// as zeros), splits them into bf16 hi/lo and stores them fragment-major;
// also sum(hi + lo) per token, in a fixed order.
template <int FMT>
__global__ __launch_bounds__(256) void k_xprep(MmArgs a, const float *__restrict__ x, int64_t ldx)
{
    using T = MF<FMT>;
    __shared__ float red[4][kTPP];
    const int gp = blockIdx.x;
    if (gp >= n_group_passes(a)) return;
    const GP d = decode_gp(a, gp);
    const int tid = threadIdx.x, t = tid % kTPP;
    int row = -1;
    if (t < d.nt) {
        const int tok = d.t0 + t;
        if (!a.xrow_token) row = d.r0 + tok;
        else if (d.extra) row = tok;
        else row = a.row_pair[d.r0 + tok] / a.K;
    }
    const float *xr = row >= 0 ? x + (int64_t)row * ldx : nullptr;
    uint16_t *dst = a.xf + (int64_t)gp * a.xf_stride;
    const int nchunks = a.kpad / 8;
    float sum = 0.f;
    for (int item = tid; item < nchunks * kTPP; item += 256) {
        const int c = item / kTPP;
        const int kbi = c / (T::STEPS * 4), s = (c >> 2) % T::STEPS, q = c & 3;
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int j2 = 0; j2 < 4; ++j2) {
            uint32_t hp = 0, lp = 0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int e = elem_of<FMT>(kbi, s, q, 2 * j2 + h);
                const float v = (xr && e < a.I) ? xr[e] : 0.f;
                const uint16_t hv = bf16_rne(v);
                const uint16_t lv = bf16_rne(v - bf16_f(hv));
                sum += bf16_f(hv) + bf16_f(lv);
                hp |= (uint32_t)hv << (16 * h);
                lp |= (uint32_t)lv << (16 * h);
            }
            hw[j2] = hp;
            lw[j2] = lp;
        }
        *reinterpret_cast<uint4 *>(dst + ((int64_t)c * kCols + 2 * t) * 8) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        *reinterpret_cast<uint4 *>(dst + ((int64_t)c * kCols + 2 * t + 1) * 8) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
    // lanes with the same t (= lane % 16): xor over the higher lane bits
    sum += __shfl_xor(sum, 16, kWave);
    sum += __shfl_xor(sum, 32, kWave);
    if ((tid & 63) < kTPP) red[tid >> 6][t] = sum;
    __syncthreads();
    if (tid < kTPP)
        a.xsum[(int64_t)gp * kTPP + tid] = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
}

// ---------------------------------------------------------------- main kernel
// NTL = N-tiles (of 16 columns = 8 tokens) processed per pass: 1 when the
// pass has at most 8 live tokens, else 2.
template <int FMT, int M, int NTL>
__device__ __forceinline__ void mm_kloop(const MmArgs &a, const uint8_t *const (&wr)[M][2],
                                         int64_t last_seg, int src_lane, const uint4 *bglob,
                                         int live_units, int nkb, int tid, int lane,
                                         uint4 (*bsh)[MF<FMT>::STEPS * 4 * kCols],
                                         floatx4 (&acc)[M][2][2])
{
    using T = MF<FMT>;
    constexpr int SEGS = T::SEGS, SPS = T::SPS, STEPS = T::STEPS, KB = T::KB, BITS = T::BITS;
    constexpr int CH = STEPS * 4;                 // chunks per k-block
    constexpr int UMAX = (CH * kCols + 255) / 256;
    const int q = lane >> 4, col = lane & 15;
    // k-block kbi: segment sg of each row at byte kbi*KB*BITS/8 + 64 sg + 16
    // chunk.  Its activations are loaded once per block -- only the live
    // columns, live_units = CH * 2nt 16-byte units, spread over the block --
    // and shared through LDS, so the weights are nearly the only global
    // loads (every 16-byte-per-lane load costs the texture path about the
    // same, whatever it reads).
    const int lc = live_units / CH;               // live columns per chunk
    auto load = [&](int kbi, uint4 (&wv)[M][2][SEGS], uint4 (&bv)[UMAX]) {
        const int64_t b0 = (int64_t)kbi * KB * BITS / 8;
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int sg = 0; sg < SEGS; ++sg)
                    wv[m][mt][sg] = gload16(wr[m][mt] + min(b0 + 64 * sg, last_seg));
#pragma unroll
        for (int i = 0; i < UMAX; ++i) {
            const int u = tid + 256 * i;
            if (u < live_units) {
                const int ch = u / lc, cu = u - ch * lc;
                bv[i] = gload16(bglob + ((int64_t)kbi * CH + ch) * kCols + cu);
            }
        }
    };
    auto stage = [&](int buf, const uint4 (&bv)[UMAX]) {
#pragma unroll
        for (int i = 0; i < UMAX; ++i) {
            const int u = tid + 256 * i;
            if (u < live_units) {
                const int ch = u / lc, cu = u - ch * lc;
                bsh[buf][ch * kCols + cu] = bv[i];
            }
        }
    };
    auto compute = [&](const uint4 (&wl)[M][2][SEGS], int buf) {
        uint4 wv[M][2][SEGS];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int sg = 0; sg < SEGS; ++sg) {
                    const uint4 v = wl[m][mt][sg];
                    wv[m][mt][sg] = make_uint4(
                        (uint32_t)__builtin_amdgcn_ds_bpermute(4 * src_lane, (int)v.x),
                        (uint32_t)__builtin_amdgcn_ds_bpermute(4 * src_lane, (int)v.y),
                        (uint32_t)__builtin_amdgcn_ds_bpermute(4 * src_lane, (int)v.z),
                        (uint32_t)__builtin_amdgcn_ds_bpermute(4 * src_lane, (int)v.w));
                }
#pragma unroll
        for (int s2 = 0; s2 < STEPS; ++s2) {
            uint4 xb[NTL];
#pragma unroll
            for (int n = 0; n < NTL; ++n) xb[n] = bsh[buf][(s2 * 4 + q) * kCols + 16 * n + col];
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const uint4 cw = codes<FMT>(wv[m][mt][s2 / SPS], s2 % SPS);
#pragma unroll
                    for (int n = 0; n < NTL; ++n) acc[m][mt][n] = mfma(cw, xb[n], acc[m][mt][n]);
                }
        }
    };
    // Weights double-buffered in registers, activations in LDS, one k-block
    // ahead; straight-line body (the last prefetch re-reads a valid k-block
    // and is not used).  sched_barrier keeps the scheduler from sinking a
    // prefetch below the products.
    uint4 wa[M][2][SEGS], wb[M][2][SEGS], ba[UMAX], bb[UMAX];
    __syncthreads();   // bsh of the previous item is no longer read
    load(0, wa, ba);
    stage(0, ba);
    __syncthreads();
    for (int kbi = 0; kbi < nkb; kbi += 2) {
        load(kbi + 1, wb, bb);
        __builtin_amdgcn_sched_barrier(0);
        compute(wa, 0);
        __builtin_amdgcn_sched_barrier(0);
        stage(1, bb);
        __syncthreads();
        load(min(kbi + 2, nkb - 1), wa, ba);
        __builtin_amdgcn_sched_barrier(0);
        compute(wb, 1);
        __builtin_amdgcn_sched_barrier(0);
        // every wave finished reading buffer 0 before the barrier that
        // published buffer 1
        stage(0, ba);
        __syncthreads();
    }
}

template <int FMT, int M>
__global__ __launch_bounds__(256) void k_mm(MmArgs a)
{
    using T = MF<FMT>;
    constexpr int STEPS = T::STEPS, KB = T::KB;
    constexpr float OFF = T::OFF;
    __shared__ float red[4][kTPP];
    __shared__ uint4 bsh[2][STEPS * 4 * kCols];   // activations of one k-block, double-buffered

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, q = lane >> 4;
    const int xcd = blockIdx.x % kXcds, lb = blockIdx.x / kXcds;
    const int bpx = gridDim.x / kXcds;                 // blocks per XCD (grid is a multiple of 8)
    const int n_gp = n_group_passes(a);
    const int gp_per_xcd = (n_gp + kXcds - 1 - xcd) / kXcds;   // group-passes gp = xcd + 8 i
    const int n_items = gp_per_xcd * a.tiles;
    const int nkb = a.kpad / KB;                       // even: kpad is a multiple of 512

    for (int it = lb; it < n_items; it += bpx) {
        const int gp = xcd + kXcds * (it / a.tiles);
        const int tile = it % a.tiles;
        const GP d = decode_gp(a, gp);
        const uint8_t *W[M];
        const float *SC[M];
        int Og;
        if (d.extra) {
            Og = a.xO;
#pragma unroll
            for (int m = 0; m < M; ++m) { W[m] = a.xw[m]; SC[m] = a.xs[m]; }
        } else {
            Og = a.O;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                W[m] = a.w[m] + (int64_t)d.g * a.w_gstride;
                SC[m] = a.s[m] + (int64_t)d.g * a.s_gstride;
            }
        }
        const int obase = tile * kRowsPerBlock + wave * kRowsPerWave;
        // Weights are loaded row-contiguously -- lane L reads row L/4, chunk
        // L%4, so a quarter-wave touches 4 rows x 64 bytes -- and moved into
        // the MFMA operand layout (lane (q, col) holds row col, chunk q) with
        // ds_bpermute, which runs on the LDS crossbar instead of the texture
        // path.  Rows past Og are clamped (never written); segments past the
        // row end are clamped to its last segment and meet zero activations.
        const int lrow = lane >> 2, lchunk = lane & 3;
        const uint8_t *wr[M][2];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                wr[m][mt] = W[m] + (int64_t)min(obase + 16 * mt + lrow, Og - 1) * a.rb + 16 * lchunk;
        const int64_t last_seg = a.rb - 16 - 16 * lchunk;
        const uint4 *bglob = reinterpret_cast<const uint4 *>(a.xf + (int64_t)gp * a.xf_stride);
        const int live_units = STEPS * 4 * 2 * d.nt;
        floatx4 acc[M][2][2];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int n = 0; n < 2; ++n) acc[m][mt][n] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (nkb > 0) {
            if (d.nt > 8)
                mm_kloop<FMT, M, 2>(a, wr, last_seg, 4 * col + q, bglob, live_units, nkb, tid, lane, bsh, acc);
            else
                mm_kloop<FMT, M, 1>(a, wr, last_seg, 4 * col + q, bglob, live_units, nkb, tid, lane, bsh, acc);
        }
        // ---- epilogue: D[4q + r][16n + col]; add the lo column to the hi column
        float hpart[2] = {0.f, 0.f};   // per N-tile: this lane's hi + lo outputs (M == 2)
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int tok = 8 * n + (col >> 1);
            if (n == 1 && d.nt <= 8) break;            // uniform
            const bool live = tok < d.nt;
            float xs_t = 0.f;
            if (live)
                for (int p = 0; p < a.xsum_parts; ++p)
                    xs_t += gloadf(a.xsum + (int64_t)p * a.xsum_stride + (int64_t)gp * kTPP + tok);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                float v[M][4];
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[m][r] = acc[m][mt][n][r] + __shfl_xor(acc[m][mt][n][r], 1, kWave);
                const bool writer = (col & 1) == 0 && live;
                const int ob = obase + 16 * mt + 4 * q;
                float res[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int o = ob + r;
                    float y = 0.f;
                    if (o < Og) {
                        y = gloadf(SC[0] + o) * (v[0][r] - OFF * xs_t);
                        if constexpr (M == 2) {
                            const float u = gloadf(SC[1] + o) * (v[1][r] - OFF * xs_t);
                            y = silu_f(y) * u;
                        }
                    }
                    res[r] = y;
                }
                if (writer) {
                    float *op = a.out + (int64_t)(d.r0 + d.t0 + tok) * a.ldo;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (ob + r < Og) op[ob + r] = res[r];
                    if constexpr (M == 2) {
                        if (a.hf) {
                            uint16_t *hb = a.hf + (int64_t)gp * a.hf_stride + 2 * tok * 8;
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int o = ob + r;
                                if (o < a.hf_rows) {
                                    const uint16_t hv = bf16_rne(res[r]);
                                    const uint16_t lv = bf16_rne(res[r] - bf16_f(hv));
                                    int c, j;
                                    pos_any(a.hf_fmt, o, c, j);
                                    hb[(int64_t)c * kCols * 8 + j] = hv;
                                    hb[(int64_t)c * kCols * 8 + 8 + j] = lv;
                                    hpart[n] += bf16_f(hv) + bf16_f(lv);
                                }
                            }
                        }
                    }
                }
            }
        }
        if constexpr (M == 2) {
            if (a.hsum) {
                // sum over the 4 lane groups (rows), then over the 4 waves, per token
                __syncthreads();   // red[] of the previous item is consumed
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    float hp = hpart[n];
                    hp += __shfl_xor(hp, 16, kWave);
                    hp += __shfl_xor(hp, 32, kWave);
                    if (q == 0 && (col & 1) == 0) red[wave][8 * n + (col >> 1)] = hp;
                }
                __syncthreads();
                if (tid < d.nt)
                    a.hsum[(int64_t)tile * a.hsum_stride + (int64_t)gp * kTPP + tid] =
                        (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
            }
        }
    }
}

// Resident blocks of one kernel on the whole device (occupancy x CUs),
// queried once per kernel and device.
int resident_blocks(const void *kern, int *cache)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] > 0) return cache[dev];
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, 256, 0) != hipSuccess || per <= 0)
        per = 1;
    cache[dev] = cus * per;
    return cache[dev];
}

template <int FMT, int M>
hipError_t launch_fm(const MmArgs &a, int64_t items, hipStream_t st)
{
    static int cache[64] = {0};
    const void *kern = (const void *)k_mm<FMT, M>;
    int64_t cap = resident_blocks(kern, cache) / kXcds * kXcds;
    if (cap < kXcds) cap = kXcds;
    int64_t grid = (items + kXcds - 1) / kXcds * kXcds;
    if (grid > cap) grid = cap;
    if (grid < kXcds) grid = kXcds;
    hipLaunchKernelGGL((k_mm<FMT, M>), dim3((unsigned)grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const MmArgs &a, int M, int64_t items, hipStream_t st)
{
    return M == 2 ? launch_fm<FMT, 2>(a, items, st) : launch_fm<FMT, 1>(a, items, st);
}

}  // namespace

int mm_rows_per_block() { return kRowsPerBlock; }
int64_t mm_kpad(int64_t I) { return (I + 511) / 512 * 512; }

hipError_t xprep_launch(int fmt, const MmArgs &a, const float *x, int64_t ldx, int64_t max_group_passes,
                        hipStream_t st)
{
    if (max_group_passes <= 0) return hipSuccess;
    if (max_group_passes > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 g((unsigned)max_group_passes), b(256);
    switch (fmt) {
    case kI8: hipLaunchKernelGGL(k_xprep<kI8>, g, b, 0, st, a, x, ldx); break;
    case kI4: hipLaunchKernelGGL(k_xprep<kI4>, g, b, 0, st, a, x, ldx); break;
    case kI2: hipLaunchKernelGGL(k_xprep<kI2>, g, b, 0, st, a, x, ldx); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t mm_launch(MmArgs a, int fmt, int M, int64_t max_group_passes, hipStream_t st)
{
    const int Ocover = a.hf && a.hf_rows > a.O ? a.hf_rows : a.O;
    const int Omax = a.has_extra && a.xO > Ocover ? a.xO : Ocover;
    a.tiles = (Omax + kRowsPerBlock - 1) / kRowsPerBlock;
    const int64_t items = max_group_passes * a.tiles;
    switch (fmt) {
    case kI8: return launch_fmt<kI8>(a, M, items, st);
    case kI4: return launch_fmt<kI4>(a, M, items, st);
    case kI2: return launch_fmt<kI2>(a, M, items, st);
    default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------- work list
// One block: passes of kTPP rows per group (the extra group has x_rows rows),
// exclusive scan, then (g | pass << 11) entries in group order.
__global__ __launch_bounds__(1024) void k_build_work(const int32_t *__restrict__ offsets, int E,
                                                     int extra_rows, int32_t *__restrict__ work,
                                                     int32_t *__restrict__ n_work)
{
    __shared__ int32_t scan[1024];
    __shared__ int32_t carry;
    const int G = E + (extra_rows > 0 ? 1 : 0);
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < G; base += 1024) {
        const int g = base + threadIdx.x;
        int np = 0;
        if (g < G) {
            const int cnt = g < E ? offsets[g + 1] - offsets[g] : extra_rows;
            np = (cnt + kTPP - 1) / kTPP;
        }
        scan[threadIdx.x] = np;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int v = threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
            __syncthreads();
            scan[threadIdx.x] += v;
            __syncthreads();
        }
        const int start = carry + scan[threadIdx.x] - np;
        for (int p = 0; p < np; ++p) work[start + p] = g | (p << 11);
        __syncthreads();
        if (threadIdx.x == 1023) carry += scan[1023];
        __syncthreads();
    }
    if (threadIdx.x == 0) *n_work = carry;
}

hipError_t build_work_launch(const int32_t *offsets, int E, int extra_rows, int32_t *work,
                             int32_t *n_work, hipStream_t st)
{
    hipLaunchKernelGGL(k_build_work, dim3(1), dim3(1024), 0, st, offsets, E, extra_rows, work, n_work);
    return hipGetLastError();
}

}  // namespace coli
