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
#include "coli_internal.h"
#include "coli_frag.h"
#include "coli_mfma.h"

namespace coli {

namespace {

constexpr int kWavesPerBlock = 4;
// Row tiles of 16 per wave: 2, except for the paired gate/up product with
// two-N-tile passes, where 1 keeps the register footprint of the others.
template <int M, int NT> struct RowTiles { static constexpr int MT = (M == 2 && NT == 2) ? 1 : 2; };
constexpr int kXcds = 8;

// ---------------------------------------------------------------- layout
// Work is cut into passes of activation rows ("tokens") of one group, of
// 16 NT columns (NT MFMA N-tiles of 16).  fp32 precision: NT = 1, up to 8
// tokens, token t in columns 2t (bf16 hi) and 2t+1 (bf16 lo).  bf16
// precision: NT = 2, up to 32 tokens, token t in column t (x rounded once).
// A pass's activations are stored "fragment-major": for k-block kbi, MFMA
// step s and lane group q, chunk c = (kbi*STEPS + s)*4 + q holds, for each
// column, the 8 bf16 values of the slots that lane (col, q) feeds to that
// step; the live columns are a prefix of every chunk, and a pass whose live
// columns fit one N-tile runs the products of that tile only.  A k-block's activations are one contiguous
// STEPS*2 KB run, and the live tokens' columns are a prefix of every chunk.
// Element e of the product's input sits in chunk c, slot j = pos_of(e).
static_assert(2 * COLI_MM_TPP_FP32 == 16 && COLI_MM_TPP_BF16 == 32, "pass widths: 1 and 2 N-tiles");
constexpr int nt_of(int bf16) { return bf16 ? 2 : 1; }

// Group-pass decode shared by the prep and the product kernels (gp uniform).
struct GP {
    int g, pass, r0, cnt, t0, nt;
    bool extra;
};
__device__ __forceinline__ GP decode_gp(const MmArgs &a, int gp)
{
    GP d;
    if (a.work) {
        const int wv = cload(a.work + gp);
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
        d.r0 = cload(a.offsets + d.g);
        d.cnt = cload(a.offsets + d.g + 1) - d.r0;
    } else {
        d.r0 = 0;
        d.cnt = a.x_rows;
    }
    d.t0 = d.pass * a.tpp;
    d.nt = min(a.tpp, d.cnt - d.t0);
    return d;
}

__device__ __forceinline__ int n_group_passes(const MmArgs &a)
{
    return a.work ? cload(a.n_work) : (a.x_rows + a.tpp - 1) / a.tpp;
}

// ---------------------------------------------------------------- x prep
// Block (group-pass, token): the block reads the token's activation row in
// coalesced runs of RUN consecutive elements (all of a thread's loads are
// issued before any is used), splits each value into bf16 hi/lo and stores
// the run as the 16-byte units of the chunk(s) it feeds.  A run of 8 (int8,
// int4) is exactly one chunk; a run of 16 (int2) is the two chunks of an
// even/odd step pair.  Only live columns are written: the product kernel
// reads nothing else.  Also the sum of the stored values (hi + lo, or hi
// alone in bf16 precision) per token, in a fixed order.
constexpr int kPrepThreads = 256;
constexpr int kPrepRuns = 4;   // runs per thread per round
template <int FMT, int NT>
__global__ __launch_bounds__(kPrepThreads) void k_xprep(MmArgs a, const float *__restrict__ x,
                                                        int64_t ldx, int vec)
{
    constexpr int RUN = FMT == kI2 ? 16 : 8;
    constexpr int kCols = 16 * NT;
    __shared__ float red[kPrepThreads / kWave];
    const int gp = blockIdx.x, t = blockIdx.y;
    if (gp >= n_group_passes(a)) return;
    const GP d = decode_gp(a, gp);
    if (t >= d.nt) return;   // uniform over the block
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tok = d.t0 + t;
    int row;
    if (!a.xrow_token) row = d.r0 + tok;
    else if (d.extra) row = tok;
    else row = a.row_pair[d.r0 + tok] / a.K;
    const float *xr = x + (int64_t)row * ldx;
    uint16_t *dst = a.xf + (int64_t)gp * a.xf_stride;
    const int nruns = a.kpad / RUN;
    float sum = 0.f;
    for (int r0 = 0; r0 < nruns; r0 += kPrepThreads * kPrepRuns) {
        float v[kPrepRuns][RUN];
#pragma unroll
        for (int k = 0; k < kPrepRuns; ++k) {
            const int e0 = (r0 + k * kPrepThreads + tid) * RUN;
            if (vec && e0 + RUN <= a.I) {
#pragma unroll
                for (int i = 0; i < RUN / 4; ++i) {
                    const float4 f = *reinterpret_cast<const float4 *>(xr + e0 + 4 * i);
                    v[k][4 * i] = f.x;
                    v[k][4 * i + 1] = f.y;
                    v[k][4 * i + 2] = f.z;
                    v[k][4 * i + 3] = f.w;
                }
            } else {
#pragma unroll
                for (int i = 0; i < RUN; ++i) v[k][i] = e0 + i < a.I ? xr[e0 + i] : 0.f;
            }
        }
#pragma unroll
        for (int k = 0; k < kPrepRuns; ++k) {
            const int r = r0 + k * kPrepThreads + tid;
            if (r >= nruns) break;
            uint16_t hv[RUN], lv[RUN];
#pragma unroll
            for (int i = 0; i < RUN; ++i) {
                hv[i] = bf16_rne(v[k][i]);
                lv[i] = bf16_rne(v[k][i] - bf16_f(hv[i]));
                sum += a.bf16 ? bf16_f(hv[i]) : bf16_f(hv[i]) + bf16_f(lv[i]);
            }
            // slot pairs (2m, 2m+1) of each chunk, as the unpacking orders them
            int c, j;
            pos_of<FMT>(r * RUN, c, j);
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
                uint16_t *u = dst + ((int64_t)(c + 4 * h) * kCols + (a.bf16 ? t : 2 * t)) * 8;
                *reinterpret_cast<uint4 *>(u) = make_uint4(hw[4 * h], hw[4 * h + 1], hw[4 * h + 2], hw[4 * h + 3]);
                if (!a.bf16)
                    *reinterpret_cast<uint4 *>(u + 8) = make_uint4(lw[4 * h], lw[4 * h + 1], lw[4 * h + 2], lw[4 * h + 3]);
            }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, kWave);
    if (lane == 0) red[wave] = sum;
    __syncthreads();
    if (tid == 0) {
        float tot = 0.f;
        for (int w = 0; w < kPrepThreads / kWave; ++w) tot += red[w];
        a.xsum[(int64_t)gp * kCols + t] = tot;
    }
}

// ---------------------------------------------------------------- main kernel
// One MFMA k-block step of a wave: weights (row-contiguous registers) moved
// into the operand layout in place with ds_bpermute -- lane (q, col) gets
// row col, chunk q, from lane 4 col + q -- then STEPS x M x 2 x NTL products
// against the activations staged in LDS (bs), for the first NTL N-tiles.
template <int FMT, int M, int MT, int NT, int NTL>
__device__ __forceinline__ void mm_step(uint4 (&wl)[M][MT][MF<FMT>::SEGS], const uint4 *bs,
                                        int src4, int q, int col, floatx4 (&acc)[M][MT][NT])
{
    using T = MF<FMT>;
    constexpr int SEGS = T::SEGS, SPS = T::SPS, STEPS = T::STEPS;
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int sg = 0; sg < SEGS; ++sg) {
                const uint4 v = wl[m][mt][sg];
                wl[m][mt][sg] = make_uint4((uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)v.x),
                                           (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)v.y),
                                           (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)v.z),
                                           (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)v.w));
            }
#pragma unroll
    for (int s2 = 0; s2 < STEPS; ++s2) {
        uint4 xb[NTL];
#pragma unroll
        for (int n = 0; n < NTL; ++n) xb[n] = bs[(s2 * 4 + q) * (16 * NT) + 16 * n + col];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint4 cw = codes<FMT>(wl[m][mt][s2 / SPS], s2 % SPS);
#pragma unroll
                for (int n = 0; n < NTL; ++n) acc[m][mt][n] = mfma(cw, xb[n], acc[m][mt][n]);
            }
    }
}

// Everything about one item -- (group-pass gp, 128-row tile) -- that its
// loads, its activation staging and its epilogue need.
template <int M, int MT, int UMAX>
struct Item {
    int gp, tile, nt, row0, Og;
    const uint8_t *wb[M];      // the group's matrices (uniform)
    uint32_t roff[MT];         // this lane's row (clamped) * rb + its 16-byte chunk, per row tile
    const float *sc[M];
    const uint4 *bglob;        // the group-pass's activation fragments (uniform)
    int boff[UMAX];            // this thread's activation units in a k-block (-1: dead)
};

// Persistent blocks walk the items of their XCD (block b of XCD x takes
// items b, b + blocks-per-XCD, ...; all tiles of one group-pass run on the
// same XCD, so its activations are fetched into one L2) as ONE pipeline of
// k-block steps that runs across item boundaries:
//   * weights are loaded two steps ahead into a ring of three register
//     buffers, activations three steps ahead into another ring of three
//     (the loop body is three steps, so every buffer has a fixed name); at
//     the end of each step the next step's activations go to a ring of
//     three LDS buffers;
//   * loads complete in issue order, so per step they are issued as: the
//     epilogue's scales and token sums (second-to-last step of an item),
//     the activations three steps ahead, the weights two steps ahead.  The
//     staging wait (activations issued two steps earlier) then never covers
//     the weights in flight, the products wait only for their own k-block,
//     and the epilogue never waits for the next item's k-blocks; two
//     k-blocks of weights per wave stay in flight all the time.
//   * kpad is a multiple of 1024, so an item has at least 4 k-blocks and
//     three steps ahead is at most the next item.
template <int FMT, int M, int NT>
__global__ __launch_bounds__(256) void k_mm(MmArgs a)
{
    using T = MF<FMT>;
    constexpr int STEPS = T::STEPS, KB = T::KB, SEGS = T::SEGS, BITS = T::BITS;
    constexpr int MT = RowTiles<M, NT>::MT;
    constexpr int kNT = NT, kCols = 16 * NT, kMaxTok = kCols;
    constexpr int kRowsPerWave = 16 * MT, kRowsPerBlock = kWavesPerBlock * kRowsPerWave;
    constexpr int CH = STEPS * 4;                 // activation chunks per k-block
    constexpr int UMAX = (CH * kCols + 255) / 256;
    constexpr float OFF = T::OFF;
    __shared__ float red[4][kMaxTok];
    __shared__ uint4 bsh[3][CH * kCols];
    __shared__ uint4 btrash[256];   // dead staging lanes write here: every load and store is unconditional

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, q = lane >> 4;
    const int lrow = lane >> 2, lchunk = lane & 3;
    const int src4 = 4 * (4 * col + q);
    const int xcd = blockIdx.x % kXcds, lb = blockIdx.x / kXcds;
    const int bpx = gridDim.x / kXcds;                 // blocks per XCD (grid is a multiple of 8)
    const int n_gp = n_group_passes(a);
    // XCD x takes the contiguous run of group-passes [gp_lo, gp_hi): the
    // passes of one group are adjacent, so they run on the same XCD at about
    // the same time and the later passes find the weights in its L2
    const int gp_lo = (int)((int64_t)n_gp * xcd / kXcds);
    const int gp_per_xcd = (int)((int64_t)n_gp * (xcd + 1) / kXcds) - gp_lo;
    const int n_items = gp_per_xcd * a.tiles;
    const int nkb = a.kpad / KB;                       // >= 4: kpad is a multiple of 1024
    if (lb >= n_items) return;                         // whole block, before any barrier
    const int64_t kbytes = (int64_t)KB * BITS / 8;
    // segments past the row end are clamped to its last segment (they meet
    // zero activations)
    const uint32_t last_seg = (uint32_t)(a.rb - 16 - 16 * lchunk);

    using It = Item<M, MT, UMAX>;
    auto make = [&](It &c, int it) {
        // uniform: the work-list and offset lookups below are scalar loads
        c.gp = __builtin_amdgcn_readfirstlane(gp_lo + it / a.tiles);
        c.tile = __builtin_amdgcn_readfirstlane(it % a.tiles);
        const GP d = decode_gp(a, c.gp);
        c.nt = d.nt;
        c.row0 = d.r0 + d.t0;
        const uint8_t *W[M];
        if (d.extra) {
            c.Og = a.xO;
#pragma unroll
            for (int m = 0; m < M; ++m) { W[m] = a.xw[m]; c.sc[m] = a.xs[m]; }
        } else {
            c.Og = a.O;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                W[m] = a.w[m] + (int64_t)d.g * a.w_gstride;
                c.sc[m] = a.s[m] + (int64_t)d.g * a.s_gstride;
            }
        }
        // lane L loads row L/4, chunk L%4 (a quarter-wave reads 4 rows x 64
        // contiguous bytes); rows past Og are clamped and never written
        const int obase = c.tile * kRowsPerBlock + wave * kRowsPerWave;
#pragma unroll
        for (int m = 0; m < M; ++m) c.wb[m] = W[m];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            c.roff[mt] = (uint32_t)(min(obase + 16 * mt + lrow, c.Og - 1) * a.rb) + 16 * lchunk;
        c.bglob = reinterpret_cast<const uint4 *>(a.xf + (int64_t)c.gp * a.xf_stride);
        // live activation units of a k-block: CH chunks x (2 nt or nt) columns
        const int lc = a.bf16 ? d.nt : 2 * d.nt, live = CH * lc;
#pragma unroll
        for (int i = 0; i < UMAX; ++i) {
            const int u = tid + 256 * i;
            const int ch = u / lc;
            c.boff[i] = u < live ? ch * kCols + (u - ch * lc) : -1;
        }
    };
    // weights: uniform matrix base + 32-bit lane offset (scalar-base loads);
    // past the row end (only when the row is shorter than kpad) each lane's
    // segment is clamped to the row's last one
    auto loadW = [&](const It &c, int kbi, uint4 (&w)[M][MT][SEGS]) {
        const uint32_t b0 = (uint32_t)kbi * (uint32_t)kbytes;
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int sg = 0; sg < SEGS; ++sg)
                    w[m][mt][sg] = gload16(c.wb[m] + (c.roff[mt] + min(b0 + 64 * sg, last_seg)));
    };
    // activations: dead units re-read unit 0 and are written to the trash
    // slot, so every load and store is unconditional
    auto loadB = [&](const It &c, int kbi, uint4 (&bv)[UMAX]) {
        const uint4 *src = c.bglob + (int64_t)kbi * CH * kCols;
#pragma unroll
        for (int i = 0; i < UMAX; ++i) bv[i] = gload16(src + (uint32_t)max(c.boff[i], 0));
    };
    auto stage = [&](const It &c, int buf, const uint4 (&bv)[UMAX]) {
#pragma unroll
        for (int i = 0; i < UMAX; ++i) {
            uint4 *dst = c.boff[i] >= 0 ? &bsh[buf][c.boff[i]] : &btrash[tid];
            *dst = bv[i];
        }
    };
    // epilogue inputs: the scales of the lane's 4 rows per (matrix, row tile)
    // and the sums of its tokens (clamped indexes, unconditional loads; rows
    // and tokens out of range are never written)
    // this lane's token in N-tile n: column 16 n + col (bf16) or half of it
    // (hi/lo pairs)
    auto ltok = [&](int n) { return a.bf16 ? 16 * n + col : 8 * n + (col >> 1); };
    float sreg[M][MT][4], xsr[kNT];
    auto load_epi = [&](const It &c) {
        const int obase = c.tile * kRowsPerBlock + wave * kRowsPerWave;
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sreg[m][mt][r] = gloadf(c.sc[m] + min(obase + 16 * mt + 4 * q + r, c.Og - 1));
#pragma unroll
        for (int n = 0; n < kNT; ++n)
            xsr[n] = gloadf(a.xsum + (int64_t)c.gp * kMaxTok + min(ltok(n), c.nt - 1));
    };

    floatx4 acc[M][MT][kNT];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int n = 0; n < kNT; ++n) acc[m][mt][n] = floatx4{0.f, 0.f, 0.f, 0.f};

    // ---- epilogue: D[4q + r][16 n + col]; in hi/lo precision the lo
    // column is added to the hi column
    auto epilogue = [&](const It &c) {
        const int obase = c.tile * kRowsPerBlock + wave * kRowsPerWave;
        const int ncols = a.bf16 ? c.nt : 2 * c.nt;
        float hpart[kNT] = {};   // this lane's stored h values per N-tile (M == 2)
#pragma unroll
        for (int n = 0; n < kNT; ++n) {
            if (16 * n >= ncols) break;                  // uniform: tile not live
            const int tok = ltok(n);
            const bool writer = tok < c.nt && (a.bf16 || (col & 1) == 0);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                float v[M][4];
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float other = __shfl_xor(acc[m][mt][n][r], 1, kWave);
                        v[m][r] = a.bf16 ? acc[m][mt][n][r] : acc[m][mt][n][r] + other;
                    }
                const int ob = obase + 16 * mt + 4 * q;
                float res[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float y = 0.f;
                    if (ob + r < c.Og) {
                        y = sreg[0][mt][r] * (v[0][r] - OFF * xsr[n]);
                        if constexpr (M == 2) {
                            const float u = sreg[1][mt][r] * (v[1][r] - OFF * xsr[n]);
                            y = silu_f(y) * u;
                        }
                    }
                    res[r] = y;
                }
                if (writer) {
                    float *op = a.out + (int64_t)(c.row0 + tok) * a.ldo;
                    if (a.out_vec4 && ob + 3 < c.Og) {
                        *reinterpret_cast<float4 *>(op + ob) = make_float4(res[0], res[1], res[2], res[3]);
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (ob + r < c.Og) op[ob + r] = res[r];
                    }
                }
                if constexpr (M == 2) {
                    if (a.hf) {
                        // h as the down product's activations: this lane's 4
                        // outputs are half of one 16-byte unit (8 slots of one
                        // chunk and column), the partner lane (q ^ 1, or q ^ 2
                        // for int2) holds the other half; the lower lane of
                        // the pair stores the whole unit.  Column 16 n + col:
                        // bf16 hi (even col) or lo (odd col) in fp32 precision.
                        constexpr int PX = FMT == kI2 ? 32 : 16;
                        const bool lowq = FMT == kI2 ? q < 2 : (q & 1) == 0;
                        const bool lo_col = !a.bf16 && (col & 1);
                        uint32_t hv[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const uint16_t h16 = bf16_rne(res[r]);
                            const uint16_t l16 = bf16_rne(res[r] - bf16_f(h16));
                            if (writer && ob + r < a.hf_rows)
                                hpart[n] += a.bf16 ? bf16_f(h16) : bf16_f(h16) + bf16_f(l16);
                            hv[r] = lo_col ? l16 : h16;
                        }
                        uint32_t pv[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) pv[r] = (uint32_t)__shfl_xor((int)hv[r], PX, kWave);
                        if (lowq && tok < c.nt && ob < a.hf_rows) {
                            int cc, j;
                            pos_of<FMT>(ob, cc, j);
                            uint4 u;
                            if constexpr (FMT == kI8)
                                u = make_uint4(hv[0] | hv[1] << 16, hv[2] | hv[3] << 16,
                                               pv[0] | pv[1] << 16, pv[2] | pv[3] << 16);
                            else
                                u = make_uint4(hv[0] | pv[0] << 16, hv[1] | pv[1] << 16,
                                               hv[2] | pv[2] << 16, hv[3] | pv[3] << 16);
                            *reinterpret_cast<uint4 *>(a.hf + (int64_t)c.gp * a.hf_stride +
                                                       ((int64_t)cc * kCols + 16 * n + col) * 8) = u;
                        }
                    }
                }
            }
        }
        if constexpr (M == 2) {
            if (a.hsum) {
                // sum over the 4 lane groups (rows), then over the 4 waves, per token
#pragma unroll
                for (int n = 0; n < kNT; ++n) {
                    float hp = hpart[n];
                    hp += __shfl_xor(hp, 16, kWave);
                    hp += __shfl_xor(hp, 32, kWave);
                    const int tok = ltok(n);
                    if (q == 0 && tok < c.nt && (a.bf16 || (col & 1) == 0)) red[wave][tok] = hp;
                }
                __syncthreads();
                if (tid < c.nt)
                    a.hsum[(int64_t)c.tile * a.hsum_stride + (int64_t)c.gp * kMaxTok + tid] =
                        (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
                __syncthreads();   // red[] is free again
            }
        }
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int n = 0; n < kNT; ++n) acc[m][mt][n] = floatx4{0.f, 0.f, 0.f, 0.f};
    };

    // nxt is the block's next item, or a copy of cur after the last one (its
    // loads then re-read valid data that nothing uses)
    It cur, nxt;
    make(cur, lb);
    int jn = lb + bpx;
    bool has_nxt = jn < n_items;
    if (has_nxt) make(nxt, jn);
    else nxt = cur;

    uint4 w0[M][MT][SEGS], w1[M][MT][SEGS], w2[M][MT][SEGS];
    uint4 breg[UMAX];
    int k = 0, buf = 0;
    // prologue: W(0), W(1), B(0) -> LDS
    loadW(cur, 0, w0);
    loadW(cur, 1, w1);
    loadB(cur, 0, breg);
    stage(cur, 0, breg);
    __syncthreads();

    // one k-block step s = (cur, k): returns true after the block's last item
    //   wc = W(s), wl <- W(s+2); B(s+1) loaded and staged to LDS
    auto step = [&](uint4 (&wc)[M][MT][SEGS], uint4 (&wl)[M][MT][SEGS]) -> bool {
        if (k == nkb - 2) load_epi(cur);
        // the sources are selected, not branched on: the same loads are
        // issued on every path, so the waits count them exactly
        It bsrc = cur;
        if (k + 1 >= nkb) bsrc = nxt;
        loadB(bsrc, k + 1 < nkb ? k + 1 : 0, breg);
        It src = cur;
        if (k + 2 >= nkb) src = nxt;
        loadW(src, k + 2 < nkb ? k + 2 : k + 2 - nkb, wl);
        __builtin_amdgcn_sched_barrier(0);
        if (NT == 2 && (a.bf16 ? cur.nt : 2 * cur.nt) > 16)
            mm_step<FMT, M, MT, NT, NT>(wc, bsh[buf], src4, q, col, acc);
        else
            mm_step<FMT, M, MT, NT, 1>(wc, bsh[buf], src4, q, col, acc);
        __builtin_amdgcn_sched_barrier(0);
        const int nb = buf == 2 ? 0 : buf + 1;
        // every wave finished reading buffer nb (two steps ago) before the
        // barrier at the end of the previous step
        stage(bsrc, nb, breg);
        __syncthreads();
        buf = nb;
        if (k != nkb - 1) {
            ++k;
            return false;
        }
        epilogue(cur);
        if (!has_nxt) return true;
        cur = nxt;
        k = 0;
        jn += bpx;
        has_nxt = jn < n_items;
        if (has_nxt) make(nxt, jn);
        else nxt = cur;
        return false;
    };
    for (;;) {
        if (step(w0, w2)) break;
        if (step(w1, w0)) break;
        if (step(w2, w1)) break;
    }
}

// xsum of the down product's passes: the gate/up epilogue leaves one partial
// sum per 128-row tile; add them in tile order (one thread per pass token).
__global__ void k_sum_parts(const float *__restrict__ parts, int nparts, int64_t stride, int n,
                            float *__restrict__ out)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float s = 0.f;
    for (int p = 0; p < nparts; ++p) s += parts[(int64_t)p * stride + i];
    out[i] = s;
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

template <int FMT, int M, int NT>
hipError_t launch_fm(const MmArgs &a, int64_t items, hipStream_t st)
{
    static int cache[64] = {0};
    const void *kern = (const void *)k_mm<FMT, M, NT>;
    int64_t cap = resident_blocks(kern, cache) / kXcds * kXcds;
    if (cap < kXcds) cap = kXcds;
    int64_t grid = (items + kXcds - 1) / kXcds * kXcds;
    if (grid > cap) grid = cap;
    if (grid < kXcds) grid = kXcds;
    hipLaunchKernelGGL((k_mm<FMT, M, NT>), dim3((unsigned)grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const MmArgs &a, int M, int64_t items, hipStream_t st)
{
    if (a.bf16) return M == 2 ? launch_fm<FMT, 2, 2>(a, items, st) : launch_fm<FMT, 1, 2>(a, items, st);
    return M == 2 ? launch_fm<FMT, 2, 1>(a, items, st) : launch_fm<FMT, 1, 1>(a, items, st);
}

}  // namespace

int mm_rows_per_block(int M, int bf16)
{
    const int mt = bf16 ? (M == 2 ? RowTiles<2, 2>::MT : RowTiles<1, 2>::MT)
                        : (M == 2 ? RowTiles<2, 1>::MT : RowTiles<1, 1>::MT);
    return kWavesPerBlock * 16 * mt;
}
int mm_pass_slots(int bf16) { return 16 * nt_of(bf16); }
int64_t mm_kpad(int64_t I) { return (I + 1023) / 1024 * 1024; }

hipError_t xprep_launch(int fmt, const MmArgs &a, const float *x, int64_t ldx, int64_t max_group_passes,
                        hipStream_t st)
{
    if (max_group_passes <= 0) return hipSuccess;
    if (max_group_passes > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 g((unsigned)max_group_passes, 16 * nt_of(a.bf16)), b(kPrepThreads);
    const int vec = ldx % 4 == 0 && ((uintptr_t)x & 15u) == 0;
    switch (fmt) {
    case kI8:
        if (a.bf16) hipLaunchKernelGGL((k_xprep<kI8, 2>), g, b, 0, st, a, x, ldx, vec);
        else hipLaunchKernelGGL((k_xprep<kI8, 1>), g, b, 0, st, a, x, ldx, vec);
        break;
    case kI4:
        if (a.bf16) hipLaunchKernelGGL((k_xprep<kI4, 2>), g, b, 0, st, a, x, ldx, vec);
        else hipLaunchKernelGGL((k_xprep<kI4, 1>), g, b, 0, st, a, x, ldx, vec);
        break;
    case kI2:
        if (a.bf16) hipLaunchKernelGGL((k_xprep<kI2, 2>), g, b, 0, st, a, x, ldx, vec);
        else hipLaunchKernelGGL((k_xprep<kI2, 1>), g, b, 0, st, a, x, ldx, vec);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t sum_parts_launch(const float *parts, int nparts, int64_t stride, int64_t n, float *out,
                           hipStream_t st)
{
    if (n <= 0) return hipSuccess;
    if (n > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_sum_parts, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, parts,
                       nparts, stride, (int)n, out);
    return hipGetLastError();
}

hipError_t mm_launch(MmArgs a, int fmt, int M, int64_t max_group_passes, hipStream_t st)
{
    const int Ocover = a.hf && a.hf_rows > a.O ? a.hf_rows : a.O;
    const int Omax = a.has_extra && a.xO > Ocover ? a.xO : Ocover;
    const int rpb = mm_rows_per_block(M, a.bf16);
    a.tiles = (Omax + rpb - 1) / rpb;
    const int64_t items = max_group_passes * a.tiles;
    switch (fmt) {
    case kI8: return launch_fmt<kI8>(a, M, items, st);
    case kI4: return launch_fmt<kI4>(a, M, items, st);
    case kI2: return launch_fmt<kI2>(a, M, items, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace coli
