// coli_pre.hip -- grouped expert products for prefill batches on the bf16
// matrix cores (activations rounded once to bf16, fp32 accumulation).
//
// The products of the pages' MoE block [glm.c@98759bf -- moe, phase D;
// glm.c@97c756a -- expert_gate_up, matmul_i4_pair; metal@93cde63 --
// moe_gemv, moe_silu], for batches where an expert meets tens to thousands
// of rows: per expert (group) and pass of up to 64 of its rows,
//   gate/up:  h = silu(sg * (Vg x)) * (su * (Vu x))
//   down:     y = sd * (Vd h)
// Weight codes are exact bf16 values v + OFF (coli_frag.h); OFF * sum(x),
// sum(x) being the sum of the stored bf16 activations of the row, is
// removed per output.
//
// An item is (group-pass, 256 weight rows for gate/up, 512 for down); a
// block of 8 waves takes it, each wave 32 (64) weight rows x the pass's live
// rows (up to 4 MFMA N-tiles of 16), so each weight byte read from memory
// meets up to 64 activation rows.  Per k-block the pass rows' activations
// are staged from their bf16 row tables into LDS (double-buffered, units
// XOR-swizzled by chunk so that the operand reads spread over the banks),
// while each wave has the next weights in flight (tiled weights: two
// k-blocks ahead).  The row-table rows of an item's pass rows and their
// activation sums are fetched one item ahead into LDS, so no wait on global
// memory ever drains the weight stream.
#include <hip/hip_ext.h>

#include "coli_device.h"
#include "coli_frag.h"
#include "coli_stages.h"
#include "coli_pre.h"

namespace coli {

namespace {

typedef __attribute__((address_space(3))) const void lds_void;

constexpr int kPreWaves = 8;
constexpr int kPreXcds = 8;
constexpr int kPreNT = kPreTpp / 16;   // N-tiles per pass
constexpr int kPreMT = 2;              // 16-row weight tiles per wave (gate/up)
constexpr int kPreMTDown = 4;          // the same for the single product (down)

// ---------------------------------------------------------------- row tables
template <int FMT>
__global__ __launch_bounds__(256) void k_xrows_bf16(const float *__restrict__ x, int64_t ldx, int I,
                                                    int kpad, uint16_t *__restrict__ table,
                                                    float *__restrict__ sums, int vec)
{
    constexpr int RUN = FMT == kI2 ? 16 : 8;
    __shared__ float red[4];
    const int row = blockIdx.x, tid = threadIdx.x;
    const float *xr = x + (int64_t)row * ldx;
    uint16_t *dst = table + (int64_t)row * kpad;
    const int nruns = kpad / RUN;
    float sum = 0.f;
    for (int r = tid; r < nruns; r += 256) {
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
        uint16_t hv[RUN];
#pragma unroll
        for (int i = 0; i < RUN; ++i) {
            hv[i] = bf16_rne(v[i]);
            sum += bf16_f(hv[i]);
        }
        int c, j;
        pos_of<FMT>(e0, c, j);
        uint32_t hw[RUN / 2];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            int k0, k1;
            if constexpr (FMT == kI8) { k0 = 2 * m; k1 = 2 * m + 1; }
            else if constexpr (FMT == kI4) { k0 = m; k1 = m + 4; }
            else { k0 = m; k1 = m + 8; }
            hw[m] = (uint32_t)hv[k0] | ((uint32_t)hv[k1] << 16);
            if constexpr (FMT == kI2) hw[4 + m] = (uint32_t)hv[m + 4] | ((uint32_t)hv[m + 12] << 16);
        }
#pragma unroll
        for (int h = 0; h < RUN / 8; ++h)
            *reinterpret_cast<uint4 *>(dst + (int64_t)(c + 4 * h) * 8) =
                make_uint4(hw[4 * h], hw[4 * h + 1], hw[4 * h + 2], hw[4 * h + 3]);
    }
    sum = wave_sum(sum);
    if ((tid & 63) == 0) red[tid >> 6] = sum;
    __syncthreads();
    if (tid == 0) sums[row] = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ void k_pre_rows(const int32_t *__restrict__ row_pair, int P, int K, int S, int n,
                           const float *__restrict__ token_sum, int32_t *__restrict__ act_row,
                           float *__restrict__ row_sum)
{
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= n) return;
    int t = r < P ? row_pair[r] / K : r - P;
    if (t < 0 || t >= S) t = 0;   // rows past the grouped slots (never read)
    act_row[r] = t;
    row_sum[r] = token_sum[t];
}

__global__ void k_pre_sum(const float *__restrict__ hpart, int nparts, int rows, float *__restrict__ row_sum)
{
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    const float *p = hpart + (int64_t)r * nparts;
    float s = 0.f;
    for (int i = 0; i < nparts; ++i) s += p[i];
    row_sum[r] = s;
}

// ---------------------------------------------------------------- products
// LDS DMA of 16 bytes per lane (lane L's bytes land at lds + 16 L), issued
// from inline assembly: the compiler does not see it, so it neither makes
// LDS reads wait for it nor counts it in its own waits -- the kernel orders
// and waits for these loads itself (s_nop: the wait state an LDS DMA needs
// after an SALU write of M0).
__device__ __forceinline__ void dma16(const void *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}

// SPG > 0: grouped-scale int4 (one scale per 32 SPG elements; SPG = 8
// stands for every group of 256 or more, a.gs_spg steps) on the grouped
// tiled layout, whose segments hold MFMA step s' of lane q as elements
// 32 s' + 8 q .. + 7, so each step covers 32 consecutive elements: the pass
// rows' units are staged from the row tables in that order, a group's
// products start from zero (groups of one or two steps: from -OFF times
// their column sums, made by the matrix cores) and at its last step are
// scaled by the group's scales (staged per k-block beside the activations)
// into a running total per output.
template <int FMT, int M, bool TILED, int SPG = 0>
__global__ __launch_bounds__(64 * kPreWaves) void k_pre(PreArgs a)
{
    using T = MF<FMT>;
    constexpr int STEPS = T::STEPS, KB = T::KB, SEGS = T::SEGS, BITS = T::BITS, SPS = T::SPS;
    constexpr bool GS = SPG > 0;
    static_assert(!GS || (TILED && FMT == kI4), "grouped scales: tiled int4");
    constexpr int MT = (M == 2 ? kPreMT : kPreMTDown) / (GS ? 2 : 1), NT = kPreNT, RPW = 16 * MT,
                  RPB = kPreWaves * RPW;
    static_assert(RPB == pre_rows_per_item(M, GS), "rows per item");
    // grouped scales: per wave and k-block its M x MT row tiles' scales of
    // the k-block's NGK groups, 16 rows each (64 bytes): one DMA per wave
    constexpr int NGK = GS ? (SPG < 8 ? 8 / SPG : 1) : 1;
    constexpr int SREG = M * MT * NGK * 64;
    static_assert(!GS || SREG <= 1024, "a wave's k-block scales in one DMA");
    __shared__ float4 ssA[GS ? kPreWaves * 64 : 1], ssB[GS ? kPreWaves * 64 : 1];
    constexpr float OFF = T::OFF;
    constexpr int CH = STEPS * 4;               // 16-byte chunks of a row per k-block
    constexpr int UNITS = CH * kPreTpp;         // units of one staged k-block
    constexpr uint32_t kbytes = KB * BITS / 8;
    __shared__ uint4 bsA[UNITS], bsB[UNITS];    // staged k-blocks (even, odd)
    __shared__ int lrow[2][kPreTpp];            // row-table rows of an item's pass rows
    __shared__ float lsum[2][kPreTpp];          // their activation sums

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, q = lane >> 4;
    const int xcd = blockIdx.x % kPreXcds, lb = blockIdx.x / kPreXcds;
    const int bpx = gridDim.x / kPreXcds;               // grid is a multiple of 8
    const int nkb = a.kpad / KB;                        // even and >= 4
    // a chunk past the end of a row shorter than 64 bytes is read at the
    // row's last chunk (it meets zero activations)
    const uint32_t coff = (uint32_t)min(16 * q, (int)(a.rb - 16));
    const uint32_t last_seg = (uint32_t)(a.rb - 16) - coff;
    // tiled layout: segments per row; a k-block past the row end reads the
    // last segment (it meets zero activations)
    const int ns = (int)((a.rb + 63) / 64);
    const uint8_t *actb = reinterpret_cast<const uint8_t *>(a.act);
    const uint32_t arow = (uint32_t)(2 * a.kpad);       // bytes per row-table row
    const int dq = (lane & 3) ^ ((lane >> 3) & 3);

    // The work list is sorted by the passes' live N-tiles (NL = 4, 3, 2, 1:
    // with skewed routing most groups are a few rows, and a pass multiplies
    // only its live tiles); the classes run one after the other, each with
    // its own code, so no N-tile branch sits in the product loop.
    auto run = [&](auto nlc, int w0, int w1) {
    constexpr int NL = decltype(nlc)::value;
    // XCD x: a contiguous run of the class's group-passes, pass-major: the
    // blocks of an XCD work on all weight tiles of a few consecutive passes
    // at a time, so a pass's activations are read from memory once for all
    // its tiles, and consecutive passes of a large group share each tile's
    // weights through the XCD's L2 (this measured less memory traffic and
    // time than tile-major order)
    const int n_gp = w1 - w0;
    const int gp_lo = w0 + (int)((int64_t)n_gp * xcd / kPreXcds);
    const int gp_cnt = w0 + (int)((int64_t)n_gp * (xcd + 1) / kPreXcds) - gp_lo;
    const int n_items = gp_cnt * a.tiles;
    if (lb >= n_items) return;                          // whole block, before any barrier

    struct It {
        int gp, tile, nt, r0t, Og;
        const uint8_t *wb[M];
        const float *sc[M];
        uint32_t roff[MT];   // rows: this lane's row (clamped) * rb + its chunk;
                             // tiled: its row tile's first unit + 16 lane
        uint32_t gstr;       // tiled: bytes from one segment's unit to the next
    };
    auto make = [&](It &c, int it) {
        c.gp = __builtin_amdgcn_readfirstlane(gp_lo + it / a.tiles);
        c.tile = __builtin_amdgcn_readfirstlane(it % a.tiles);
        const int wv = cload(a.work + c.gp);
        const int g = wv & 0x7FF, pass = wv >> 11;
        const bool extra = a.has_extra && g == a.ngroups;
        int r0, cnt;
        if (extra) {
            r0 = a.x_row0;
            cnt = a.x_rows;
        } else {
            r0 = cload(a.offsets + g);
            cnt = cload(a.offsets + g + 1) - r0;
        }
        c.nt = min(kPreTpp, cnt - pass * kPreTpp);
        c.r0t = r0 + pass * kPreTpp;
        if (extra) {
            c.Og = a.xO;
#pragma unroll
            for (int m = 0; m < M; ++m) { c.wb[m] = a.xw[m]; c.sc[m] = a.xs[m]; }
        } else {
            c.Og = a.O;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                c.wb[m] = a.w[m] + (int64_t)g * a.w_gstride;
                c.sc[m] = a.s[m] + (int64_t)g * a.s_gstride;
            }
        }
        const int obase = c.tile * RPB + wave * RPW;
        if constexpr (TILED) {
            // the wave's row tiles lie in one group of the layout (a row tile
            // past the matrix is clamped to the last one: never stored)
            const int mt16 = (c.Og + 15) / 16;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) c.roff[mt] = tiled_base(min(obase / 16 + mt, mt16 - 1), ns) + 16 * lane;
            c.gstr = tiled_gstride(min(obase / 16, mt16 - 1), mt16);
        } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                c.roff[mt] = (uint32_t)(min(obase + 16 * mt + col, c.Og - 1) * a.rb) + coff;
            c.gstr = 0;
        }
    };
    // pass rows of an item: row-table row and activation sum (threads < 64;
    // dead rows repeat the last live one)
    auto loadList = [&](const It &c, int &ar, float &rs) {
        const int gr = c.r0t + min(tid & 63, c.nt - 1);
        ar = a.act_row ? a.act_row[gr] : gr;
        rs = a.row_sum[gr];
    };
    auto storeList = [&](int par, int ar, float rs) {
        if (tid < kPreTpp) {
            lrow[par][tid] = ar;
            lsum[par][tid] = rs;
        }
    };
    auto loadW = [&](const It &c, int kbi, uint4 (&w)[M][MT][SEGS]) {
        if constexpr (TILED) {
#pragma unroll
            for (int sg = 0; sg < SEGS; ++sg) {
                const uint32_t go = (uint32_t)min(kbi * SEGS + sg, ns - 1) * c.gstr;
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) w[m][mt][sg] = gload16(c.wb[m] + (c.roff[mt] + go));
            }
            return;
        }
        const uint32_t b0 = (uint32_t)kbi * kbytes;
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int sg = 0; sg < SEGS; ++sg)
                    w[m][mt][sg] = gload16(c.wb[m] + (c.roff[mt] + min(b0 + 64 * sg, last_seg)));
    };
    // tiled: segment sg of k-block kbi of item c's weights into w[.][.][sg]
    auto loadSeg = [&](const It &c, int kbi, int sg, uint4 (&w)[M][MT][SEGS]) {
        const uint32_t go = (uint32_t)min(kbi * SEGS + sg, ns - 1) * c.gstr;
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) w[m][mt][sg] = gload16(c.wb[m] + (c.roff[mt] + go));
    };
    // Staging by LDS DMA (each lane's 16 bytes land at the instruction's LDS
    // base + 16 lane): staged unit (pass row t = 16 n + col, chunk c = 4 s +
    // q) sits at ((n STEPS + s) 16 + col) 4 + (q ^ ((col >> 1) & 3)), a
    // swizzle under which the operand reads (ds_read_b128) measured free of
    // bank conflicts on gfx950 (q ^ (col >> 2) cost 4 conflict cycles per
    // read).  One instruction fills one (n, s): lane L takes row 16 n + L / 4
    // and chunk 4 s + ((L & 3) ^ ((L >> 3) & 3)) -- 64 contiguous bytes of
    // each of 16 rows.  Instruction i = n STEPS + s of the NL x STEPS is
    // issued by wave i % 8.
    constexpr int NI = NL * STEPS, IPW = (NI + kPreWaves - 1) / kPreWaves;
    // this lane's byte offset, in the row tables, of its unit of instruction
    // j at k-block 0 for the pass rows of list par (an LDS read)
    auto stage_base = [&](int par, uint32_t (&rb)[IPW]) {
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
            const int i = min(wave + kPreWaves * j, NI - 1);
            const int n = i / STEPS, s = i % STEPS;
            // the unit of (step s, chunk dq): fragment-order unit 4 s + dq of
            // the k-block; on the grouped layout unit 4 dq + s' of segment s / 4
            const uint32_t u = GS ? (uint32_t)((s >> 2) * 256 + dq * 64 + (s & 3) * 16)
                                  : (uint32_t)(s * 64 + dq * 16);
            rb[j] = (uint32_t)lrow[par][16 * n + (lane >> 2)] * arow + u;
        }
    };
    auto stageB_r = [&](const uint32_t (&rb)[IPW], int kbi, const uint4 *buf) {
        const uint32_t lbuf = (uint32_t)(uintptr_t)(const lds_void *)buf;
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
            const int i = wave + kPreWaves * j;
            if (NI % kPreWaves == 0 || i < NI)          // uniform
                dma16(actb + (rb[j] + (uint32_t)kbi * (CH * 16)),
                      __builtin_amdgcn_readfirstlane(lbuf + (uint32_t)i * 1024));
        }
    };
    auto stageB = [&](int par, int kbi, const uint4 *buf) {
        uint32_t rb[IPW];
        stage_base(par, rb);
        stageB_r(rb, kbi, buf);
    };

    // Grouped scales of k-block kbi of item c into this wave's 1 KB of sbuf:
    // the scale tensors are packed [row tile][group][16 rows], so a row
    // tile's NGK groups of one k-block are 64 NGK contiguous bytes; byte b of
    // the region is row tile b / (64 NGK) (m major), its byte b % (64 NGK);
    // lanes past the region read its last 16 bytes again.
    const int ngp = GS ? a.gs_ngp : 0;
    auto stageS = [&](const It &c, int kbi, const float4 *sbuf) {
        if constexpr (GS) {
            const int g0 = kbi * 8 / a.gs_spg;
            const uint32_t lbase = (uint32_t)(uintptr_t)(const lds_void *)(sbuf + wave * 64);
            const int mt16 = (c.Og + 15) / 16;
            const int obt = (c.tile * RPB + wave * RPW) / 16;
            const int b = min(16 * lane, SREG - 16);
            const int ti = b / (64 * NGK), within = b - ti * (64 * NGK);
            const int m = ti / MT, mt = ti - m * MT;
            const int rt = min(obt + mt, mt16 - 1);
            // m varies across lanes: a select, not an index
            const float *sb = c.sc[0];
#pragma unroll
            for (int mm = 1; mm < M; ++mm) sb = m == mm ? c.sc[mm] : sb;
            dma16(sb + ((int64_t)rt * ngp + g0) * 16 + within / 4, __builtin_amdgcn_readfirstlane(lbase));
        }
    };

    floatx4 acc[M][MT][NL];
    // grouped scales: the group's column sums (times -OFF for groups of one
    // or two steps) and the scaled total of the finished groups
    floatx4 accs[GS ? NL : 1], tot[GS ? M : 1][GS ? MT : 1][GS ? NL : 1];
    const floatx4 zero4 = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int n = 0; n < NL; ++n) acc[m][mt][n] = zero4;
    if constexpr (GS) {
#pragma unroll
        for (int n = 0; n < NL; ++n) {
            accs[n] = zero4;
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) tot[m][mt][n] = zero4;
        }
    }
    constexpr bool CI = GS && SPG <= 2;
    constexpr uint32_t noff_bf = __builtin_bit_cast(uint32_t, -OFF) >> 16;
    static_assert(!CI || (__builtin_bit_cast(uint32_t, -OFF) & 0xFFFFu) == 0, "-OFF is a bf16 value");
    const uint32_t noff2 = opaque_v(CI ? noff_bf | noff_bf << 16 : 0x3F803F80u);   // bf16 -OFF pairs, else ones
    const uint4 cs_op = make_uint4(noff2, noff2, noff2, noff2);
    // after the last step of group gl of the k-block whose scales are in
    // sbuf: its products (less OFF times its column sums) times its scales
    // into tot
    auto flush = [&](const float4 *sbuf, int gl) {
        if constexpr (GS) {
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const float4 sv = sbuf[wave * 64 + ((m * MT + mt) * NGK + gl) * 4 + q];
#pragma unroll
                    for (int n = 0; n < NL; ++n) {
                        floatx4 v = acc[m][mt][n];
                        if constexpr (!CI) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) v[r] = fmaf(-OFF, accs[n][r], v[r]);
                        }
                        tot[m][mt][n][0] = fmaf(sv.x, v[0], tot[m][mt][n][0]);
                        tot[m][mt][n][1] = fmaf(sv.y, v[1], tot[m][mt][n][1]);
                        tot[m][mt][n][2] = fmaf(sv.z, v[2], tot[m][mt][n][2]);
                        tot[m][mt][n][3] = fmaf(sv.w, v[3], tot[m][mt][n][3]);
                    }
                }
        }
    };

    // one k-block: per MFMA step the live N-tiles' activation units from LDS
    // and the M x MT x NL products; the weights were loaded in the operand
    // layout (lane (q, col) holds row col, chunk q of each 64-byte segment)
    // (sg >= 0: only the steps of segment sg; grouped scales: sbuf holds the
    // scales of this k-block, ckb)
    auto compute = [&](const uint4 (&w)[M][MT][SEGS], const uint4 *buf, int sg = -1,
                       const float4 *sbuf = nullptr, int ckb = 0) {
#pragma unroll
        for (int s2 = 0; s2 < STEPS; ++s2) {
            if (sg >= 0 && s2 / SPS != sg) continue;
            uint4 b[NL];
#pragma unroll
            for (int n = 0; n < NL; ++n) b[n] = buf[((n * STEPS + s2) * 16 + col) * 4 + (q ^ ((col >> 1) & 3))];
            if constexpr (GS) {
                // a group of fewer than 8 steps starts at steps s2 % SPG == 0;
                // one of a k-block or more (SPG = 8) finds its sums zeroed by
                // the last group's flush
                const bool fresh = SPG < 8 && s2 % (SPG < 8 ? SPG : 1) == 0;
                if constexpr (CI) {
                    if (fresh) {   // the group's steps: this one and (SPG = 2) the next
#pragma unroll
                        for (int n = 0; n < NL; ++n) {
                            accs[n] = mfma(cs_op, b[n], zero4);
                            if constexpr (SPG == 2)
                                accs[n] = mfma(cs_op, buf[((n * STEPS + s2 + 1) * 16 + col) * 4 + (q ^ ((col >> 1) & 3))],
                                               accs[n]);
                        }
                    }
                }
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const uint4 cw = codes<FMT>(w[m][mt][s2 / SPS], s2 % SPS);
#pragma unroll
                        for (int n = 0; n < NL; ++n)
                            acc[m][mt][n] = mfma(cw, b[n], fresh ? (CI ? accs[n] : zero4) : acc[m][mt][n]);
                    }
                if constexpr (!CI) {
#pragma unroll
                    for (int n = 0; n < NL; ++n) accs[n] = mfma(cs_op, b[n], fresh ? zero4 : accs[n]);
                }
                if constexpr (SPG < 8) {
                    // a uniform branch the compiler cannot fold (a.gs_spg is
                    // SPG here) keeps each flush a scheduling region of its
                    // own; without it the scheduler runs later steps' work
                    // ahead of the flushes and spills (gs 32: 2.2 KB per lane)
                    if ((s2 + 1) % SPG == 0 && a.gs_spg == SPG) flush(sbuf, s2 / SPG);
                } else if (s2 == STEPS - 1 && (ckb == nkb - 1 || ((ckb + 1) * 8) % a.gs_spg == 0)) {
                    flush(sbuf, 0);   // uniform
#pragma unroll
                    for (int n = 0; n < NL; ++n) {
#pragma unroll
                        for (int m = 0; m < M; ++m)
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt) acc[m][mt][n] = zero4;
                        accs[n] = zero4;
                    }
                }
                continue;
            }
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const uint4 cw = codes<FMT>(w[m][mt][s2 / SPS], s2 % SPS);
#pragma unroll
                    for (int n = 0; n < NL; ++n) acc[m][mt][n] = mfma(cw, b[n], acc[m][mt][n]);
                }
        }
    };

    float sreg[M][MT][4];
    auto load_epi = [&](const It &c) {
        if constexpr (GS) return;   // grouped scales were applied group by group
        const int obase = c.tile * RPB + wave * RPW;
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sreg[m][mt][r] = gloadf(c.sc[m] + min(obase + 16 * mt + 4 * q + r, c.Og - 1));
    };
    // D[4q + r][col] of tile (m, mt, n): weight row obase + 16 mt + 4 q + r,
    // pass row 16 n + col; xsv[n]: that row's activation sum
    float xsv[NL];
    // Stores of the uniform fast path (the wave's rows inside the matrix and,
    // for gate/up, inside h's row table; 16-byte (bf16: 8-byte) result
    // stores): per N-tile one per row tile (gate/up: only with a result
    // array), and for gate/up one more per row tile (h's row table) and one
    // (its partial sums).  Every one is issued: each of the NL tiles has a
    // live row.
    constexpr int kStores = NL * (MT + (M == 2 ? MT + 1 : 0));
    constexpr int kStoresT = NL * (M == 2 ? MT + 1 : MT);   // gate/up without a result array
    const bool has_out = M == 1 || a.out != nullptr;
    // returns kStores (kStoresT) on the fast path, else 0
    auto epilogue = [&](const It &c) -> int {
        const int obase = c.tile * RPB + wave * RPW;
        const bool fast = (!has_out || a.out_vec4) && obase + RPW <= c.Og &&
                          (M == 1 || obase + RPW <= a.hf_kpad);
#pragma unroll
        for (int n = 0; n < NL; ++n) {
            const int t = 16 * n + col;
            const bool live = t < c.nt;
            const int64_t gr = c.r0t + t;
            float hp = 0.f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int ob = obase + 16 * mt + 4 * q;
                float res[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float y, u = 0.f;
                    if constexpr (GS) {
                        y = tot[0][mt][n][r];
                        if constexpr (M == 2) u = tot[GS ? 1 : 0][mt][n][r];
                    } else {
                        y = sreg[0][mt][r] * (acc[0][mt][n][r] - OFF * xsv[n]);
                        if constexpr (M == 2) u = sreg[1][mt][r] * (acc[1][mt][n][r] - OFF * xsv[n]);
                    }
                    if constexpr (M == 2) y = silu_f(y) * u;
                    res[r] = ob + r < c.Og ? y : 0.f;
                }
                if (live && has_out) {
                    if (M == 1 && a.out_bf16) {
                        uint16_t *op = reinterpret_cast<uint16_t *>(a.out) + gr * a.ldo;
                        uint32_t hb[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) hb[r] = bf16_rne(res[r]);
                        if (fast || (a.out_vec4 && ob + 3 < c.Og)) {
                            *reinterpret_cast<uint2 *>(op + ob) = make_uint2(hb[0] | hb[1] << 16, hb[2] | hb[3] << 16);
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (ob + r < c.Og) op[ob + r] = (uint16_t)hb[r];
                        }
                    } else {
                        float *op = a.out + gr * a.ldo;
                        if (fast || (a.out_vec4 && ob + 3 < c.Og)) {
                            *reinterpret_cast<float4 *>(op + ob) = make_float4(res[0], res[1], res[2], res[3]);
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (ob + r < c.Og) op[ob + r] = res[r];
                        }
                    }
                }
                if constexpr (M == 2) {
                    // h as the down product's bf16 row table: this lane's
                    // 4 outputs are half of one unit, the partner lane (q ^ 1,
                    // int2: q ^ 2) holds the other half, the lower lane stores
                    constexpr int PX = FMT == kI2 ? 32 : 16;
                    const bool lowq = FMT == kI2 ? q < 2 : (q & 1) == 0;
                    uint32_t hv[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        hv[r] = bf16_rne(res[r]);
                        if (ob + r < a.hf_kpad) hp += bf16_f((uint16_t)hv[r]);
                    }
                    uint32_t pv[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) pv[r] = (uint32_t)__shfl_xor((int)hv[r], PX, kWave);
                    if (lowq && live && (fast || ob < a.hf_kpad)) {
                        int cc, j;
                        pos_of<FMT>(ob, cc, j);
                        uint4 u;
                        if constexpr (FMT == kI8)
                            u = make_uint4(hv[0] | hv[1] << 16, hv[2] | hv[3] << 16,
                                           pv[0] | pv[1] << 16, pv[2] | pv[3] << 16);
                        else
                            u = make_uint4(hv[0] | pv[0] << 16, hv[1] | pv[1] << 16,
                                           hv[2] | pv[2] << 16, hv[3] | pv[3] << 16);
                        *reinterpret_cast<uint4 *>(a.hf + gr * a.hf_kpad + (int64_t)cc * 8) = u;
                    }
                }
            }
            if constexpr (M == 2) {
                // partial sum of the stored h of pass row t over this wave's
                // 32 weight rows (4 lane groups q), in a fixed order
                hp += __shfl_xor(hp, 16, kWave);
                hp += __shfl_xor(hp, 32, kWave);
                if (q == 0 && live) a.hpart[gr * a.nparts + c.tile * kPreWaves + wave] = hp;
            }
        }
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int n = 0; n < NL; ++n) {
                    acc[m][mt][n] = zero4;
                    if constexpr (GS) tot[m][mt][n] = zero4;
                }
        return fast ? (has_out ? kStores : kStoresT) : 0;
    };

    // the staged k-block is complete once this wave's DMA loads are: they
    // were issued before the NW weight loads of the next k-block
    constexpr int NW = M * MT * SEGS;
    // Half-step j (k-block j in LDS buffer rd, the next in wr):
    //   1. the next weights are requested (NW loads);
    //   2. wait until only those are in flight: this k-block's weights and
    //      this wave's DMA of its activations (issued before them) are done;
    //   3. barrier: every wave's DMA of k-block j is done, and every wave is
    //      past the products of k-block j-1, which read wr;
    //   4. the next k-block's activations are requested into wr (DMA);
    //   5. the products of k-block j.
    // The compiler's own wait for this k-block's weights is met by step 2.
    auto step_sync = [&]() {
        // vmcnt <= NW (bits 3:0 and 15:14), lgkmcnt = 0, expcnt not waited on
        __builtin_amdgcn_s_waitcnt((NW & 15) | ((NW >> 4) << 14) | (7 << 4));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    auto half = [&](const uint4 *rd, const uint4 *wr, int spar, int skb, const It &wsrc, int wkb,
                    uint4 (&wn)[M][MT][SEGS], const uint4 (&wc)[M][MT][SEGS]) {
        loadW(wsrc, wkb, wn);
        step_sync();
        stageB(spar, skb, wr);
        __builtin_amdgcn_sched_barrier(0);
        compute(wc, rd);
        __builtin_amdgcn_sched_barrier(0);
    };

    // prologue: the first item's pass rows; its first weights, then the DMA
    // of its first k-block's activations into bsA
    It cur;
    make(cur, lb);
    int par = 0;
    {
        int ar;
        float rs;
        loadList(cur, ar, rs);
        storeList(0, ar, rs);
    }
    __syncthreads();
    uint4 wA[M][MT][SEGS], wB[M][MT][SEGS];
    loadW(cur, 0, wA);
    stageB(0, 0, bsA);
    stageS(cur, 0, ssA);
    int jn = lb + bpx;

    if constexpr (TILED) {
        // Tiled weights: the loads of k-block j + 2 are issued into k-block
        // j's registers while j is multiplied, segment by segment as each is
        // consumed, so the wait at k-block j + 2 is for loads issued two
        // k-blocks earlier.  VMEM order per k-block j: wait, barrier, DMA of
        // j + 1, [the epilogue's scale loads], products of j with W(j + 2)
        // after each segment.  The wait before j needs W(j) and DMA(j): only
        // W(j + 1) (NW), plus what came after it -- the next item's pass-row
        // loads (2, or 1 without a row map) and the last epilogue's stores --
        // may stay in flight.
        // K-blocks past an item's end are the next item's first two (the
        // block's last item re-reads its own last k-block, from L2).
        loadW(cur, 1, wB);
        auto wait_vm = [&](auto nc) {
            constexpr int N = decltype(nc)::value;
            static_assert(N < 64, "vmcnt field");
            __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
        };
        // after is 0, or the pass-row loads (nlist: 2 with a row map, else
        // 1) plus 0, kStores or kStoresT
        const int nlist = a.act_row ? 2 : 1;
        auto sync_x = [&](int after) {
            asm volatile("" ::: "memory");
            if (after == 2 + kStores) wait_vm(std::integral_constant<int, NW + 2 + kStores>{});
            else if (after == 1 + kStores) wait_vm(std::integral_constant<int, NW + 1 + kStores>{});
            else if (after == 2 + kStoresT) wait_vm(std::integral_constant<int, NW + 2 + kStoresT>{});
            else if (after == 1 + kStoresT) wait_vm(std::integral_constant<int, NW + 1 + kStoresT>{});
            else if (after == 2) wait_vm(std::integral_constant<int, NW + 2>{});
            else if (after == 1) wait_vm(std::integral_constant<int, NW + 1>{});
            else wait_vm(std::integral_constant<int, NW>{});
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        // products of k-block kb from w and buf; DMA of (spar, skb) into
        // nbuf; W(lc, lkb) recycled into w
        // the current item's staging offsets, taken once per item (the
        // next item's first k-block is staged from its list directly)
        uint32_t rbc[IPW];
        // (grouped scales: k-block skb's scales, of item si, are staged with
        // its activations, into the scale buffer of the same parity)
        auto kstep = [&](uint4 (&w)[M][MT][SEGS], const uint4 *buf, int spar, int skb, const uint4 *nbuf,
                         const It &lc, int lkb, const It &si, bool epi = false, int after = 0) {
            sync_x(after);
            if (spar == par) stageB_r(rbc, skb, nbuf);
            else stageB(spar, skb, nbuf);
            const bool even = buf == bsA;
            stageS(si, skb, even ? ssB : ssA);
            if (epi) load_epi(cur);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int sg = 0; sg < SEGS; ++sg) {
                compute(w, buf, sg, even ? ssA : ssB, skb > 0 ? skb - 1 : nkb - 1);
                __builtin_amdgcn_sched_barrier(0);
                loadSeg(lc, lkb, sg, w);
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        int stores = 0;
        for (;;) {
            const bool has_nxt = jn < n_items;
            It nxt = cur;
            if (has_nxt) make(nxt, jn);
            int ar;
            float rs;
            loadList(nxt, ar, rs);
            stage_base(par, rbc);
            kstep(wA, bsA, par, 1, bsB, cur, 2, cur, false, nlist + stores);
            storeList(par ^ 1, ar, rs);
            kstep(wB, bsB, par, 2, bsA, cur, 3, cur);
            for (int k = 2; k < nkb - 2; k += 2) {
                kstep(wA, bsA, par, k + 1, bsB, cur, k + 2, cur);
                kstep(wB, bsB, par, k + 2, bsA, cur, k + 3, cur);
            }
            kstep(wA, bsA, par, nkb - 1, bsB, has_nxt ? nxt : cur, has_nxt ? 0 : nkb - 1, cur, true);
#pragma unroll
            for (int n = 0; n < NL; ++n) xsv[n] = lsum[par][min(16 * n + col, cur.nt - 1)];
            kstep(wB, bsB, par ^ 1, 0, bsA, has_nxt ? nxt : cur, has_nxt ? 1 : nkb - 1, nxt);
            stores = epilogue(cur);
            if (!has_nxt) break;
            cur = nxt;
            par ^= 1;
            jn += bpx;
        }
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }
    // Even k-blocks are staged in bsA, odd ones in bsB (nkb is even).
    for (;;) {
        const bool has_nxt = jn < n_items;
        It nxt = cur;
        if (has_nxt) make(nxt, jn);
        int ar;
        float rs;
        loadList(nxt, ar, rs);     // stored after the first k-block
        for (int k = 0; k < nkb - 2; k += 2) {
            half(bsA, bsB, par, k + 1, cur, k + 1, wB, wA);
            if (k == 0) storeList(par ^ 1, ar, rs);
            half(bsB, bsA, par, k + 2, cur, k + 2, wA, wB);
        }
        // last two k-blocks: the epilogue's scales and row sums, then the
        // next item's first k-block (a copy of this item's when there is none)
        load_epi(cur);
        half(bsA, bsB, par, nkb - 1, cur, nkb - 1, wB, wA);
#pragma unroll
        for (int n = 0; n < NL; ++n) xsv[n] = lsum[par][min(16 * n + col, cur.nt - 1)];
        half(bsB, bsA, par ^ 1, 0, nxt, 0, wA, wB);
        (void)epilogue(cur);
        if (!has_nxt) break;
        cur = nxt;
        par ^= 1;
        jn += bpx;
    }
    // every wave's DMA is complete before the class ends (the next class's
    // first DMA, after a barrier, may fill the same LDS)
    __builtin_amdgcn_s_waitcnt(0);
    };

    static_assert(NT == 4, "classes of 4, 3, 2 and 1 live N-tiles");
    const int e0 = cload(a.n_work + 1), e1 = cload(a.n_work + 2), e2 = cload(a.n_work + 3);
    const int e3 = cload(a.n_work + 4);
    run(std::integral_constant<int, 4>{}, 0, e0);
    __syncthreads();
    run(std::integral_constant<int, 3>{}, e0, e1);
    __syncthreads();
    run(std::integral_constant<int, 2>{}, e1, e2);
    __syncthreads();
    run(std::integral_constant<int, 1>{}, e2, e3);
}

int pre_resident_blocks(const void *kern, int *cache)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] > 0) return cache[dev];
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, 64 * kPreWaves, 0) != hipSuccess || per <= 0)
        per = 1;
    cache[dev] = cus * per;
    return cache[dev];
}

template <int FMT, int M, bool TILED, int SPG = 0>
hipError_t launch_pre(const PreArgs &a, int64_t items, hipStream_t st)
{
    static int cache[64] = {0};
    const void *kern = (const void *)k_pre<FMT, M, TILED, SPG>;
    int64_t cap = pre_resident_blocks(kern, cache) / kPreXcds * kPreXcds;
    if (cap < kPreXcds) cap = kPreXcds;
    int64_t grid = (items + kPreXcds - 1) / kPreXcds * kPreXcds;
    if (grid > cap) grid = cap;
    if (grid < kPreXcds) grid = kPreXcds;
    const KernelEvents ev = take_kernel_events();   // timed stage: events at the kernel's bounds
    if (ev.start)
        hipExtLaunchKernelGGL((k_pre<FMT, M, TILED, SPG>), dim3((unsigned)grid), dim3(64 * kPreWaves), 0, st,
                              ev.start, ev.stop, 0, a);
    else
        hipLaunchKernelGGL((k_pre<FMT, M, TILED, SPG>), dim3((unsigned)grid), dim3(64 * kPreWaves), 0, st, a);
    return hipGetLastError();
}

}  // namespace

int pre_parts(int hf_kpad, bool gs)
{
    return (hf_kpad + pre_rows_per_item(2, gs) - 1) / pre_rows_per_item(2, gs) * kPreWaves;
}

hipError_t xrows_bf16_launch(int fmt, const float *x, int64_t ldx, int rows, int I, int kpad,
                             uint16_t *table, float *sums, hipStream_t st)
{
    if (rows <= 0) return hipSuccess;
    const int vec = ldx % 4 == 0 && ((uintptr_t)x & 15u) == 0;
    switch (fmt) {
    case kI8: hipLaunchKernelGGL(k_xrows_bf16<kI8>, dim3(rows), dim3(256), 0, st, x, ldx, I, kpad, table, sums, vec); break;
    case kI4: hipLaunchKernelGGL(k_xrows_bf16<kI4>, dim3(rows), dim3(256), 0, st, x, ldx, I, kpad, table, sums, vec); break;
    case kI2: hipLaunchKernelGGL(k_xrows_bf16<kI2>, dim3(rows), dim3(256), 0, st, x, ldx, I, kpad, table, sums, vec); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t pre_rows_launch(const int32_t *row_pair, int P, int K, int S, int extra, const float *token_sum,
                           int32_t *act_row, float *row_sum, hipStream_t st)
{
    const int n = P + extra;
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_pre_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, row_pair, P, K, S, n,
                       token_sum, act_row, row_sum);
    return hipGetLastError();
}

hipError_t pre_sum_launch(const float *hpart, int nparts, int rows, float *row_sum, hipStream_t st)
{
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_pre_sum, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, hpart, nparts,
                       rows, row_sum);
    return hipGetLastError();
}

hipError_t pre_launch(PreArgs a, int fmt, int M, int64_t max_group_passes, hipStream_t st)
{
    int Ocover = a.O;
    if (M == 2 && a.hf && a.hf_kpad > Ocover) Ocover = a.hf_kpad;
    if (a.has_extra && a.xO > Ocover) Ocover = a.xO;
    const bool gs = a.gs_spg > 0;
    const int rpi = pre_rows_per_item(M, gs);
    a.tiles = (Ocover + rpi - 1) / rpi;
    if (M == 2 && a.nparts < a.tiles * kPreWaves) return hipErrorInvalidValue;
    const int64_t items = max_group_passes * a.tiles;
    if (gs) {   // grouped-scale int4, grouped tiled layout
        if (fmt != kI4 || !a.tiled) return hipErrorInvalidValue;
        const int spg = a.gs_spg;
#define COLI_PRE_GS(MM)                                                          \
        if (spg == 1) return launch_pre<kI4, MM, true, 1>(a, items, st);         \
        if (spg == 2) return launch_pre<kI4, MM, true, 2>(a, items, st);         \
        if (spg == 4) return launch_pre<kI4, MM, true, 4>(a, items, st);         \
        if (spg % 8 == 0) return launch_pre<kI4, MM, true, 8>(a, items, st);     \
        return hipErrorInvalidValue;
        if (M == 2) { COLI_PRE_GS(2) }
        COLI_PRE_GS(1)
#undef COLI_PRE_GS
    }
#define COLI_PRE_CASES(MM, TT)                                      \
    switch (fmt) {                                                 \
    case kI8: return launch_pre<kI8, MM, TT>(a, items, st);        \
    case kI4: return launch_pre<kI4, MM, TT>(a, items, st);        \
    case kI2: return launch_pre<kI2, MM, TT>(a, items, st);        \
    default: return hipErrorInvalidValue;                          \
    }
    if (M == 2) {
        if (a.tiled) COLI_PRE_CASES(2, true)
        COLI_PRE_CASES(2, false)
    }
    if (a.tiled) COLI_PRE_CASES(1, true)
    COLI_PRE_CASES(1, false)
#undef COLI_PRE_CASES
}

}  // namespace coli
