// coli_dec.hip -- grouped expert products for decode batches on the bf16
// matrix cores, fp32-level accuracy.
//
// The products of the pages' MoE block [glm.c@98759bf -- moe, phase D;
// glm.c@97c756a -- expert_gate_up, matmul_i4_pair; metal@93cde63 --
// moe_gemv, moe_silu]: for every expert (group) and the rows routed to it,
//   gate/up:  h = silu(sg * (Vg x)) * (su * (Vu x))
//   down:     y = sd * (Vd h)
// with Vg, Vu, Vd the dequantised int8 / int4 / int2 weights.
//
// Layout of the work:
//   * a pass is up to 16 rows of one group, two MFMA N-tiles of 8 rows; row
//     t of a tile takes columns 2t (bf16 hi of its activations) and 2t+1
//     (bf16 lo), so the tile carries fp32-accurate activations (|x - hi -
//     lo| <= 2^-16 |x|); the second tile's products are skipped when the
//     pass has 8 rows or fewer;
//   * activations come from "row tables" (coli_dec.h): one row per
//     activation row, in fragment order.  Per k-block the waves of a block
//     copy the pass's units into LDS by DMA (each unit once per block), one
//     k-block ahead of the products, with one barrier per k-block;
//   * sum(x) per column, needed to remove OFF * sum(x) from the code
//     products, is one more MFMA per step against a tile of ones, over the
//     very bf16 values the products use;
//   * an item is (group-pass, 128-row tile) for gate/up (4 waves of 32
//     rows), (group-pass, 128-row tile) for down (2 waves of 64 rows); the items
//     are shared out to the XCDs so that the passes of one group run on the
//     same XCD at about the same time (later passes find the weights in its
//     L2), persistent blocks walk them in order, and each wave loads the
//     next k-block's weights while it multiplies the current one, and the
//     next item's first k-block during the current item's last.
#include <hip/hip_ext.h>

#include "coli_device.h"
#include "coli_frag.h"
#include "coli_stages.h"
#include "coli_dec.h"
#include "coli_xrows.h"

namespace coli {

namespace {

constexpr int kDecXcds = 8;
constexpr int kDecNT = kDecTpp / 8;   // MFMA N-tiles per pass (8 rows: hi/lo column pairs)
// per product: 16-row tiles per wave, waves per block (gate/up 4 x 32 rows,
// down 2 x 64 rows: measured fastest for each on the 64- and 16-token layers)
template <int M> struct DecTiles { static constexpr int MT = M == 2 ? 2 : 4, W = M == 2 ? 4 : 2; };

// ---------------------------------------------------------------- row tables
// Block (row, part): the row's runs (coli_xrows.h), 256 per part.
template <int FMT>
__global__ __launch_bounds__(256) void k_xrows(const float *__restrict__ x, int64_t ldx, int I,
                                               int kpad, uint16_t *__restrict__ table, int vec)
{
    const int row = blockIdx.x;
    const float *xr = x + (int64_t)row * ldx;
    uint16_t *dst = table + (int64_t)row * 2 * kpad;
    const int nruns = kpad / xrows_run_len<FMT>();
    for (int r = blockIdx.y * 256 + threadIdx.x; r < nruns; r += gridDim.y * 256) xrows_run<FMT>(xr, I, r, dst, vec);
}

// ---------------------------------------------------------------- products
// LDS DMA of 16 bytes per lane (lane L's bytes land at lds + 16 L), issued
// from inline assembly: the compiler does not see it, so it neither makes
// LDS reads wait for it nor counts it in its own waits -- the kernel orders
// and waits for these loads itself.  On this GPU family an LDS DMA that
// reads M0 right after an SALU write of M0 needs one wait state (the s_nop),
// which the compiler cannot insert inside the asm.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}

typedef __attribute__((address_space(3))) const void lds_void;

// SPG > 0: grouped-scale int4 (one scale per 32 SPG elements; SPG = 8
// stands for every group of 256 or more, a.gs_spg steps) on the grouped
// tiled layout, whose segments hold MFMA step s' of lane q as elements
// 32 s' + 8 q .. + 7, so that each step covers 32 consecutive elements.
template <int FMT, int M, bool TILED, int SPG = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(SPG > 0 ? 2 : 1))) void k_dec(DecArgs a)
{
    using T = MF<FMT>;
    constexpr int STEPS = T::STEPS, KB = T::KB, SEGS = T::SEGS, BITS = T::BITS, SPS = T::SPS;
    constexpr int MT = DecTiles<M>::MT, kDecWaves = DecTiles<M>::W, RPW = 16 * MT, RPB = kDecWaves * RPW;
    constexpr int NT = kDecNT;
    constexpr float OFF = T::OFF;
    constexpr uint32_t kChunkStep = 4 * 32;   // bytes between one step's chunks and the next's
    constexpr int UNITS = NT * STEPS * kWave; // 16-byte units of one staged k-block
    constexpr int IPW = NT * STEPS / kDecWaves;   // DMA instructions per wave and k-block
    static_assert(IPW >= 1 && STEPS % IPW == 0, "a wave stages steps of one N-tile");
    __shared__ uint4 bsA[UNITS], bsB[UNITS];   // staged k-blocks (even, odd)
    // grouped scales: per wave and k-block its M x MT row tiles' scales of
    // the k-block's NGK groups, 16 rows each (64 bytes), NSI KB a wave
    constexpr bool GS = SPG > 0;
    static_assert(!GS || (TILED && FMT == kI4), "grouped scales: tiled int4");
    constexpr int NGK = GS ? (SPG < 8 ? 8 / SPG : 1) : 1;
    constexpr int NSI = GS ? (M * MT * NGK * 64 + 1023) / 1024 : 0;
    __shared__ float4 ssA[GS ? kDecWaves * NSI * 64 : 1], ssB[GS ? kDecWaves * NSI * 64 : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, q = lane >> 4, lrow = lane >> 2, lchunk = lane & 3;
    const int src4 = 4 * (4 * col + q);
    const int xcd = blockIdx.x % kDecXcds, lb = blockIdx.x / kDecXcds;
    const int bpx = gridDim.x / kDecXcds;               // grid is a multiple of 8
    // Items of an XCD, in order (adjacent items: the passes of one group,
    // which then run there at about the same time and meet the weights in
    // its L2):
    //   gate/up (M = 2): all tiles of a contiguous run of group-passes;
    //   down (M = 1): tiles x, x + 8, ... of every group-pass, so each XCD
    //   streams the same share of every matrix.
    // (each measured faster for its kernel on the 64-token layer)
    const int n_gp = cload(a.n_work);
    constexpr bool RUNS = M == 2;
    const int gp_lo = RUNS ? (int)((int64_t)n_gp * xcd / kDecXcds) : 0;
    const int gp_cnt = RUNS ? (int)((int64_t)n_gp * (xcd + 1) / kDecXcds) - gp_lo : n_gp;
    const int tpx = RUNS ? a.tiles : (a.tiles - xcd + kDecXcds - 1) / kDecXcds;   // tiles per pass here
    const int n_items = gp_cnt * tpx;
    if (lb >= n_items) return;                          // whole block, before any barrier
    const int nkb = a.kpad / KB;                        // even and >= 4 (kpad: multiple of 1024)
    constexpr uint32_t kbytes = KB * BITS / 8;
    // a lane's 16-byte segment past the row end is clamped to the row's last
    // one (it meets zero activations)
    // (rows of fewer than 64 bytes: a chunk past the row end is read at the
    // row's last chunk; it too meets zero activations)
    const uint32_t coff = (uint32_t)min(16 * lchunk, (int)(a.rb - 16));
    const uint32_t last_seg = (uint32_t)(a.rb - 16) - coff;
    // tiled layout: segments per row; a k-block past the row end reads the
    // last segment (it meets zero activations)
    const int ns = (int)((a.rb + 63) / 64);
    const uint8_t *actb = reinterpret_cast<const uint8_t *>(a.act);
    const uint32_t arow = (uint32_t)(4 * a.kpad);       // bytes per row-table row
    // the N-tile and the first step this wave stages
    const int nw = wave * IPW / STEPS, s0 = wave * IPW % STEPS;

    struct It {
        int gp, tile, nt, r0t, Og;
        const uint8_t *wb[M];
        const float *sc[M];
        uint32_t roff[MT];   // rows: this lane's row (clamped) * rb + its 16-byte chunk;
                             // tiled: its row tile's first unit + 16 lane
        uint32_t gstr;       // tiled: bytes from one segment's unit to the next
        uint32_t doff;       // the unit this lane stages, in its activation row (bytes)
    };
    auto make = [&](It &c, int it) {
        c.gp = __builtin_amdgcn_readfirstlane(gp_lo + it / tpx);
        c.tile = __builtin_amdgcn_readfirstlane(RUNS ? it % tpx : xcd + kDecXcds * (it % tpx));
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
        c.nt = min(kDecTpp, cnt - pass * kDecTpp);
        c.r0t = r0 + pass * kDecTpp;
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
            // past the matrix is clamped to the last one: its results are
            // never stored)
            const int mt16 = (c.Og + 15) / 16;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) c.roff[mt] = tiled_base(min(obase / 16 + mt, mt16 - 1), ns) + 16 * lane;
            c.gstr = __builtin_amdgcn_readfirstlane(tiled_gstride(min(obase / 16, mt16 - 1), mt16));
        } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                c.roff[mt] = (uint32_t)(min(obase + 16 * mt + lrow, c.Og - 1) * a.rb) + coff;
            c.gstr = 0;
        }
        // activation row of the pass row whose unit this lane stages (pass
        // row 8 nw + col / 2), from scalar loads; dead rows repeat the last
        // live one (their results are never stored)
        const int t = 8 * nw + (col >> 1);
        int ar = 0;
#pragma unroll
        for (int u = 0; u < kDecTpp; ++u) {
            const int gr = c.r0t + min(u, c.nt - 1);
            int au;
            if (!a.act_by_token) au = gr;
            else if (extra) au = gr - a.x_row0;
            else au = cload(a.row_pair + gr) / a.K;
            ar = t == u ? au : ar;
        }
        // the unit of chunk q of step s' of a segment sits at byte 32 (4 s' +
        // q) of the segment's 512 bytes; on the grouped layout lane q of step
        // s' takes the unit at 32 (4 q + s')
        c.doff = (uint32_t)ar * arow + (GS ? 128 * q : 32 * q) + 16 * (col & 1);
    };
    // Tiled weights are loaded with the non-temporal hint: each unit is read
    // once per pass, and keeping that stream out of L2 leaves the activation
    // row tables, reused by every tile of a pass, resident there (64-token
    // layer: gate/up 322 -> 301 us).  Row-major weights keep plain loads:
    // there the two 64-byte halves of a 128-byte line come from two load
    // instructions, which then fetch the line twice (gate/up 337 -> 411 us).
    auto loadW = [&](const It &c, int kbi, uint4 (&w)[M][MT][SEGS]) {
        if constexpr (TILED) {
#pragma unroll
            for (int sg = 0; sg < SEGS; ++sg) {
                const uint32_t go = (uint32_t)min(kbi * SEGS + sg, ns - 1) * c.gstr;
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) w[m][mt][sg] = gload16_nt(c.wb[m] + (c.roff[mt] + go));
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
    // tiled layout: the loads of one k-block, by value (a pointer to an
    // item would keep it in memory and its uniform bases in vector registers)
    struct Ld {
        const uint8_t *wb[M];
        uint32_t roff[MT];
        uint32_t gstr;
        int kbi;
        bool on;
    };
    auto ld_of = [&](const It &c, int kbi) {
        Ld l;
#pragma unroll
        for (int m = 0; m < M; ++m) l.wb[m] = c.wb[m];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) l.roff[mt] = c.roff[mt];
        l.gstr = c.gstr;
        l.kbi = kbi;
        l.on = true;
        return l;
    };
    // segment sg of that k-block's weights into w[.][.][sg]
    auto loadSeg = [&](const Ld &l, int sg, uint4 (&w)[M][MT][SEGS]) {
        const uint32_t go = (uint32_t)min(l.kbi * SEGS + sg, ns - 1) * l.gstr;
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) w[m][mt][sg] = gload16_nt(l.wb[m] + (l.roff[mt] + go));
    };
    // Activations of k-block kbi into LDS by DMA: unit (n, step s, lane L)
    // at (n STEPS + s) 64 + L is the B operand of lane L for N-tile n (pass
    // rows 8n..8n+7) at step s.  Wave w issues IPW of the NT x STEPS
    // instructions -- N-tile nw, steps s0.. -- none for a dead N-tile.
    auto stageB = [&](const It &c, int kbi, const uint4 *buf) {
        if (8 * nw >= c.nt) return;                     // uniform
        const uint32_t lbase = (uint32_t)(uintptr_t)(const lds_void *)(buf + (nw * STEPS + s0) * kWave);
        if constexpr (GS) {
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const uint32_t st = (uint32_t)(kbi * STEPS + s0 + i);
                dma16(actb + (c.doff + 512u * (st >> 2) + 32u * (st & 3u)),
                      __builtin_amdgcn_readfirstlane(lbase + i * 1024));
            }
            return;
        }
        const uint32_t o = c.doff + (uint32_t)(kbi * STEPS + s0) * kChunkStep;
#pragma unroll
        for (int i = 0; i < IPW; ++i)
            dma16(actb + (o + (uint32_t)i * kChunkStep), __builtin_amdgcn_readfirstlane(lbase + i * 1024));
    };
    // Grouped scales of k-block kbi into this wave's region of sbuf: scale
    // tensors packed as [row tile][group][16 rows] (coli_pack_scales_grouped),
    // so a row tile's NGK groups of one k-block are 64 NGK contiguous bytes;
    // byte b of the region is row tile b / (64 NGK) (m major), its byte
    // b % (64 NGK); lanes past the region read its last 16 bytes again.
    const int ngp = GS ? a.gs_ngp : 0;
    auto stageS = [&](const It &c, int kbi, const float4 *sbuf) {
        if constexpr (GS) {
            const int g0 = kbi * 8 / a.gs_spg;
            const uint32_t lbase = (uint32_t)(uintptr_t)(const lds_void *)(sbuf + wave * NSI * 64);
            const int mt16 = (c.Og + 15) / 16;
            const int obt = (c.tile * RPB + wave * RPW) / 16;
#pragma unroll
            for (int k = 0; k < NSI; ++k) {
                const int b = min(1024 * k + 16 * lane, M * MT * NGK * 64 - 16);
                const int ti = b / (64 * NGK), within = b - ti * (64 * NGK);
                const int m = ti / MT, mt = ti - m * MT;
                const int rt = min(obt + mt, mt16 - 1);
                // m varies across lanes: a select, not an index (an indexed
                // per-lane read of c.sc would put the item in scratch memory)
                const float *sb = c.sc[0];
#pragma unroll
                for (int mm = 1; mm < M; ++mm) sb = m == mm ? c.sc[mm] : sb;
                const float *src = sb + ((int64_t)rt * ngp + g0) * 16 + within / 4;
                dma16(src, __builtin_amdgcn_readfirstlane(lbase + k * 1024));
            }
        }
    };

    floatx4 acc[M][MT][NT], accs[NT];
    // grouped scales: the scaled sum of the finished groups
    floatx4 tot[GS ? M : 1][GS ? MT : 1][GS ? NT : 1];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[m][mt][n] = floatx4{0.f, 0.f, 0.f, 0.f};
        accs[n] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (GS) {
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) tot[m][mt][n] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    const floatx4 zero4 = floatx4{0.f, 0.f, 0.f, 0.f};
    const uint32_t one2 = opaque_v(0x3F803F80u);       // bf16 (1, 1)
    const uint4 ones = make_uint4(one2, one2, one2, one2);
    // groups of one or two steps: the group's -OFF times its column sums is
    // made by the matrix cores (A = bf16 -OFF, exact) and is the C operand
    // the group's first product starts from, so a group's flush is one
    // multiply-add per output (the VALU work is what bounds these groups)
    constexpr bool CI = GS && SPG <= 2;
    constexpr uint32_t noff_bf = __builtin_bit_cast(uint32_t, -OFF) >> 16;
    static_assert(!CI || (__builtin_bit_cast(uint32_t, -OFF) & 0xFFFFu) == 0, "-OFF is a bf16 value");
    const uint32_t noff2 = opaque_v(noff_bf | noff_bf << 16);
    const uint4 noffs = make_uint4(noff2, noff2, noff2, noff2);

    // one k-block over the first NL N-tiles: weights moved into the operand
    // layout in place (lane (q, col) gets row col, chunk q, from lane 4 col
    // + q), then per MFMA step the M x MT code products and the column sums
    // GS: after the last step of each group its products, less OFF times its
    // column sums, are scaled by the group's scales (from sbuf, the k-block
    // ckb's) and added to tot; the next group starts from zero
    auto flush = [&](auto nl, const float4 *sbuf, int gl) {
        constexpr int NL = decltype(nl)::value;
        if constexpr (GS) {
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const float4 sv = sbuf[wave * NSI * 64 + ((m * MT + mt) * NGK + gl) * 4 + q];
#pragma unroll
                    for (int n = 0; n < NL; ++n) {
                        if constexpr (CI) {   // the products started from -OFF times the column sums
                            tot[m][mt][n][0] = fmaf(sv.x, acc[m][mt][n][0], tot[m][mt][n][0]);
                            tot[m][mt][n][1] = fmaf(sv.y, acc[m][mt][n][1], tot[m][mt][n][1]);
                            tot[m][mt][n][2] = fmaf(sv.z, acc[m][mt][n][2], tot[m][mt][n][2]);
                            tot[m][mt][n][3] = fmaf(sv.w, acc[m][mt][n][3], tot[m][mt][n][3]);
                        } else {
                            tot[m][mt][n][0] = fmaf(sv.x, fmaf(-OFF, accs[n][0], acc[m][mt][n][0]), tot[m][mt][n][0]);
                            tot[m][mt][n][1] = fmaf(sv.y, fmaf(-OFF, accs[n][1], acc[m][mt][n][1]), tot[m][mt][n][1]);
                            tot[m][mt][n][2] = fmaf(sv.z, fmaf(-OFF, accs[n][2], acc[m][mt][n][2]), tot[m][mt][n][2]);
                            tot[m][mt][n][3] = fmaf(sv.w, fmaf(-OFF, accs[n][3], acc[m][mt][n][3]), tot[m][mt][n][3]);
                        }
                    }
                }
        }
    };
    auto compute_n = [&](auto nl, uint4 (&w)[M][MT][SEGS], const uint4 *buf, int rkb,
                         const float4 *sbuf = nullptr, int ckb = 0) {
        constexpr int NL = decltype(nl)::value;
        if constexpr (!TILED) {   // the tiled layout arrives in the operand layout
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int sg = 0; sg < SEGS; ++sg) {
                        const uint4 v = w[m][mt][sg];
                        w[m][mt][sg] = make_uint4((uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)v.x),
                                                  (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)v.y),
                                                  (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)v.z),
                                                  (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)v.w));
                    }
        }
        if constexpr (TILED) {
            // One MFMA step at a time behind a scheduling barrier, each
            // weight word passed through an empty asm first (codes_late):
            // left free, the compiler computes every step's nibble shifts up
            // front (merging them from both N-tile branches into the block
            // before the branch) and needs ~90 more registers, half the
            // occupancy.  The next step's activation units are read before
            // the barrier.  Only the steps of segment rc_sg (< 0: all).
            const int sg = rkb;
            uint4 b[NL], bn[NL];
            const int s_lo = sg < 0 ? 0 : sg * SPS, s_hi = sg < 0 ? STEPS : s_lo + SPS;
#pragma unroll
            for (int n = 0; n < NL; ++n) b[n] = buf[(n * STEPS + s_lo) * kWave + lane];
#pragma unroll
            for (int s2 = 0; s2 < STEPS; ++s2) {
                if (s2 < s_lo || s2 >= s_hi) continue;
                if (s2 + 1 < s_hi) {
#pragma unroll
                    for (int n = 0; n < NL; ++n) bn[n] = buf[(n * STEPS + s2 + 1) * kWave + lane];
                }
                // grouped scales: a group of fewer than 8 steps starts from
                // zero at steps s2 % SPG == 0 (a group of a k-block or more,
                // SPG = 8, finds its sums zeroed by the last group's flush)
                const bool fresh = GS && SPG < 8 && s2 % (SPG < 8 ? SPG : 1) == 0;
                if constexpr (CI) {
                    if (fresh) {   // the group's steps: this one and (SPG = 2) the next
#pragma unroll
                        for (int n = 0; n < NL; ++n) {
                            accs[n] = mfma(noffs, b[n], zero4);
                            if constexpr (SPG == 2) accs[n] = mfma(noffs, bn[n], accs[n]);
                        }
                    }
                }
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const uint4 cw = codes_late<FMT>(w[m][mt][s2 / SPS], s2 % SPS);
#pragma unroll
                        for (int n = 0; n < NL; ++n)
                            acc[m][mt][n] = mfma(cw, b[n], fresh ? (CI ? accs[n] : zero4) : acc[m][mt][n]);
                    }
                if constexpr (!CI) {
#pragma unroll
                    for (int n = 0; n < NL; ++n) accs[n] = mfma(ones, b[n], fresh ? zero4 : accs[n]);
                }
                if constexpr (GS) {
                    if constexpr (SPG < 8) {
                        if ((s2 + 1) % SPG == 0) flush(nl, sbuf, s2 / SPG);
                    } else if (s2 == STEPS - 1 && (ckb == nkb - 1 || ((ckb + 1) * 8) % a.gs_spg == 0)) {
                        flush(nl, sbuf, 0);   // uniform
#pragma unroll
                        for (int n = 0; n < NL; ++n) {
#pragma unroll
                            for (int m = 0; m < M; ++m)
#pragma unroll
                                for (int mt = 0; mt < MT; ++mt) acc[m][mt][n] = zero4;
                            accs[n] = zero4;
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int n = 0; n < NL; ++n) b[n] = bn[n];
            }
            return;
        }
#pragma unroll
        for (int s2 = 0; s2 < STEPS; ++s2) {
            uint4 b[NL];
#pragma unroll
            for (int n = 0; n < NL; ++n) b[n] = buf[(n * STEPS + s2) * kWave + lane];
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const uint4 cw = codes<FMT>(w[m][mt][s2 / SPS], s2 % SPS);
#pragma unroll
                    for (int n = 0; n < NL; ++n) acc[m][mt][n] = mfma(cw, b[n], acc[m][mt][n]);
                }
#pragma unroll
            for (int n = 0; n < NL; ++n) accs[n] = mfma(ones, b[n], accs[n]);
        }
    };
    // the products of k-block buf (tiled: of segment sg only, sg < 0: all)
    // over the live N-tiles
    auto compute_s = [&](uint4 (&w)[M][MT][SEGS], const uint4 *buf, int ntl, int sg,
                         const float4 *sbuf = nullptr, int ckb = 0) {
        if constexpr (NT == 2) {
            if (ntl == 2) { compute_n(std::integral_constant<int, 2>{}, w, buf, sg, sbuf, ckb); return; }
        }
        compute_n(std::integral_constant<int, 1>{}, w, buf, sg, sbuf, ckb);
    };
    auto compute = [&](uint4 (&w)[M][MT][SEGS], const uint4 *buf, int ntl) { compute_s(w, buf, ntl, -1); };
    // Tiled: segment by segment, and as soon as a segment's products are
    // done that segment of rc's k-block is requested into the same
    // registers.  The loads sit after the N-tile branch has joined: a
    // register with a load in flight that the branches had placed apart
    // would be copied at the join, and the copy waits for every load.
    auto compute_r = [&](uint4 (&w)[M][MT][SEGS], const uint4 *buf, int ntl, Ld rc,
                         const float4 *sbuf = nullptr, int ckb = 0) {
#pragma unroll
        for (int sg = 0; sg < SEGS; ++sg) {
            compute_s(w, buf, ntl, sg, sbuf, ckb);
            __builtin_amdgcn_sched_barrier(0);
            if (rc.on) loadSeg(rc, sg, w);
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
    // D[4q + r][col] of tile (m, mt, n); the lo column is added to the hi one.
    // Returns the number of store instructions issued when that number is
    // known (the uniform fast path: the wave's rows inside the matrix -- and
    // for gate/up inside the down product's row table -- and 16-byte stores:
    // one per live N-tile and row tile, and one more for the row table), else
    // 0.  The tiled loop's next wait lets exactly that many stores stay in
    // flight.
    auto epilogue = [&](const It &c) -> int {
        const int obase = c.tile * RPB + wave * RPW;
        const int ntl = (c.nt + 7) / 8;
        const bool fast = a.out_vec4 && obase + RPW <= c.Og;
        const bool hfast = M == 2 && a.hf && obase + RPW <= a.hf_kpad;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            if (n >= ntl) break;                        // uniform
            const int tok = 8 * n + (col >> 1);
            const bool live = tok < c.nt;
            const float xs = accs[n][0] + __shfl_xor(accs[n][0], 1, kWave);   // sum of hi + lo over k
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                float v[M][4];
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if constexpr (GS)
                            v[m][r] = tot[m][mt][n][r] + __shfl_xor(tot[m][mt][n][r], 1, kWave);
                        else
                            v[m][r] = acc[m][mt][n][r] + __shfl_xor(acc[m][mt][n][r], 1, kWave);
                    }
                const int ob = obase + 16 * mt + 4 * q;
                float res[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float y, u;
                    if constexpr (GS) {
                        y = v[0][r];
                        u = M == 2 ? v[M - 1][r] : 0.f;
                    } else {
                        y = sreg[0][mt][r] * (v[0][r] - OFF * xs);
                        u = M == 2 ? sreg[M - 1][mt][r] * (v[M - 1][r] - OFF * xs) : 0.f;
                    }
                    if constexpr (M == 2) y = silu_f(y) * u;
                    res[r] = ob + r < c.Og ? y : 0.f;
                }
                float *op = a.out + (int64_t)(c.r0t + tok) * a.ldo;
                if (fast) {   // uniform
                    if (live && (col & 1) == 0)
                        *reinterpret_cast<float4 *>(op + ob) = make_float4(res[0], res[1], res[2], res[3]);
                } else if (live && (col & 1) == 0) {
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
                        // h as the down product's row table: this lane's 4
                        // outputs are half of one unit (8 slots of a chunk),
                        // the partner lane (q ^ 1, int2: q ^ 2) holds the
                        // other half, and the lower lane of the pair stores
                        // the unit; even columns store hi units, odd columns
                        // lo units
                        constexpr int PX = FMT == kI2 ? 32 : 16;
                        const bool lowq = FMT == kI2 ? q < 2 : (q & 1) == 0;
                        uint32_t hv[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const uint16_t h16 = bf16_rne(res[r]);
                            hv[r] = (col & 1) ? bf16_rne(res[r] - bf16_f(h16)) : h16;
                        }
                        uint32_t pv[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) pv[r] = (uint32_t)__shfl_xor((int)hv[r], PX, kWave);
                        if (lowq && live && (hfast || ob < a.hf_kpad)) {
                            int cc, j;
                            pos_of<FMT>(ob, cc, j);
                            uint4 u;
                            if constexpr (FMT == kI8)
                                u = make_uint4(hv[0] | hv[1] << 16, hv[2] | hv[3] << 16,
                                               pv[0] | pv[1] << 16, pv[2] | pv[3] << 16);
                            else
                                u = make_uint4(hv[0] | pv[0] << 16, hv[1] | pv[1] << 16,
                                               hv[2] | pv[2] << 16, hv[3] | pv[3] << 16);
                            *reinterpret_cast<uint4 *>(a.hf + (int64_t)(c.r0t + tok) * 2 * a.hf_kpad +
                                                       (int64_t)(2 * cc + (col & 1)) * 8) = u;
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    acc[m][mt][n] = floatx4{0.f, 0.f, 0.f, 0.f};
                    if constexpr (GS) tot[m][mt][n] = floatx4{0.f, 0.f, 0.f, 0.f};
                }
            accs[n] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
        if (!fast || (M == 2 && a.hf && !hfast)) return 0;
        return ntl * MT * (M == 2 && a.hf ? 2 : 1);
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
    // the same with `extra` more VMEM operations (stores) issued after the
    // next k-block's weights: 0, or an epilogue's known store count
    auto step_sync_x = [&](int extra) {
        constexpr int L = 7 << 4;
        switch (extra) {   // uniform; an unexpected count waits for everything but NW
        case 4: __builtin_amdgcn_s_waitcnt(((NW + 4) & 15) | (((NW + 4) >> 4) << 14) | L); break;
        case 8: __builtin_amdgcn_s_waitcnt(((NW + 8) & 15) | (((NW + 8) >> 4) << 14) | L); break;
        case 16: __builtin_amdgcn_s_waitcnt(((NW + 16) & 15) | (((NW + 16) >> 4) << 14) | L); break;
        default: __builtin_amdgcn_s_waitcnt((NW & 15) | ((NW >> 4) << 14) | L); break;
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    auto half = [&](const uint4 *rd, const uint4 *wr, const It &snext, int skb, const It &wsrc, int wkb,
                    uint4 (&wn)[M][MT][SEGS], uint4 (&wc)[M][MT][SEGS], int ntl) {
        loadW(wsrc, wkb, wn);
        step_sync();
        stageB(snext, skb, wr);
        __builtin_amdgcn_sched_barrier(0);
        compute(wc, rd, ntl);
        __builtin_amdgcn_sched_barrier(0);
    };

    if constexpr (TILED) {
        // Tiled weights: the loads of k-block j + 2 are issued into k-block
        // j's registers while j is multiplied (segment by segment, as each
        // is consumed), so the wait at k-block j + 2 is for loads issued two
        // k-blocks earlier -- the latency tolerance of three weight buffers
        // in the registers of two.  VMEM order: ... DMA(j), [compute j - 1:
        // W(j + 1)], wait (vmcnt <= NW: W(j) and DMA(j) done), DMA(j + 1),
        // [compute j: W(j + 2)], ...; k-blocks past an item's end are the
        // next item's first two (the block's last item re-reads its own last
        // k-block, from L2).  The epilogue's scale loads are issued after a
        // wait, so they never hold back the weight loads.
        It cur;
        make(cur, lb);
        int jn = lb + bpx;
        uint4 wA[M][MT][SEGS], wB[M][MT][SEGS];
        loadW(cur, 0, wA);
        stageB(cur, 0, bsA);
        stageS(cur, 0, ssA);
        loadW(cur, 1, wB);
        // one k-block: its products from weights w and activations buf
        // (k-block kb in LDS), the next k-block's activations (and grouped
        // scales) staged into nbuf, and the loads of l recycled into w; the
        // scale DMA is issued with the activation DMA, before the weights
        auto kstep = [&](int ntl, uint4 (&w)[M][MT][SEGS], const uint4 *buf, const It &sc, int skb,
                         const uint4 *nbuf, const Ld &l, bool epi = false, int extra = 0) {
            step_sync_x(extra);
            stageB(sc, skb, nbuf);
            const bool even = buf == bsA;
            stageS(sc, skb, even ? ssB : ssA);
            if (epi) load_epi(cur);   // after the wait: it does not hold back the weights
            __builtin_amdgcn_sched_barrier(0);
            compute_r(w, buf, ntl, l, even ? ssA : ssB, skb > 0 ? skb - 1 : nkb - 1);
            __builtin_amdgcn_sched_barrier(0);
        };
        // extra: the stores the previous item's epilogue left in flight
        auto kloop = [&](int nl, int extra) {
            kstep(nl, wA, bsA, cur, 1, bsB, ld_of(cur, 2), false, extra);
            kstep(nl, wB, bsB, cur, 2, bsA, ld_of(cur, 3));
            for (int k = 2; k < nkb - 2; k += 2) {
                kstep(nl, wA, bsA, cur, k + 1, bsB, ld_of(cur, k + 2));
                kstep(nl, wB, bsB, cur, k + 2, bsA, ld_of(cur, k + 3));
            }
            // the last two: the epilogue's scales, then the next item's
            // first two k-blocks (the block's last item re-reads its own
            // last k-block, from L2) and its first activations
            const bool has_nxt = jn < n_items;
            It nxt = cur;
            if (has_nxt) make(nxt, jn);
            kstep(nl, wA, bsA, cur, nkb - 1, bsB, has_nxt ? ld_of(nxt, 0) : ld_of(cur, nkb - 1), true);
            kstep(nl, wB, bsB, nxt, 0, bsA, has_nxt ? ld_of(nxt, 1) : ld_of(cur, nkb - 1));
            return nxt;
        };
        int extra = 0;
        for (;;) {
            It nxt = kloop((cur.nt + 7) / 8, extra);
            extra = epilogue(cur);
            if (jn >= n_items) break;
            cur = nxt;
            jn += bpx;
        }
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }

    // prologue: the first item's first weights, then the DMA of its first
    // k-block's activations into bsA.  Even k-blocks are staged in bsA, odd
    // ones in bsB (nkb is even).
    It cur;
    make(cur, lb);
    uint4 wA[M][MT][SEGS], wB[M][MT][SEGS];
    loadW(cur, 0, wA);
    stageB(cur, 0, bsA);
    int jn = lb + bpx;
    for (;;) {
        const int ntl = (cur.nt + 7) / 8;            // live N-tiles
        for (int k = 0; k < nkb - 2; k += 2) {
            half(bsA, bsB, cur, k + 1, cur, k + 1, wB, wA, ntl);
            half(bsB, bsA, cur, k + 2, cur, k + 2, wA, wB, ntl);
        }
        // last two k-blocks: the epilogue's scales, then the next item's
        // first k-block (a copy of this item's when there is none)
        const bool has_nxt = jn < n_items;
        It nxt = cur;
        if (has_nxt) make(nxt, jn);
        load_epi(cur);
        half(bsA, bsB, cur, nkb - 1, cur, nkb - 1, wB, wA, ntl);
        half(bsB, bsA, nxt, 0, nxt, 0, wA, wB, ntl);
        epilogue(cur);
        if (!has_nxt) break;
        cur = nxt;
        jn += bpx;
    }
    // every wave's DMA is complete before the block ends
    __builtin_amdgcn_s_waitcnt(0);
}

int dec_resident_blocks(const void *kern, int threads, int *cache)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] > 0) return cache[dev];
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, threads, 0) != hipSuccess || per <= 0)
        per = 1;
    cache[dev] = cus * per;
    return cache[dev];
}

template <int FMT, int M, bool TILED, int SPG = 0>
hipError_t launch_dec(const DecArgs &a, int64_t items, hipStream_t st)
{
    static int cache[64] = {0};
    const void *kern = (const void *)k_dec<FMT, M, TILED, SPG>;
    constexpr int threads = 64 * DecTiles<M>::W;
    int64_t cap = dec_resident_blocks(kern, threads, cache) / kDecXcds * kDecXcds;
    if (cap < kDecXcds) cap = kDecXcds;
    int64_t grid = (items + kDecXcds - 1) / kDecXcds * kDecXcds;
    if (grid > cap) grid = cap;
    if (grid < kDecXcds) grid = kDecXcds;
    const KernelEvents ev = take_kernel_events();   // timed stage: events at the kernel's bounds
    if (ev.start)
        hipExtLaunchKernelGGL((k_dec<FMT, M, TILED, SPG>), dim3((unsigned)grid), dim3(threads), 0, st,
                              ev.start, ev.stop, 0, a);
    else
        hipLaunchKernelGGL((k_dec<FMT, M, TILED, SPG>), dim3((unsigned)grid), dim3(threads), 0, st, a);
    return hipGetLastError();
}

}  // namespace

int dec_rows_per_block(int M)
{
    return M == 2 ? DecTiles<2>::W * 16 * DecTiles<2>::MT : DecTiles<1>::W * 16 * DecTiles<1>::MT;
}

hipError_t xrows_launch(int fmt, const float *x, int64_t ldx, int rows, int I, int kpad,
                        uint16_t *table, hipStream_t st)
{
    if (rows <= 0) return hipSuccess;
    const int run = fmt == kI2 ? 16 : 8;
    const int parts = (kpad / run + 255) / 256;
    const dim3 g((unsigned)rows, (unsigned)parts);
    const int vec = ldx % 4 == 0 && ((uintptr_t)x & 15u) == 0;
    switch (fmt) {
    case kI8: hipLaunchKernelGGL(k_xrows<kI8>, g, dim3(256), 0, st, x, ldx, I, kpad, table, vec); break;
    case kI4: hipLaunchKernelGGL(k_xrows<kI4>, g, dim3(256), 0, st, x, ldx, I, kpad, table, vec); break;
    case kI2: hipLaunchKernelGGL(k_xrows<kI2>, g, dim3(256), 0, st, x, ldx, I, kpad, table, vec); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t dec_launch(DecArgs a, int fmt, int M, int64_t max_group_passes, hipStream_t st)
{
    int Ocover = a.O;
    if (M == 2 && a.hf && a.hf_kpad > Ocover) Ocover = a.hf_kpad;
    if (a.has_extra && a.xO > Ocover) Ocover = a.xO;
    const int rpb = dec_rows_per_block(M);
    a.tiles = (Ocover + rpb - 1) / rpb;
    const int64_t items = max_group_passes * a.tiles;
    if (a.gs_spg > 0) {   // grouped-scale int4, grouped tiled layout
        if (fmt != kI4 || !a.tiled) return hipErrorInvalidValue;
        const int spg = a.gs_spg;
#define COLI_DEC_GS(MM)                                                          \
        if (spg == 1) return launch_dec<kI4, MM, true, 1>(a, items, st);         \
        if (spg == 2) return launch_dec<kI4, MM, true, 2>(a, items, st);         \
        if (spg == 4) return launch_dec<kI4, MM, true, 4>(a, items, st);         \
        if (spg % 8 == 0) return launch_dec<kI4, MM, true, 8>(a, items, st);     \
        return hipErrorInvalidValue;
        if (M == 2) { COLI_DEC_GS(2) }
        COLI_DEC_GS(1)
#undef COLI_DEC_GS
    }
#define COLI_DEC_CASES(MM, TT)                                      \
    switch (fmt) {                                                 \
    case kI8: return launch_dec<kI8, MM, TT>(a, items, st);        \
    case kI4: return launch_dec<kI4, MM, TT>(a, items, st);        \
    case kI2: return launch_dec<kI2, MM, TT>(a, items, st);        \
    default: return hipErrorInvalidValue;                          \
    }
    if (M == 2) {
        if (a.tiled) COLI_DEC_CASES(2, true)
        COLI_DEC_CASES(2, false)
    }
    if (a.tiled) COLI_DEC_CASES(1, true)
    COLI_DEC_CASES(1, false)
#undef COLI_DEC_CASES
}

}  // namespace coli
