// coli_qmv.hip -- the dense quantised matrix-vector product on the matrix
// cores, fp32-level accuracy:
//   y[s, o] = scale[o] * sum_i v(o, i) x[s, i]
// over int8 / int4 (nibble - 8) / int2 (crumb - 2) rows on the bf16 matrix
// cores, fp32 rows on the fp32 ones, and int4 rows with one scale per gs
// elements [glm.c@98759bf -- typedef QT, matmul_qt, matmul_q, matmul_i4,
// matmul_i2; metal@93cde63 -- mm_gemv; docs-quickstart -- qt_resolve_fmt].
//
// k_qmv1 (one or two activation rows) issues every weight load of the call
// up front; see its comment.  k_qmv (more rows): a block of 8 waves owns
// 16 MT consecutive output rows for one pass of up to 8 activation rows;
// wave w multiplies the rows' k-blocks w, w + 8, ... (a K-slice) in rounds
// of 8 k-blocks, so one block's loads cover its rows' whole width and there
// are enough blocks for the chip even for a few thousand rows; with GPS > 0
// it applies group scales segment by segment.  k_qmvg: group scales for one
// or two rows.  k_qmvf: fp32 rows.  In the integer kernels each lane loads
// its matrix-core operand straight from the row-major rows (lane 16 q + c:
// row c, bytes 16 q .. 16 q + 15 of each 64-byte segment; measured faster
// than coalesced row loads transposed with ds_bpermute, except for int8
// rows in k_qmv), and the activations are split into bf16 hi/lo in the
// kernel (column 2t: hi of row t, column 2t+1: lo) straight from the fp32
// input, so the call needs no scratch memory.  sum(x), needed to remove
// OFF * sum(x) from the code products, is one more MFMA per step against a
// tile of ones.  The 8 waves' partial tiles are added in wave order through
// LDS.
#include "coli_device.h"
#include "coli_frag.h"
#include "coli_qmv.h"

namespace coli {

namespace {

constexpr int kQmvWaves = 8;
constexpr int kQmvTpp = 8;   // activation rows per pass

typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 b2v __attribute__((ext_vector_type(2)));

// bf16 pair (a, b) -> one dword; `lo` lanes get the rounding residue instead:
// round(a - hi(a)), round(b - hi(b)).
__device__ __forceinline__ uint32_t hilo_pair(float a, float b, float lo)
{
    const b2v h = __builtin_convertvector(f2v{a, b}, b2v);
    const uint32_t hu = __builtin_bit_cast(uint32_t, h);
    const float ha = __uint_as_float(hu << 16), hb = __uint_as_float(hu & 0xFFFF0000u);
    const b2v r = __builtin_convertvector(f2v{fmaf(-lo, ha, a), fmaf(-lo, hb, b)}, b2v);
    return __builtin_bit_cast(uint32_t, r);
}

// LDS slot of a staged activation unit inside its chunk.  One LDS pass of a
// 16-byte access serves 8 lanes; the staging lanes of a pass write 8
// different chunks of one column (in each format's chunk order), the
// products' lanes read 8 columns of one chunk.  XOR-ing the column with these
// bits of the chunk index puts every pass's 8 writes into 8 different bank
// groups for the int8, int4 and int2 chunk orders alike (with the column
// alone, int4 and int2 writes collided 2- to 8-way); a read pass keeps its
// one chunk, so its columns stay distinct.  swz16: chunks of 16 column
// units; swz4: chunks of 4.
__device__ __forceinline__ int swz16(int c) { return ((c ^ (c >> 2)) & 6) | (c & 9); }
__device__ __forceinline__ int swz4(int c) { return (((c >> 1) ^ (c >> 3)) & 1) | ((((c >> 2) ^ (c >> 4)) & 1) << 1); }

// Staging loads of one run of RUN activations (elements e0 .. e0 + RUN - 1
// of row xr): unconditional 16-byte loads, from the run when it lies whole
// inside the row, else from x0 (the first row's first elements, always in
// bounds: rows hold at least RUN elements on these kernels) -- a value the
// staging then discards: it stages zeros for a run past the row end, and
// reads the one run crossing it element by element in a branch of its own.  A divergent choice between vector and element loads writing
// the same registers made the compiler wait for the first loads before
// issuing the second, for every run, before the weight loads were issued.
template <int RUN>
__device__ __forceinline__ void xrun_issue(const float *xr, const float *x0, int e0, int I,
                                           float4 (&v)[RUN / 4])
{
    const float *src = e0 + RUN <= I ? xr + e0 : x0;
#pragma unroll
    for (int i = 0; i < RUN / 4; ++i) v[i] = gload4f(src + 4 * i);
}
template <int RUN>
__device__ __forceinline__ void xrun_values(const float4 (&xv)[RUN / 4], float (&v)[RUN])
{
#pragma unroll
    for (int i = 0; i < RUN / 4; ++i) {
        v[4 * i] = xv[i].x;
        v[4 * i + 1] = xv[i].y;
        v[4 * i + 2] = xv[i].z;
        v[4 * i + 3] = xv[i].w;
    }
}
template <int RUN>
__device__ __forceinline__ void xrun_elements(const float *xr, int e0, int I, float (&v)[RUN])
{
#pragma unroll
    for (int i = 0; i < RUN; ++i) v[i] = e0 + i < I ? xr[e0 + i] : 0.f;
}

// GPS > 0: int4 rows with one scale per gs elements, GPS groups per 64-byte
// segment (128 elements): 1 (gs a multiple of 128), 2 (gs 64) or 4 (gs 32).
// Lane group q holds the segment's elements 32 q .. 32 q + 31, so group j is
// lane groups q with q / (4 / GPS) = j: per step one product per group with
// the activation operand zero in the other lane groups.  Each segment's
// products and activation sums start from zero and are then scaled into the
// running total, tot += scale[o, g] (products - OFF sums); the block's
// scales are staged in LDS after the round buffers.
// LDS of the rounds kernel: two round buffers, with group scales their
// block's scales (16 MT rows of ng | 1 floats), then the 8 waves' partial
// tiles -- past the rest when that keeps as many blocks on a CU (160 KB of
// LDS), else over the round buffers behind one more barrier.  The byte
// offset of the partial tiles (0: over the buffers) is shared by the kernel
// and its launch.
constexpr size_t kLdsMax = 160 * 1024;
__host__ __device__ inline bool lds_apart(size_t stage, size_t red)
{
    const size_t both = stage > red ? stage : red;
    return stage + red <= kLdsMax && kLdsMax / (stage + red) >= kLdsMax / both;
}
template <int FMT, int MT, int GPS>
__host__ __device__ inline size_t qmv_stage_bytes(int ng)
{
    return (size_t)2 * kQmvWaves * MF<FMT>::STEPS * 4 * 16 * 16 + (GPS > 0 ? (size_t)16 * MT * (size_t)(ng | 1) * 4 : 0);
}
template <int MT>
constexpr size_t qmv_red_bytes = (size_t)kQmvWaves * (MT + 1) * kWave * 16;
template <int FMT, int MT, int GPS>
__host__ __device__ inline size_t qmv_red_at(int ng)
{
    const size_t st = qmv_stage_bytes<FMT, MT, GPS>(ng);
    return lds_apart(st, qmv_red_bytes<MT>) ? st : 0;
}

template <int FMT, int MT, int GPS = 0>
__global__ __launch_bounds__(512) void k_qmv(QmvArgs a)
{
    constexpr bool GS = GPS > 0;
    static_assert(!GS || FMT == kI4, "group scales: int4 rows");
    using T = MF<FMT>;
    constexpr int STEPS = T::STEPS, KB = T::KB, SEGS = T::SEGS, BITS = T::BITS, SPS = T::SPS;
    constexpr int RB = 16 * MT;
    constexpr float OFF = T::OFF;
    constexpr uint32_t kbytes = KB * BITS / 8;
    constexpr int RUN = FMT == kI2 ? 16 : 8;          // elements per staging run
    // two round buffers of activation units -- per chunk 16 column units (hi
    // and lo of each row) at column ^ swz16(chunk); the partial tiles at the
    // end go past them or over them (qmv_red_at)
    extern __shared__ uint4 lds[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, q = lane >> 4;
    // int8: coalesced row loads (lane 4 r + k: row r, bytes 16 k ..)
    // transposed into the operand layout with ds_bpermute -- 2-3% faster
    // here than the direct operand loads the other formats take
    constexpr bool XPOSE = FMT == kI8;
    const int lrow = XPOSE ? lane >> 2 : col, lchunk = XPOSE ? lane & 3 : q;
    const int src4 = 4 * (4 * col + q);
    const int row0 = blockIdx.x * RB;
    const int t0 = blockIdx.y * kQmvTpp;
    const int nt = min(kQmvTpp, a.S - t0);
    const int nkb = a.nkb;
    const int rounds = (nkb + kQmvWaves - 1) / kQmvWaves;
    constexpr int units = kQmvWaves * STEPS * 4 * 16;   // units per round buffer
    float *sl = reinterpret_cast<float *>(lds + 2 * units);   // GS: the block's scales
    const int ngp = a.ng | 1;

    // a chunk past the end of a row shorter than 64 bytes is read at the
    // row's last chunk (it meets zero activations)
    const uint32_t coff = (uint32_t)min(16 * lchunk, (int)(a.rb - 16));
    uint32_t roff[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        roff[mt] = (uint32_t)(min(row0 + 16 * mt + lrow, a.O - 1) * a.rb) + coff;
    const uint32_t last_seg = (uint32_t)(a.rb - 16) - coff;

    floatx4 acc[MT], accs = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    const uint32_t one2 = opaque_v(0x3F803F80u);   // bf16 (1, 1)
    const uint4 ones = make_uint4(one2, one2, one2, one2);

    // weights of this wave's k-block in round r (a clamped copy when it has
    // none: the loads stay unconditional, the products are skipped)
    auto loadW = [&](int r, uint4 (&w)[MT][SEGS]) {
        const int kb = min(r * kQmvWaves + wave, nkb - 1);
        const uint32_t b0 = (uint32_t)kb * kbytes;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int sg = 0; sg < SEGS; ++sg)
                w[mt][sg] = gload16(a.W + (roff[mt] + min(b0 + 64 * sg, last_seg)));
    };
    // staging of round r: run u of the round (RUN consecutive elements of
    // one live row) per thread and pass; zeros past I
    constexpr int RUNS_PER_ROW = kQmvWaves * KB / RUN;
    constexpr int PASSES = (RUNS_PER_ROW * kQmvTpp + 511) / 512;
    auto loadX = [&](int r, float4 (&xv)[PASSES][RUN / 4]) {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int u = tid + 512 * p;
            const int t = min(u / RUNS_PER_ROW, nt - 1);
            const int e0 = r * kQmvWaves * KB + (u % RUNS_PER_ROW) * RUN;
            const float *xr = a.x + (int64_t)(t0 + t) * a.I;
            if (e0 + RUN <= a.I) {
#pragma unroll
                for (int i = 0; i < RUN / 4; ++i) xv[p][i] = gload4f(xr + e0 + 4 * i);
            } else {
#pragma unroll
                for (int i = 0; i < RUN / 4; ++i) {
                    float f[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) f[j] = e0 + 4 * i + j < a.I ? xr[e0 + 4 * i + j] : 0.f;
                    xv[p][i] = make_float4(f[0], f[1], f[2], f[3]);
                }
            }
        }
    };
    // ... split into bf16 hi (column 2t) and lo (column 2t+1) units in
    // fragment order: slot pairs (2m, 2m+1) are elements int8 (2m, 2m+1),
    // int4 (m, m+4), int2 (m, m+8) (and (m+4, m+12) for the odd step)
    auto stageX = [&](int r, const float4 (&xv)[PASSES][RUN / 4], uint4 *buf) {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int u = tid + 512 * p;
            if (u >= RUNS_PER_ROW * nt) break;   // live rows only
            const int t = u / RUNS_PER_ROW;
            const int e0 = (u % RUNS_PER_ROW) * RUN;   // inside the round
            int c, j;
            pos_of<FMT>(e0, c, j);   // chunk inside the round (k-blocks from 0)
            auto put = [&](const float (&v)[RUN]) {
#pragma unroll
                for (int h = 0; h < RUN / 8; ++h) {
                    uint32_t hw[4], lw[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        int k0, k1;
                        if constexpr (FMT == kI8) { k0 = 2 * m; k1 = 2 * m + 1; }
                        else if constexpr (FMT == kI4) { k0 = m; k1 = m + 4; }
                        else { k0 = m + 4 * h; k1 = m + 4 * h + 8; }
                        hw[m] = hilo_pair(v[k0], v[k1], 0.f);
                        lw[m] = hilo_pair(v[k0], v[k1], 1.f);
                    }
                    const int cc = c + 4 * h;
                    uint4 *dst = buf + cc * 16;
                    dst[(2 * t) ^ swz16(cc)] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
                    dst[(2 * t + 1) ^ swz16(cc)] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
                }
            };
            float v[RUN];
            xrun_values<RUN>(xv[p], v);   // loadX left zeros past I
            put(v);
        }
    };
    auto compute = [&](uint4 (&w)[MT][SEGS], const uint4 *buf, int kb) {
        if constexpr (XPOSE) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int sg = 0; sg < SEGS; ++sg) {
                    const uint4 u = w[mt][sg];
                    w[mt][sg] = make_uint4((uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)u.x),
                                           (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)u.y),
                                           (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)u.z),
                                           (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)u.w));
                }
        }
        // dead columns read the last live row's units
        const int bcol = (col >> 1) < nt ? col : 2 * (nt - 1) + (col & 1);
        if constexpr (GS) {
            constexpr int GPSX = GS ? GPS : 1;
            const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
            for (int sg = 0; sg < SEGS; ++sg) {
                floatx4 ap[GPSX][MT], sp[GPSX];
#pragma unroll
                for (int jg = 0; jg < GPSX; ++jg) {
                    sp[jg] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) ap[jg][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int sub = 0; sub < SPS; ++sub) {
                    const int cq = (wave * STEPS + sg * SPS + sub) * 4 + q;
                    const uint4 b = buf[cq * 16 + (bcol ^ swz16(cq))];
#pragma unroll
                    for (int jg = 0; jg < GPSX; ++jg) {
                        const uint4 bj = (GPSX == 1 || q / (4 / GPSX) == jg) ? b : zero;
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) ap[jg][mt] = mfma(codes<FMT>(w[mt][sg], sub), bj, ap[jg][mt]);
                        sp[jg] = mfma(ones, bj, sp[jg]);
                    }
                }
                // each group's scale (segments past the row end meet zero
                // activations: their products and sums are zero)
#pragma unroll
                for (int jg = 0; jg < GPSX; ++jg) {
                    const int g = min((kb * KB + sg * 128 + jg * (128 / GPSX)) / a.gs, a.ng - 1);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[mt][r] += sl[(16 * mt + 4 * q + r) * ngp + g] * (ap[jg][mt][r] - OFF * sp[jg][r]);
                }
            }
            return;
        }
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            const int cq = (wave * STEPS + s) * 4 + q;
            const uint4 b = buf[cq * 16 + (bcol ^ swz16(cq))];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma(codes<FMT>(w[mt][s / SPS], s % SPS), b, acc[mt]);
            accs = mfma(ones, b, accs);
        }
    };

    // Round r: the next round's activations and weights are requested (in
    // that order: the wait before staging then covers the activations only),
    // this round's products run from LDS, the next round is staged into the
    // other buffer, barrier.
    // the epilogue wave's (wave mt < MT) scales, requested before anything else
    float scp[4] = {1.f, 1.f, 1.f, 1.f};
    if (!GS && wave < MT && a.scale) {
#pragma unroll
        for (int r = 0; r < 4; ++r) scp[r] = a.scale[min(row0 + 16 * wave + 4 * q + r, a.O - 1)];
    }
    uint4 wA[MT][SEGS], wB[MT][SEGS];
    float4 xv[PASSES][RUN / 4];
    loadX(0, xv);
    loadW(0, wA);
    if constexpr (GS) {
        // the block's rows' scales (one contiguous span of ng per row) at
        // sl[row * ngp + g]; an odd row stride puts the 4 rows a read meets
        // (4 q + r, q = 0..3) in different banks
        const int nsc = (min(row0 + RB, a.O) - row0) * a.ng;
        const float *sb = a.scale + (int64_t)row0 * a.ng;
        for (int e = tid; e < nsc; e += 512) {
            const int rr = e / a.ng, g = e - rr * a.ng;
            sl[rr * ngp + g] = sb[e];
        }
    }
    stageX(0, xv, lds);
    __syncthreads();
    for (int r = 0; r < rounds; r += 2) {
        loadX(r + 1 < rounds ? r + 1 : r, xv);
        loadW(r + 1 < rounds ? r + 1 : r, wB);
        __builtin_amdgcn_sched_barrier(0);
        if (r * kQmvWaves + wave < nkb) compute(wA, lds, r * kQmvWaves + wave);
        __builtin_amdgcn_sched_barrier(0);
        if (r + 1 >= rounds) break;
        stageX(r + 1, xv, lds + units);
        __syncthreads();
        loadX(r + 2 < rounds ? r + 2 : r + 1, xv);
        loadW(r + 2 < rounds ? r + 2 : r + 1, wA);
        __builtin_amdgcn_sched_barrier(0);
        if ((r + 1) * kQmvWaves + wave < nkb) compute(wB, lds + units, (r + 1) * kQmvWaves + wave);
        __builtin_amdgcn_sched_barrier(0);
        if (r + 2 >= rounds) break;
        stageX(r + 2, xv, lds);
        __syncthreads();
    }

    // partial tiles of the 8 waves, added in wave order
    const size_t red_at = qmv_red_at<FMT, MT, GPS>(a.ng);
    if (red_at == 0) __syncthreads();   // every wave is done with the round buffers
    floatx4 *red = reinterpret_cast<floatx4 *>(reinterpret_cast<char *>(lds) + red_at);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[(wave * (MT + 1) + mt) * kWave + lane] = acc[mt];
    red[(wave * (MT + 1) + MT) * kWave + lane] = accs;
    __syncthreads();
    if (wave >= MT) return;
    const int mt = wave;
    floatx4 v = red[mt * kWave + lane], xs4 = red[MT * kWave + lane];
#pragma unroll
    for (int w = 1; w < kQmvWaves; ++w) {
        v += red[(w * (MT + 1) + mt) * kWave + lane];
        xs4 += red[(w * (MT + 1) + MT) * kWave + lane];
    }
    // D[4q + r][col]: the lo column is added to the hi one
    const float xs = xs4[0] + __shfl_xor(xs4[0], 1, kWave);
    const int ob = row0 + 16 * mt + 4 * q;
    float res[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float vv = v[r] + __shfl_xor(v[r], 1, kWave);
        res[r] = GS ? vv : scp[r] * (vv - OFF * xs);   // GS: scaled segment by segment
    }
    const int tok = col >> 1;
    if ((col & 1) == 0 && tok < nt) {
        float *yp = a.y + (int64_t)(t0 + tok) * a.O;
        if (a.y_vec4 && ob + 3 < a.O) {
            *reinterpret_cast<float4 *>(yp + ob) = make_float4(res[0], res[1], res[2], res[3]);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (ob + r < a.O) yp[ob + r] = res[r];
        }
    }
}

// ---------------------------------------------------------------- one shot
// For few activation rows the whole product fits one round: a block of 8
// waves owns MTB tiles of 16 output rows for a pass of up to kQ1Tpp
// activation rows, wave w takes the NKW consecutive k-blocks w NKW, ... of
// the rows, and every weight load of the block is issued before anything
// waits.  Several tiles per block keep the launch near one block per CU
// (12288 rows: 256 blocks of 48 rows) -- fewer, longer-lived waves, and
// the activations staged once per 16 MTB rows.  The
// pass's activations (the full width, as bf16 hi/lo units in fragment order)
// are staged into LDS while the weights are in flight; their loads are
// issued first, so the wait for them leaves the weight loads outstanding.
// Blocks on one XCD (block id mod 8) take the passes of a row tile next to
// each other, so the later passes find the tile's weights in that XCD's L2.
constexpr int kQ1Tpp = 2;   // activation rows per pass

template <int FMT, int NKW, int MTB>
__global__ __launch_bounds__(512) void k_qmv1(QmvArgs a, int passes, int ntiles)
{
    using T = MF<FMT>;
    constexpr int STEPS = T::STEPS, KB = T::KB, SEGS = T::SEGS, BITS = T::BITS, SPS = T::SPS;
    constexpr float OFF = T::OFF;
    constexpr uint32_t kbytes = KB * BITS / 8;
    constexpr int RUN = FMT == kI2 ? 16 : 8;              // elements per staging run
    constexpr int RW = NKW * KB / RUN;                    // staging runs per row in a wave's k-blocks
    constexpr int XP = (RW * kQ1Tpp + kWave - 1) / kWave; // runs per lane
    extern __shared__ uint4 lds[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, q = lane >> 4;
    const int xcd = blockIdx.x % 8, jb = blockIdx.x / 8;
    const int tgroup = (jb / passes) * 8 + xcd, pass = jb % passes;
    if (tgroup * MTB >= ntiles) return;                   // whole block, before any barrier
    const int row0 = tgroup * MTB * 16;                   // the block's first row
    const int t0 = pass * kQ1Tpp;
    const int nt = min(kQ1Tpp, a.S - t0);
    const int nkb = a.nkb;
    // this wave's k-blocks: kw0 .. kw0 + NKW - 1, those below nkb staged and
    // multiplied
    const int kw0 = wave * NKW;
    const int rw = max(0, min(RW, (nkb - kw0) * (KB / RUN)));   // live runs per row

    // wave mt < MTB finishes tile mt: its 4 scales per lane are requested first
    float scp[4] = {1.f, 1.f, 1.f, 1.f};
    if (wave < MTB && a.scale) {
#pragma unroll
        for (int r = 0; r < 4; ++r) scp[r] = a.scale[min(row0 + 16 * wave + 4 * q + r, a.O - 1)];
    }
    // activations next: each wave stages the runs of its own k-blocks (a
    // lane's dead runs read nothing: they start at I)
    float4 xv[XP][RUN / 4];
#pragma unroll
    for (int p = 0; p < XP; ++p) {
        const int u = lane + kWave * p;
        const bool live = u < RW * nt && u % RW < rw;
        const int t = live ? u / RW : 0, e0 = live ? kw0 * KB + (u % RW) * RUN : a.I;
        xrun_issue<RUN>(a.x + (int64_t)(t0 + t) * a.I, a.x, e0, a.I, xv[p]);
    }
    // then every weight load of this wave (a clamped copy for k-blocks past
    // the end: the loads stay unconditional, the products are skipped)
    const uint32_t coff = (uint32_t)min(16 * q, (int)(a.rb - 16));   // short rows: see k_qmv
    const uint32_t last_seg = (uint32_t)(a.rb - 16) - coff;
    uint4 w[MTB][NKW][SEGS];
#pragma unroll
    for (int mt = 0; mt < MTB; ++mt) {
        const uint32_t roff = (uint32_t)(min(row0 + 16 * mt + col, a.O - 1) * a.rb) + coff;
#pragma unroll
        for (int i = 0; i < NKW; ++i) {
            const uint32_t b0 = (uint32_t)min(wave * NKW + i, nkb - 1) * kbytes;
#pragma unroll
            for (int sg = 0; sg < SEGS; ++sg)
                w[mt][i][sg] = gload16(a.W + (roff + min(b0 + 64 * sg, last_seg)));
        }
    }
    // stage: run -> bf16 hi (column 2t) and lo (column 2t+1) units; the
    // wave reads back only what it wrote, so no block barrier is needed
#pragma unroll
    for (int p = 0; p < XP; ++p) {
        const int u = lane + kWave * p;
        if (u >= RW * nt) break;
        if (u % RW >= rw) continue;                   // past the last k-block
        const int t = u / RW, e0 = kw0 * KB + (u % RW) * RUN;
        int c, j;
        pos_of<FMT>(e0, c, j);
        auto put = [&](const float (&v)[RUN]) {
#pragma unroll
            for (int h = 0; h < RUN / 8; ++h) {
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    int k0, k1;
                    if constexpr (FMT == kI8) { k0 = 2 * m; k1 = 2 * m + 1; }
                    else if constexpr (FMT == kI4) { k0 = m; k1 = m + 4; }
                    else { k0 = m + 4 * h; k1 = m + 4 * h + 8; }
                    hw[m] = hilo_pair(v[k0], v[k1], 0.f);
                    lw[m] = hilo_pair(v[k0], v[k1], 1.f);
                }
                const int cc = c + 4 * h;
                uint4 *dst = lds + cc * 4;
                dst[(2 * t) ^ swz4(cc)] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
                dst[(2 * t + 1) ^ swz4(cc)] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
            }
        };
        float v[RUN];
        if (e0 + RUN <= a.I) {
            xrun_values<RUN>(xv[p], v);
            put(v);
        } else if (e0 >= a.I) {   // the k-block's padding past the row end
#pragma unroll
            for (int i = 0; i < RUN; ++i) v[i] = 0.f;
            put(v);
        } else {   // the run crossing the row end
            xrun_elements<RUN>(a.x + (int64_t)(t0 + t) * a.I, e0, a.I, v);
            put(v);
        }
    }

    floatx4 acc[MTB], accs = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < MTB; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    const uint32_t one2 = opaque_v(0x3F803F80u);   // bf16 (1, 1)
    const uint4 ones = make_uint4(one2, one2, one2, one2);
    // dead columns read the last live row's units
    const int bcol = (col >> 1) < nt ? col : 2 * (nt - 1) + (col & 1);
#pragma unroll
    for (int i = 0; i < NKW; ++i) {
        const int kb = wave * NKW + i;
        if (kb >= nkb) break;                         // uniform
#pragma unroll
        for (int s2 = 0; s2 < STEPS; ++s2) {
            const int cq = (kb * STEPS + s2) * 4 + q;
            const uint4 b = lds[cq * 4 + (bcol ^ swz4(cq))];
#pragma unroll
            for (int mt = 0; mt < MTB; ++mt) acc[mt] = mfma(codes<FMT>(w[mt][i][s2 / SPS], s2 % SPS), b, acc[mt]);
            accs = mfma(ones, b, accs);
        }
    }

    // partial tiles of the 8 waves, added in wave order; wave mt < MTB adds
    // tile mt.  They go to LDS past the staged activations, so one barrier
    // suffices (measured 0.1-0.4 us faster than reusing the staging area
    // behind a second barrier at 12288 x 6144)
    floatx4 *red = reinterpret_cast<floatx4 *>(lds + nkb * STEPS * 4 * 4);
#pragma unroll
    for (int mt = 0; mt < MTB; ++mt) red[(wave * (MTB + 1) + mt) * kWave + lane] = acc[mt];
    red[(wave * (MTB + 1) + MTB) * kWave + lane] = accs;
    __syncthreads();
    if (wave >= MTB) return;
    const int mt = wave;
    floatx4 v = red[mt * kWave + lane], xs4 = red[MTB * kWave + lane];
#pragma unroll
    for (int ww = 1; ww < kQmvWaves; ++ww) {
        v += red[(ww * (MTB + 1) + mt) * kWave + lane];
        xs4 += red[(ww * (MTB + 1) + MTB) * kWave + lane];
    }
    // D[4q + r][col]: the lo column is added to the hi one
    const float xs = xs4[0] + __shfl_xor(xs4[0], 1, kWave);
    const int ob = row0 + 16 * mt + 4 * q;
    float res[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float vv = v[r] + __shfl_xor(v[r], 1, kWave);
        res[r] = scp[r] * (vv - OFF * xs);
    }
    const int tok = col >> 1;
    if ((col & 1) == 0 && tok < nt) {
        float *yp = a.y + (int64_t)(t0 + tok) * a.O;
        if (a.y_vec4 && ob + 3 < a.O) {
            *reinterpret_cast<float4 *>(yp + ob) = make_float4(res[0], res[1], res[2], res[3]);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (ob + r < a.O) yp[ob + r] = res[r];
        }
    }
}

template <int FMT, int NKW, int MTB>
hipError_t launch_q1(const QmvArgs &a, hipStream_t st)
{
    const int ntiles = (a.O + 15) / 16;
    const int ngroups = (ntiles + MTB - 1) / MTB;
    const int passes = (a.S + kQ1Tpp - 1) / kQ1Tpp;
    const int64_t grid = (int64_t)(ngroups + 7) / 8 * 8 * passes;
    if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    const size_t stage = (size_t)a.nkb * MF<FMT>::STEPS * 4 * 4 * 16;   // 4 column units per chunk
    const size_t red = (size_t)kQmvWaves * (MTB + 1) * kWave * 16;
    const size_t lds = stage + red;   // at most 96 + 32 KB (nkw <= 6)
    auto kern = k_qmv1<FMT, NKW, MTB>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * kQmvWaves), lds, st, a, passes, ntiles);
    return hipGetLastError();
}

// Tiles per block: about one block per CU (256), at most three, and at most
// as many weight loads per wave as measured to fit the registers.
template <int FMT, int NKW>
hipError_t launch_q1_mtb(const QmvArgs &a, hipStream_t st)
{
    const int ntiles = (a.O + 15) / 16;
    int mtb = (ntiles + 255) / 256;
    if (mtb > 3) mtb = 3;
    if (NKW * mtb > 9) mtb = 9 / NKW;
    if (mtb >= 3) return launch_q1<FMT, NKW, (NKW <= 3 ? 3 : 1)>(a, st);
    if (mtb == 2) return launch_q1<FMT, NKW, (NKW <= 4 ? 2 : 1)>(a, st);
    return launch_q1<FMT, NKW, 1>(a, st);
}
template <int FMT>
hipError_t launch_q1_nkw(const QmvArgs &a, int nkw, hipStream_t st)
{
    switch (nkw) {
    case 1: return launch_q1_mtb<FMT, 1>(a, st);
    case 2: return launch_q1_mtb<FMT, 2>(a, st);
    case 3: return launch_q1_mtb<FMT, 3>(a, st);
    case 4: return launch_q1_mtb<FMT, 4>(a, st);
    case 5: return launch_q1_mtb<FMT, 5>(a, st);
    case 6: return launch_q1_mtb<FMT, 6>(a, st);
    default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------- fp32 rows
// fp32 weights on the fp32 matrix cores (v_mfma_f32_16x16x4_f32): the
// products need neither codes nor a hi/lo split, and no activation staging.
// A block of 8 waves owns MTB tiles of 16 rows for a pass of up to 16
// activation rows (one MFMA column each); wave w takes the w-th eighth of the
// row width in steps of 16 elements: lane (c, q) loads 16 bytes of weight
// row c and 16 of activation row c at element 16 j + 4 q and feeds them to 4
// consecutive MFMAs (k-slot q of product i is element 16 j + 4 q + i).  The
// loads of the next 4 steps are in flight while the current 4 are
// multiplied; the 8 waves' tiles are added in wave order through LDS.
constexpr int kQfTpp = 16;   // activation rows per pass
constexpr int kQfUnr = 4;    // steps per load batch

template <int MTB>
__global__ __launch_bounds__(512) void k_qmvf(QmvArgs a, int passes, int ntiles, int kw)
{
    __shared__ floatx4 red[kQmvWaves * MTB * kWave];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, q = lane >> 4;
    const int xcd = blockIdx.x % 8, jb = blockIdx.x / 8;
    const int tgroup = (jb / passes) * 8 + xcd, pass = jb % passes;
    if (tgroup * MTB >= ntiles) return;                   // whole block, before any barrier
    const int row0 = tgroup * MTB * 16;
    const int t0 = pass * kQfTpp;
    const int nt = min(kQfTpp, a.S - t0);

    // wave mt < MTB finishes tile mt: its 4 scales per lane are requested first
    float scp[4] = {1.f, 1.f, 1.f, 1.f};
    if (wave < MTB && a.scale) {
#pragma unroll
        for (int r = 0; r < 4; ++r) scp[r] = a.scale[min(row0 + 16 * wave + 4 * q + r, a.O - 1)];
    }
    const float *wr[MTB];
#pragma unroll
    for (int mt = 0; mt < MTB; ++mt)
        wr[mt] = reinterpret_cast<const float *>(a.W) + (int64_t)min(row0 + 16 * mt + col, a.O - 1) * a.I;
    // dead columns repeat the last live activation row (never stored)
    const float *xr = a.x + (int64_t)(t0 + min(col, nt - 1)) * a.I;
    const int k0 = wave * kw, k1 = min(a.I, k0 + kw);      // this wave's elements
    constexpr int BATCH = 16 * kQfUnr;

    floatx4 acc[MTB];
#pragma unroll
    for (int mt = 0; mt < MTB; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    // batch at element e: lane (c, q) takes elements e + 16 u + 4 q .. + 3
    // (I is a multiple of 4: a run is wholly inside the wave's part or not
    // loaded at all, its values zero)
    auto load = [&](int e, float4 (&wv)[kQfUnr][MTB], float4 (&xv)[kQfUnr]) {
#pragma unroll
        for (int u = 0; u < kQfUnr; ++u) {
            const int k = e + 16 * u + 4 * q;
            const bool in = k < k1;
#pragma unroll
            for (int mt = 0; mt < MTB; ++mt) wv[u][mt] = in ? gload4f(wr[mt] + k) : make_float4(0.f, 0.f, 0.f, 0.f);
            xv[u] = in ? gload4f(xr + k) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto product = [&](const float4 (&wv)[kQfUnr][MTB], const float4 (&xv)[kQfUnr]) {
#pragma unroll
        for (int u = 0; u < kQfUnr; ++u) {
            const float xa[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int mt = 0; mt < MTB; ++mt) {
                    const float wa[4] = {wv[u][mt].x, wv[u][mt].y, wv[u][mt].z, wv[u][mt].w};
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[i], xa[i], acc[mt], 0, 0, 0);
                }
        }
    };
    float4 wA[kQfUnr][MTB], xA[kQfUnr], wB[kQfUnr][MTB], xB[kQfUnr];
    if (k0 < k1) load(k0, wA, xA);
    for (int e = k0; e < k1; e += 2 * BATCH) {
        if (e + BATCH < k1) load(e + BATCH, wB, xB);
        product(wA, xA);
        if (e + BATCH >= k1) break;
        if (e + 2 * BATCH < k1) load(e + 2 * BATCH, wA, xA);
        product(wB, xB);
    }

    // partial tiles of the 8 waves, added in wave order; wave mt < MTB adds
    // tile mt
#pragma unroll
    for (int mt = 0; mt < MTB; ++mt) red[(wave * MTB + mt) * kWave + lane] = acc[mt];
    __syncthreads();
    if (wave >= MTB) return;
    const int mt = wave;
    floatx4 v = red[mt * kWave + lane];
#pragma unroll
    for (int ww = 1; ww < kQmvWaves; ++ww) v += red[(ww * MTB + mt) * kWave + lane];
    // D[4 q + r][col]: weight row row0 + 16 mt + 4 q + r, activation row t0 + col
    const int ob = row0 + 16 * mt + 4 * q;
    if (col < nt) {
        float *yp = a.y + (int64_t)(t0 + col) * a.O;
        if (a.y_vec4 && ob + 3 < a.O) {
            *reinterpret_cast<float4 *>(yp + ob) = make_float4(scp[0] * v[0], scp[1] * v[1], scp[2] * v[2], scp[3] * v[3]);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (ob + r < a.O) yp[ob + r] = scp[r] * v[r];
        }
    }
}

template <int MTB>
hipError_t launch_qf(const QmvArgs &a, hipStream_t st)
{
    const int ntiles = (a.O + 15) / 16;
    const int ngroups = (ntiles + MTB - 1) / MTB;
    const int passes = (a.S + kQfTpp - 1) / kQfTpp;
    const int64_t grid = (int64_t)(ngroups + 7) / 8 * 8 * passes;
    if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int kw = ((a.I + kQmvWaves - 1) / kQmvWaves + 15) / 16 * 16;
    hipLaunchKernelGGL((k_qmvf<MTB>), dim3((unsigned)grid), dim3(64 * kQmvWaves), 0, st, a, passes, ntiles, kw);
    return hipGetLastError();
}

// compute units of the current device (cached per device)
int64_t qmv_cus()
{
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] <= 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cache[dev] = cus;
    }
    return cache[dev];
}

template <int FMT, int MT, int GPS = 0>
hipError_t launch_q(const QmvArgs &a, hipStream_t st)
{
    const int rb = 16 * MT;
    const dim3 grid((unsigned)((a.O + rb - 1) / rb), (unsigned)((a.S + kQmvTpp - 1) / kQmvTpp));
    // LDS: two round buffers (GS: and the block's scales), then or over
    // them the partial tiles
    const size_t stage = qmv_stage_bytes<FMT, MT, GPS>(a.ng), red = qmv_red_bytes<MT>;
    const size_t red_at = qmv_red_at<FMT, MT, GPS>(a.ng);
    const size_t lds = red_at ? red_at + red : (stage > red ? stage : red);
    if (lds > kLdsMax) return hipErrorInvalidValue;
    auto kern = k_qmv<FMT, MT, GPS>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, grid, dim3(64 * kQmvWaves), lds, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- grouped int4
// Grouped-scale int4 (one fp32 scale per gs elements along I) [docs-quickstart
// -- qt_resolve_fmt; glm.c@98759bf -- qt_from_disk]: the one-shot structure
// of k_qmv1, with the scale applied per group inside the sum.  A 64-byte
// segment (128 elements) lies in one group when gs is a multiple of 128; for
// gs = 64 / 32 it holds GPS = 2 / 4 groups, lane group q's 32 elements in
// group q / (4 / GPS).  The groups take the product's spare columns: column
// col = h + 2 t + 4 j holds token t's hi / lo part (h) restricted to the
// segment's group j (the B operand is zero in the lane groups of other
// groups), so one code product and one column-sum product per step serve
// every group.  Per segment each lane adds scale[o, g(j)] * (products -
// OFF * sum) for its column's group; the columns of one token are summed at
// the end.  The block's scales (16 consecutive rows: one contiguous span of
// 16 ng floats) are staged in LDS in row order.
// LDS of k_qmvg: the staged activations, the block's scales (ng + 15 rows
// of 16 floats), then the 8 waves' partial tiles -- past the rest when that
// keeps as many blocks on a CU, else over the staging behind one more
// barrier.
__host__ __device__ inline size_t qmvg_stage_bytes(int nkb, int ng)
{
    return (size_t)nkb * MF<kI4>::STEPS * 4 * 4 * 16 + (size_t)(ng + 15) * 16 * 4;
}
constexpr size_t kQgRedBytes = (size_t)kQmvWaves * kWave * 16;
__host__ __device__ inline size_t qmvg_red_at(int nkb, int ng)
{
    const size_t st = qmvg_stage_bytes(nkb, ng);
    return lds_apart(st, kQgRedBytes) ? st : 0;
}

template <int GPS, int NKW>
__global__ __launch_bounds__(512) void k_qmvg(QmvArgs a, int passes, int ntiles)
{
    using T = MF<kI4>;
    constexpr int STEPS = T::STEPS, KB = T::KB, SPS = T::SPS;
    constexpr float OFF = T::OFF;
    constexpr uint32_t kbytes = KB / 2;
    constexpr int RUN = 8;
    constexpr int RW = NKW * KB / RUN;
    constexpr int XP = (RW * kQ1Tpp + kWave - 1) / kWave;
    static_assert(kQ1Tpp == 2, "columns h + 2t + 4j");
    extern __shared__ uint4 lds[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, q = lane >> 4;
    const int xcd = blockIdx.x % 8, jb = blockIdx.x / 8;
    const int tile = (jb / passes) * 8 + xcd, pass = jb % passes;
    if (tile >= ntiles) return;                           // whole block, before any barrier
    const int row0 = tile * 16;
    const int t0 = pass * kQ1Tpp;
    const int nt = min(kQ1Tpp, a.S - t0);
    const int nkb = a.nkb, ng = a.ng, gs = a.gs;
    const int kw0 = wave * NKW;
    const int rw = max(0, min(RW, (nkb - kw0) * (KB / RUN)));
    // scales of the block's rows after the staged activations (4 column
    // units per chunk, at column ^ swz4(chunk))
    float *sl = reinterpret_cast<float *>(lds + (int64_t)nkb * STEPS * 4 * 4);

    // the block's scales first: rows row0 .. row0 + 15 (those below O) are
    // the contiguous span scale[row0 * ng ..], 16-byte aligned (row0 * ng is a
    // multiple of 16 and the base is aligned).  A k-block holds at most
    // 2 GPS groups and a block at most 8 NKW k-blocks, so the span is at most
    // 16 x 16 GPS NKW floats: SCN float4 per thread (checked at launch)
    const int nsc = (min(row0 + 16, a.O) - row0) * ng;
    const float *sbase = a.scale + (int64_t)row0 * ng;
    constexpr int SCN = (GPS * NKW + 7) / 8;
    float4 sv[SCN];
#pragma unroll
    for (int k = 0; k < SCN; ++k) {
        const int e = 4 * (tid + 512 * k);
        if (e + 3 < nsc) {
            sv[k] = gload4f(sbase + e);
        } else {
            float f[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) f[c] = e + c < nsc ? sbase[e + c] : 0.f;
            sv[k] = make_float4(f[0], f[1], f[2], f[3]);
        }
    }
    // activations next
    float4 xv[XP][RUN / 4];
#pragma unroll
    for (int p = 0; p < XP; ++p) {
        const int u = lane + kWave * p;
        const bool live = u < RW * nt && u % RW < rw;
        const int t = live ? u / RW : 0, e0 = live ? kw0 * KB + (u % RW) * RUN : a.I;
        // rows are whole 16-byte segments (I a multiple of 32): a live run
        // is whole inside the row or wholly past it (staged as zeros)
        xrun_issue<RUN>(a.x + (int64_t)(t0 + t) * a.I, a.x, e0, a.I, xv[p]);
    }
    // then every weight load of this wave
    const uint32_t coff = (uint32_t)min(16 * q, (int)(a.rb - 16));   // short rows: see k_qmv
    const uint32_t roff = (uint32_t)(min(row0 + col, a.O - 1) * a.rb) + coff;
    const uint32_t last_seg = (uint32_t)(a.rb - 16) - coff;
    uint4 w[NKW][2];
#pragma unroll
    for (int i = 0; i < NKW; ++i) {
        const uint32_t b0 = (uint32_t)min(kw0 + i, nkb - 1) * kbytes;
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) w[i][sg] = gload16(a.W + (roff + min(b0 + 64 * sg, last_seg)));
    }
    // scales into LDS in row order, row stride ngp = ng rounded up to 4 mod 16
    // (the span's float4 land on consecutive banks; the epilogue's 16 reads,
    // rows 4q .. 4q + 3 x four groups, on distinct banks)
    const int ngp = (ng + 11) / 16 * 16 + 4;
    {
        const float inv = 1.0f / (float)ng;
        auto split = [&](int e, int &r, int &g) {          // e = r ng + g, e < 6144
            r = (int)((float)e * inv);                     // off by at most one
            g = e - r * ng;
            if (g < 0) { --r; g += ng; }
            if (g >= ng) { ++r; g -= ng; }
        };
        if (ng % 4 == 0) {                                 // a float4 stays in one row
#pragma unroll
            for (int k = 0; k < SCN; ++k) {
                const int e = 4 * (tid + 512 * k);
                if (e < nsc) {
                    int r, g;
                    split(e, r, g);
                    *reinterpret_cast<float4 *>(sl + r * ngp + g) = sv[k];
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < SCN; ++k) {
                const float f[4] = {sv[k].x, sv[k].y, sv[k].z, sv[k].w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int e = 4 * (tid + 512 * k) + c;
                    if (e < nsc) {
                        int r, g;
                        split(e, r, g);
                        sl[r * ngp + g] = f[c];
                    }
                }
            }
        }
    }
    // activations into LDS: run -> bf16 hi / lo units (this wave's k-blocks)
#pragma unroll
    for (int p = 0; p < XP; ++p) {
        const int u = lane + kWave * p;
        if (u >= RW * nt) break;
        if (u % RW >= rw) continue;
        const int t = u / RW, e0 = kw0 * KB + (u % RW) * RUN;
        float v[RUN];
        // I is a multiple of 32: a run is whole inside the row or wholly in
        // the k-block's padding past I (zeros)
        xrun_values<RUN>(xv[p], v);
        if (e0 >= a.I) {
#pragma unroll
            for (int i = 0; i < RUN; ++i) v[i] = 0.f;
        }
        int c, j;
        pos_of<kI4>(e0, c, j);
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            hw[m] = hilo_pair(v[m], v[m + 4], 0.f);
            lw[m] = hilo_pair(v[m], v[m + 4], 1.f);
        }
        uint4 *dst = lds + c * 4;
        dst[(2 * t) ^ swz4(c)] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        dst[(2 * t + 1) ^ swz4(c)] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
    __syncthreads();                                      // the scales are read by every wave

    floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
    const uint32_t one2 = opaque_v(0x3F803F80u);           // bf16 (1, 1)
    const uint4 ones = make_uint4(one2, one2, one2, one2);
    // column col = h + 2 t + 4 j: token t (dead tokens read the last live
    // one's units and are never written), group j of the segment
    const int tcol = (col >> 1) & 1, jcol = col >> 2;
    const int bcol = tcol < nt ? (col & 3) : 2 * (nt - 1) + (col & 1);
    const bool mine = jcol == q / (4 / GPS);              // this lane group's elements are in group j
    const int jofs = jcol * (128 / GPS);                  // first element of group j in a segment
#pragma unroll
    for (int i = 0; i < NKW; ++i) {
        const int kb = kw0 + i;
        if (kb >= nkb) break;                             // uniform
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
            floatx4 ap = floatx4{0.f, 0.f, 0.f, 0.f}, sp = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sub = 0; sub < SPS; ++sub) {
                const int s2 = sg * SPS + sub;
                const int cq = (kb * STEPS + s2) * 4 + q;
                const uint4 b0 = lds[cq * 4 + (bcol ^ swz4(cq))];
                const uint4 b = mine ? b0 : make_uint4(0u, 0u, 0u, 0u);
                ap = mfma(codes<kI4>(w[i][sg], sub), b, ap);
                sp = mfma(ones, b, sp);
            }
            // rows 4q + r, this column's group (dead groups: zero products)
            const int g = min((kb * KB + sg * 128 + jofs) / gs, ng - 1);
            const float *sr = sl + 4 * q * ngp + g;
            const float4 s4 = make_float4(sr[0], sr[ngp], sr[2 * ngp], sr[3 * ngp]);
            const float xs = sp[0];
            acc[0] += s4.x * (ap[0] - OFF * xs);
            acc[1] += s4.y * (ap[1] - OFF * xs);
            acc[2] += s4.z * (ap[2] - OFF * xs);
            acc[3] += s4.w * (ap[3] - OFF * xs);
        }
    }

    // partial tiles of the 8 waves, added in wave order
    // (past the staged activations and scales when they fit, else over them
    // behind one more barrier)
    const size_t red_at = qmvg_red_at(nkb, ng);
    if (red_at == 0) __syncthreads();
    floatx4 *red = reinterpret_cast<floatx4 *>(reinterpret_cast<char *>(lds) + red_at);
    red[wave * kWave + lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    floatx4 v = red[lane];
#pragma unroll
    for (int ww = 1; ww < kQmvWaves; ++ww) v += red[ww * kWave + lane];
    const int ob = row0 + 4 * q;
    float res[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float t = v[r] + __shfl_xor(v[r], 1, kWave);      // hi + lo
        if (GPS > 1) t += __shfl_xor(t, 4, kWave);        // groups j: 0 + 1, 2 + 3
        if (GPS > 2) t += __shfl_xor(t, 8, kWave);        // (0 + 1) + (2 + 3)
        res[r] = t;
    }
    const int tok = tcol;
    if ((col & 1) == 0 && jcol == 0 && tok < nt) {
        float *yp = a.y + (int64_t)(t0 + tok) * a.O;
        if (a.y_vec4 && ob + 3 < a.O) {
            *reinterpret_cast<float4 *>(yp + ob) = make_float4(res[0], res[1], res[2], res[3]);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (ob + r < a.O) yp[ob + r] = res[r];
        }
    }
}

template <int GPS, int NKW>
hipError_t launch_qg(const QmvArgs &a, hipStream_t st)
{
    const int ntiles = (a.O + 15) / 16;
    const int passes = (a.S + kQ1Tpp - 1) / kQ1Tpp;
    const int64_t grid = (int64_t)(ntiles + 7) / 8 * 8 * passes;
    if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    const size_t stage = qmvg_stage_bytes(a.nkb, a.ng), red = kQgRedBytes;
    const size_t red_at = qmvg_red_at(a.nkb, a.ng);
    const size_t lds = red_at ? red_at + red : (stage > red ? stage : red);
    if (lds > kLdsMax) return hipErrorInvalidValue;
    if (16 * a.ng > 4 * 512 * ((GPS * NKW + 7) / 8)) return hipErrorInvalidValue;   // the scale span
    auto kern = k_qmvg<GPS, NKW>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * kQmvWaves), lds, st, a, passes, ntiles);
    return hipGetLastError();
}

template <int GPS>
hipError_t launch_qg_nkw(const QmvArgs &a, int nkw, hipStream_t st)
{
    switch (nkw) {
    case 1: return launch_qg<GPS, 1>(a, st);
    case 2: return launch_qg<GPS, 2>(a, st);
    case 3: return launch_qg<GPS, 3>(a, st);
    case 4: return launch_qg<GPS, 4>(a, st);
    case 5: return launch_qg<GPS, 5>(a, st);
    case 6: return launch_qg<GPS, 6>(a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Row tiles per block of the rounds kernel: 64 or 48 rows once that still
// gives at least 128 blocks, else 32 (each block stages every activation
// row, so fewer rows per block cost activation traffic): of 64 and 48 the one
// whose blocks fill the last round of CUs best, 64 on a tie (12288 rows: 256
// blocks of 48 against 192 of 64 -- int8 8 rows 22.0 -> 20.0 us, int4 16.7
// -> 16.3 us)
int rounds_mt(int O)
{
    if ((int64_t)O < 64 * 128) return 2;
    const int64_t cus = qmv_cus();
    auto fill = [&](int rows) {
        const int64_t blocks = (O + rows - 1) / rows, rounds = (blocks + cus - 1) / cus;
        return (double)blocks / (double)(rounds * cus);
    };
    return fill(48) > fill(64) ? 3 : 4;
}

bool qmv_f32_supported(int I, const void *W, const float *x)
{
    return I >= 4 && I % 4 == 0 && ((uintptr_t)W & 15u) == 0 && ((uintptr_t)x & 15u) == 0;
}

// fp32 rows: up to 4 activation rows one row tile per block (more blocks
// per CU; 12288 x 6144: S = 1 58.4 us against 65.1 with 3 tiles); from 5 rows
// on about one block per CU with at most 3 tiles, so fewer blocks re-read the
// activations (S = 8: 69.9 against 74.5 us, S = 16: 75.3 against 90.3 us)
hipError_t qmv_f32_launch(QmvArgs a, hipStream_t st)
{
    if (a.S <= 0 || a.O <= 0) return hipSuccess;
    a.y_vec4 = a.O % 4 == 0 && ((uintptr_t)a.y & 15u) == 0;
    const int64_t ntiles = (a.O + 15) / 16;
    const int64_t mtb = a.S <= 4 ? 1 : (ntiles + qmv_cus() - 1) / qmv_cus();
    if (mtb >= 3) return launch_qf<3>(a, st);
    if (mtb == 2) return launch_qf<2>(a, st);
    return launch_qf<1>(a, st);
}

bool qmv_supported(int fmt, int64_t rb, int I, int O, const void *W, const float *x)
{
    if (fmt != kI8 && fmt != kI4 && fmt != kI2) return false;
    return rb >= 16 && rb % 16 == 0 && I % 4 == 0 && ((uintptr_t)W & 15u) == 0 && ((uintptr_t)x & 15u) == 0 &&
           (int64_t)O * rb < ((int64_t)1 << 32) - 4096;
}

hipError_t qmv_launch(QmvArgs a, int fmt, hipStream_t st)
{
    if (a.S <= 0 || a.O <= 0) return hipSuccess;
    const int KB = fmt == kI8 ? MF<kI8>::KB : fmt == kI4 ? MF<kI4>::KB : MF<kI2>::KB;
    a.nkb = (a.I + KB - 1) / KB;
    a.y_vec4 = a.O % 4 == 0 && ((uintptr_t)a.y & 15u) == 0;
    // one shot for one pass (measured faster there: int4 12288 x 6144 at one
    // row 10.9 us against 14.8 us for the rounds below; from two passes on
    // the rounds win) while a wave's k-blocks fit its registers
    const int nkw = (a.nkb + kQmvWaves - 1) / kQmvWaves;
    if (a.S <= kQ1Tpp && nkw <= 6) {
        switch (fmt) {
        case kI8: return launch_q1_nkw<kI8>(a, nkw, st);
        case kI4: return launch_q1_nkw<kI4>(a, nkw, st);
        case kI2: return launch_q1_nkw<kI2>(a, nkw, st);
        default: return hipErrorInvalidValue;
        }
    }
    const int mt = rounds_mt(a.O);
#define COLI_Q_MT(F) return mt == 4 ? launch_q<F, 4>(a, st) : mt == 3 ? launch_q<F, 3>(a, st) : launch_q<F, 2>(a, st)
    switch (fmt) {
    case kI8: COLI_Q_MT(kI8);
    case kI4: COLI_Q_MT(kI4);
    case kI2: COLI_Q_MT(kI2);
    default: return hipErrorInvalidValue;
    }
#undef COLI_Q_MT
}

}  // namespace coli

namespace coli {

bool qmv_grouped_supported(int64_t rb, int I, int gs, const void *W, const float *scale, const float *x)
{
    const int nkb = (I + MF<kI4>::KB - 1) / MF<kI4>::KB;
    return (gs == 32 || gs == 64 || (gs >= 128 && gs % 128 == 0)) && rb >= 16 && rb % 16 == 0 &&
           I % 4 == 0 && ((uintptr_t)W & 15u) == 0 && ((uintptr_t)x & 15u) == 0 &&
           ((uintptr_t)scale & 15u) == 0 &&
           (nkb + kQmvWaves - 1) / kQmvWaves <= 6;
}

hipError_t qmv_grouped_launch(QmvArgs a, hipStream_t st)
{
    if (a.S <= 0 || a.O <= 0) return hipSuccess;
    a.nkb = (a.I + MF<kI4>::KB - 1) / MF<kI4>::KB;
    a.ng = (a.I + a.gs - 1) / a.gs;
    a.y_vec4 = a.O % 4 == 0 && ((uintptr_t)a.y & 15u) == 0;
    // more rows than one pass of k_qmvg holds: the rounds kernel with group
    // scales takes 8 rows per pass (12288 x 6144, gs 128: 4 rows 15.3 us
    // against 21.7 us for two passes, 8 rows 16.0 against 38.9 us; gs 64:
    // 18.1 / 19.5 against 23.7 / 43.1 us).  gs 32 costs it four products and
    // four flushes per step and segment (4 rows: 36.2 against 24.3 us for two
    // passes, 8 rows: 38.0 against 44.2 us), so gs 32 takes it from 7 rows on.
    // Only when the block's scales fit LDS beside the two round buffers;
    // else, for the widest rows at gs 32 / 64, passes of k_qmvg.
    if (a.S > kQ1Tpp && (a.gs != 32 || a.S > 3 * kQ1Tpp)) {
        int mt = rounds_mt(a.O);
        if (a.gs == 32) mt = 2;                           // 48 rows: 4 x 3 group tiles spill
        else if (a.gs == 64 && mt > 3) mt = 3;
        const size_t need = (size_t)2 * kQmvWaves * MF<kI4>::STEPS * 4 * 16 * 16 + (size_t)16 * mt * (size_t)(a.ng | 1) * 4;
        if (need <= kLdsMax) {
            if (a.gs == 32) return launch_q<kI4, 2, 4>(a, st);
            if (a.gs == 64) return mt == 3 ? launch_q<kI4, 3, 2>(a, st) : launch_q<kI4, 2, 2>(a, st);
            return mt == 4 ? launch_q<kI4, 4, 1>(a, st) : mt == 3 ? launch_q<kI4, 3, 1>(a, st)
                                                            : launch_q<kI4, 2, 1>(a, st);
        }
    }
    const int nkw = (a.nkb + kQmvWaves - 1) / kQmvWaves;
    if (a.gs == 32) return launch_qg_nkw<4>(a, nkw, st);
    if (a.gs == 64) return launch_qg_nkw<2>(a, nkw, st);
    return launch_qg_nkw<1>(a, nkw, st);
}

}  // namespace coli
