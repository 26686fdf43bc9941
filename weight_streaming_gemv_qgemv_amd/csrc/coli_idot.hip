// coli_idot.hip -- the integer-dot qgemv (IDOT) on the int8 matrix cores
// [glm.c@98759bf -- qrow_i8, dot_i8i8, dot_i4i8, matmul_q_idot,
// matmul_i4_idot]: each activation row is quantised to int8 by its absolute
// maximum (s = max|x| / 127, at least 1e-12; q = round-half-even(x * (1/s))),
// the dot product with the int8 / int4 weight values is exact in int32, and
//   y[s, o] = ((float)dot * scale[o]) * s_row,
// each step rounded in fp32 as the pages order it -- so the result is the
// definition's, bit for bit.
//
// k_qrow quantises one row per block and writes it in fragment order (below);
// k_idot is one-shot like the dense bf16 qgemv: a block of 8 waves owns 16
// output rows for a pass of up to 16 activation rows (one MFMA column each:
// no hi/lo pair is needed, the values are exact integers), wave w takes the
// NKW consecutive k-blocks w NKW, ..., every load of the call is issued before
// anything waits, and the 8 partial tiles are added in LDS (int32: exact in
// any order).
//
// Fragment order (v_mfma_i32_16x16x64_i8, 16 bytes per lane and step): lane
// (q, col) holds row col, 16-byte chunk q of a 64-byte weight segment.
//   int8: one step per chunk; byte b of the chunk is element 16 q + b of the
//         step's 64 (natural order).
//   int4: two steps per chunk (its low and high 8 bytes); for the 16
//         elements e0..e0+15 of a step the A operand's dwords are the low
//         nibbles of bytes 0-3, their high nibbles, the low nibbles of bytes
//         4-7, their high nibbles -- element order [0 2 4 6 | 1 3 5 7 |
//         8 10 12 14 | 9 11 13 15] -- and the quantised activations are
//         stored in that order.  Nibbles are taken as codes 0..15 (value +
//         8): 8 * sum(q) is removed from the integer dot.
// A step st of a row is 4 units of 16 bytes (q = 0..3) at byte 64 st.
#include <hip/hip_ext.h>

#include "coli_device.h"
#include "coli_frag.h"
#include "coli_idot.h"
#include "coli_pre.h"
#include "coli_stages.h"

namespace coli {

namespace {

constexpr int kIdWaves = 8;
constexpr int kIdTpp = 16;        // activation rows per pass
constexpr int kIdMaxNkw = 8;      // k-blocks a wave holds in registers
typedef int int4v __attribute__((ext_vector_type(4)));

// k-block: 128 bytes of a weight row (two 64-byte segments)
template <int FMT> struct ID;
template <> struct ID<kI8> { static constexpr int KB = 128, SPK = 2; };   // elements, MFMA steps
template <> struct ID<kI4> { static constexpr int KB = 256, SPK = 4; };

// ---------------------------------------------------------------- quantiser
// Block (row, part): the row's absolute maximum (every part takes it over the
// whole row: a max is exact in any order), then part p quantises elements
// 4096 p .. 4096 p + 4095 -- 16 per thread -- and stores them in fragment
// order with its partial sum of the quantised values (int32, exact).
constexpr int kQPart = 4096;
constexpr int kQMaxParts = 4;

template <int FMT>
__global__ __launch_bounds__(256) void k_qrow(const float *__restrict__ x, int I, int64_t kq, int vec,
                                              int8_t *__restrict__ table, float *__restrict__ sx,
                                              int *__restrict__ psq)
{
    __shared__ float redf[4];
    __shared__ int redi[4];
    const int row = blockIdx.x, part = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float *xr = x + (int64_t)row * I;
    float amax = 0.f;
    if (vec) {
        for (int i = 4 * tid; i < I; i += 1024) {
            const float4 v = *reinterpret_cast<const float4 *>(xr + i);
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
    } else {
        for (int i = tid; i < I; i += 256) amax = fmaxf(amax, fabsf(xr[i]));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
    if (lane == 0) redf[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(redf[0], redf[1]), fmaxf(redf[2], redf[3]));
    float s = amax / 127.f;
    if (s < 1e-12f) s = 1e-12f;
    const float inv = 1.f / s;
    int sum = 0;
    const int64_t e0 = (int64_t)part * kQPart + 16 * tid;
    if (e0 < kq) {
        float xv[16];
        if (vec && e0 + 16 <= I) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float4 v = *reinterpret_cast<const float4 *>(xr + e0 + 4 * k);
                xv[4 * k] = v.x;
                xv[4 * k + 1] = v.y;
                xv[4 * k + 2] = v.z;
                xv[4 * k + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k) xv[k] = e0 + k < I ? xr[e0 + k] : 0.f;
        }
        int qv[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            qv[k] = (int)__builtin_rintf(xv[k] * inv);   // round half to even
            sum += qv[k];
        }
        int64_t off;
        uint32_t d[4];
        if constexpr (FMT == kI8) {
            off = e0;
#pragma unroll
            for (int m = 0; m < 4; ++m)
                d[m] = (uint32_t)(qv[4 * m] & 255) | (uint32_t)(qv[4 * m + 1] & 255) << 8 |
                       (uint32_t)(qv[4 * m + 2] & 255) << 16 | (uint32_t)(qv[4 * m + 3] & 255) << 24;
        } else {
            // run e0 = 256 kb + 128 sg + 32 q + 16 sub -> step 4 kb + 2 sg + sub, unit q
            const int64_t kb = e0 / 256;
            const int r = (int)(e0 % 256), sg = r / 128, q = (r % 128) / 32, sub = (r % 32) / 16;
            off = 16 * (4 * (4 * kb + 2 * sg + sub) + q);
            static constexpr int ord[4][4] = {{0, 2, 4, 6}, {1, 3, 5, 7}, {8, 10, 12, 14}, {9, 11, 13, 15}};
#pragma unroll
            for (int m = 0; m < 4; ++m)
                d[m] = (uint32_t)(qv[ord[m][0]] & 255) | (uint32_t)(qv[ord[m][1]] & 255) << 8 |
                       (uint32_t)(qv[ord[m][2]] & 255) << 16 | (uint32_t)(qv[ord[m][3]] & 255) << 24;
        }
        *reinterpret_cast<uint4 *>(table + (int64_t)row * kq + off) = make_uint4(d[0], d[1], d[2], d[3]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, kWave);
    if (lane == 0) redi[wave] = sum;
    __syncthreads();
    if (tid == 0) {
        if (part == 0) sx[row] = s;
        psq[(int64_t)row * kQMaxParts + part] = redi[0] + redi[1] + redi[2] + redi[3];
    }
}

// ---------------------------------------------------------------- product
template <int FMT>
__device__ __forceinline__ int4v icodes(const uint4 &w, int sub)
{
    if constexpr (FMT == kI8) {
        return int4v{(int)w.x, (int)w.y, (int)w.z, (int)w.w};
    } else {
        const uint32_t m = opaque_s(0x0F0F0F0Fu);
        const uint32_t d0 = sub ? w.z : w.x, d1 = sub ? w.w : w.y;
        return int4v{(int)(d0 & m), (int)((d0 >> 4) & m), (int)(d1 & m), (int)((d1 >> 4) & m)};
    }
}

template <int FMT, int NKW>
__global__ __launch_bounds__(512) void k_idot(IdotArgs a, int passes, int ntiles)
{
    using P = ID<FMT>;
    constexpr int SPK = P::SPK;
    constexpr uint32_t kbytes = 128;
    __shared__ int4v red[kIdWaves * kWave];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, q = lane >> 4, lrow = lane >> 2, lchunk = lane & 3;
    const int src4 = 4 * (4 * col + q);
    const int xcd = blockIdx.x % 8, jb = blockIdx.x / 8;
    const int tile = (jb / passes) * 8 + xcd, pass = jb % passes;
    if (tile >= ntiles) return;                           // whole block, before any barrier
    const int row0 = tile * 16;
    const int t0 = pass * kIdTpp;
    const int nt = min(kIdTpp, a.S - t0);
    const int nkb = a.nkb;
    const int kw0 = wave * NKW;

    // activations first: this lane's units of its k-blocks (dead columns
    // read the last live row; their results are never stored)
    const int8_t *brow = a.table + (int64_t)(t0 + min(col, nt - 1)) * a.kq;
    uint4 b[NKW][SPK];
#pragma unroll
    for (int i = 0; i < NKW; ++i) {
        const int kb = min(kw0 + i, nkb - 1);
#pragma unroll
        for (int st = 0; st < SPK; ++st) b[i][st] = gload16(brow + 16 * (4 * (kb * SPK + st) + q));
    }
    // then every weight load of this wave (clamped copies past the end)
    // a chunk past the end of a row shorter than 64 bytes is read at the
    // row's last chunk (it meets zero activations)
    const uint32_t coff = (uint32_t)min(16 * lchunk, (int)(a.rb - 16));
    const uint32_t roff = (uint32_t)(min(row0 + lrow, a.O - 1) * a.rb) + coff;
    const uint32_t last_seg = (uint32_t)(a.rb - 16) - coff;
    uint4 w[NKW][2];
#pragma unroll
    for (int i = 0; i < NKW; ++i) {
        const uint32_t b0 = (uint32_t)min(kw0 + i, nkb - 1) * kbytes;
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) w[i][sg] = gload16(a.W + (roff + min(b0 + 64 * sg, last_seg)));
    }
    // the finishing wave's scales and row factors
    float scp[4] = {1.f, 1.f, 1.f, 1.f};
    if (wave == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) scp[r] = a.scale[min(row0 + 4 * q + r, a.O - 1)];
    }

    int4v acc = int4v{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < NKW; ++i) {
        if (kw0 + i >= nkb) break;                         // uniform
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
            const uint4 u = w[i][sg];
            w[i][sg] = make_uint4((uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)u.x),
                                  (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)u.y),
                                  (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)u.z),
                                  (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)u.w));
        }
#pragma unroll
        for (int st = 0; st < SPK; ++st) {
            const int4v A = icodes<FMT>(w[i][st / (SPK / 2)], st % (SPK / 2));
            const int4v B = int4v{(int)b[i][st].x, (int)b[i][st].y, (int)b[i][st].z, (int)b[i][st].w};
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, acc, 0, 0, 0);
        }
    }
    red[wave * kWave + lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    int4v v = red[lane];
#pragma unroll
    for (int ww = 1; ww < kIdWaves; ++ww) v += red[ww * kWave + lane];
    // D[4q + r][col]: weight row row0 + 4 q + r, activation row t0 + col
    if (col >= nt) return;
    const int tok = t0 + col;
    int sqt = 0;
    if constexpr (FMT == kI4) {
#pragma unroll
        for (int p = 0; p < kQMaxParts; ++p) sqt += a.sq[(int64_t)tok * kQMaxParts + p];
    }
    const int corr = 8 * sqt;
    const float srow = a.sx[tok];
    const int ob = row0 + 4 * q;
    float res[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float d = (float)(v[r] - corr);
        res[r] = (d * scp[r]) * srow;
    }
    float *yp = a.y + (int64_t)tok * a.O;
    if (a.y_vec4 && ob + 3 < a.O) {
        *reinterpret_cast<float4 *>(yp + ob) = make_float4(res[0], res[1], res[2], res[3]);
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (ob + r < a.O) yp[ob + r] = res[r];
    }
}

// ---------------------------------------------------------------- experts
// Integer-dot grouped expert products for prefill batches: the items,
// classes (passes sorted by live 16-row N-tiles), pass-major XCD order and
// pipeline of the bf16 prefill kernel on tiled weights -- each wave 32
// (gate/up) or 64 (down) weight rows x the pass's live rows; per k-block the
// pass rows' int8 units are staged into LDS by direct-to-LDS loads (double
// buffered), and the weights of k-block j + 2 are loaded into k-block j's
// registers as each segment is consumed -- but the products are exact int32
// dots on v_mfma_i32_16x16x64_i8, and the epilogue is the pages' fp32 one.
// The tiled weight unit (16 rows x 64 bytes, lane 16 q + c = row c, bytes
// 16 q..16 q + 15) is the A operand's layout as it is.
__global__ void k_idrows(const int32_t *__restrict__ row_pair, int P, int K, int S, int rows,
                         const float *__restrict__ sx, const int *__restrict__ sq,
                         int32_t *__restrict__ act_row, float *__restrict__ row_sx,
                         int *__restrict__ row_sq)
{
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    int t = r;
    if (row_pair) {
        t = r < P ? row_pair[r] / K : r - P;
        if (t < 0 || t >= S) t = 0;   // rows past the grouped slots (never read)
        act_row[r] = t;
    }
    row_sx[r] = sx[t];
    int v = 0;
#pragma unroll
    for (int p = 0; p < kQMaxParts; ++p) v += sq[(int64_t)t * kQMaxParts + p];
    row_sq[r] = v;
}

typedef __attribute__((address_space(3))) const void lds_void_i;

__device__ __forceinline__ void dma16_i(const void *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}

constexpr int kPidWaves = 8;
constexpr int kPidXcds = 8;
constexpr int kPidNT = kPreTpp / 16;

template <int FMT, int M>
__global__ __launch_bounds__(64 * kPidWaves) void k_preid(PreIdArgs a)
{
    constexpr int SEGS = 2;                          // 64-byte tiled segments per k-block
    constexpr int SPSI = FMT == kI4 ? 2 : 1;         // i8 MFMA steps per segment
    constexpr int STEPS = SEGS * SPSI;
    constexpr int KB = ID<FMT>::KB;                  // elements per k-block
    static_assert(ID<FMT>::SPK == STEPS, "steps per k-block");
    constexpr int MT = M == 2 ? 2 : 4, NT = kPidNT, RPW = 16 * MT, RPB = kPidWaves * RPW;
    static_assert(RPB == pre_rows_per_item(M), "rows per item");
    constexpr int UNITS = NT * STEPS * 64;           // 16-byte units of one staged k-block
    __shared__ uint4 bsA[UNITS], bsB[UNITS];
    __shared__ int lrow[2][kPreTpp];
    __shared__ float lsx[2][kPreTpp];
    __shared__ int lsq[2][kPreTpp];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, q = lane >> 4;
    const int xcd = blockIdx.x % kPidXcds, lb = blockIdx.x / kPidXcds;
    const int bpx = gridDim.x / kPidXcds;
    const int nkb = (int)(a.kq / KB);                  // a multiple of 4
    const int ns = (int)((a.rb + 63) / 64);
    const uint8_t *actb = reinterpret_cast<const uint8_t *>(a.act);
    const uint32_t arow = (uint32_t)a.kq;
    const int dq = (lane & 3) ^ ((lane >> 3) & 3);
    // VMEM loads of one loadList: the table row (with a row map), the scale,
    // and for int4 the int8 sum (int8 codes need no correction: the compiler
    // drops that load, and the count below must match what is issued)
    const int nlist = (a.act_row ? 2 : 1) + (FMT == kI4 ? 1 : 0);

    auto run = [&](auto nlc, int w0, int w1) {
    constexpr int NL = decltype(nlc)::value;
    const int n_gp = w1 - w0;
    const int gp_lo = w0 + (int)((int64_t)n_gp * xcd / kPidXcds);
    const int gp_cnt = w0 + (int)((int64_t)n_gp * (xcd + 1) / kPidXcds) - gp_lo;
    const int n_items = gp_cnt * a.tiles;
    if (lb >= n_items) return;                       // whole block, before any barrier

    struct It {
        int tile, nt, r0t, Og;
        const uint8_t *wb[M];
        const float *sc[M];
        uint32_t roff[MT];
        uint32_t gstr;
    };
    auto make = [&](It &c, int it) {
        const int gp = __builtin_amdgcn_readfirstlane(gp_lo + it / a.tiles);
        c.tile = __builtin_amdgcn_readfirstlane(it % a.tiles);
        const int wv = cload(a.work + gp);
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
        const int mt16 = (c.Og + 15) / 16;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) c.roff[mt] = tiled_base(min(obase / 16 + mt, mt16 - 1), ns) + 16 * lane;
        c.gstr = tiled_gstride(min(obase / 16, mt16 - 1), mt16);
    };
    // pass rows: table row, scale and (int4) int8 sum (dead rows repeat the
    // last live one); nlist loads
    auto loadList = [&](const It &c, int &ar, float &rs, int &rq) {
        const int gr = c.r0t + min(tid & 63, c.nt - 1);
        ar = a.act_row ? a.act_row[gr] : gr;
        rs = a.row_sx[gr];
        rq = FMT == kI4 ? a.row_sq[gr] : 0;
    };
    auto storeList = [&](int par, int ar, float rs, int rq) {
        if (tid < kPreTpp) {
            lrow[par][tid] = ar;
            lsx[par][tid] = rs;
            lsq[par][tid] = rq;
        }
    };
    auto loadSeg = [&](const It &c, int kbi, int sg, uint4 (&w)[M][MT][SEGS]) {
        const uint32_t go = (uint32_t)min(kbi * SEGS + sg, ns - 1) * c.gstr;
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) w[m][mt][sg] = gload16(c.wb[m] + (c.roff[mt] + go));
    };
    auto loadW = [&](const It &c, int kbi, uint4 (&w)[M][MT][SEGS]) {
#pragma unroll
        for (int sg = 0; sg < SEGS; ++sg) loadSeg(c, kbi, sg, w);
    };
    // Staging: unit (pass row t = 16 n + col, step s, chunk q) at
    // ((n STEPS + s) 16 + col) 4 + (q ^ ((col >> 1) & 3)); instruction
    // i = n STEPS + s fills one (n, s) -- lane L takes row 16 n + L / 4,
    // chunk (L & 3) ^ ((L >> 3) & 3) -- and is issued by wave i % 8.
    constexpr int NI = NL * STEPS, IPW = (NI + kPidWaves - 1) / kPidWaves;
    auto stageB = [&](int par, int kbi, const uint4 *buf) {
        const uint32_t lbuf = (uint32_t)(uintptr_t)(lds_void_i *)buf;
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
            const int i = wave + kPidWaves * j;
            if (NI % kPidWaves == 0 || i < NI) {        // uniform
                const int n = i / STEPS, st = i % STEPS;
                const uint32_t off = (uint32_t)lrow[par][16 * n + (lane >> 2)] * arow +
                                     (uint32_t)(kbi * STEPS + st) * 64u + (uint32_t)dq * 16u;
                dma16_i(actb + off, __builtin_amdgcn_readfirstlane(lbuf + (uint32_t)i * 1024));
            }
        }
    };

    int4v acc[M][MT][NL];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int n = 0; n < NL; ++n) acc[m][mt][n] = int4v{0, 0, 0, 0};

    // the steps of segment sg of one k-block
    auto compute = [&](const uint4 (&w)[M][MT][SEGS], const uint4 *buf, int sg) {
#pragma unroll
        for (int s2 = 0; s2 < STEPS; ++s2) {
            if (s2 / SPSI != sg) continue;
            int4v b[NL];
#pragma unroll
            for (int n = 0; n < NL; ++n) {
                const uint4 u = buf[((n * STEPS + s2) * 16 + col) * 4 + (q ^ ((col >> 1) & 3))];
                b[n] = int4v{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
            }
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const int4v A = icodes<FMT>(w[m][mt][sg], s2 % SPSI);
#pragma unroll
                    for (int n = 0; n < NL; ++n)
                        acc[m][mt][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, b[n], acc[m][mt][n], 0, 0, 0);
                }
        }
    };

    float sreg[M][MT][4];
    auto load_epi = [&](const It &c) {
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
    // pass row 16 n + col.  The pages' epilogue, each step rounded in fp32:
    // ((float)dot * scale) * s_row, dot less 8 * sum(q) for int4 (the codes
    // are nibbles 0..15); gate/up: silu(g) * u.  Stores of the uniform fast
    // path (16-byte stores, the wave's rows inside the matrix): one per live
    // N-tile and row tile, every one issued (each tile has a live row).
    float rsx[NL];
    int rsq[NL];
    constexpr int kStores = NL * MT;
    auto epilogue = [&](const It &c) -> int {
        const int obase = c.tile * RPB + wave * RPW;
        const bool fast = a.out_vec4 && obase + RPW <= c.Og;
#pragma unroll
        for (int n = 0; n < NL; ++n) {
            const int t = 16 * n + col;
            const bool live = t < c.nt;
            const int64_t gr = c.r0t + t;
            const int corr = FMT == kI4 ? 8 * rsq[n] : 0;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int ob = obase + 16 * mt + 4 * q;
                float res[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float y = ((float)(acc[0][mt][n][r] - corr) * sreg[0][mt][r]) * rsx[n];
                    if constexpr (M == 2) {
                        const float u = ((float)(acc[1][mt][n][r] - corr) * sreg[1][mt][r]) * rsx[n];
                        y = silu_f(y) * u;
                    }
                    res[r] = y;
                }
                if (live) {
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
        }
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int n = 0; n < NL; ++n) acc[m][mt][n] = int4v{0, 0, 0, 0};
        return fast ? kStores : 0;
    };

    constexpr int NW = M * MT * SEGS;
    auto wait_vm = [&](auto nc) {
        constexpr int N = decltype(nc)::value;
        static_assert(N < 64, "vmcnt field");
        __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
    };
    // Before k-block j's products: W(j) and DMA(j) must be done; W(j + 1)
    // (NW) and what followed it -- the next item's pass-row loads (nlist)
    // and the last epilogue's stores -- may stay in flight.
    auto sync_x = [&](int after) {
        asm volatile("" ::: "memory");
        if (after == 3 + kStores) wait_vm(std::integral_constant<int, NW + 3 + kStores>{});
        else if (after == 2 + kStores) wait_vm(std::integral_constant<int, NW + 2 + kStores>{});
        else if (after == 1 + kStores) wait_vm(std::integral_constant<int, NW + 1 + kStores>{});
        else if (after == 3) wait_vm(std::integral_constant<int, NW + 3>{});
        else if (after == 2) wait_vm(std::integral_constant<int, NW + 2>{});
        else if (after == 1) wait_vm(std::integral_constant<int, NW + 1>{});
        else wait_vm(std::integral_constant<int, NW>{});
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    It cur;
    make(cur, lb);
    int par = 0;
    {
        int ar, rq;
        float rs;
        loadList(cur, ar, rs, rq);
        storeList(0, ar, rs, rq);
    }
    __syncthreads();
    uint4 wA[M][MT][SEGS], wB[M][MT][SEGS];
    loadW(cur, 0, wA);
    stageB(0, 0, bsA);
    loadW(cur, 1, wB);
    int jn = lb + bpx;
    auto kstep = [&](uint4 (&w)[M][MT][SEGS], const uint4 *buf, int spar, int skb, const uint4 *nbuf,
                     const It &lc, int lkb, bool epi = false, int after = 0) {
        sync_x(after);
        stageB(spar, skb, nbuf);
        if (epi) load_epi(cur);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int sg = 0; sg < SEGS; ++sg) {
            compute(w, buf, sg);
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
        int ar, rq;
        float rs;
        loadList(nxt, ar, rs, rq);
        kstep(wA, bsA, par, 1, bsB, cur, 2, false, nlist + stores);
        storeList(par ^ 1, ar, rs, rq);
        kstep(wB, bsB, par, 2, bsA, cur, 3);
        for (int k = 2; k < nkb - 2; k += 2) {
            kstep(wA, bsA, par, k + 1, bsB, cur, k + 2);
            kstep(wB, bsB, par, k + 2, bsA, cur, k + 3);
        }
        kstep(wA, bsA, par, nkb - 1, bsB, has_nxt ? nxt : cur, has_nxt ? 0 : nkb - 1, true);
#pragma unroll
        for (int n = 0; n < NL; ++n) {
            rsx[n] = lsx[par][min(16 * n + col, cur.nt - 1)];
            rsq[n] = lsq[par][min(16 * n + col, cur.nt - 1)];
        }
        kstep(wB, bsB, par ^ 1, 0, bsA, has_nxt ? nxt : cur, has_nxt ? 1 : nkb - 1);
        stores = epilogue(cur);
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

template <int FMT, int M>
hipError_t launch_preid(const PreIdArgs &a, int64_t items, hipStream_t st)
{
    static int cache[64] = {0};
    const void *kern = (const void *)k_preid<FMT, M>;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cache[dev] <= 0) {
        int cus = 0, per = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, 64 * kPidWaves, 0) != hipSuccess || per <= 0)
            per = 1;
        cache[dev] = cus * per;
    }
    int64_t cap = cache[dev] / kPidXcds * kPidXcds;
    if (cap < kPidXcds) cap = kPidXcds;
    int64_t grid = (items + kPidXcds - 1) / kPidXcds * kPidXcds;
    if (grid > cap) grid = cap;
    if (grid < kPidXcds) grid = kPidXcds;
    const KernelEvents ev = take_kernel_events();   // timed stage: events at the kernel's bounds
    if (ev.start)
        hipExtLaunchKernelGGL((k_preid<FMT, M>), dim3((unsigned)grid), dim3(64 * kPidWaves), 0, st, ev.start,
                              ev.stop, 0, a);
    else
        hipLaunchKernelGGL((k_preid<FMT, M>), dim3((unsigned)grid), dim3(64 * kPidWaves), 0, st, a);
    return hipGetLastError();
}

template <int FMT, int NKW>
hipError_t launch_idot(const IdotArgs &a, hipStream_t st)
{
    const int ntiles = (a.O + 15) / 16;
    const int passes = (a.S + kIdTpp - 1) / kIdTpp;
    const int64_t grid = (int64_t)(ntiles + 7) / 8 * 8 * passes;
    if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_idot<FMT, NKW>), dim3((unsigned)grid), dim3(64 * kIdWaves), 0, st, a, passes, ntiles);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_idot_nkw(const IdotArgs &a, int nkw, hipStream_t st)
{
    switch (nkw) {
    case 1: return launch_idot<FMT, 1>(a, st);
    case 2: return launch_idot<FMT, 2>(a, st);
    case 3: return launch_idot<FMT, 3>(a, st);
    case 4: return launch_idot<FMT, 4>(a, st);
    case 5: return launch_idot<FMT, 5>(a, st);
    case 6: return launch_idot<FMT, 6>(a, st);
    case 7: return launch_idot<FMT, 7>(a, st);
    case 8: return launch_idot<FMT, 8>(a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int64_t idot_workspace_bytes(int S, int I)
{
    if (S < 0 || I < 1) return 0;
    const int64_t t = (int64_t)S * idot_row_bytes(I);
    return (t + 255) / 256 * 256 + (int64_t)S * 4 * (1 + kQMaxParts) + 256;
}

int idot_max_kblocks_per_wave() { return kIdMaxNkw; }
int idot_kblock(int fmt) { return fmt == kI8 ? ID<kI8>::KB : ID<kI4>::KB; }

hipError_t qrow_launch(int fmt, const float *x, int rows, int I, int64_t kq, int8_t *table, float *sx,
                       int *sq, hipStream_t st)
{
    if (rows <= 0) return hipSuccess;
    if (kq < I || kq % 256 || kq > (int64_t)kQPart * kQMaxParts || (fmt != kI8 && fmt != kI4))
        return hipErrorInvalidValue;
    const int vec = I % 4 == 0 && ((uintptr_t)x & 15u) == 0;
    const dim3 qg((unsigned)rows, kQMaxParts);
    if (fmt == kI8)
        hipLaunchKernelGGL(k_qrow<kI8>, qg, dim3(256), 0, st, x, I, kq, vec, table, sx, sq);
    else
        hipLaunchKernelGGL(k_qrow<kI4>, qg, dim3(256), 0, st, x, I, kq, vec, table, sx, sq);
    return hipGetLastError();
}

hipError_t idrows_launch(const int32_t *row_pair, int P, int K, int S, int rows, const float *sx,
                         const int *sq, int32_t *act_row, float *row_sx, int *row_sq, hipStream_t st)
{
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_idrows, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, row_pair, P, K, S, rows,
                       sx, sq, act_row, row_sx, row_sq);
    return hipGetLastError();
}

hipError_t preid_launch(PreIdArgs a, int fmt, int M, int64_t max_group_passes, hipStream_t st)
{
    if (fmt != kI8 && fmt != kI4) return hipErrorInvalidValue;
    if (a.kq % idot_kblock(fmt) || (a.kq / idot_kblock(fmt)) % 4 || a.kq < 4 * idot_kblock(fmt))
        return hipErrorInvalidValue;
    int Ocover = a.O;
    if (a.has_extra && a.xO > Ocover) Ocover = a.xO;
    a.tiles = (Ocover + pre_rows_per_item(M) - 1) / pre_rows_per_item(M);
    const int64_t items = max_group_passes * a.tiles;
    if (M == 2) return fmt == kI8 ? launch_preid<kI8, 2>(a, items, st) : launch_preid<kI4, 2>(a, items, st);
    return fmt == kI8 ? launch_preid<kI8, 1>(a, items, st) : launch_preid<kI4, 1>(a, items, st);
}

hipError_t idot_launch(IdotArgs a, int fmt, hipStream_t st)
{
    if (a.S <= 0 || a.O <= 0) return hipSuccess;
    if (fmt != kI8 && fmt != kI4) return hipErrorInvalidValue;
    const int KB = idot_kblock(fmt);
    a.nkb = (a.I + KB - 1) / KB;
    const int nkw = (a.nkb + kIdWaves - 1) / kIdWaves;
    if (nkw > kIdMaxNkw) return hipErrorInvalidValue;
    a.kq = idot_row_bytes(a.I);
    a.y_vec4 = a.O % 4 == 0 && ((uintptr_t)a.y & 15u) == 0;
    const int vec = a.I % 4 == 0 && ((uintptr_t)a.x & 15u) == 0;
    // all kQMaxParts parts run (a part past kq writes a zero partial sum)
    if (a.kq > (int64_t)kQPart * kQMaxParts) return hipErrorInvalidValue;
    const dim3 qg((unsigned)a.S, kQMaxParts);
    if (fmt == kI8)
        hipLaunchKernelGGL(k_qrow<kI8>, qg, dim3(256), 0, st, a.x, a.I, a.kq, vec, a.table, a.sx, a.sq);
    else
        hipLaunchKernelGGL(k_qrow<kI4>, qg, dim3(256), 0, st, a.x, a.I, a.kq, vec, a.table, a.sx, a.sq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return fmt == kI8 ? launch_idot_nkw<kI8>(a, nkw, st) : launch_idot_nkw<kI4>(a, nkw, st);
}

}  // namespace coli
