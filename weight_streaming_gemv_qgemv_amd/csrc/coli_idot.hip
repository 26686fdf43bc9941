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
#include "coli_device.h"
#include "coli_frag.h"
#include "coli_idot.h"

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
