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
// EPL: elements in a lane's 16-byte weight load; STEPS: MFMA k-steps (8
// elements each) it feeds; KB: elements per k-block (4 lane groups);
// GRP: size of the element group whose order the unpacking permutes;
// OFF: code - value.
template <> struct MF<kI8> { static constexpr int EPL = 16, STEPS = 2, KB = 64, GRP = 1; static constexpr float OFF = 128.f; };
template <> struct MF<kI4> { static constexpr int EPL = 32, STEPS = 4, KB = 128, GRP = 8; static constexpr float OFF = 136.f; };
template <> struct MF<kI2> { static constexpr int EPL = 64, STEPS = 8, KB = 256, GRP = 16; static constexpr float OFF = 130.f; };

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

// Slot of element e inside its group for the weights' unpacking order.
template <int FMT> __device__ __forceinline__ int slot_of(int e)
{
    if constexpr (FMT == kI4) { const int r = e & 7; return (e & ~7) + 2 * (r & 3) + (r >> 2); }
    if constexpr (FMT == kI2) { const int r = e & 15; return (e & ~15) + 2 * (r & 7) + (r >> 3); }
    return e;
}

__device__ __forceinline__ floatx4 mfma(const uint4 &a, const uint4 &b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- x prep
// One block per activation row: hi/lo bf16 planes in the weights' slot
// order, zero past I up to ld, and sum(hi + lo) in a fixed order.
template <int FMT>
__global__ __launch_bounds__(256) void k_xprep(const float *__restrict__ x, int64_t ldx, int I,
                                               int ld, uint16_t *__restrict__ xq,
                                               float *__restrict__ xsum)
{
    __shared__ float red[4];
    const int row = blockIdx.x;
    const float *xr = x + (int64_t)row * ldx;
    uint16_t *hi = xq + (int64_t)row * 2 * ld;
    uint16_t *lo = hi + ld;
    float acc = 0.f;
    for (int e = threadIdx.x; e < ld; e += blockDim.x) {
        const float v = e < I ? xr[e] : 0.f;
        const uint16_t h = bf16_rne(v);
        const uint16_t l = bf16_rne(v - bf16_f(h));
        const int p = slot_of<FMT>(e);
        hi[p] = h;
        lo[p] = l;
        acc += bf16_f(h) + bf16_f(l);
    }
    acc = wave_sum(acc);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) xsum[row] = (red[0] + red[1]) + (red[2] + red[3]);
}

// ---------------------------------------------------------------- main kernel
template <int FMT, int M>
__global__ __launch_bounds__(256) void k_mm(MmArgs a)
{
    using T = MF<FMT>;
    constexpr int EPL = T::EPL, STEPS = T::STEPS, KB = T::KB;
    constexpr float OFF = T::OFF;
    constexpr int BITS = FMT == kI8 ? 8 : FMT == kI4 ? 4 : 2;
    __shared__ float red[4][8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, q = lane >> 4;
    const int xcd = blockIdx.x % kXcds, lb = blockIdx.x / kXcds;
    const int bpx = gridDim.x / kXcds;                 // blocks per XCD (grid is a multiple of 8)
    const int n_gp = a.work ? *a.n_work : (a.x_rows + 7) / 8;
    const int gp_per_xcd = (n_gp + kXcds - 1 - xcd) / kXcds;   // group-passes gp = xcd + 8 i
    const int n_items = gp_per_xcd * a.tiles;
    const int Iblk = (a.I + KB - 1) / KB * KB;

    for (int it = lb; it < n_items; it += bpx) {
        const int gp = xcd + kXcds * (it / a.tiles);
        const int tile = it % a.tiles;
        int g, pass;
        if (a.work) {
            const int wv = a.work[gp];
            g = wv & 0x7FF;
            pass = wv >> 11;
        } else {
            g = 0;
            pass = gp;
        }
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
                SC[m] = a.s[m] + (int64_t)g * a.s_gstride;
            }
        }
        const int t0 = pass * 8;
        const int nt = min(8, cnt - t0);
        // activation row of this lane's column (token t0 + col/2), -1 if dead
        const int tcol = col >> 1;
        int arow = -1;
        if (tcol < nt) {
            const int tok = t0 + tcol;
            if (!a.xrow_token) arow = r0 + tok;
            else if (extra) arow = tok;
            else arow = a.row_pair[r0 + tok] / a.K;
        }
        const uint16_t *xp = arow >= 0 ? a.xq + ((int64_t)arow * 2 + (col & 1)) * a.xld : nullptr;
        const int obase = tile * kRowsPerBlock + wave * kRowsPerWave;
        const int orow0 = obase + col, orow1 = obase + 16 + col;   // A rows of this lane
        const uint8_t *wr[M][2];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            wr[m][0] = orow0 < Og ? W[m] + (int64_t)orow0 * a.rb : nullptr;
            wr[m][1] = orow1 < Og ? W[m] + (int64_t)orow1 * a.rb : nullptr;
        }
        floatx4 acc[M][2];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            acc[m][0] = floatx4{0.f, 0.f, 0.f, 0.f};
            acc[m][1] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
        for (int kb = 0; kb < Iblk; kb += KB) {
            const int64_t boff = (int64_t)kb * BITS / 8 + 16 * q;
            const bool segok = boff < a.rb;
            uint4 wv[M][2];
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    wv[m][mt] = (wr[m][mt] && segok)
                                    ? *reinterpret_cast<const uint4 *>(wr[m][mt] + boff)
                                    : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                const uint4 xb = xp ? *reinterpret_cast<const uint4 *>(xp + kb + EPL * q + 8 * s)
                                    : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
                        acc[m][mt] = mfma(codes<FMT>(wv[m][mt], s), xb, acc[m][mt]);
            }
        }
        // ---- epilogue: D[4q + r][col]; add the lo column to the hi column
        float xs_t = 0.f;
        if (arow >= 0) {
            for (int p = 0; p < a.xsum_parts; ++p) xs_t += a.xsum[(int64_t)p * a.xsum_stride + arow];
        }
        float hpart = 0.f;   // partial sum of this lane's outputs (M == 2)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            float v[M][4];
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) v[m][r] = acc[m][mt][r] + __shfl_xor(acc[m][mt][r], 1, kWave);
            const bool writer = (col & 1) == 0 && tcol < nt;
            const int ob = obase + 16 * mt + 4 * q;
            float res[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = ob + r;
                float y = 0.f;
                if (o < Og) {
                    y = SC[0][o] * (v[0][r] - OFF * xs_t);
                    if constexpr (M == 2) {
                        const float u = SC[1][o] * (v[1][r] - OFF * xs_t);
                        y = silu_f(y) * u;
                    }
                }
                res[r] = y;
            }
            if (writer) {
                const int64_t orow = (int64_t)(r0 + t0 + tcol);
                float *op = a.out + orow * a.ldo;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (ob + r < Og) op[ob + r] = res[r];
                if constexpr (M == 2) {
                    if (a.hq) {
                        uint16_t *hh = a.hq + orow * 2 * a.hq_ld;
                        uint16_t *hl = hh + a.hq_ld;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int o = ob + r;
                            if (o < a.hq_rows) {
                                const uint16_t h = bf16_rne(res[r]);
                                const uint16_t l = bf16_rne(res[r] - bf16_f(h));
                                const int p = a.hq_fmt == kI4 ? slot_of<kI4>(o)
                                              : a.hq_fmt == kI2 ? slot_of<kI2>(o) : o;
                                hh[p] = h;
                                hl[p] = l;
                                hpart += bf16_f(h) + bf16_f(l);
                            }
                        }
                    }
                }
            }
        }
        if constexpr (M == 2) {
            if (a.hsum_part) {
                // sum over the 4 lane groups (rows), then over the 4 waves, per token
                hpart += __shfl_xor(hpart, 16, kWave);
                hpart += __shfl_xor(hpart, 32, kWave);
                __syncthreads();   // red[] of the previous item is consumed
                if (q == 0 && (col & 1) == 0) red[wave][col >> 1] = hpart;
                __syncthreads();
                if (tid < 8 && tid < nt)
                    a.hsum_part[(int64_t)tile * a.hsum_stride + r0 + t0 + tid] =
                        (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
            }
        }
    }
}

template <int FMT>
hipError_t launch_fmt(const MmArgs &a, int M, int grid, hipStream_t st)
{
    if (M == 2) hipLaunchKernelGGL((k_mm<FMT, 2>), dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_mm<FMT, 1>), dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace

int mm_kblock(int fmt) { return fmt == kI8 ? 64 : fmt == kI4 ? 128 : 256; }
int mm_rows_per_block() { return kRowsPerBlock; }

hipError_t xprep_launch(int fmt, const float *x, int64_t ldx, int rows, int I, int ld,
                        uint16_t *xq, float *xsum, hipStream_t st)
{
    if (rows <= 0) return hipSuccess;
    switch (fmt) {
    case kI8: hipLaunchKernelGGL(k_xprep<kI8>, dim3(rows), dim3(256), 0, st, x, ldx, I, ld, xq, xsum); break;
    case kI4: hipLaunchKernelGGL(k_xprep<kI4>, dim3(rows), dim3(256), 0, st, x, ldx, I, ld, xq, xsum); break;
    case kI2: hipLaunchKernelGGL(k_xprep<kI2>, dim3(rows), dim3(256), 0, st, x, ldx, I, ld, xq, xsum); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t mm_launch(MmArgs a, int fmt, int M, int64_t max_group_passes, hipStream_t st)
{
    const int Ocover = a.hq && a.hq_rows > a.O ? a.hq_rows : a.O;
    const int Omax = a.has_extra && a.xO > Ocover ? a.xO : Ocover;
    a.tiles = (Omax + kRowsPerBlock - 1) / kRowsPerBlock;
    int64_t items = max_group_passes * a.tiles;
    int64_t grid = (items + kXcds - 1) / kXcds * kXcds;
    const int64_t cap = 256 * 4;   // persistent: four blocks per CU
    if (grid > cap) grid = cap;
    if (grid < kXcds) grid = kXcds;
    switch (fmt) {
    case kI8: return launch_fmt<kI8>(a, M, (int)grid, st);
    case kI4: return launch_fmt<kI4>(a, M, (int)grid, st);
    case kI2: return launch_fmt<kI2>(a, M, (int)grid, st);
    default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------- work list
// One block: passes of 8 rows per group (the extra group has x_rows rows),
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
            np = (cnt + 7) / 8;
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
