// coli_tiled.hip -- coli_pack_tiled: the tiled copy of stacked weight
// matrices that the matrix-core expert kernels read with contiguous 1 KB
// loads per wave; coli_pack_tiled_grouped / coli_pack_scales_grouped: the
// same for int4 with one scale per group of gs elements.  The values are the pages' packed rows unchanged
// [glm.c@98759bf -- typedef QT, pack_int4, pack_int2]; only their order in
// memory changes (unit layout: coli_frag.h, tiled_base / tiled_gstride).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "coli.h"
#include "coli_device.h"
#include "coli_frag.h"
#include "coli_internal.h"

namespace coli {
namespace {

// One thread per 16-byte lane chunk: block (unit column, matrix) with 4 units
// of 64 lanes; unit u = (m, g) in row-tile-major numbering u = m * ns + g.
__global__ __launch_bounds__(256) void k_pack_tiled(const uint8_t *__restrict__ W, int O, int64_t rb,
                                                    int ns, int mt16, int64_t src_mat,
                                                    int64_t dst_mat, uint8_t *__restrict__ dst)
{
    const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (u >= (int64_t)mt16 * ns) return;
    const int lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15;
    const int m = (int)(u / ns), g = (int)(u - (int64_t)m * ns);
    const int64_t mat = blockIdx.y;
    const int row = 16 * m + c;
    const int64_t off = 64 * (int64_t)g + 16 * q;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < O && off < rb)   // rb is a multiple of 16: the chunk is whole
        v = *reinterpret_cast<const uint4 *>(W + mat * src_mat + (int64_t)row * rb + off);
    const int64_t d = mat * dst_mat + (int64_t)tiled_base(m, ns) + (int64_t)g * tiled_gstride(m, mt16) + 16 * lane;
    *reinterpret_cast<uint4 *>(dst + d) = v;
}

// The grouped tiled layout: as k_pack_tiled, but the thread of lane chunk q
// gathers word q of each of the segment's four 16-byte chunks, so that word
// s of chunk q (the matrix cores' step s) holds elements 32 s + 8 q .. + 7.
__global__ __launch_bounds__(256) void k_pack_tiled_grouped(const uint8_t *__restrict__ W, int O, int64_t rb,
                                                            int ns, int mt16, int64_t src_mat,
                                                            int64_t dst_mat, uint8_t *__restrict__ dst)
{
    const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (u >= (int64_t)mt16 * ns) return;
    const int lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15;
    const int m = (int)(u / ns), g = (int)(u - (int64_t)m * ns);
    const int64_t mat = blockIdx.y;
    const int row = 16 * m + c;
    uint32_t v[4] = {0u, 0u, 0u, 0u};
    if (row < O) {
        const uint8_t *src = W + mat * src_mat + (int64_t)row * rb;
        for (int s = 0; s < 4; ++s) {
            const int64_t off = 64 * (int64_t)g + 16 * s;   // chunk s; rb is a multiple of 16
            if (off < rb) v[s] = *reinterpret_cast<const uint32_t *>(src + off + 4 * q);
        }
    }
    const int64_t d = mat * dst_mat + (int64_t)tiled_base(m, ns) + (int64_t)g * tiled_gstride(m, mt16) + 16 * lane;
    *reinterpret_cast<uint4 *>(dst + d) = make_uint4(v[0], v[1], v[2], v[3]);
}

// One thread per (matrix, row tile, group): the 16 rows' scales of the group.
__global__ __launch_bounds__(256) void k_pack_scales_grouped(const float *__restrict__ S, int O, int ng,
                                                             int ngp, int mt16, int64_t total,
                                                             float *__restrict__ dst)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= total) return;
    const int g = (int)(t % ngp);
    const int64_t mr = t / ngp;                 // matrix * mt16 + row tile
    const int m = (int)(mr % mt16);
    const int64_t mat = mr / mt16;
    float v[16];
    for (int r = 0; r < 16; ++r) {
        const int row = 16 * m + r;
        v[r] = (row < O && g < ng) ? S[(mat * O + row) * ng + g] : 0.f;
    }
    float4 *d = reinterpret_cast<float4 *>(dst + t * 16);
    for (int i = 0; i < 4; ++i) d[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

}  // namespace
}  // namespace coli

using namespace coli;

extern "C" int coli_pack_tiled(int fmt, const void *W, int64_t count, int O, int I, void *dst, void *stream)
{
    int rc = coli__check_pack(fmt, W, count, O, I, dst);
    if (rc != COLI_OK) return rc;
    if (count == 0 || O == 0 || I == 0) return COLI_OK;
    const int64_t rb = coli_row_bytes(fmt, I);
    const int ns = (int)((rb + 63) / 64), mt16 = (O + 15) / 16;
    const int64_t units = (int64_t)mt16 * ns;
    if ((units + 3) / 4 > 0x7FFFFFFF || count > 65535) return COLI_ERANGE;
    const int64_t dst_mat = coli_tiled_bytes(fmt, 1, O, I);
    hipLaunchKernelGGL(k_pack_tiled, dim3((unsigned)((units + 3) / 4), (unsigned)count), dim3(256), 0,
                       (hipStream_t)stream, (const uint8_t *)W, O, rb, ns, mt16, rb * O, dst_mat,
                       (uint8_t *)dst);
    return hipGetLastError() == hipSuccess ? COLI_OK : COLI_EDEVICE;
}

extern "C" int coli_pack_tiled_grouped(const void *W, int64_t count, int O, int I, void *dst, void *stream)
{
    int rc = coli__check_pack(COLI_I4, W, count, O, I, dst);
    if (rc != COLI_OK) return rc;
    if (count == 0 || O == 0 || I == 0) return COLI_OK;
    const int64_t rb = coli_row_bytes(COLI_I4, I);
    const int ns = (int)((rb + 63) / 64), mt16 = (O + 15) / 16;
    const int64_t units = (int64_t)mt16 * ns;
    if ((units + 3) / 4 > 0x7FFFFFFF || count > 65535) return COLI_ERANGE;
    const int64_t dst_mat = coli_tiled_bytes(COLI_I4, 1, O, I);
    hipLaunchKernelGGL(k_pack_tiled_grouped, dim3((unsigned)((units + 3) / 4), (unsigned)count), dim3(256), 0,
                       (hipStream_t)stream, (const uint8_t *)W, O, rb, ns, mt16, rb * O, dst_mat,
                       (uint8_t *)dst);
    return hipGetLastError() == hipSuccess ? COLI_OK : COLI_EDEVICE;
}

extern "C" int coli_pack_scales_grouped(const float *S, int64_t count, int O, int I, int gs, float *dst,
                                        void *stream)
{
    int rc = coli__check_pack_scales(S, count, O, I, gs, dst);
    if (rc != COLI_OK) return rc;
    if (count == 0 || O == 0 || I == 0) return COLI_OK;
    const int ng = (I + gs - 1) / gs, ngp = (int)(coli__kpad(I) / gs), mt16 = (O + 15) / 16;
    const int64_t total = count * mt16 * (int64_t)ngp;
    if ((total + 255) / 256 > 0x7FFFFFFF) return COLI_ERANGE;
    hipLaunchKernelGGL(k_pack_scales_grouped, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, S, O, ng, ngp, mt16, total, dst);
    return hipGetLastError() == hipSuccess ? COLI_OK : COLI_EDEVICE;
}
