// coli_tiled.hip -- coli_pack_tiled: the tiled copy of stacked weight
// matrices that the matrix-core expert kernels read with contiguous 1 KB
// loads per wave.  The values are the pages' packed rows unchanged
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
