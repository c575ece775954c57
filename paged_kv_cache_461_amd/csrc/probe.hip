// probe.hip -- HBM read-ceiling probe: the bandwidth this GPU delivers for reads of 4 KiB tiles
// in a caller-given order (a random order mimics the scattered physical blocks of a paged KV
// pool).  It is a measurement helper beside the attention path, not part of it.
//
// Each wave reads two whole tiles per iteration (8 nontemporal loads of 16 bytes per lane,
// each one contiguous 1 KiB, as the decode kernel's K/V stream does), grid-striding over the
// order list; the XOR of everything read goes to
// `sink` only in an impossible case, so the loads cannot be removed.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace {

constexpr int kProbeTile = 4096;

__global__ __launch_bounds__(256) void tile_read_kernel(const unsigned char* __restrict__ buf, int64_t buf_tiles,
                                                        int64_t ntiles, const int32_t* __restrict__ order,
                                                        uint32_t* sink)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = __builtin_amdgcn_readfirstlane((int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6));
    const int64_t nwaves = (int64_t)gridDim.x * blockDim.x / 64;
    uint32_t acc = 0;
    for (int64_t t = wave * 2; t < ntiles; t += nwaves * 2) {
        uint4 v[2][4];
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int64_t tt = min(t + u, ntiles - 1);
            int64_t o = order[tt];
            o = o < 0 || o >= buf_tiles ? 0 : o;  // an order entry outside the buffer reads tile 0
            const unsigned char* p = buf + o * kProbeTile + lane * 16;
#pragma unroll
            for (int c = 0; c < 4; c++) v[u][c] = load16_stream(p + c * 1024);
        }
#pragma unroll
        for (int u = 0; u < 2; u++)
#pragma unroll
            for (int c = 0; c < 4; c++) acc ^= v[u][c].x ^ v[u][c].y ^ v[u][c].z ^ v[u][c].w;
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

hipError_t launch_tile_read(const void* buf, int64_t buf_tiles, int64_t ntiles, const int32_t* order, int grid,
                            uint32_t* sink, hipStream_t stream)
{
    hipLaunchKernelGGL(tile_read_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       static_cast<const unsigned char*>(buf), buf_tiles, ntiles, order, sink);
    return hipGetLastError();
}

}  // namespace pa
