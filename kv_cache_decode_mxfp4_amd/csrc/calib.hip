// Streaming-read calibration kernel: the fastest plain read of a buffer that
// the GPU sustains, the ceiling the indexer scan's bandwidth is compared with
// (the scan streams 72 bytes per cache entry once, so its bound is HBM
// bandwidth, of which a plain read is the practical maximum).
//
// Each workgroup reads one contiguous slice of the buffer with 16-byte
// non-temporal buffer loads, `depth` loads per lane in flight per round; the
// data are folded into a checksum that is stored (to sink[workgroup]) only if
// it equals one fixed 32-bit value, so the reads cannot be optimised away and
// the kernel in practice writes nothing: its time is its reads.  Loads past the slice end read zero (buffer range check).
#include "device_common.h"
#include "launch.h"

namespace csa2 {
namespace {

constexpr int kThreads = 256;
constexpr int kBufferConfig = 0x00020000;  // raw (untyped) buffer, 32-bit data
constexpr int kNonTemporal = 2;

template <int kDepth>
__global__ void __launch_bounds__(kThreads)
stream_read_kernel(const uint8_t* __restrict__ src, int64_t bytes, int64_t slice,
                   uint32_t* __restrict__ sink)
{
    const int64_t s = (int64_t)blockIdx.x * slice;
    const int64_t e = s + slice < bytes ? s + slice : bytes;
    if (s >= e)
        return;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(src + s), 0, (int32_t)(e - s), kBufferConfig);
    uint32_t acc = 0;
    constexpr int kRound = kThreads * kDepth * 16;  // bytes per round
    for (int64_t off = 0; off < e - s; off += kRound) {
        u32x4 v[kDepth];
#pragma unroll
        for (int j = 0; j < kDepth; ++j)
            v[j] = __builtin_amdgcn_raw_buffer_load_b128(
                r, (int32_t)(off + (j * kThreads + threadIdx.x) * 16), 0, kNonTemporal);
#pragma unroll
        for (int j = 0; j < kDepth; ++j)
            acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    }
    if (acc == 0x9E3779B9u)
        sink[blockIdx.x] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, int32_t workgroups, int32_t depth,
                              uint32_t* sink, hipStream_t stream)
{
    if (bytes == 0)
        return hipSuccess;
    if (!grid_fits(workgroups, kThreads))
        return hipErrorInvalidConfiguration;
    // slices of whole 16-byte units
    const int64_t slice = ((bytes + workgroups - 1) / workgroups + 15) / 16 * 16;
    const dim3 grid((uint32_t)workgroups), block(kThreads);
    const uint8_t* p = static_cast<const uint8_t*>(src);
    switch (depth) {
    case 1: stream_read_kernel<1><<<grid, block, 0, stream>>>(p, bytes, slice, sink); break;
    case 2: stream_read_kernel<2><<<grid, block, 0, stream>>>(p, bytes, slice, sink); break;
    case 4: stream_read_kernel<4><<<grid, block, 0, stream>>>(p, bytes, slice, sink); break;
    default: stream_read_kernel<8><<<grid, block, 0, stream>>>(p, bytes, slice, sink); break;
    }
    return hipGetLastError();
}

}  // namespace csa2
