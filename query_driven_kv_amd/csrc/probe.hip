// probe.hip - a calibration kernel, not part of the method: one launch that
// reads `read_bytes` and writes `write_bytes` as fast as the part allows, so a
// benchmark can state the single-launch ceiling for a path's byte counts
// (a launch of ~100 MB cannot reach the sustained bandwidth of a long stream:
// the launch ramp and the drain of the last workgroups weigh on it).
//
// 2048 workgroups of 512 threads; workgroup w reads the w-th of 2048
// contiguous slices of the source with 16-byte non-temporal buffer loads,
// eight in flight per thread, and writes the w-th slice of the destination
// with 16-byte non-temporal stores of values that depend on what it read (so
// no load can be dropped).  Of a sweep over 256-2048 workgroups of 256-1024
// threads with 4-16 loads in flight, issued in batches or two batches
// overlapped, this shape was within 1.6 % of the fastest at both 100 MB
// (15.6 us) and 400 MB (59.2 us against 58.3): more workgroups than the
// compute units hold at once let the dispatcher even out the last ones.
#include "think_common.h"

namespace thinkkv {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeWgs = 2048;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void k_probe_stream(const char* __restrict__ src,
                                                                size_t rd_per_wg, size_t rd_total,
                                                                char* __restrict__ dst,
                                                                size_t wr_per_wg, size_t wr_total) {
    const int tid = threadIdx.x;
    const size_t r0 = (size_t)blockIdx.x * rd_per_wg;
    const size_t r1 = r0 + rd_per_wg < rd_total ? r0 + rd_per_wg : rd_total;
    uint32_t acc = 0;
    if (r0 < r1) {
        // the slice through one descriptor (slices stay below 4 GiB)
        const auto rs = make_rsrc(src + r0, (uint32_t)(r1 - r0));
        const uint32_t n = (uint32_t)(r1 - r0);
        for (uint32_t base = 0; base < n; base += 16u * kProbeThreads * kProbeUnroll) {
            u32x4_t v[kProbeUnroll];
#pragma unroll
            for (int u = 0; u < kProbeUnroll; ++u)
                v[u] = __builtin_amdgcn_raw_buffer_load_b128(
                        rs, (int)(base + 16u * (tid + u * kProbeThreads)), 0, kNonTemporal);
#pragma unroll
            for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
    }
    const size_t w0 = (size_t)blockIdx.x * wr_per_wg;
    const size_t w1 = w0 + wr_per_wg < wr_total ? w0 + wr_per_wg : wr_total;
    if (w0 < w1) {
        const auto ws = make_rsrc(dst + w0, (uint32_t)(w1 - w0));
        const uint32_t n = (uint32_t)(w1 - w0);
        const u32x4_t x = {acc, acc + 1u, acc + 2u, acc + 3u};
        for (uint32_t o = 16u * tid; o < n; o += 16u * kProbeThreads)
            __builtin_amdgcn_raw_buffer_store_b128(x, ws, (int)o, 0, kNonTemporal);
    }
}

}  // namespace

hipError_t launch_probe_stream(const void* src, size_t read_bytes, void* dst, size_t write_bytes,
                               hipStream_t s) {
    // slices of whole 16-byte vectors that together cover the byte counts
    const size_t rd = ((read_bytes + kProbeWgs - 1) / kProbeWgs + 15) / 16 * 16;
    const size_t wr = ((write_bytes + kProbeWgs - 1) / kProbeWgs + 15) / 16 * 16;
    k_probe_stream<<<kProbeWgs, kProbeThreads, 0, s>>>(static_cast<const char*>(src), rd,
                                                       read_bytes, static_cast<char*>(dst), wr,
                                                       write_bytes);
    return hipGetLastError();
}

}  // namespace thinkkv
