// ssd_probe.hip -- HBM streaming probe: the read/write rate the device sustains for a given
// mix of read and written bytes.  A measurement aid for the benchmark (the ceiling an
// HBM-bound kernel with that byte mix could reach), not a step of the scan.
//
// Each workgroup is a reader or a writer, fixed once per workgroup: R of the nb workgroups
// read (R / nb as close to the requested read share as nb allows) and they are spread
// evenly over the grid, so readers and writers run side by side through the whole launch.
// Reader j streams its contiguous 1/R share of the source, writer i its 1/(nb - R) share of
// the destination, in 16-byte items, four per thread per pass with no division in the
// loop.  Writes are non-temporal (they stream past the caches, as checkpoint and output
// writes do).  The loaded values feed a sum that is written only if it equals a value no
// finite input produces, so the loads cannot be dropped.
#include <cstdint>

#include "ssd_params.h"
#include "ssd_probe.h"

namespace ssd {

constexpr int kProbeThreads = 256, kProbeUnroll = 4, kProbeBlocks = 2048;

__global__ __launch_bounds__(kProbeThreads) void k_probe_stream(const float4_v* __restrict__ src,
                                                                int64_t nr,
                                                                float4_v* __restrict__ dst,
                                                                int64_t nw, int readers,
                                                                float* sink) {
  const int b = blockIdx.x, nb = gridDim.x;
  // readers are the workgroups where floor(b * R / nb) advances; the readers before b
  // number floor(b * R / nb)
  const int before = int(int64_t(b) * readers / nb);
  const bool reader = int(int64_t(b + 1) * readers / nb) > before;
  const int parts = reader ? readers : nb - readers;
  const int j = reader ? before : b - before;
  const int64_t total = reader ? nr : nw;
  const int64_t lo = total * j / parts, hi = total * (j + 1) / parts;
  constexpr int kStep = kProbeThreads * kProbeUnroll;
  float acc = 0.f;
  if (reader) {
    for (int64_t base = lo + threadIdx.x; base < hi; base += kStep) {
      float4_v v[kProbeUnroll];
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) {
        const int64_t i = base + u * kProbeThreads;
        v[u] = i < hi ? src[i] : float4_v{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) acc += v[u].x + v[u].y + v[u].z + v[u].w;
    }
  } else {
    const float4_v v = float4_v{1.f, 2.f, 3.f, float(b)};
    for (int64_t base = lo + threadIdx.x; base < hi; base += kStep) {
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) {
        const int64_t i = base + u * kProbeThreads;
        if (i < hi) __builtin_nontemporal_store(v, dst + i);
      }
    }
  }
  if (acc == -1.2345678e-30f) sink[0] = acc;
}

}  // namespace ssd

extern "C" ssd_status ssd_probe_stream(const void* src, size_t read_bytes, void* dst,
                                       size_t write_bytes, float* sink, ssd_stream_t stream) {
  if ((read_bytes && !src) || (write_bytes && !dst) || !sink) return SSD_ERR_NULL_POINTER;
  if (read_bytes % 16 || write_bytes % 16) return SSD_ERR_BAD_SHAPE;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16)
    return SSD_ERR_UNSUPPORTED;
  const int64_t nr = int64_t(read_bytes / 16), nw = int64_t(write_bytes / 16);
  if (nr == 0 && nw == 0) return SSD_OK;
  if (nr > (int64_t(1) << 31) || nw > (int64_t(1) << 31)) return SSD_ERR_BAD_SHAPE;
  // readers in proportion to the read share; at least one of each role that has bytes
  const int nb = ssd::kProbeBlocks;
  int readers = int((nr * nb + (nr + nw) / 2) / (nr + nw));
  if (nr > 0 && readers < 1) readers = 1;
  if (nw > 0 && readers > nb - 1) readers = nb - 1;
  if (nr == 0) readers = 0;
  if (nw == 0) readers = nb;
  hipLaunchKernelGGL(ssd::k_probe_stream, dim3(nb), dim3(ssd::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream),
                     static_cast<const ssd::float4_v*>(src), nr, static_cast<ssd::float4_v*>(dst),
                     nw, readers, sink);
  return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}
