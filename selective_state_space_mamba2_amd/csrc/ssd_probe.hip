// ssd_probe.hip -- HBM streaming probe: the read/write rate the device sustains for a given
// mix of read and written bytes.  A measurement aid for the benchmark (the ceiling an
// HBM-bound kernel with that byte mix could reach), not a step of the scan.
//
// Each workgroup is a reader or a writer, fixed once per workgroup: R of the nb workgroups
// read (R / nb as close to the requested read share as nb allows) and they are spread
// evenly over the grid, so readers and writers run side by side through the whole launch.
// In the contiguous form reader j streams its 1/R share of the source and writer i its
// 1/(nb - R) share of the destination; in the strided form the readers (writers) walk the
// source (destination) together, 256 items per workgroup and step.  Items are 16 bytes,
// four per thread per pass.  Writes are non-temporal (they stream past the caches, as
// checkpoint and output writes do) or plain.  The loaded values feed a sum that is written
// only if it equals a value no finite input produces, so the loads cannot be dropped.
#include <cstdint>

#include "ssd_params.h"
#include "ssd_probe.h"

namespace ssd {

constexpr int kProbeThreads = 256, kProbeUnroll = 4;

template <bool kStride, bool kNt>
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
  // items base + u * gap (u < kProbeUnroll) for base = first, first + step, ... below end
  const int64_t gap = kStride ? int64_t(parts) * kProbeThreads : kProbeThreads;
  const int64_t step = gap * kProbeUnroll;
  const int64_t first = kStride ? int64_t(j) * kProbeThreads : total * j / parts;
  const int64_t end = kStride ? total : total * (j + 1) / parts;
  float acc = 0.f;
  if (reader) {
    for (int64_t base = first + threadIdx.x; base < end; base += step) {
      float4_v v[kProbeUnroll];
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) {
        const int64_t i = base + u * gap;
        v[u] = i < end ? src[i] : float4_v{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) acc += v[u].x + v[u].y + v[u].z + v[u].w;
    }
  } else {
    const float4_v v = float4_v{1.f, 2.f, 3.f, float(b)};
    for (int64_t base = first + threadIdx.x; base < end; base += step) {
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) {
        const int64_t i = base + u * gap;
        if (i < end) {
          if (kNt) __builtin_nontemporal_store(v, dst + i);
          else dst[i] = v;
        }
      }
    }
  }
  if (acc == -1.2345678e-30f) sink[0] = acc;
}

template <bool kStride, bool kNt>
static void launch_probe(int nb, hipStream_t s, const float4_v* src, int64_t nr, float4_v* dst,
                         int64_t nw, int readers, float* sink) {
  hipLaunchKernelGGL((k_probe_stream<kStride, kNt>), dim3(nb), dim3(kProbeThreads), 0, s, src, nr,
                     dst, nw, readers, sink);
}

}  // namespace ssd

extern "C" ssd_status ssd_probe_stream(const void* src, size_t read_bytes, void* dst,
                                       size_t write_bytes, float* sink, int32_t variant,
                                       ssd_stream_t stream) {
  if ((read_bytes && !src) || (write_bytes && !dst) || !sink) return SSD_ERR_NULL_POINTER;
  if (read_bytes % 16 || write_bytes % 16 || variant < 0 || variant > 11) return SSD_ERR_BAD_SHAPE;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16)
    return SSD_ERR_UNSUPPORTED;
  const int64_t nr = int64_t(read_bytes / 16), nw = int64_t(write_bytes / 16);
  if (nr == 0 && nw == 0) return SSD_OK;
  if (nr > (int64_t(1) << 31) || nw > (int64_t(1) << 31)) return SSD_ERR_BAD_SHAPE;
  // readers in proportion to the read share; at least one of each role that has bytes
  const int nb = 2048 << (variant >> 2);
  int readers = int((nr * nb + (nr + nw) / 2) / (nr + nw));
  if (nr > 0 && readers < 1) readers = 1;
  if (nw > 0 && readers > nb - 1) readers = nb - 1;
  if (nr == 0) readers = 0;
  if (nw == 0) readers = nb;
  const auto* s4 = static_cast<const ssd::float4_v*>(src);
  auto* d4 = static_cast<ssd::float4_v*>(dst);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  switch (variant & 3) {
    case 0: ssd::launch_probe<false, true>(nb, s, s4, nr, d4, nw, readers, sink); break;
    case 1: ssd::launch_probe<false, false>(nb, s, s4, nr, d4, nw, readers, sink); break;
    case 2: ssd::launch_probe<true, true>(nb, s, s4, nr, d4, nw, readers, sink); break;
    default: ssd::launch_probe<true, false>(nb, s, s4, nr, d4, nw, readers, sink); break;
  }
  return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}
