// ssd_conv.hip -- the causal depthwise conv1d ahead of the scan ("vLLM Mamba2 SSD kernel
// warm-up", mamba_mixer2.py section: x, B and C are taken after a depthwise convolution;
// conv state shapes from "vLLM v0.20.0 adds disaggregated serving for hybrid SSM models").
//
//   k_conv_prefill  per (chunk, 256-channel block, half of the chunk): four wavefronts
//                   split the half's tokens; a lane owns 4 consecutive channels (8-byte
//                   rows for bf16, 70 VGPRs, seven wavefronts per SIMD), keeps the last W-1
//                   inputs in registers and streams the tokens in straight-line batches of
//                   8 whose loads go out together.  A window reaching before the sequence
//                   start reads the sequence's conv state.
//   k_conv_state    per (sequence, 512 channels): the new conv state (the last W-1
//                   inputs), written after every output kernel read of the old one.
//   k_conv_update   per (decode row, 512 channels): the row's inputs continue its state,
//                   which is replaced in place.
// Streaming work: each is bound by HBM bandwidth (bytes per unit in the header of each
// kernel).  With SiLU an output costs about 18 VALU cycles per lane (4 FMAs, two
// quarter-rate transcendentals, the bf16 conversions), enough to matter: an IEEE divide
// in the sigmoid (about 10 more) made the prefill VALU-bound.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "ssd.h"
#include "ssd_device.h"
#include "ssd_params.h"

namespace ssd {
namespace {

constexpr int kConvW = 4;                              // instantiated kernel width
constexpr int kConvVec = 8;                            // channels per lane (state, update)
constexpr int kConvChan = 64 * kConvVec;               // channels per wavefront (state, update)
constexpr int kPreVec = 4;                             // channels per lane (prefill outputs)
constexpr int kPreChan = 64 * kPreVec;                 // channels per wavefront (prefill)
constexpr int kConvWaves = 4;                          // wavefronts per workgroup
constexpr int kConvSplit = 2;                          // workgroups per (chunk, channel block)
constexpr int kConvBatch = 8;                          // tokens whose loads go out together
constexpr int kConvMaxTokens = 16;                     // decode inputs per row

struct ConvParams {
  int T, D, S;
  const void* x; int64_t x_st;
  void* out; int64_t out_st;
  const float* w;        // [D, W]
  const float* bias;     // [D] or NULL
  int silu;
  const int* cu_seqlens;
  const int* cu_chunk;
  const int* seq_idx;
  void* cs;              // conv state pool or NULL
  int64_t slot_stride;
  int num_slots;
  int layout;            // SSD_CONV_LAYOUT_SD or _DS
  const int* sidx;
  const int* has_init;
  int* flag;
  int ntok, null_id;     // decode
};

// A raw buffer resource over rows of one tensor: a wave-uniform base, a per-lane byte
// offset (the lane's channels, < 1 KB) and a wave-uniform row offset in a scalar register.
struct RowBuf {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ explicit RowBuf(const void* base)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff,
                                            0x00020000)) {}
};

// V consecutive channels (V = 4 or 8) of one row, as fp32: bf16 rows move 2V bytes, fp32
// rows 4V bytes, in 8- or 16-byte pieces.  ld/st take a flat pointer; bld/bst a buffer
// resource, a per-lane byte offset and a wave-uniform byte offset.
template <int V> struct BF16Row;
template <> struct BF16Row<4> {
  using W = u32x2_v;
  static __device__ __forceinline__ W load(const RowBuf& b, uint32_t vo, uint32_t so) {
    return __builtin_amdgcn_raw_buffer_load_b64(b.r, vo, so, 0);
  }
  static __device__ __forceinline__ void store(const RowBuf& b, uint32_t vo, uint32_t so, W w) {
    __builtin_amdgcn_raw_buffer_store_b64(w, b.r, vo, so, 0);
  }
};
template <> struct BF16Row<8> {
  using W = u32x4_v;
  static __device__ __forceinline__ W load(const RowBuf& b, uint32_t vo, uint32_t so) {
    return __builtin_amdgcn_raw_buffer_load_b128(b.r, vo, so, 0);
  }
  static __device__ __forceinline__ void store(const RowBuf& b, uint32_t vo, uint32_t so, W w) {
    __builtin_amdgcn_raw_buffer_store_b128(w, b.r, vo, so, 0);
  }
};

template <typename T, int V> struct RowV;
template <int V> struct RowV<bf16_t, V> {
  using W = typename BF16Row<V>::W;
  static __device__ __forceinline__ void unpack(const W& w, float* v) {
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ W pack(const float* v) {
    W w;
#pragma unroll
    for (int i = 0; i < V / 2; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    return w;
  }
  static __device__ __forceinline__ void ld(const bf16_t* p, float* v) {
    unpack(*reinterpret_cast<const W*>(p), v);
  }
  static __device__ __forceinline__ void st(bf16_t* p, const float* v) {
    *reinterpret_cast<W*>(p) = pack(v);
  }
  static __device__ __forceinline__ void bld(const RowBuf& b, uint32_t vo, uint32_t so, float* v) {
    unpack(BF16Row<V>::load(b, vo, so), v);
  }
  static __device__ __forceinline__ void bst(const RowBuf& b, uint32_t vo, uint32_t so, const float* v) {
    BF16Row<V>::store(b, vo, so, pack(v));
  }
};
template <int V> struct RowV<float, V> {
  static __device__ __forceinline__ void ld(const float* p, float* v) {
#pragma unroll
    for (int q = 0; q < V / 4; ++q) {
      const float4_v a = reinterpret_cast<const float4_v*>(p)[q];
      v[4 * q] = a.x; v[4 * q + 1] = a.y; v[4 * q + 2] = a.z; v[4 * q + 3] = a.w;
    }
  }
  static __device__ __forceinline__ void st(float* p, const float* v) {
#pragma unroll
    for (int q = 0; q < V / 4; ++q)
      reinterpret_cast<float4_v*>(p)[q] = float4_v{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
  }
  static __device__ __forceinline__ void bld(const RowBuf& b, uint32_t vo, uint32_t so, float* v) {
#pragma unroll
    for (int q = 0; q < V / 4; ++q) {
      const u32x4_v w = __builtin_amdgcn_raw_buffer_load_b128(b.r, vo + 16 * q, so, 0);
      v[4 * q] = __uint_as_float(w.x); v[4 * q + 1] = __uint_as_float(w.y);
      v[4 * q + 2] = __uint_as_float(w.z); v[4 * q + 3] = __uint_as_float(w.w);
    }
  }
  static __device__ __forceinline__ void bst(const RowBuf& b, uint32_t vo, uint32_t so, const float* v) {
#pragma unroll
    for (int q = 0; q < V / 4; ++q)
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4_v{__float_as_uint(v[4 * q]), __float_as_uint(v[4 * q + 1]),
                  __float_as_uint(v[4 * q + 2]), __float_as_uint(v[4 * q + 3])},
          b.r, vo + 16 * q, so, 0);
  }
};

// Entry k (0 = oldest input) of channels c0..c0+V-1 of a pool slot, in either layout.
template <typename T, int V>
__device__ __forceinline__ void state_ld(const ConvParams& p, int slot, int k, int c0, float* v) {
  const T* base = static_cast<const T*>(p.cs) + int64_t(slot) * p.slot_stride;
  if (p.layout == SSD_CONV_LAYOUT_SD) {
    RowV<T, V>::ld(base + int64_t(k) * p.D + c0, v);
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = Elem<T>::load(base + int64_t(c0 + i) * (kConvW - 1) + k);
  }
}
template <typename T, int V>
__device__ __forceinline__ void state_st(const ConvParams& p, int slot, int k, int c0, const float* v) {
  T* base = static_cast<T*>(p.cs) + int64_t(slot) * p.slot_stride;
  if (p.layout == SSD_CONV_LAYOUT_SD) {
    RowV<T, V>::st(base + int64_t(k) * p.D + c0, v);
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) Elem<T>::store(base + int64_t(c0 + i) * (kConvW - 1) + k, v[i]);
  }
}

// The lane's filter taps wk[k][i] = weight[c0 + i, k] and biases.
template <int V>
__device__ __forceinline__ void load_taps(const ConvParams& p, int c0, float (&wk)[kConvW][V],
                                          float (&bv)[V]) {
  const float4_v* w4 = reinterpret_cast<const float4_v*>(p.w + int64_t(c0) * kConvW);
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const float4_v t = w4[i];   // weight[c0 + i, 0..3]
    wk[0][i] = t.x; wk[1][i] = t.y; wk[2][i] = t.z; wk[3][i] = t.w;
  }
#pragma unroll
  for (int q = 0; q < V / 4; ++q) {
    const float4_v b4 = p.bias ? reinterpret_cast<const float4_v*>(p.bias + c0)[q]
                               : float4_v{0.f, 0.f, 0.f, 0.f};
    bv[4 * q] = b4.x; bv[4 * q + 1] = b4.y; bv[4 * q + 2] = b4.z; bv[4 * q + 3] = b4.w;
  }
}

// act(bias + sum_k w[k] u[k]) for the window u[0..W-1] (oldest first) of V channels.
// SiLU is v * sigmoid(v) with the sigmoid as the hardware reciprocal of 1 + e^-v (about
// 1 ulp; e^-v = inf for very negative v gives -0, the limit).
template <bool SILU, int V>
__device__ __forceinline__ void conv_out(const float (&wk)[kConvW][V], const float (&bv)[V],
                                         const float (*u)[V], float* o) {
#pragma unroll
  for (int i = 0; i < V; ++i) {
    float v = bv[i];
#pragma unroll
    for (int k = 0; k < kConvW; ++k) v += wk[k][i] * u[k][i];
    if (SILU) v = v * __builtin_amdgcn_rcpf(1.f + fast_exp(-v));
    o[i] = v;
  }
}

// One output row from the window u (oldest first) and the new input xv; then the window
// moves on by one input.
template <int V>
__device__ __forceinline__ void conv_step(const float (&wk)[kConvW][V], const float (&bv)[V],
                                          float (&u)[kConvW - 1][V], const float* xv,
                                          int silu, float* o) {
  float win[kConvW][V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
#pragma unroll
    for (int k = 0; k < kConvW - 1; ++k) win[k][i] = u[k][i];
    win[kConvW - 1][i] = xv[i];
  }
  if (silu) conv_out<true, V>(wk, bv, win, o);
  else conv_out<false, V>(wk, bv, win, o);
#pragma unroll
  for (int i = 0; i < V; ++i) {
#pragma unroll
    for (int k = 0; k < kConvW - 1; ++k) u[k][i] = win[k + 1][i];
  }
}

// ---------------------------------------------------------------------------------------
// k_conv_prefill: per chunk and token, x row in and out row out (2 D b bytes), plus the
// sequence's conv state (3 D b) for the windows reaching before its first token.
// ---------------------------------------------------------------------------------------
template <typename T, bool SILU>
__global__ __launch_bounds__(256) void k_conv_prefill(ConvParams p, int C) {
  const int k = blockIdx.x, cb = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (k >= C) return;
  const int cs0 = p.cu_chunk[k], cs1 = p.cu_chunk[k + 1], r = p.seq_idx[k];
  bool ok = r >= 0 && r < p.S && cs0 >= 0 && cs1 > cs0 && cs1 <= p.T;
  int t0 = 0;
  if (ok) {
    t0 = p.cu_seqlens[r];
    ok = t0 >= 0 && cs0 >= t0 && cs1 <= p.cu_seqlens[r + 1];
  }
  if (!ok) {
    if (threadIdx.x == 0 && cb == 0) raise_flag(p.flag, SSD_DEVERR_CHUNK_RANGE);
    return;
  }
  const int c0 = cb * kPreChan + lane * kPreVec;
  const int parts = kConvWaves * int(gridDim.z), part = int(blockIdx.z) * kConvWaves + wave;
  const int L = cs1 - cs0, per = (L + parts - 1) / parts;
  const int a = cs0 + part * per, b = min(cs1, a + per);
  if (c0 >= p.D || a >= b) return;

  // the sequence's conv state, needed only by windows reaching before t0
  int slot = -1;
  if (a - (kConvW - 1) < t0 && p.cs && p.sidx && p.has_init && p.has_init[r]) {
    slot = p.sidx[r];
    if (slot < 0 || slot >= p.num_slots) {
      if (lane == 0) raise_flag(p.flag, SSD_DEVERR_SLOT_RANGE);
      slot = -1;
    }
  }
  const T* xg = static_cast<const T*>(p.x) + c0;
  // the window: W-1 inputs before the batch, then the batch's inputs
  float win[kConvW - 1 + kConvBatch][kPreVec];
#pragma unroll
  for (int j = 0; j < kConvW - 1; ++j) {
    const int t = a - (kConvW - 1) + j;
    if (t >= t0) {
      RowV<T, kPreVec>::ld(xg + int64_t(t) * p.x_st, win[j]);
    } else if (slot >= 0) {
      state_ld<T, kPreVec>(p, slot, (kConvW - 1) + (t - t0), c0, win[j]);
    } else {
#pragma unroll
      for (int i = 0; i < kPreVec; ++i) win[j][i] = 0.f;
    }
  }
  float wk[kConvW][kPreVec], bv[kPreVec];
  load_taps<kPreVec>(p, c0, wk, bv);

  // straight-line batches over rows t .. t+7 of this wave's range: buffer accesses with the
  // wave's first row as the base, the lane's channels as the vector offset and the row as
  // a scalar offset (the host keeps (T / 8 + 1) rows under 2 GiB).  Rows past b load row
  // b-1 again (in bounds; their outputs are not stored), so no load is predicated and the
  // window is only re-arranged by the slide at the end of a full batch.
  const RowBuf xb(static_cast<const T*>(p.x) + int64_t(a) * p.x_st + cb * kPreChan);
  const RowBuf ob(static_cast<T*>(p.out) + int64_t(a) * p.out_st + cb * kPreChan);
  const uint32_t lane_b = uint32_t(lane * kPreVec * sizeof(T));
  const uint32_t xrow_b = uint32_t(p.x_st * int64_t(sizeof(T)));
  const uint32_t orow_b = uint32_t(p.out_st * int64_t(sizeof(T)));
  for (int t = a; t < b; t += kConvBatch) {
#pragma unroll
    for (int i = 0; i < kConvBatch; ++i) {
      const int row = (t + i < b ? t + i : b - 1) - a;
      RowV<T, kPreVec>::bld(xb, lane_b, uint32_t(row) * xrow_b, win[kConvW - 1 + i]);
    }
#pragma unroll
    for (int i = 0; i < kConvBatch; ++i) {
      float o[kPreVec];
      conv_out<SILU, kPreVec>(wk, bv, &win[i], o);
      if (t + i < b) RowV<T, kPreVec>::bst(ob, lane_b, uint32_t(t + i - a) * orow_b, o);
    }
#pragma unroll
    for (int j = 0; j < kConvW - 1; ++j)
#pragma unroll
      for (int c = 0; c < kPreVec; ++c) win[j][c] = win[kConvBatch + j][c];
  }
}

// ---------------------------------------------------------------------------------------
// k_conv_state: per sequence, 3 D b bytes of new state out (plus the old state or the last
// inputs read back: 3 D b).
// ---------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void k_conv_state(ConvParams p) {
  const int r = blockIdx.x;
  const int c0 = blockIdx.y * kConvChan + threadIdx.x * kConvVec;
  if (c0 >= p.D) return;
  const int t0 = p.cu_seqlens[r], t1 = p.cu_seqlens[r + 1];
  if (t0 < 0 || t1 <= t0 || t1 > p.T) return;   // the output kernel flags such a sequence
  const int slot = p.sidx[r];
  if (slot < 0 || slot >= p.num_slots) {
    if (threadIdx.x == 0 && blockIdx.y == 0) raise_flag(p.flag, SSD_DEVERR_SLOT_RANGE);
    return;
  }
  const bool init = p.has_init && p.has_init[r];
  const int L = t1 - t0;
  const T* xg = static_cast<const T*>(p.x) + c0;
  // entry j of the new state is input L + j of (old state, new inputs): new input
  // q = L - (W-1) + j when q >= 0, else old entry (W-1) + q; every read before any write
  float nv[kConvW - 1][kConvVec];
#pragma unroll
  for (int j = 0; j < kConvW - 1; ++j) {
    const int q = L - (kConvW - 1) + j;
    if (q >= 0) {
      RowV<T, kConvVec>::ld(xg + int64_t(t0 + q) * p.x_st, nv[j]);
    } else if (init) {
      state_ld<T, kConvVec>(p, slot, (kConvW - 1) + q, c0, nv[j]);
    } else {
#pragma unroll
      for (int i = 0; i < kConvVec; ++i) nv[j][i] = 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < kConvW - 1; ++j) state_st<T, kConvVec>(p, slot, j, c0, nv[j]);
}

// ---------------------------------------------------------------------------------------
// k_conv_update: per live row, 3 D b state bytes in and out, ntok D b inputs in and out.
// ---------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void k_conv_update(ConvParams p) {
  const int r = blockIdx.x;
  const int c0 = blockIdx.y * kConvChan + threadIdx.x * kConvVec;
  if (c0 >= p.D) return;
  const int slot = p.sidx[r];
  if (slot == p.null_id) return;   // padding row: nothing read, nothing written
  if (slot < 0 || slot >= p.num_slots) {
    if (threadIdx.x == 0 && blockIdx.y == 0) raise_flag(p.flag, SSD_DEVERR_SLOT_RANGE);
    return;
  }
  float u[kConvW - 1][kConvVec];
#pragma unroll
  for (int j = 0; j < kConvW - 1; ++j) state_ld<T, kConvVec>(p, slot, j, c0, u[j]);
  float wk[kConvW][kConvVec], bv[kConvVec];
  load_taps<kConvVec>(p, c0, wk, bv);
  const T* xg = static_cast<const T*>(p.x) + int64_t(r) * p.ntok * p.D + c0;
  T* og = static_cast<T*>(p.out) + int64_t(r) * p.ntok * p.D + c0;
  for (int j = 0; j < p.ntok; ++j) {
    float xv[kConvVec], o[kConvVec];
    RowV<T, kConvVec>::ld(xg + int64_t(j) * p.D, xv);
    conv_step<kConvVec>(wk, bv, u, xv, p.silu, o);
    RowV<T, kConvVec>::st(og + int64_t(j) * p.D, o);
  }
#pragma unroll
  for (int j = 0; j < kConvW - 1; ++j) state_st<T, kConvVec>(p, slot, j, c0, u[j]);
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }
bool valid_dtype(int32_t d) { return d == SSD_F32 || d == SSD_BF16; }

// Checks shared by both calls: sizes, dtype, activation, layout, the instantiated width,
// 16-byte vector access to rows of 8 channels.
ssd_status check_common(int D, int W, int dtype, int act, int layout) {
  if (D < 1 || W < 2) return SSD_ERR_BAD_SHAPE;
  if (!valid_dtype(dtype) || (act != 0 && act != 1)) return SSD_ERR_BAD_SHAPE;
  if (layout != SSD_CONV_LAYOUT_SD && layout != SSD_CONV_LAYOUT_DS) return SSD_ERR_BAD_SHAPE;
  if (W != kConvW || D % kConvVec != 0) return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

ssd_status check_pool(const void* cs, int64_t slot_stride, int num_slots, int D, int W) {
  if (num_slots < 1 || slot_stride < int64_t(W - 1) * D) return SSD_ERR_BAD_SHAPE;
  if (!aligned16(cs) || slot_stride % kConvVec != 0) return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

}  // namespace
}  // namespace ssd

extern "C" {

ssd_status ssd_conv1d_prefill(const ssd_conv1d_args* a, ssd_stream_t stream) {
  using namespace ssd;
  if (!a) return SSD_ERR_NULL_POINTER;
  if (a->T < 0 || a->num_seqs < 0 || a->num_chunks < 0) return SSD_ERR_BAD_SHAPE;
  ssd_status st = check_common(a->D, a->W, a->in_dtype, a->activation, a->state_layout);
  if (st != SSD_OK) return st;
  if (a->num_seqs == 0) return (a->T != 0 || a->num_chunks != 0) ? SSD_ERR_BAD_SHAPE : SSD_OK;
  if (a->T < a->num_seqs || a->num_chunks < a->num_seqs || a->num_chunks > a->T)
    return SSD_ERR_BAD_SHAPE;
  if (a->x_stride_t < a->D || a->out_stride_t < a->D) return SSD_ERR_BAD_SHAPE;
  if (!a->x || !a->out || !a->weight || !a->cu_seqlens || !a->cu_chunk_seqlens || !a->seq_idx)
    return SSD_ERR_NULL_POINTER;
  if (a->conv_states) {
    if (!a->state_indices) return SSD_ERR_NULL_POINTER;
    st = check_pool(a->conv_states, a->slot_stride, a->num_slots, a->D, a->W);
    if (st != SSD_OK) return st;
  }
  if (!aligned16(a->x) || !aligned16(a->out) || !aligned16(a->weight) ||
      (a->bias && !aligned16(a->bias)) || a->x_stride_t % kConvVec || a->out_stride_t % kConvVec)
    return SSD_ERR_UNSUPPORTED;
  {
    // a wave covers at most ceil(T / 8) rows, addressed as 32-bit offsets from its first row
    const int64_t esz = a->in_dtype == SSD_BF16 ? 2 : 4;
    const int64_t rows = int64_t(a->T) / (kConvWaves * kConvSplit) + 1;
    if (rows * std::max(a->x_stride_t, a->out_stride_t) * esz >= (int64_t(1) << 31))
      return SSD_ERR_UNSUPPORTED;
  }

  ConvParams p{};
  p.T = a->T; p.D = a->D; p.S = a->num_seqs;
  p.x = a->x; p.x_st = a->x_stride_t; p.out = a->out; p.out_st = a->out_stride_t;
  p.w = a->weight; p.bias = a->bias; p.silu = a->activation;
  p.cu_seqlens = a->cu_seqlens; p.cu_chunk = a->cu_chunk_seqlens; p.seq_idx = a->seq_idx;
  p.cs = a->conv_states; p.slot_stride = a->slot_stride; p.num_slots = a->num_slots;
  p.layout = a->state_layout; p.sidx = a->state_indices; p.has_init = a->has_initial_state;
  p.flag = a->device_error_flag;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int nb = (a->D + kConvChan - 1) / kConvChan;
  record_event(a->profile_events, 0, s);
  const dim3 grid(a->num_chunks, (a->D + kPreChan - 1) / kPreChan, kConvSplit), block(64 * kConvWaves);
  if (a->in_dtype == SSD_BF16) {
    if (a->activation) hipLaunchKernelGGL((k_conv_prefill<bf16_t, true>), grid, block, 0, s, p, a->num_chunks);
    else hipLaunchKernelGGL((k_conv_prefill<bf16_t, false>), grid, block, 0, s, p, a->num_chunks);
  } else {
    if (a->activation) hipLaunchKernelGGL((k_conv_prefill<float, true>), grid, block, 0, s, p, a->num_chunks);
    else hipLaunchKernelGGL((k_conv_prefill<float, false>), grid, block, 0, s, p, a->num_chunks);
  }
  if (a->conv_states) {
    record_event(a->profile_events, 1, s);
    if (a->in_dtype == SSD_BF16)
      hipLaunchKernelGGL(k_conv_state<bf16_t>, dim3(a->num_seqs, nb), dim3(64), 0, s, p);
    else
      hipLaunchKernelGGL(k_conv_state<float>, dim3(a->num_seqs, nb), dim3(64), 0, s, p);
    record_event(a->profile_events, 2, s);
  } else {
    record_event(a->profile_events, 1, s);
  }
  return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

ssd_status ssd_conv1d_update(const ssd_conv1d_update_args* a, ssd_stream_t stream) {
  using namespace ssd;
  if (!a) return SSD_ERR_NULL_POINTER;
  if (a->B_pad < 0 || a->ntok < 1) return SSD_ERR_BAD_SHAPE;
  ssd_status st = check_common(a->D, a->W, a->in_dtype, a->activation, a->state_layout);
  if (st != SSD_OK) return st;
  if (a->ntok > kConvMaxTokens) return SSD_ERR_UNSUPPORTED;
  if (a->B_pad == 0) return SSD_OK;
  if (!a->x || !a->out || !a->weight || !a->conv_states || !a->state_indices)
    return SSD_ERR_NULL_POINTER;
  st = check_pool(a->conv_states, a->slot_stride, a->num_slots, a->D, a->W);
  if (st != SSD_OK) return st;
  if (!aligned16(a->x) || !aligned16(a->out) || !aligned16(a->weight) ||
      (a->bias && !aligned16(a->bias)))
    return SSD_ERR_UNSUPPORTED;

  ConvParams p{};
  p.D = a->D; p.x = a->x; p.out = a->out; p.w = a->weight; p.bias = a->bias;
  p.silu = a->activation; p.cs = a->conv_states; p.slot_stride = a->slot_stride;
  p.num_slots = a->num_slots; p.layout = a->state_layout; p.sidx = a->state_indices;
  p.flag = a->device_error_flag; p.ntok = a->ntok; p.null_id = a->null_block_id;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int nb = (a->D + kConvChan - 1) / kConvChan;
  record_event(a->profile_events, 0, s);
  if (a->in_dtype == SSD_BF16)
    hipLaunchKernelGGL(k_conv_update<bf16_t>, dim3(a->B_pad, nb), dim3(64), 0, s, p);
  else
    hipLaunchKernelGGL(k_conv_update<float>, dim3(a->B_pad, nb), dim3(64), 0, s, p);
  record_event(a->profile_events, 1, s);
  return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

}  // extern "C"
