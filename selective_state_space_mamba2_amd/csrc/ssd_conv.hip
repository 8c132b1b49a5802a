// ssd_conv.hip -- the causal depthwise conv1d ahead of the scan ("vLLM Mamba2 SSD kernel
// warm-up", mamba_mixer2.py section: x, B and C are taken after a depthwise convolution;
// conv state shapes from "vLLM v0.20.0 adds disaggregated serving for hybrid SSM models").
//
//   k_conv_prefill  per (chunk, 512-channel block): four wavefronts split the chunk's
//                   tokens; a lane owns 8 consecutive channels (16-byte rows for bf16),
//                   keeps the last W-1 inputs in registers and streams the tokens, loads
//                   issued 8 tokens ahead.  A window reaching before the sequence start
//                   reads the sequence's conv state.
//   k_conv_state    per (sequence, 512 channels): the new conv state (the last W-1
//                   inputs), written after every output kernel read of the old one.
//   k_conv_update   per (decode row, 512 channels): the row's inputs continue its state,
//                   which is replaced in place.
// Pure streaming work: each is bound by HBM bandwidth (bytes per unit in the header of
// each kernel), not by its 4 FMAs per channel and token.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ssd.h"
#include "ssd_device.h"
#include "ssd_params.h"

namespace ssd {
namespace {

constexpr int kConvW = 4;                              // instantiated kernel width
constexpr int kConvVec = 8;                            // channels per lane
constexpr int kConvChan = 64 * kConvVec;               // channels per wavefront
constexpr int kConvWaves = 4;                          // token quarters of a chunk
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

// 8 consecutive channels of one row: bf16 (16 bytes) or fp32 (32 bytes).
template <typename T> struct Row8;
template <> struct Row8<bf16_t> {
  static __device__ __forceinline__ void ld(const bf16_t* p, float* v) {
    const u32x4_v w = *reinterpret_cast<const u32x4_v*>(p);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(ws[i] << 16);
      v[2 * i + 1] = __uint_as_float(ws[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void st(bf16_t* p, const float* v) {
    *reinterpret_cast<u32x4_v*>(p) = u32x4_v{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                             pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
  }
};
template <> struct Row8<float> {
  static __device__ __forceinline__ void ld(const float* p, float* v) {
    const float4_v a = reinterpret_cast<const float4_v*>(p)[0];
    const float4_v b = reinterpret_cast<const float4_v*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void st(float* p, const float* v) {
    reinterpret_cast<float4_v*>(p)[0] = float4_v{v[0], v[1], v[2], v[3]};
    reinterpret_cast<float4_v*>(p)[1] = float4_v{v[4], v[5], v[6], v[7]};
  }
};

// Entry k (0 = oldest input) of channels c0..c0+7 of a pool slot, in either layout.
template <typename T>
__device__ __forceinline__ void state_ld(const ConvParams& p, int slot, int k, int c0, float* v) {
  const T* base = static_cast<const T*>(p.cs) + int64_t(slot) * p.slot_stride;
  if (p.layout == SSD_CONV_LAYOUT_SD) {
    Row8<T>::ld(base + int64_t(k) * p.D + c0, v);
  } else {
#pragma unroll
    for (int i = 0; i < kConvVec; ++i) v[i] = Elem<T>::load(base + int64_t(c0 + i) * (kConvW - 1) + k);
  }
}
template <typename T>
__device__ __forceinline__ void state_st(const ConvParams& p, int slot, int k, int c0, const float* v) {
  T* base = static_cast<T*>(p.cs) + int64_t(slot) * p.slot_stride;
  if (p.layout == SSD_CONV_LAYOUT_SD) {
    Row8<T>::st(base + int64_t(k) * p.D + c0, v);
  } else {
#pragma unroll
    for (int i = 0; i < kConvVec; ++i) Elem<T>::store(base + int64_t(c0 + i) * (kConvW - 1) + k, v[i]);
  }
}

// The lane's filter taps wk[k][i] = weight[c0 + i, k] and biases.
__device__ __forceinline__ void load_taps(const ConvParams& p, int c0, float (&wk)[kConvW][kConvVec],
                                          float (&bv)[kConvVec]) {
  const float4_v* w4 = reinterpret_cast<const float4_v*>(p.w + int64_t(c0) * kConvW);
#pragma unroll
  for (int i = 0; i < kConvVec; ++i) {
    const float4_v t = w4[i];   // weight[c0 + i, 0..3]
    wk[0][i] = t.x; wk[1][i] = t.y; wk[2][i] = t.z; wk[3][i] = t.w;
  }
  if (p.bias) {
    const float4_v b0 = reinterpret_cast<const float4_v*>(p.bias + c0)[0];
    const float4_v b1 = reinterpret_cast<const float4_v*>(p.bias + c0)[1];
    bv[0] = b0.x; bv[1] = b0.y; bv[2] = b0.z; bv[3] = b0.w;
    bv[4] = b1.x; bv[5] = b1.y; bv[6] = b1.z; bv[7] = b1.w;
  } else {
#pragma unroll
    for (int i = 0; i < kConvVec; ++i) bv[i] = 0.f;
  }
}

// One output row from the window u (oldest first) and the new input xv; then the window
// moves on by one input.
__device__ __forceinline__ void conv_step(const float (&wk)[kConvW][kConvVec], const float (&bv)[kConvVec],
                                          float (&u)[kConvW - 1][kConvVec], const float* xv,
                                          int silu, float* o) {
#pragma unroll
  for (int i = 0; i < kConvVec; ++i) {
    float v = bv[i] + wk[0][i] * u[0][i] + wk[1][i] * u[1][i] + wk[2][i] * u[2][i] + wk[3][i] * xv[i];
    if (silu) v = v / (1.f + fast_exp(-v));
    o[i] = v;
    u[0][i] = u[1][i];
    u[1][i] = u[2][i];
    u[2][i] = xv[i];
  }
}

// ---------------------------------------------------------------------------------------
// k_conv_prefill: per chunk and token, x row in and out row out (2 D b bytes), plus the
// sequence's conv state (3 D b) for the windows reaching before its first token.
// ---------------------------------------------------------------------------------------
template <typename T>
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
  const int c0 = cb * kConvChan + lane * kConvVec;
  const int L = cs1 - cs0, per = (L + kConvWaves - 1) / kConvWaves;
  const int a = cs0 + wave * per, b = min(cs1, a + per);
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
  T* og = static_cast<T*>(p.out) + c0;
  float u[kConvW - 1][kConvVec];
#pragma unroll
  for (int j = 0; j < kConvW - 1; ++j) {
    const int t = a - (kConvW - 1) + j;
    if (t >= t0) {
      Row8<T>::ld(xg + int64_t(t) * p.x_st, u[j]);
    } else if (slot >= 0) {
      state_ld<T>(p, slot, (kConvW - 1) + (t - t0), c0, u[j]);
    } else {
#pragma unroll
      for (int i = 0; i < kConvVec; ++i) u[j][i] = 0.f;
    }
  }
  float wk[kConvW][kConvVec], bv[kConvVec];
  load_taps(p, c0, wk, bv);

  for (int t = a; t < b; t += kConvBatch) {
    float xv[kConvBatch][kConvVec];
#pragma unroll
    for (int i = 0; i < kConvBatch; ++i)
      if (t + i < b) Row8<T>::ld(xg + int64_t(t + i) * p.x_st, xv[i]);
#pragma unroll
    for (int i = 0; i < kConvBatch; ++i) {
      if (t + i >= b) break;
      float o[kConvVec];
      conv_step(wk, bv, u, xv[i], p.silu, o);
      Row8<T>::st(og + int64_t(t + i) * p.out_st, o);
    }
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
      Row8<T>::ld(xg + int64_t(t0 + q) * p.x_st, nv[j]);
    } else if (init) {
      state_ld<T>(p, slot, (kConvW - 1) + q, c0, nv[j]);
    } else {
#pragma unroll
      for (int i = 0; i < kConvVec; ++i) nv[j][i] = 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < kConvW - 1; ++j) state_st<T>(p, slot, j, c0, nv[j]);
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
  for (int j = 0; j < kConvW - 1; ++j) state_ld<T>(p, slot, j, c0, u[j]);
  float wk[kConvW][kConvVec], bv[kConvVec];
  load_taps(p, c0, wk, bv);
  const T* xg = static_cast<const T*>(p.x) + int64_t(r) * p.ntok * p.D + c0;
  T* og = static_cast<T*>(p.out) + int64_t(r) * p.ntok * p.D + c0;
  for (int j = 0; j < p.ntok; ++j) {
    float xv[kConvVec], o[kConvVec];
    Row8<T>::ld(xg + int64_t(j) * p.D, xv);
    conv_step(wk, bv, u, xv, p.silu, o);
    Row8<T>::st(og + int64_t(j) * p.D, o);
  }
#pragma unroll
  for (int j = 0; j < kConvW - 1; ++j) state_st<T>(p, slot, j, c0, u[j]);
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
  if (a->in_dtype == SSD_BF16)
    hipLaunchKernelGGL(k_conv_prefill<bf16_t>, dim3(a->num_chunks, nb), dim3(64 * kConvWaves), 0, s, p, a->num_chunks);
  else
    hipLaunchKernelGGL(k_conv_prefill<float>, dim3(a->num_chunks, nb), dim3(64 * kConvWaves), 0, s, p, a->num_chunks);
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
