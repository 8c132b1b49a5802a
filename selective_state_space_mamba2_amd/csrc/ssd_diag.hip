// ssd_diag.hip -- Mamba1-style selective scan with a per-(channel, state) diagonal A.
//
// The S6 model of "[vLLM] Mamba (SSM)" (paper key content) with A[channel, state]:
//   h[c,n] = exp(delta[t,c] A[c,n]) h[c,n] + delta[t,c] x[t,c] B[t,n];  y[t,c] = sum_n C[t,n] h[c,n] + D[c] x[t,c]
// Mamba1 has no chunk notion of its own, so the chunk size only sets where state
// checkpoints are written ("vLLM Mamba2 SSD kernel warm-up", config/model.py section).
//
// This path is bound by the exponential (one per (token, channel, state)) and VALU work,
// not by a contraction, so it runs on the vector ALUs: one workgroup owns 64 channels of
// one sequence and walks its tokens in order; each channel's 16 states are spread over 4
// adjacent lanes (4 states each) and y is a 4-lane reduction.  Token tiles of delta, x,
// B and C are staged through LDS with coalesced loads (64 channels = 128 B per token for
// bf16), delta is prepared once per (token, channel) while staging, and y leaves through
// an LDS tile as coalesced rows.  Checkpoints are written at the chunk ends listed by the
// chunk metadata.
#include "ssd_params.h"

namespace ssd {

template <typename T>
__global__ __launch_bounds__(256) void k_diag_scan(PrefillParams p) {
  constexpr int N = kDiagN;    // 16 states per channel
  constexpr int CH = 64;       // channels per workgroup
  constexpr int TT = 32;       // tokens per LDS tile
  __shared__ float s_d[TT][CH];
  __shared__ float s_x[TT][CH];
  __shared__ float s_y[TT][CH];
  __shared__ float4_v s_b[TT][N / 4];
  __shared__ float4_v s_c[TT][N / 4];

  const int tid = threadIdx.x;
  const int cb = blockIdx.x, r = blockIdx.y;
  const int cl = tid >> 2, ng = tid & 3;
  const int H = p.H;
  const int c = cb * CH + cl;
  const bool valid = c < H;

  const int t0 = p.cu_seqlens[r], t1 = p.cu_seqlens[r + 1];
  int k = r == 0 ? 0 : p.last_chunk[r - 1] + 1;
  const int klast = p.last_chunk[r];
  if (t0 < 0 || t1 > p.T || t1 <= t0 || k < 0 || klast < k || klast >= p.C || p.cu_chunk[k] != t0 ||
      p.cu_chunk[klast + 1] != t1) {
    if (tid == 0 && cb == 0) raise_flag(p.flag, SSD_DEVERR_CHUNK_RANGE);
    return;
  }
  int next_end = p.cu_chunk[k + 1];

  float A2[4];
  float h[4] = {0.f, 0.f, 0.f, 0.f};
  int slot = -1;
  if (p.pool && p.state_idx) {
    slot = p.state_idx[r];
    if (slot < 0 || slot >= p.num_slots) {
      if (tid == 0 && cb == 0) raise_flag(p.flag, SSD_DEVERR_SLOT_RANGE);
      slot = -1;
    }
  }
  if (valid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) A2[i] = p.A[c * N + ng * 4 + i] * kLog2e;
    if (slot >= 0 && p.has_init && p.has_init[r]) {
      const float4_v v = *reinterpret_cast<const float4_v*>(
          p.pool + int64_t(slot) * p.slot_stride + int64_t(c) * N + ng * 4);
      h[0] = v.x; h[1] = v.y; h[2] = v.z; h[3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) A2[i] = 0.f;
  }
  const float Dc = (valid && p.D) ? p.D[c] : 0.f;

  const T* xg = static_cast<const T*>(p.x);
  const T* dg = static_cast<const T*>(p.dt);
  const T* bg = static_cast<const T*>(p.B);
  const T* cg = static_cast<const T*>(p.Cm);
  T* yg = static_cast<T*>(p.y);

  for (int tb = t0; tb < t1; tb += TT) {
    const int nt = min(TT, t1 - tb);
    for (int e = tid; e < TT * CH; e += 256) {
      const int tt = e / CH, cc = e % CH, ch = cb * CH + cc;
      float dv = 0.f, xv = 0.f;
      if (tt < nt && ch < H) {
        const int64_t t = tb + tt;
        dv = p.prep(Elem<T>::load(dg + t * p.dt_st + ch), ch);
        xv = Elem<T>::load(xg + t * p.x_st + ch);
      }
      s_d[tt][cc] = dv;
      s_x[tt][cc] = xv;
    }
    if (tid < TT * 2 * (N / 4)) {
      const int tt = tid / (2 * (N / 4)), q = tid % (2 * (N / 4));
      const int which = q / (N / 4), n4 = q % (N / 4);
      float4_v v = {0.f, 0.f, 0.f, 0.f};
      if (tt < nt) {
        const T* src = (which ? cg : bg) + int64_t(tb + tt) * p.bc_st + n4 * 4;
        v = float4_v{Elem<T>::load(src), Elem<T>::load(src + 1), Elem<T>::load(src + 2),
                     Elem<T>::load(src + 3)};
      }
      if (which) s_c[tt][n4] = v; else s_b[tt][n4] = v;
    }
    __syncthreads();

    for (int tt = 0; tt < nt; ++tt) {
      const float d = s_d[tt][cl];
      const float xv = s_x[tt][cl];
      const float dx = d * xv;
      const float4_v bv = s_b[tt][ng];
      const float4_v cv = s_c[tt][ng];
      const float bb[4] = {bv.x, bv.y, bv.z, bv.w};
      const float cc4[4] = {cv.x, cv.y, cv.z, cv.w};
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = __builtin_amdgcn_exp2f(d * A2[i]);
        h[i] = a * h[i] + dx * bb[i];
        acc += cc4[i] * h[i];
      }
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      if (ng == 0) s_y[tt][cl] = acc + Dc * xv;
      if (tb + tt + 1 == next_end) {  // end of chunk k: checkpoint (uniform branch)
        if (valid && p.states) {
          *reinterpret_cast<float4_v*>(p.states + (int64_t(k) * H + c) * N + ng * 4) =
              float4_v{h[0], h[1], h[2], h[3]};
        }
        ++k;
        next_end = k <= klast ? p.cu_chunk[k + 1] : -1;
      }
    }
    __syncthreads();
    for (int e = tid; e < nt * CH; e += 256) {
      const int tt = e / CH, cc = e % CH, ch = cb * CH + cc;
      if (ch < H) Elem<T>::store(yg + int64_t(tb + tt) * p.y_st + ch, s_y[tt][cc]);
    }
    __syncthreads();
  }
  if (k != klast + 1 && tid == 0 && cb == 0) raise_flag(p.flag, SSD_DEVERR_CHUNK_RANGE);
  if (valid && p.write_final && slot >= 0) {
    *reinterpret_cast<float4_v*>(p.pool + int64_t(slot) * p.slot_stride + int64_t(c) * N +
                                 ng * 4) = float4_v{h[0], h[1], h[2], h[3]};
  }
}

hipError_t launch_diag_prefill(int in_dtype, const PrefillParams& p, hipStream_t s,
                               void* const* events) {
  const dim3 grid((p.H + 63) / 64, p.S);
  record_event(events, 0, s);
  if (in_dtype == SSD_BF16) hipLaunchKernelGGL(k_diag_scan<bf16_t>, grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL(k_diag_scan<float>, grid, dim3(256), 0, s, p);
  record_event(events, 1, s);
  return hipGetLastError();
}

}  // namespace ssd
