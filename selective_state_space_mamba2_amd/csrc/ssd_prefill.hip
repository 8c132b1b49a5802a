// ssd_prefill.hip -- chunked varlen SSD prefill for gfx950.
//
// Per head h (state in R^{P x N}) the recurrence h_t = exp(delta_t A) h_{t-1} + delta_t x_t B_t^T,
// y_t = h_t C_t + D x_t is split at the chunk boundaries produced by the chunk-metadata
// builder (one sequence per chunk, a cut at every chunk_size-th absolute token: "[vLLM]
// Mamba (SSM)", chunk-metadata section).  Inside chunk k with inclusive cumsum
// c_t = sum_{r<=t} delta_r A (chunk-local), unrolling the recurrence gives
//   h_end  = exp(c_last) h_in + sum_s delta_s exp(c_last - c_s) x_s B_s^T
//   y_l    = exp(c_l) (h_in C_l) + sum_{s<=l} (C_l . B_s) exp(c_l - c_s) delta_s x_s + D x_l
// which three kernels evaluate:
//   k_chunk_state    per (chunk, head): delta, c (block scan), and the chunk's own state
//                    S_k = X^T diag(w) B with w_s = delta_s exp(c_last - c_s)  (bf16 MFMA)
//   k_state_passing  per (sequence, head, state slice): H_k = exp(c_last,k) H_{k-1} + S_k in
//                    fp32, serial over the sequence's chunks; gathers the initial state from
//                    the pool first and writes the final state back last
//   k_chunk_scan     per (chunk, head): y = exp(c_l) C H_in^T + (L o C B^T) X + D x, where
//                    L_{l,s} = exp(c_l - c_s) delta_s for s <= l (bf16 MFMA)
// The chunk state k_state_passing writes at every chunk end is the prefix-caching checkpoint
// ("why this design", item 3).  Decay factors are always exp of a difference of cumsums
// (never exp(+c) * exp(-c)), so they stay in [0, 1] for A <= 0 and delta >= 0.
//
// MFMA fragments (v_mfma_f32_16x16x32_bf16; fp32 inputs use 8 x v_mfma_f32_16x16x4_f32 on
// the same 8-values-per-lane fragments): the 16x16 fp32 result tile gives lane L rows
// 4*(L/16)+r of column L%16.  C.B^T is computed transposed (rows s, columns l), so after
// masking each lane already holds 8 values of one row l of L o CB: slots j<4 are
// s = s0+4*(L/16)+j and slots j>=4 are s = s0+16+4*(L/16)+(j-4).  The same slot -> s map is
// used when reading X^T for the B operand, so M = L o CB never goes through LDS.
#include "ssd_params.h"

namespace ssd {

// ---------------------------------------------------------------------------------------
// operand traits: bf16 inputs run bf16 MFMA, fp32 inputs run fp32 MFMA
// ---------------------------------------------------------------------------------------
template <typename T> struct Ops;

template <> struct Ops<bf16_t> {
  using lds_t = bf16_t;
  using frag = Frag8;
  static constexpr int kPad = 8;  // 16 B of row padding (spreads rows over LDS banks)
  static __device__ __forceinline__ frag ld8(const lds_t* q) {
    const u32x4_v v = *reinterpret_cast<const u32x4_v*>(q);
    return frag{{v.x, v.y, v.z, v.w}};
  }
  static __device__ __forceinline__ frag ld44(const lds_t* a, const lds_t* b) {
    const u32x2_v va = *reinterpret_cast<const u32x2_v*>(a);
    const u32x2_v vb = *reinterpret_cast<const u32x2_v*>(b);
    return frag{{va.x, va.y, vb.x, vb.y}};
  }
  static __device__ __forceinline__ frag from8(const float* v) {
    return frag{{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                 pack_bf16x2(v[6], v[7])}};
  }
  // 8 consecutive global elements (16 B aligned), zeros when !ok
  static __device__ __forceinline__ frag gld8(const bf16_t* q, bool ok) {
    if (!ok) return frag{{0u, 0u, 0u, 0u}};
    const u32x4_v v = *reinterpret_cast<const u32x4_v*>(q);
    return frag{{v.x, v.y, v.z, v.w}};
  }
  static __device__ __forceinline__ f32x4_v mma(const frag& a, const frag& b, f32x4_v c) {
    return mma_bf16(a, b, c);
  }
  static __device__ __forceinline__ lds_t cvt(float v) { return f32_to_bf16(v); }
  static __device__ __forceinline__ float tof(lds_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ float val(const frag& f, int j) {
    return bf16_to_f32(bf16_t(f.w[j >> 1] >> ((j & 1) * 16)));
  }
};

template <> struct Ops<float> {
  using lds_t = float;
  using frag = Frag8f;
  static constexpr int kPad = 4;
  static __device__ __forceinline__ frag ld8(const lds_t* q) {
    const float4_v a = *reinterpret_cast<const float4_v*>(q);
    const float4_v b = *reinterpret_cast<const float4_v*>(q + 4);
    return frag{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
  }
  static __device__ __forceinline__ frag ld44(const lds_t* a, const lds_t* b) {
    const float4_v va = *reinterpret_cast<const float4_v*>(a);
    const float4_v vb = *reinterpret_cast<const float4_v*>(b);
    return frag{{va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w}};
  }
  static __device__ __forceinline__ frag from8(const float* v) {
    return frag{{v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]}};
  }
  static __device__ __forceinline__ frag gld8(const float* q, bool ok) {
    if (!ok) return frag{{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}};
    return ld8(q);
  }
  static __device__ __forceinline__ f32x4_v mma(const frag& a, const frag& b, f32x4_v c) {
    return mma_f32(a, b, c);
  }
  static __device__ __forceinline__ lds_t cvt(float v) { return v; }
  static __device__ __forceinline__ float tof(lds_t v) { return v; }
  static __device__ __forceinline__ float val(const frag& f, int j) { return f.v[j]; }
};

// Chunk k's token range and sequence; false (and the flag raised) if the metadata is bad.
__device__ __forceinline__ bool chunk_bounds(const PrefillParams& p, int k, int cs_max,
                                             int& cs0, int& L, int& r) {
  cs0 = p.cu_chunk[k];
  const int cs1 = p.cu_chunk[k + 1];
  r = p.seq_idx[k];
  L = cs1 - cs0;
  bool ok = L >= 1 && L <= cs_max && r >= 0 && r < p.S && cs0 >= 0;
  if (ok) ok = cs0 >= p.cu_seqlens[r] && cs1 <= p.cu_seqlens[r + 1] && cs1 <= p.T;
  return ok;
}

__device__ __forceinline__ void wave_lds_sync() {
  // s_waitcnt lgkmcnt(0): this wave's LDS writes are done before its lanes read them.
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// Stage chunk-relative tokens [s_base, s_base + KB) of a row-major [token][W] source into
// dst[W][RS] (transposed: token index contiguous), token s scaled by scale[s] when given.
// Each work item moves a 2-token x 8-column block: two 16 B row loads, eight 2-token
// column writes.  Tokens at or past L read as zero.
template <typename T, int W, int KB, int RS, int NTH>
__device__ __forceinline__ void stage_transposed(typename Ops<T>::lds_t* dst, const T* src,
                                                 int64_t stride_t, int s_base, int L,
                                                 const float* scale) {
  using O = Ops<T>;
  constexpr int NPAIR = KB / 2, NG = W / 8;
  for (int it = threadIdx.x; it < NPAIR * NG; it += NTH) {
    const int sp = it % NPAIR, g8 = it / NPAIR;
    const int s = s_base + 2 * sp;
    const typename O::frag a = O::gld8(src + int64_t(s) * stride_t + 8 * g8, s < L);
    const typename O::frag b = O::gld8(src + int64_t(s + 1) * stride_t + 8 * g8, s + 1 < L);
    if constexpr (sizeof(T) == 2) {
      uint32_t* d32 = reinterpret_cast<uint32_t*>(dst);
      if (scale) {
        const float sa = scale[s], sb = scale[s + 1];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          d32[((8 * g8 + j) * RS + 2 * sp) >> 1] = pack_bf16x2(O::val(a, j) * sa, O::val(b, j) * sb);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t lo = (a.w[j >> 1] >> ((j & 1) * 16)) & 0xffffu;
          const uint32_t hi = (b.w[j >> 1] >> ((j & 1) * 16)) & 0xffffu;
          d32[((8 * g8 + j) * RS + 2 * sp) >> 1] = lo | (hi << 16);
        }
      }
    } else {
      const float sa = scale ? scale[s] : 1.f, sb = scale ? scale[s + 1] : 1.f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<float2_v*>(dst + (8 * g8 + j) * RS + 2 * sp) =
            float2_v{O::val(a, j) * sa, O::val(b, j) * sb};
    }
  }
}

// ---------------------------------------------------------------------------------------
// k_chunk_state: delta, within-chunk cumsum, and S_k = X^T diag(w) B for one (chunk, head)
// ---------------------------------------------------------------------------------------
template <typename T, int P, int N, int CS>
__global__ __launch_bounds__(256) void k_chunk_state(PrefillParams p) {
  using O = Ops<T>;
  using lds_t = typename O::lds_t;
  constexpr int KB = CS < 64 ? CS : 64;   // tokens staged per step
  constexpr int RS = KB + O::kPad;
  constexpr int TP = P / 16, TN = N / 16, NT = TP * TN, QPW = (NT + 3) / 4;
  static_assert(CS <= 256, "one token per thread in the cumsum");
  __shared__ __attribute__((aligned(16))) lds_t xT[P * RS];
  __shared__ __attribute__((aligned(16))) lds_t bT[N * RS];
  __shared__ float s_c[CS];
  __shared__ float s_w[CS];
  __shared__ float s_scan[4];

  const int k = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  int cs0, L, r;
  if (!chunk_bounds(p, k, CS, cs0, L, r)) {
    if (tid == 0) raise_flag(p.flag, SSD_DEVERR_CHUNK_RANGE);
    return;
  }
  const int g = h / (p.H / p.G);
  const T* dtp = static_cast<const T*>(p.dt);
  float d = 0.f;
  if (tid < L) d = p.prep(Elem<T>::load(dtp + int64_t(cs0 + tid) * p.dt_st + h), h);
  const float c = block_inclusive_scan(d * p.A[h], s_scan);
  if (tid < CS) s_c[tid] = c;
  __syncthreads();
  const float c_last = s_c[L - 1];
  if (tid < CS) s_w[tid] = tid < L ? d * fast_exp(c_last - c) : 0.f;
  if (tid < L && p.dA_cumsum_out) p.dA_cumsum_out[int64_t(h) * p.T + cs0 + tid] = c;
  if (tid == 0) p.dA_last[int64_t(k) * p.H + h] = c_last;
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63, li = lane & 15, kg = lane >> 4;
  f32x4_v acc[QPW];
#pragma unroll
  for (int q = 0; q < QPW; ++q) acc[q] = f32x4_v{0.f, 0.f, 0.f, 0.f};

  const T* xs = static_cast<const T*>(p.x) + int64_t(cs0) * p.x_st + int64_t(h) * P;
  const T* bs = static_cast<const T*>(p.B) + int64_t(cs0) * p.bc_st + int64_t(g) * N;
  for (int sb = 0; sb * KB < L; ++sb) {
    stage_transposed<T, P, KB, RS, 256>(xT, xs, p.x_st, sb * KB, L, nullptr);
    stage_transposed<T, N, KB, RS, 256>(bT, bs, p.bc_st, sb * KB, L, s_w);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KB / 32; ++kk) {
#pragma unroll
      for (int q = 0; q < QPW; ++q) {
        const int tile = wave * QPW + q;
        if (tile < NT) {
          const int pt = tile / TN, nt = tile % TN;
          const typename O::frag a = O::ld8(&xT[(pt * 16 + li) * RS + kk * 32 + 8 * kg]);
          const typename O::frag b = O::ld8(&bT[(nt * 16 + li) * RS + kk * 32 + 8 * kg]);
          acc[q] = O::mma(a, b, acc[q]);
        }
      }
    }
    __syncthreads();
  }

  const int64_t base = (int64_t(k) * p.H + h) * (P * N);
#pragma unroll
  for (int q = 0; q < QPW; ++q) {
    const int tile = wave * QPW + q;
    if (tile < NT) {
      const int pt = tile / TN, nt = tile % TN;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int e = (pt * 16 + 4 * kg + rr) * N + nt * 16 + li;
        p.states[base + e] = acc[q][rr];
        if (p.local_states_out) p.local_states_out[base + e] = acc[q][rr];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// k_state_passing: H_k = exp(c_last,k) H_{k-1} + S_k over one sequence's chunks, in place
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_state_passing(PrefillParams p) {
  const int PN4 = p.P * p.N / 4;
  const int e4 = blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y, r = blockIdx.z;
  if (e4 >= PN4) return;
  const int k0 = r == 0 ? 0 : p.last_chunk[r - 1] + 1;
  const int k1 = p.last_chunk[r];
  if (k0 < 0 || k1 < k0 || k1 >= p.C) {
    if (e4 == 0) raise_flag(p.flag, SSD_DEVERR_CHUNK_RANGE);
    return;
  }
  int slot = -1;
  if (p.pool && p.state_idx) {
    slot = p.state_idx[r];
    if (slot < 0 || slot >= p.num_slots) {
      if (e4 == 0) raise_flag(p.flag, SSD_DEVERR_SLOT_RANGE);
      slot = -1;
    }
  }
  float4_v st = {0.f, 0.f, 0.f, 0.f};
  float4_v* pool_v = slot >= 0 ? reinterpret_cast<float4_v*>(
                                     p.pool + int64_t(slot) * p.slot_stride) + int64_t(h) * PN4 + e4
                               : nullptr;
  if (pool_v && p.has_init && p.has_init[r]) st = *pool_v;
  if (p.init_copy)
    reinterpret_cast<float4_v*>(p.init_copy)[(int64_t(r) * p.H + h) * PN4 + e4] = st;

  float4_v* sv = reinterpret_cast<float4_v*>(p.states) + (int64_t(k0) * p.H + h) * PN4 + e4;
  const int64_t kstride = int64_t(p.H) * PN4;
  const float* dl = p.dA_last + int64_t(k0) * p.H + h;
  const int nk = k1 - k0 + 1;
  for (int k = 0; k < nk; k += 4) {
    float4_v s[4];
    float dd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (k + i < nk) {
        s[i] = sv[(k + i) * kstride];
        dd[i] = dl[int64_t(k + i) * p.H];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (k + i < nk) {
        st = fast_exp(dd[i]) * st + s[i];
        sv[(k + i) * kstride] = st;
      }
    }
  }
  if (pool_v && p.write_final) *pool_v = st;
}

// ---------------------------------------------------------------------------------------
// k_chunk_scan: y = exp(c_l) C_l H_in^T + sum_{s<=l} CB_{l,s} exp(c_l - c_s) delta_s x_s + D x_l
// ---------------------------------------------------------------------------------------
template <typename T, int P, int N, int CS>
__global__ __launch_bounds__(CS * 2) void k_chunk_scan(PrefillParams p) {
  using O = Ops<T>;
  using lds_t = typename O::lds_t;
  using frag = typename O::frag;
  constexpr int NW = CS / 32, NTH = 64 * NW;   // each wave owns two 16-row l-tiles
  constexpr int RSX = CS + O::kPad;            // X^T rows (token contiguous)
  constexpr int NP = N < 32 ? 32 : N;          // dstate padded to the MFMA K of 32
  constexpr int RSB = NP + O::kPad;            // B and H rows
  constexpr int RSY = P + O::kPad;             // y staging rows
  constexpr int TPc = P / 16, KN = NP / 32;
  __shared__ __attribute__((aligned(16))) lds_t xT[P * RSX];
  __shared__ __attribute__((aligned(16))) lds_t Bs[CS * RSB];
  __shared__ __attribute__((aligned(16))) lds_t Hs[P * RSB];
  __shared__ __attribute__((aligned(16))) lds_t ystage[NW * 16 * RSY];
  __shared__ float s_c[CS];
  __shared__ float s_d[CS];
  __shared__ float s_scan[NW];

  const int k = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  int cs0, L, r;
  if (!chunk_bounds(p, k, CS, cs0, L, r)) {
    if (tid == 0) raise_flag(p.flag, SSD_DEVERR_CHUNK_RANGE);
    return;
  }
  const int hpg = p.H / p.G, g = h / hpg;
  const T* dtp = static_cast<const T*>(p.dt);
  float d = 0.f;
  if (tid < L) d = p.prep(Elem<T>::load(dtp + int64_t(cs0 + tid) * p.dt_st + h), h);
  const float c = block_inclusive_scan(d * p.A[h], s_scan);
  if (tid < CS) {
    s_c[tid] = c;
    s_d[tid] = d;
  }

  // stage X^T, B and the incoming state
  const T* xs = static_cast<const T*>(p.x) + int64_t(cs0) * p.x_st + int64_t(h) * P;
  stage_transposed<T, P, CS, RSX, NTH>(xT, xs, p.x_st, 0, L, nullptr);
  const T* bsrc = static_cast<const T*>(p.B) + int64_t(cs0) * p.bc_st + int64_t(g) * N;
  for (int e = tid; e < CS * (NP / 8); e += NTH) {
    const int s = e / (NP / 8), c8 = e % (NP / 8);
    const frag v = O::gld8(bsrc + int64_t(s) * p.bc_st + 8 * c8, s < L && 8 * c8 < N);
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<u32x4_v*>(&Bs[s * RSB + 8 * c8]) = u32x4_v{v.w[0], v.w[1], v.w[2], v.w[3]};
    } else {
      *reinterpret_cast<float4_v*>(&Bs[s * RSB + 8 * c8]) = float4_v{v.v[0], v.v[1], v.v[2], v.v[3]};
      *reinterpret_cast<float4_v*>(&Bs[s * RSB + 8 * c8 + 4]) = float4_v{v.v[4], v.v[5], v.v[6], v.v[7]};
    }
  }
  const bool first = k == 0 || p.seq_idx[k - 1] != r;
  const float* hin = !first ? p.states + (int64_t(k - 1) * p.H + h) * (P * N)
                            : (p.init_copy ? p.init_copy + (int64_t(r) * p.H + h) * (P * N)
                                           : nullptr);
  for (int e = tid; e < P * NP / 4; e += NTH) {
    const int pp = e / (NP / 4), n4 = e % (NP / 4);
    float4_v v = {0.f, 0.f, 0.f, 0.f};
    if (hin && 4 * n4 < N) v = reinterpret_cast<const float4_v*>(hin)[pp * (N / 4) + n4];
    lds_t* dst = &Hs[pp * RSB + 4 * n4];
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<u32x2_v*>(dst) = u32x2_v{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
    } else {
      *reinterpret_cast<float4_v*>(dst) = v;
    }
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63, li = lane & 15, kg = lane >> 4;
  const float Dh = p.D ? p.D[h] : 0.f;
  const T* cbase = static_cast<const T*>(p.Cm) + int64_t(cs0) * p.bc_st + int64_t(g) * N;
  T* ybase = static_cast<T*>(p.y) + int64_t(cs0) * p.y_st + int64_t(h) * P;
  lds_t* yst = ystage + wave * 16 * RSY;
  const bool write_cb = p.cb_out && (h % hpg) == 0;

#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    const int tile = pass == 0 ? wave : (CS / 16 - 1 - wave);
    const int l0 = tile * 16;
    if (l0 >= L) continue;   // wave-uniform; no block barrier follows
    const int lrow = l0 + li;
    frag cf[KN];
#pragma unroll
    for (int kk = 0; kk < KN; ++kk)
      cf[kk] = O::gld8(cbase + int64_t(lrow) * p.bc_st + 32 * kk + 8 * kg,
                       lrow < L && 32 * kk + 8 * kg < N);

    f32x4_v acc[TPc];
#pragma unroll
    for (int pt = 0; pt < TPc; ++pt) acc[pt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
    // inter-chunk term: C_l . H_in[p, :]
#pragma unroll
    for (int kk = 0; kk < KN; ++kk) {
#pragma unroll
      for (int pt = 0; pt < TPc; ++pt)
        acc[pt] = O::mma(cf[kk], O::ld8(&Hs[(pt * 16 + li) * RSB + 32 * kk + 8 * kg]), acc[pt]);
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float e = fast_exp(s_c[l0 + 4 * kg + rr]);
#pragma unroll
      for (int pt = 0; pt < TPc; ++pt) acc[pt][rr] *= e;
    }

    // intra-chunk term over s-blocks of 32 tokens up to the diagonal
    const float c_l = s_c[lrow];
    for (int s0 = 0; s0 <= l0; s0 += 32) {
      f32x4_v t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) {
        t0 = O::mma(O::ld8(&Bs[(s0 + li) * RSB + 32 * kk + 8 * kg]), cf[kk], t0);
        t1 = O::mma(O::ld8(&Bs[(s0 + 16 + li) * RSB + 32 * kk + 8 * kg]), cf[kk], t1);
      }
      float m[8];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int sa = s0 + 4 * kg + rr, sb = sa + 16;
        m[rr] = sa <= lrow ? t0[rr] * fast_exp(c_l - s_c[sa]) * s_d[sa] : 0.f;
        m[4 + rr] = sb <= lrow ? t1[rr] * fast_exp(c_l - s_c[sb]) * s_d[sb] : 0.f;
        if (write_cb && lrow < L) {
          float* cbrow = p.cb_out + ((int64_t(k) * p.G + g) * CS + lrow) * CS;
          if (sa <= lrow) cbrow[sa] = t0[rr];
          if (sb <= lrow) cbrow[sb] = t1[rr];
        }
      }
      const frag mf = O::from8(m);
#pragma unroll
      for (int pt = 0; pt < TPc; ++pt) {
        const lds_t* xr = &xT[(pt * 16 + li) * RSX + s0 + 4 * kg];
        acc[pt] = O::mma(mf, O::ld44(xr, xr + 16), acc[pt]);
      }
    }

    // skip connection, then stage the 16 x P tile and write whole rows
#pragma unroll
    for (int pt = 0; pt < TPc; ++pt) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int l = l0 + 4 * kg + rr;
        const float yv = acc[pt][rr] + Dh * O::tof(xT[(pt * 16 + li) * RSX + l]);
        yst[(4 * kg + rr) * RSY + pt * 16 + li] = O::cvt(yv);
      }
    }
    wave_lds_sync();
    constexpr int EPC = 16 / sizeof(T);          // elements per 16 B
    constexpr int CPR = P / EPC;                 // 16 B pieces per row
    for (int e = lane; e < 16 * CPR; e += 64) {
      const int row = e / CPR, piece = e % CPR;
      if (l0 + row < L) {
        *reinterpret_cast<u32x4_v*>(ybase + int64_t(l0 + row) * p.y_st + piece * EPC) =
            *reinterpret_cast<const u32x4_v*>(&yst[row * RSY + piece * EPC]);
      }
    }
    wave_lds_sync();
  }
}

// ---------------------------------------------------------------------------------------
// launch table (same order as kChunkedShapes)
// ---------------------------------------------------------------------------------------
template <typename T, int P, int N, int CS>
static hipError_t run_chunked(const PrefillParams& p, hipStream_t s, void* const* ev) {
  record_event(ev, 0, s);
  hipLaunchKernelGGL((k_chunk_state<T, P, N, CS>), dim3(p.C, p.H), dim3(256), 0, s, p);
  record_event(ev, 1, s);
  hipLaunchKernelGGL(k_state_passing, dim3((P * N / 4 + 255) / 256, p.H, p.S), dim3(256), 0, s, p);
  record_event(ev, 2, s);
  hipLaunchKernelGGL((k_chunk_scan<T, P, N, CS>), dim3(p.C, p.H), dim3(CS * 2), 0, s, p);
  record_event(ev, 3, s);
  return hipGetLastError();
}

typedef hipError_t (*RunFn)(const PrefillParams&, hipStream_t, void* const*);
static const RunFn kRun[] = {
    run_chunked<bf16_t, 64, 128, 256>, run_chunked<bf16_t, 64, 128, 128>,
    run_chunked<bf16_t, 64, 128, 64>,  run_chunked<bf16_t, 16, 16, 64>,
    run_chunked<float, 16, 16, 64>,    run_chunked<float, 64, 128, 64>,
};

hipError_t launch_chunked_prefill(int variant, const PrefillParams& p, hipStream_t s,
                                  void* const* events) {
  if (variant < 0 || variant >= int(sizeof(kRun) / sizeof(kRun[0]))) return hipErrorInvalidValue;
  return kRun[variant](p, s, events);
}

}  // namespace ssd
