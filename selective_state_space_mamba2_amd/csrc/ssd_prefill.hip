// ssd_prefill.hip -- chunked varlen SSD prefill for gfx950.
//
// Per head h (state in R^{P x N}) the recurrence h_t = exp(delta_t A) h_{t-1} + delta_t x_t B_t^T,
// y_t = h_t C_t + D x_t is split at the chunk boundaries produced by the chunk-metadata
// builder (one sequence per chunk, a cut at every chunk_size-th absolute token: "[vLLM]
// Mamba (SSM)", chunk-metadata section).  Inside chunk k with inclusive cumsum
// c_t = sum_{r<=t} delta_r A (chunk-local), unrolling the recurrence gives
//   h_end  = exp(c_last) h_in + sum_s delta_s exp(c_last - c_s) x_s B_s^T
//   y_l    = exp(c_l) (h_in C_l) + sum_{s<=l} (C_l . B_s) exp(c_l - c_s) delta_s x_s + D x_l
// which two kernels evaluate:
//   k_chunk_prep   per (chunk, group): C.B^T (lower-triangular 16x16 tiles) and B^T in the
//                  input dtype, computed once and shared by every head of the group
//   k_chunk_march  per (head, sequence): walks the sequence's chunks with the fp32 state in
//                  registers, producing y, the state after every chunk (the prefix-caching
//                  checkpoint, "why this design", item 3) and the final state for the pool
// Both contractions of a chunk run on bf16 MFMA with fp32 accumulation; the state and its
// decay stay fp32.  Decay factors are products of exp of cumsum differences that are all
// <= 0 for A <= 0 and delta >= 0 (never exp(+c) * exp(-c)), so they stay in [0, 1].
//
// MFMA fragments (v_mfma_f32_16x16x32_bf16; fp32 inputs use 8 x v_mfma_f32_16x16x4_f32 on
// the same 8-values-per-lane fragments): the 16x16 fp32 result tile gives lane L rows
// 4*(L/16)+r of column L%16.  k_chunk_prep computes C.B^T transposed (rows s, columns l),
// so each lane stores four consecutive s of one row l.  In k_chunk_march the A operand of
// the (L o CB) X product is a C.B^T row fragment whose slots j<4 hold s = s0+4*(L/16)+j and
// slots j>=4 hold s = s0+16+4*(L/16)+(j-4); X^T is read with the same slot -> s map.
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
  // 8 consecutive global elements (16 B aligned), always loaded: callers pass a valid
  // address and mask the values where they are used
  static __device__ __forceinline__ frag gld8u(const bf16_t* q) {
    const u32x4_v v = *reinterpret_cast<const u32x4_v*>(q);
    return frag{{v.x, v.y, v.z, v.w}};
  }
  // 4 + 4 consecutive global elements (8-byte aligned)
  static __device__ __forceinline__ frag gld44(const bf16_t* a, const bf16_t* b) {
    const u32x2_v va = *reinterpret_cast<const u32x2_v*>(a);
    const u32x2_v vb = *reinterpret_cast<const u32x2_v*>(b);
    return frag{{va.x, va.y, vb.x, vb.y}};
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
  static __device__ __forceinline__ frag gld8u(const float* q) { return ld8(q); }
  static __device__ __forceinline__ frag gld44(const float* a, const float* b) {
    return ld44(a, b);
  }
  static __device__ __forceinline__ f32x4_v mma(const frag& a, const frag& b, f32x4_v c) {
    return mma_f32(a, b, c);
  }
  static __device__ __forceinline__ lds_t cvt(float v) { return v; }
  static __device__ __forceinline__ float tof(lds_t v) { return v; }
  static __device__ __forceinline__ float val(const frag& f, int j) { return f.v[j]; }
};

// Chunk k's token range and sequence; false if the metadata is bad.
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

// The l-tiles (16 rows each) a wave owns: tiles t with t % (2*NW) in {w, 2*NW-1-w}, which
// balances the causal (lower-triangular) work across the waves.
template <int NTILES, int NW>
struct TileSet {
  static constexpr int kPer = (NTILES + NW - 1) / NW;
  __device__ static __forceinline__ int tile(int w, int q) {
    const int period = q / 2, second = q & 1;
    return period * 2 * NW + (second ? 2 * NW - 1 - w : w);
  }
};

// Staging of a row-major [token][W] chunk into LDS transposed (token index contiguous).  A
// work item moves a 4-token x 8-column block: four 16-byte row loads (eight consecutive
// lanes cover one 128-byte row, so loads are coalesced) and eight 4-token column writes.
// The loads are issued early into registers (stage_load) and written out once the scale
// factors are known (stage_store).  Loads are unguarded (rows past the chunk end repeat its
// last row) so that no branch forces an early wait on them.
template <typename T>
__device__ __forceinline__ void put4(typename Ops<T>::lds_t* d, const typename Ops<T>::frag* v,
                                     int j, const float* sc) {
  using O = Ops<T>;
  if constexpr (sizeof(T) == 2) {
    if (sc) {
      *reinterpret_cast<u32x2_v*>(d) =
          u32x2_v{pack_bf16x2(O::val(v[0], j) * sc[0], O::val(v[1], j) * sc[1]),
                  pack_bf16x2(O::val(v[2], j) * sc[2], O::val(v[3], j) * sc[3])};
    } else {
      const uint32_t sh = (j & 1) * 16;
      const uint32_t e0 = (v[0].w[j >> 1] >> sh) & 0xffffu, e1 = (v[1].w[j >> 1] >> sh) & 0xffffu;
      const uint32_t e2 = (v[2].w[j >> 1] >> sh) & 0xffffu, e3 = (v[3].w[j >> 1] >> sh) & 0xffffu;
      *reinterpret_cast<u32x2_v*>(d) = u32x2_v{e0 | (e1 << 16), e2 | (e3 << 16)};
    }
  } else {
    const float s0 = sc ? sc[0] : 1.f, s1 = sc ? sc[1] : 1.f, s2 = sc ? sc[2] : 1.f,
                s3 = sc ? sc[3] : 1.f;
    *reinterpret_cast<float4_v*>(d) = float4_v{O::val(v[0], j) * s0, O::val(v[1], j) * s1,
                                               O::val(v[2], j) * s2, O::val(v[3], j) * s3};
  }
}

// The x tile of one work item: 4 tokens x 8 columns, loaded into registers.
template <typename T, int W, int KB, int NTH>
struct StageRegs {
  static constexpr int NG = W / 8, NQ = KB / 4, NI = (NQ * NG + NTH - 1) / NTH;
  typename Ops<T>::frag v[NI][4];
};

template <typename T, int W, int KB, int NTH>
__device__ __forceinline__ void stage_load(StageRegs<T, W, KB, NTH>& st, const T* src,
                                           int64_t stride_t, int L) {
  using SR = StageRegs<T, W, KB, NTH>;
#pragma unroll
  for (int u = 0; u < SR::NI; ++u) {
    const int it = u * NTH + int(threadIdx.x);
    const int g8 = it % SR::NG;
    const int s = 4 * ((it < SR::NQ * SR::NG ? it : 0) / SR::NG);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // no guard: rows past the chunk end are clamped to its last row
      const int row = s + t < L ? s + t : L - 1;
      st.v[u][t] = Ops<T>::gld8u(src + int64_t(row) * stride_t + 8 * g8);
    }
  }
}

// Write the loaded tile transposed into dst[W][RS] (token index contiguous), token s scaled
// by scale[s] when given; when dst2 is given, a second copy scaled by scale2[s] goes there.
template <typename T, int W, int KB, int RS, int NTH>
__device__ __forceinline__ void stage_store(const StageRegs<T, W, KB, NTH>& st,
                                            typename Ops<T>::lds_t* dst, const float* scale,
                                            typename Ops<T>::lds_t* dst2 = nullptr,
                                            const float* scale2 = nullptr) {
  using SR = StageRegs<T, W, KB, NTH>;
#pragma unroll
  for (int u = 0; u < SR::NI; ++u) {
    const int it = u * NTH + int(threadIdx.x);
    if (it >= SR::NQ * SR::NG) break;
    const int g8 = it % SR::NG, s = 4 * (it / SR::NG);
    float sc[4], sc2[4];
    if (scale) {
#pragma unroll
      for (int t = 0; t < 4; ++t) sc[t] = scale[s + t];
    }
    if (dst2) {
#pragma unroll
      for (int t = 0; t < 4; ++t) sc2[t] = scale2[s + t];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      put4<T>(dst + (8 * g8 + j) * RS + s, st.v[u], j, scale ? sc : nullptr);
      if (dst2) put4<T>(dst2 + (8 * g8 + j) * RS + s, st.v[u], j, sc2);
    }
  }
}

// ---------------------------------------------------------------------------------------
// k_chunk_prep: per (chunk, group) C.B^T (lower-triangular 16x16 tiles, incl. the diagonal)
// and B^T, both in the input dtype, shared by every head of the group
// ---------------------------------------------------------------------------------------
constexpr int kPrepSplit = 2;   // workgroups per (chunk, group) in k_chunk_prep

template <typename T, int N, int CS>
__global__ __launch_bounds__(256) void k_chunk_prep(PrefillParams p) {
  using O = Ops<T>;
  using lds_t = typename O::lds_t;
  using frag = typename O::frag;
  constexpr int NW = 4;
  constexpr int NP = N < 32 ? 32 : N;    // dstate padded to the MFMA K of 32
  constexpr int RSB = NP + O::kPad;
  constexpr int KN = NP / 32, NT = CS / 16;
  __shared__ __attribute__((aligned(16))) lds_t Bs[CS * RSB];

  const int k = blockIdx.x, g = blockIdx.y, z = blockIdx.z, tid = threadIdx.x;
  int cs0, L, r;
  if (!chunk_bounds(p, k, CS, cs0, L, r)) {
    if (tid == 0 && g == 0 && z == 0) raise_flag(p.flag, SSD_DEVERR_CHUNK_RANGE);
    return;
  }
  const T* bsrc = static_cast<const T*>(p.B) + int64_t(cs0) * p.bc_st + int64_t(g) * N;
  for (int e = tid; e < CS * (NP / 8); e += 256) {
    const int s = e / (NP / 8), c8 = e % (NP / 8);
    const frag v = O::gld8(bsrc + int64_t(s) * p.bc_st + 8 * c8, s < L && 8 * c8 < N);
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<u32x4_v*>(&Bs[s * RSB + 8 * c8]) = u32x4_v{v.w[0], v.w[1], v.w[2], v.w[3]};
    } else {
      *reinterpret_cast<float4_v*>(&Bs[s * RSB + 8 * c8]) = float4_v{v.v[0], v.v[1], v.v[2], v.v[3]};
      *reinterpret_cast<float4_v*>(&Bs[s * RSB + 8 * c8 + 4]) = float4_v{v.v[4], v.v[5], v.v[6], v.v[7]};
    }
  }
  __syncthreads();

  // B^T [N][CS] (this workgroup's half of the rows): lanes walk n fastest (conflict-free
  // LDS column reads)
  constexpr int NH = N / kPrepSplit;
  T* bt = static_cast<T*>(p.btw) + (int64_t(k) * p.G + g) * N * CS;
  for (int e = tid; e < NH * (CS / 8); e += 256) {
    const int n = z * NH + e % NH, s8 = e / NH;
    if constexpr (sizeof(T) == 2) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = uint32_t(Bs[(8 * s8 + 2 * j) * RSB + n]) | (uint32_t(Bs[(8 * s8 + 2 * j + 1) * RSB + n]) << 16);
      *reinterpret_cast<u32x4_v*>(bt + int64_t(n) * CS + 8 * s8) = u32x4_v{w[0], w[1], w[2], w[3]};
    } else {
      float w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = Bs[(8 * s8 + j) * RSB + n];
      *reinterpret_cast<float4_v*>(bt + int64_t(n) * CS + 8 * s8) = float4_v{w[0], w[1], w[2], w[3]};
      *reinterpret_cast<float4_v*>(bt + int64_t(n) * CS + 8 * s8 + 4) = float4_v{w[4], w[5], w[6], w[7]};
    }
  }

  // C.B^T tiles, computed transposed (rows s, columns l) so a lane ends up with four
  // consecutive s of one row l: CB[l][s0 + 4*(L/16) + r].
  const int wave = tid >> 6, lane = tid & 63, li = lane & 15, kg = lane >> 4;
  const T* csrc = static_cast<const T*>(p.Cm) + int64_t(cs0) * p.bc_st + int64_t(g) * N;
  T* cb = static_cast<T*>(p.cbw) + (int64_t(k) * p.G + g) * CS * CS;
  float* cb_dbg = p.cb_out ? p.cb_out + (int64_t(k) * p.G + g) * CS * CS : nullptr;
  using TS = TileSet<NT, NW * kPrepSplit>;
#pragma unroll 1
  for (int q = 0; q < TS::kPer; ++q) {
    const int i = TS::tile(z * NW + wave, q);
    if (i >= NT) continue;
    const int lrow = 16 * i + li;
    frag cf[KN];
#pragma unroll
    for (int kk = 0; kk < KN; ++kk)
      cf[kk] = O::gld8(csrc + int64_t(lrow) * p.bc_st + 32 * kk + 8 * kg,
                       lrow < L && 32 * kk + 8 * kg < N);
    for (int j = 0; j <= i; ++j) {
      f32x4_v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KN; ++kk)
        acc = O::mma(O::ld8(&Bs[(16 * j + li) * RSB + 32 * kk + 8 * kg]), cf[kk], acc);
      T* dst = cb + int64_t(lrow) * CS + 16 * j + 4 * kg;
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<u32x2_v*>(dst) = u32x2_v{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
      } else {
        *reinterpret_cast<float4_v*>(dst) = float4_v{acc[0], acc[1], acc[2], acc[3]};
      }
      if (cb_dbg && lrow < L) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          if (16 * j + 4 * kg + rr <= lrow) cb_dbg[int64_t(lrow) * CS + 16 * j + 4 * kg + rr] = acc[rr];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// k_chunk_march: one workgroup per (head, sequence) walks the sequence's chunks in order
// with the fp32 state held in registers.  For chunk k with incoming state H_in:
//   y_l   = exp(c_l) C_l . H_in[p, :] + sum_{s<=l} CB_{l,s} exp(c_l - c_s) delta_s x_s + D x_l
//   H_out = exp(c_last) H_in + sum_s delta_s exp(c_last - c_s) x_s B_s^T
// and H_out is the checkpoint written at the chunk end (prefix caching, "why this design",
// item 3).  The intra-chunk sums are split at 32-token blocks b with reference
// r_b = 32b + 31: x is staged twice in LDS, raw (x^T) and as X~_s = exp(c_{r(s)} - c_s)
// delta_s x_s (X~^T).
//   * y, blocks entirely before the row's 16-row tile: raw C.B^T tiles against X~; the
//     running sum is rescaled by exp(c_{r_b} - c_{r_{b-1}}) per block and joins the row
//     with exp(c_l - c_{r_last});
//   * y, the block holding the diagonal: exp(c_l - c_s) per element, causal mask, raw x;
//   * H_out: X~^T against B^T with the same running rescale, which ends at the chunk's
//     last token (exp(c_last - c_last) = 1).
// Every factor is an exp of a non-positive cumsum difference (delta >= 0, A <= 0).
//
// Work split (2*CS threads, NW = CS/32 waves): wave w owns the 16-row y tiles w and
// NT-1-w (equal causal work) and the state columns n-tile w, w+NW, ... for every p-tile;
// the state lives in the MFMA result layout of X~^T B^T.  The next chunk's x rows and
// delta (the HBM stream) are requested as soon as the current ones sit in LDS, so HBM
// keeps streaming while the MFMAs run; the L2-resident operands (C.B^T, B^T, C rows) are
// requested at the top of each chunk.
// ---------------------------------------------------------------------------------------
template <typename T, int P, int N, int CS>
struct MarchCfg {
  static constexpr int NW = CS / 32, NTH = 64 * NW, NT = CS / 16;
  static constexpr int NP = N < 32 ? 32 : N;
  static constexpr int RSX = CS + Ops<T>::kPad, RSB = NP + Ops<T>::kPad, RSY = P + Ops<T>::kPad;
  static constexpr int TP = P / 16, TN = N / 16, NTW = (TN + NW - 1) / NW, KN = NP / 32;
  static constexpr int NSTEP = CS / 32;
  static constexpr int F0 = (NW - 1) / 2 + 1, F1 = NW;   // C.B^T fragment slots per y tile
};

// Operand fragments of one chunk held in registers by one wave.
template <typename T, int P, int N, int CS>
struct MarchFrags {
  using M = MarchCfg<T, P, N, CS>;
  using frag = typename Ops<T>::frag;
  StageRegs<T, P, CS, M::NTH> x;
  T dt;     // raw, converted where it is used
  frag cb0[M::F0], cb1[M::F1];
  frag bt[M::NSTEP][M::NTW];
  frag cf[2][M::KN];
};

struct ChunkLoc {
  int cs0, L;
};

template <typename T, int P, int N, int CS>
__device__ __forceinline__ void march_load_x(MarchFrags<T, P, N, CS>& f, const PrefillParams& p,
                                             ChunkLoc c, int h) {
  const T* xsrc = static_cast<const T*>(p.x) + int64_t(c.cs0) * p.x_st + int64_t(h) * P;
  stage_load(f.x, xsrc, p.x_st, c.L);
  const int row = int(threadIdx.x) < c.L ? int(threadIdx.x) : c.L - 1;
  f.dt = static_cast<const T*>(p.dt)[int64_t(c.cs0 + row) * p.dt_st + h];
}

template <typename T, int P, int N, int CS>
__device__ __forceinline__ void march_load_cb(MarchFrags<T, P, N, CS>& f, const PrefillParams& p,
                                              ChunkLoc c, int k, int g, const int* tiles) {
  using M = MarchCfg<T, P, N, CS>;
  const int li = threadIdx.x & 15, kg = (threadIdx.x & 63) >> 4;
  const T* cbrows = static_cast<const T*>(p.cbw) + (int64_t(k) * p.G + g) * CS * CS;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = tiles[q], bd = i / 2;
    const T* cbr = cbrows + int64_t(16 * i + li) * CS;
    constexpr int nf0 = M::F0, nf1 = M::F1;
#pragma unroll
    for (int b = 0; b < nf1; ++b) {
      if (q == 0 && b >= nf0) break;
      const int nf = q == 0 ? nf0 : nf1;
      const int blk = b == nf - 1 ? bd : b;   // last slot: the diagonal block
      const typename Ops<T>::frag v =
          Ops<T>::gld44(cbr + 32 * blk + 4 * kg, cbr + 32 * blk + 16 + 4 * kg);
      if (q == 0) f.cb0[b] = v; else f.cb1[b] = v;
    }
  }
}

template <typename T, int P, int N, int CS>
__device__ __forceinline__ void march_load_bt(MarchFrags<T, P, N, CS>& f, const PrefillParams& p,
                                              int k, int g) {
  using M = MarchCfg<T, P, N, CS>;
  const int wave = threadIdx.x >> 6, li = threadIdx.x & 15, kg = (threadIdx.x & 63) >> 4;
  const T* bt = static_cast<const T*>(p.btw) + (int64_t(k) * p.G + g) * N * CS;
#pragma unroll
  for (int ss = 0; ss < M::NSTEP; ++ss)
#pragma unroll
    for (int q = 0; q < M::NTW; ++q) {
      const int nt = wave + M::NW * q < M::TN ? wave + M::NW * q : M::TN - 1;
      f.bt[ss][q] = Ops<T>::gld8u(bt + int64_t(nt * 16 + li) * CS + 32 * ss + 8 * kg);
    }
}

template <typename T, int P, int N, int CS>
__device__ __forceinline__ void march_load_c(MarchFrags<T, P, N, CS>& f, const PrefillParams& p,
                                             ChunkLoc c, int g, const int* tiles) {
  using M = MarchCfg<T, P, N, CS>;
  const int li = threadIdx.x & 15, kg = (threadIdx.x & 63) >> 4;
  const T* cbase = static_cast<const T*>(p.Cm) + int64_t(c.cs0) * p.bc_st + int64_t(g) * N;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int lrow = 16 * tiles[q] + li < c.L ? 16 * tiles[q] + li : c.L - 1;
#pragma unroll
    for (int kk = 0; kk < M::KN; ++kk) {
      const int col = 32 * kk + 8 * kg < N ? 32 * kk + 8 * kg : 0;
      f.cf[q][kk] = Ops<T>::gld8u(cbase + int64_t(lrow) * p.bc_st + col);
    }
  }
}

template <typename T, int P, int N, int CS>
__global__ __launch_bounds__(CS * 2) void k_chunk_march(PrefillParams p) {
  using O = Ops<T>;
  using lds_t = typename O::lds_t;
  using frag = typename O::frag;
  using M = MarchCfg<T, P, N, CS>;
  constexpr int NW = M::NW, NTH = M::NTH, NT = M::NT, NP = M::NP;
  constexpr int RSX = M::RSX, RSB = M::RSB, RSY = M::RSY;
  constexpr int TP = M::TP, TN = M::TN, NTW = M::NTW, KN = M::KN, NSTEP = M::NSTEP;
  constexpr int F0 = M::F0, F1 = M::F1;
  static_assert(CS <= 256 && CS % 64 == 0, "chunk size");
  __shared__ __attribute__((aligned(16))) lds_t xT[P * RSX];    // raw x^T
  __shared__ __attribute__((aligned(16))) lds_t xv[P * RSX];    // X~^T
  __shared__ __attribute__((aligned(16))) lds_t Hs[P * RSB];    // incoming state, bf16
  __shared__ __attribute__((aligned(16))) lds_t ystage[NW * 16 * RSY];
  __shared__ float s_c[CS];
  __shared__ float s_d[CS];
  __shared__ float s_v[CS];
  __shared__ float s_scan[NW];

  const int h = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, li = lane & 15, kg = lane >> 4;
  const int hpg = p.H / p.G, g = h / hpg;
  const int tiles[2] = {wave, NT - 1 - wave};

  // the sequence's chunks; all of them are checked before anything is read or written
  const int k0 = r == 0 ? 0 : p.last_chunk[r - 1] + 1;
  const int k1 = p.last_chunk[r];
  bool ok = k0 >= 0 && k1 >= k0 && k1 < p.C;
  if (ok) {
    const int t0 = p.cu_seqlens[r], t1 = p.cu_seqlens[r + 1];
    ok = t0 >= 0 && t1 <= p.T && p.cu_chunk[k0] == t0 && p.cu_chunk[k1 + 1] == t1;
    for (int k = k0; ok && k <= k1; ++k) {
      const int L = p.cu_chunk[k + 1] - p.cu_chunk[k];
      ok = L >= 1 && L <= CS && p.seq_idx[k] == r;
    }
  }
  if (!ok) {
    if (tid == 0) raise_flag(p.flag, SSD_DEVERR_CHUNK_RANGE);
    return;
  }
  int slot = -1;
  if (p.pool && p.state_idx) {
    slot = p.state_idx[r];
    if (slot < 0 || slot >= p.num_slots) {
      if (tid == 0) raise_flag(p.flag, SSD_DEVERR_SLOT_RANGE);
      slot = -1;
    }
  }
  float* pool_h = slot >= 0 ? p.pool + int64_t(slot) * p.slot_stride + int64_t(h) * P * N : nullptr;

  // the state: lane holds H[pt*16 + 4*kg + rr][nt*16 + li] for its n-tiles nt = wave + NW*q
  f32x4_v hreg[NTW][TP];
  const bool init = pool_h && p.has_init && p.has_init[r];
#pragma unroll
  for (int q = 0; q < NTW; ++q)
#pragma unroll
    for (int pt = 0; pt < TP; ++pt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int nt = wave + NW * q;
        hreg[q][pt][rr] = (init && nt < TN)
                              ? pool_h[(pt * 16 + 4 * kg + rr) * N + nt * 16 + li]
                              : 0.f;
      }

  const float Ah = p.A[h];
  const float Dh = p.D ? p.D[h] : 0.f;
  MarchFrags<T, P, N, CS> f;
  ChunkLoc cur{p.cu_chunk[k0], p.cu_chunk[k0 + 1] - p.cu_chunk[k0]};
  march_load_x(f, p, cur, h);

  for (int k = k0; k <= k1; ++k) {
    const int L = cur.L, cs0 = cur.cs0;
    const bool more = k < k1;
    const ChunkLoc nxt = more ? ChunkLoc{p.cu_chunk[k + 1], p.cu_chunk[k + 2] - p.cu_chunk[k + 1]}
                              : cur;
    __syncthreads();   // the previous chunk is done with every LDS buffer
    // L2-resident operands of this chunk; the scan and the staging below cover their latency
    march_load_bt(f, p, k, g);
    march_load_cb(f, p, cur, k, g, tiles);

    // incoming state as bf16 for the inter-chunk MFMA
#pragma unroll
    for (int q = 0; q < NTW; ++q) {
      const int nt = wave + NW * q;
      if (nt >= TN) continue;
#pragma unroll
      for (int pt = 0; pt < TP; ++pt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) Hs[(pt * 16 + 4 * kg + rr) * RSB + nt * 16 + li] = O::cvt(hreg[q][pt][rr]);
    }
    if constexpr (NP > N) {   // the padding columns of H must be zero for the K=32 MFMA
      for (int e = tid; e < P * (NP - N); e += NTH)
        Hs[(e / (NP - N)) * RSB + N + e % (NP - N)] = O::cvt(0.f);
    }

    // delta, cumsum, staging scale
    const float d = tid < L ? p.prep(to_f32(f.dt), h) : 0.f;
    const float c = block_inclusive_scan(d * Ah, s_scan);
    if (tid < CS) {
      s_c[tid] = c;
      s_d[tid] = d;
    }
    __syncthreads();
    if (tid < CS) {
      const int ref = (tid | 31) < CS ? (tid | 31) : CS - 1;
      s_v[tid] = d * fast_exp(s_c[ref] - c);
    }
    if (tid < L && p.dA_cumsum_out) p.dA_cumsum_out[int64_t(h) * p.T + cs0 + tid] = c;
    __syncthreads();
    stage_store<T, P, CS, RSX, NTH>(f.x, xT, nullptr, xv, s_v);
    __syncthreads();
    const float c_last = s_c[L - 1];
    if (more) march_load_x(f, p, nxt, h);

    // the chunk's own state X~^T B^T with the running block rescale
    f32x4_v sacc[NTW][TP];
#pragma unroll
    for (int q = 0; q < NTW; ++q)
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) sacc[q][pt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ss = 0; ss < NSTEP; ++ss) {
      if (ss > 0) {
        const float al = fast_exp(s_c[32 * ss + 31] - s_c[32 * ss - 1]);
#pragma unroll
        for (int q = 0; q < NTW; ++q)
#pragma unroll
          for (int pt = 0; pt < TP; ++pt) sacc[q][pt] *= al;
      }
      frag a[TP];
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) a[pt] = O::ld8(&xv[(pt * 16 + li) * RSX + 32 * ss + 8 * kg]);
#pragma unroll
      for (int q = 0; q < NTW; ++q) {
        if (TN % NW == 0 || wave + NW * q < TN) {
#pragma unroll
          for (int pt = 0; pt < TP; ++pt) sacc[q][pt] = O::mma(a[pt], f.bt[ss][q], sacc[q][pt]);
        }
      }
    }
    // H_out = exp(c_last) H_in + S_k: the checkpoint at the chunk end
    const float dec = fast_exp(c_last);
    const int64_t cbase = (int64_t(k) * p.H + h) * (P * N);
#pragma unroll
    for (int q = 0; q < NTW; ++q) {
      const int nt = wave + NW * q;
      if (nt >= TN) continue;
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        hreg[q][pt] = dec * hreg[q][pt] + sacc[q][pt];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int e = (pt * 16 + 4 * kg + rr) * N + nt * 16 + li;
          if (p.states) p.states[cbase + e] = hreg[q][pt][rr];
          if (p.local_states_out) p.local_states_out[cbase + e] = sacc[q][pt][rr];
        }
      }
    }
    march_load_c(f, p, cur, g, tiles);

    // y, one 16-row tile at a time: inter-chunk term, intra-chunk terms, skip connection,
    // then whole rows out through the wave's staging tile
    T* ybase = static_cast<T*>(p.y) + int64_t(cs0) * p.y_st + int64_t(h) * P;
    lds_t* yst = ystage + wave * 16 * RSY;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int i = tiles[q];
      if (16 * i >= L) continue;
      const int l0 = 16 * i, lrow = l0 + li, bd = i / 2;
      // inter-chunk term: exp(c_l) C_l . H_in[p, :]
      f32x4_v acc[TP];
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) acc[pt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) {
#pragma unroll
        for (int pt = 0; pt < TP; ++pt)
          acc[pt] = O::mma(f.cf[q][kk], O::ld8(&Hs[(pt * 16 + li) * RSB + 32 * kk + 8 * kg]), acc[pt]);
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float e = fast_exp(s_c[l0 + 4 * kg + rr]);
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) acc[pt][rr] *= e;
      }
      // blocks entirely before this tile, with the running rescale
      if (bd > 0) {
        f32x4_v acc2[TP];
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) acc2[pt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < F1 - 1; ++b) {
          if (b >= bd || (q == 0 && b >= F0 - 1)) break;
          if (b > 0) {
            const float al = fast_exp(s_c[32 * b + 31] - s_c[32 * b - 1]);
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) acc2[pt] *= al;
          }
          const frag& a = q == 0 ? f.cb0[b] : f.cb1[b];
#pragma unroll
          for (int pt = 0; pt < TP; ++pt) {
            const lds_t* xr = &xv[(pt * 16 + li) * RSX + 32 * b + 4 * kg];
            acc2[pt] = O::mma(a, O::ld44(xr, xr + 16), acc2[pt]);
          }
        }
        const float cref = s_c[32 * bd - 1];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float fct = fast_exp(s_c[l0 + 4 * kg + rr] - cref);
#pragma unroll
          for (int pt = 0; pt < TP; ++pt) acc[pt][rr] += fct * acc2[pt][rr];
        }
      }
      // the block holding the diagonal: exact decay per element, causal mask
      {
        const int s0 = 32 * bd;
        const frag& cbd = q == 0 ? f.cb0[F0 - 1] : f.cb1[F1 - 1];
        const float c_l = s_c[lrow];
        float m[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int sj = s0 + (j < 4 ? 4 * kg + j : 16 + 4 * kg + (j - 4));
          const float val = O::val(cbd, j) * fast_exp(c_l - s_c[sj]) * s_d[sj];
          m[j] = sj <= lrow ? val : 0.f;
        }
        const frag mf = O::from8(m);
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
          const lds_t* xr = &xT[(pt * 16 + li) * RSX + s0 + 4 * kg];
          acc[pt] = O::mma(mf, O::ld44(xr, xr + 16), acc[pt]);
        }
      }
      // skip connection, then the tile leaves as whole rows
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int l = l0 + 4 * kg + rr;
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
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

    cur = nxt;
  }

  // final state back to the pool slot (read at the start by this same workgroup)
  if (pool_h && p.write_final) {
#pragma unroll
    for (int q = 0; q < NTW; ++q) {
      const int nt = wave + NW * q;
      if (nt >= TN) continue;
#pragma unroll
      for (int pt = 0; pt < TP; ++pt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          pool_h[(pt * 16 + 4 * kg + rr) * N + nt * 16 + li] = hreg[q][pt][rr];
    }
  }
}

// ---------------------------------------------------------------------------------------
// launch table (same order as kChunkedShapes)
// ---------------------------------------------------------------------------------------
template <typename T, int P, int N, int CS>
static hipError_t run_chunked(const PrefillParams& p, hipStream_t s, void* const* ev) {
  record_event(ev, 0, s);
  hipLaunchKernelGGL((k_chunk_prep<T, N, CS>), dim3(p.C, p.G, kPrepSplit), dim3(256), 0, s, p);
  record_event(ev, 1, s);
  hipLaunchKernelGGL((k_chunk_march<T, P, N, CS>), dim3(p.H, p.S), dim3(CS * 2), 0, s, p);
  record_event(ev, 2, s);
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
