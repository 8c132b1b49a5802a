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
//   k_chunk_prep   per (chunk, group): delta and the chunk-local cumsum c of delta*A of the
//                  group's heads (one wavefront scan per head), and B^T and the
//                  lower-triangular C.B^T blocks in the input dtype, written in
//                  MFMA-fragment order and shared by every head of the group
//   k_chunk_march  per (head, sequence, slice of the head dim): walks the sequence's chunks
//                  with the fp32 state in registers, producing y, the state after every
//                  chunk (the prefix-caching checkpoint, "why this design", item 3) and the
//                  final state for the pool
// The contractions run on bf16 MFMA with fp32 accumulation; the state and its decay stay
// fp32.  Decay factors are products of exp of cumsum differences that are all <= 0 for
// A <= 0 and delta >= 0 (never exp(+c) * exp(-c)), so they stay in [0, 1].
//
// MFMA fragments (v_mfma_f32_16x16x32_bf16; fp32 inputs use 8 x v_mfma_f32_16x16x4_f32 on
// the same 8-values-per-lane fragments): lane L supplies row (A) or column (B) L%16 and
// the contracted indices 8*(L/16) + j, j = 0..7; the 16x16 fp32 result gives lane L rows
// 4*(L/16) + r of column L%16.  The march kernel computes y transposed (rows p, columns l)
// so that a lane's result is four consecutive p of one token row, stored directly.
#include "ssd_params.h"

namespace ssd {

// ---------------------------------------------------------------------------------------
// operand traits: bf16 inputs run bf16 MFMA, fp32 inputs run fp32 MFMA
// ---------------------------------------------------------------------------------------
template <typename T> struct Ops;

template <> struct Ops<bf16_t> {
  using lds_t = bf16_t;
  using frag = Frag8;
  static constexpr int kPad = 8;  // 16 B of row padding
  static __device__ __forceinline__ frag ld8(const lds_t* q) {
    const u32x4_v v = *reinterpret_cast<const u32x4_v*>(q);
    return frag{{v.x, v.y, v.z, v.w}};
  }
  static __device__ __forceinline__ frag from8(const float* v) {
    return frag{{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                 pack_bf16x2(v[6], v[7])}};
  }
  // 8 consecutive global elements (16 B aligned), always loaded: callers pass a valid
  // address and mask the values where they are used
  static __device__ __forceinline__ frag gld8u(const bf16_t* q) {
    const u32x4_v v = *reinterpret_cast<const u32x4_v*>(q);
    return frag{{v.x, v.y, v.z, v.w}};
  }
  // 8 consecutive global elements (16 B aligned), zeros when !ok
  static __device__ __forceinline__ frag gld8(const bf16_t* q, bool ok) {
    if (!ok) return frag{{0u, 0u, 0u, 0u}};
    return gld8u(q);
  }
  static __device__ __forceinline__ void st8(bf16_t* q, const frag& f) {
    *reinterpret_cast<u32x4_v*>(q) = u32x4_v{f.w[0], f.w[1], f.w[2], f.w[3]};
  }
  // four fp32 values -> 4 consecutive elements
  static __device__ __forceinline__ void st4(bf16_t* q, f32x4_v v) {
    *reinterpret_cast<u32x2_v*>(q) = u32x2_v{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
  static __device__ __forceinline__ f32x4_v mma(const frag& a, const frag& b, f32x4_v c) {
    return mma_bf16(a, b, c);
  }
  // four fp32 values -> 4 consecutive LDS elements
  static __device__ __forceinline__ void st4lds(lds_t* q, f32x4_v v) { st4(q, v); }
  static __device__ __forceinline__ lds_t cvt(float v) { return f32_to_bf16(v); }
  static __device__ __forceinline__ float val(const frag& f, int j) {
    return bf16_to_f32(bf16_t(f.w[j >> 1] >> ((j & 1) * 16)));
  }
  // elements j of four fragments, scaled, as 4 consecutive LDS elements
  static __device__ __forceinline__ void put4(lds_t* d, const frag* v, int j, const float* sc) {
    *reinterpret_cast<u32x2_v*>(d) =
        u32x2_v{pack_bf16x2(val(v[0], j) * sc[0], val(v[1], j) * sc[1]),
                pack_bf16x2(val(v[2], j) * sc[2], val(v[3], j) * sc[3])};
  }
  // the same, unscaled (a pure 16-bit shuffle)
  static __device__ __forceinline__ void put4raw(lds_t* d, const frag* v, int j) {
    const uint32_t sh = (j & 1) * 16;
    const uint32_t e0 = (v[0].w[j >> 1] >> sh) & 0xffffu, e1 = (v[1].w[j >> 1] >> sh) & 0xffffu;
    const uint32_t e2 = (v[2].w[j >> 1] >> sh) & 0xffffu, e3 = (v[3].w[j >> 1] >> sh) & 0xffffu;
    *reinterpret_cast<u32x2_v*>(d) = u32x2_v{e0 | (e1 << 16), e2 | (e3 << 16)};
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
  static __device__ __forceinline__ frag from8(const float* v) {
    return frag{{v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]}};
  }
  static __device__ __forceinline__ frag gld8u(const float* q) { return ld8(q); }
  static __device__ __forceinline__ frag gld8(const float* q, bool ok) {
    if (!ok) return frag{{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}};
    return ld8(q);
  }
  static __device__ __forceinline__ void st8(float* q, const frag& f) {
    *reinterpret_cast<float4_v*>(q) = float4_v{f.v[0], f.v[1], f.v[2], f.v[3]};
    *reinterpret_cast<float4_v*>(q + 4) = float4_v{f.v[4], f.v[5], f.v[6], f.v[7]};
  }
  static __device__ __forceinline__ void st4(float* q, f32x4_v v) {
    *reinterpret_cast<float4_v*>(q) = float4_v{v[0], v[1], v[2], v[3]};
  }
  static __device__ __forceinline__ f32x4_v mma(const frag& a, const frag& b, f32x4_v c) {
    return mma_f32(a, b, c);
  }
  static __device__ __forceinline__ void st4lds(lds_t* q, f32x4_v v) { st4(q, v); }
  static __device__ __forceinline__ lds_t cvt(float v) { return v; }
  static __device__ __forceinline__ float val(const frag& f, int j) { return f.v[j]; }
  static __device__ __forceinline__ void put4(lds_t* d, const frag* v, int j, const float* sc) {
    *reinterpret_cast<float4_v*>(d) = float4_v{v[0].v[j] * sc[0], v[1].v[j] * sc[1],
                                               v[2].v[j] * sc[2], v[3].v[j] * sc[3]};
  }
  static __device__ __forceinline__ void put4raw(lds_t* d, const frag* v, int j) {
    *reinterpret_cast<float4_v*>(d) = float4_v{v[0].v[j], v[1].v[j], v[2].v[j], v[3].v[j]};
  }
};

// Raw buffer resource over a wave-uniform base (gfx9 descriptor: 32-bit data format, no
// swizzle): loads through it take a scalar offset plus one 32-bit vector offset, so the
// per-load address math is a scalar add.  Offsets must stay below 2^31 bytes.
struct BufRes {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ explicit BufRes(const void* base)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff,
                                            0x00020000)) {}
  __device__ __forceinline__ u32x4_v ld16(uint32_t voff, uint32_t soff) const {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  }
};

// 8 consecutive elements at byte offset voff + soff of a buffer
template <typename T>
__device__ __forceinline__ typename Ops<T>::frag buf_ld8(const BufRes& b, uint32_t voff, uint32_t soff) {
  if constexpr (sizeof(T) == 2) {
    const u32x4_v v = b.ld16(voff, soff);
    return Frag8{{v.x, v.y, v.z, v.w}};
  } else {
    const u32x4_v v0 = b.ld16(voff, soff), v1 = b.ld16(voff + 16, soff);
    return Frag8f{{__uint_as_float(v0.x), __uint_as_float(v0.y), __uint_as_float(v0.z),
                   __uint_as_float(v0.w), __uint_as_float(v1.x), __uint_as_float(v1.y),
                   __uint_as_float(v1.z), __uint_as_float(v1.w)}};
  }
}

// Fragment f (64 lanes x 8 values, stored contiguously) of a buffer; lane_b = this lane's
// byte offset inside a fragment.
template <typename T>
__device__ __forceinline__ typename Ops<T>::frag ld_frag(const BufRes& b, int f, uint32_t lane_b) {
  return buf_ld8<T>(b, lane_b, uint32_t(f) * (512 * sizeof(T)));
}

// One y^T tile of a lane: acc[pt] holds p = pt*16 + 4*kg + 0..3 of token row l.  With two
// p-tiles in bf16, lanes kg and kg^1 (lane ^ 16) swap halves so each lane stores 8
// consecutive p (16 bytes): even kg keeps p-tile 0, odd kg keeps p-tile 1.
template <typename T, int TPW>
__device__ __forceinline__ void store_yt(T* ybase, int64_t y_st, int l, int L, int kg,
                                         const f32x4_v* acc) {
  if constexpr (sizeof(T) == 2 && TPW == 2) {
    const bool odd = kg & 1;
    const uint32_t u0 = pack_bf16x2(acc[0][0], acc[0][1]), u1 = pack_bf16x2(acc[0][2], acc[0][3]);
    const uint32_t w0 = pack_bf16x2(acc[1][0], acc[1][1]), w1 = pack_bf16x2(acc[1][2], acc[1][3]);
    // send the p-tile the partner keeps
    const uint32_t r0 = __builtin_amdgcn_ds_swizzle(int(odd ? u0 : w0), 0x1F | (16 << 10));
    const uint32_t r1 = __builtin_amdgcn_ds_swizzle(int(odd ? u1 : w1), 0x1F | (16 << 10));
    if (l < L) {
      const u32x4_v v = odd ? u32x4_v{r0, r1, w0, w1} : u32x4_v{u0, u1, r0, r1};
      const int col = odd ? 16 + 4 * (kg - 1) : 4 * kg;
      *reinterpret_cast<u32x4_v*>(ybase + int64_t(l) * y_st + col) = v;
    }
  } else {
    if (l < L) {
#pragma unroll
      for (int pt = 0; pt < TPW; ++pt) Ops<T>::st4(ybase + int64_t(l) * y_st + pt * 16 + 4 * kg, acc[pt]);
    }
  }
}

__device__ __forceinline__ void st_f4(float* q, f32x4_v v) {
  *reinterpret_cast<float4_v*>(q) = float4_v{v[0], v[1], v[2], v[3]};
}

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

// The transposed x tiles in LDS are [column p][token s]; token groups of 16 are XOR-ed with
// bits 3..4 of p, which spreads the staging writes of consecutive column groups over all
// banks and keeps every 8-token fragment contiguous and 16 B aligned.
__device__ __forceinline__ int xsw(int p, int s) { return s ^ (((p >> 3) & 3) << 4); }

// ---------------------------------------------------------------------------------------
// Chunk-local cumsum (dA cumsum) and the march's sequence order, both produced inside
// k_chunk_prep.
// ---------------------------------------------------------------------------------------
// The march kernel walks each sequence's chunks in order, so a long sequence is a serial
// chain: its workgroups are dispatched first (longest first, ties by index) so the chain
// starts at once and shorter sequences fill the remaining slots.  The order is computed by
// one workgroup of k_chunk_prep (a rank count over at most kOrderMaxSeqs sequences;
// larger batches keep the given order).  `nch` is kOrderMaxSeqs ints of LDS.
constexpr int kOrderMaxSeqs = kChainOrderMaxSeqs;

__device__ __forceinline__ void sequence_order(const PrefillParams& p, int* nch, int* rank_of) {
  const int S = p.S;
  for (int r = threadIdx.x; r < S; r += blockDim.x) {
    const int n = p.last_chunk[r] - (r == 0 ? -1 : p.last_chunk[r - 1]);
    nch[r] = n < 0 ? 0 : (n > p.C ? p.C : n);
  }
  __syncthreads();
  for (int r = threadIdx.x; r < S; r += blockDim.x) {
    const int n = nch[r];
    int rank = 0;
    for (int q = 0; q < S; ++q) {
      const int m = nch[q];
      rank += (m > n) || (m == n && q < r);
    }
    p.seq_ord[rank] = r;
    rank_of[r] = rank;
  }
  __syncthreads();
}

// The chain kernel's work items: (chunk k, head h) runs as workgroup 8 * slot + x, i.e. on
// the XCD of run x (workgroups are dispatched round-robin over the 8 XCDs, starting at an
// XCD that varies from launch to launch, so the ids of one residue mod 8 share an XCD).
// The chains (sequence rank q, head h), taken in the order c = q * H + h (longest sequences
// first), are cut into 8 contiguous runs of equal work (chunks), one per XCD, and every run
// is laid out row by row: row j holds the run's chains with more than j chunks, which are a
// prefix of the run since lengths do not increase along it.  So all chunks of a chain share
// one XCD (the publisher can leave the state in its L2), the heads of a (sequence, group)
// share one XCD except at the cuts (their operand fragments are fetched into one L2 rather
// than into every one), and every predecessor sits in an earlier row of the same XCD.  Slot
// of chain c at row j: sum over the run of min(length, j), plus c minus the run's first
// chain; entries no chunk claims (bad metadata, the padding of the last rows) hold -1.
// `len_q` and `wq` are kOrderMaxSeqs + 1 ints of LDS each, `kinfo` C ints of LDS.
__device__ void chain_items(const PrefillParams& p, const int* nch, const int* rank_of, int* len_q,
                            int* wq, int* kinfo) {
  const int S = p.S, H = p.H, tid = threadIdx.x, nt = blockDim.x;
  __shared__ int cut[kXcds + 1];
  __shared__ int part[256];
  for (int i = tid; i < p.chain_grid; i += nt) p.items[i] = -1;
  for (int q = tid; q < S; q += nt) len_q[q] = nch[p.seq_ord[q]];
  // every chunk's sequence rank and position in the sequence (-1: bad metadata)
  for (int k = tid; k < p.C; k += nt) {
    const int r = p.seq_idx[k];
    int info = -1;
    if (r >= 0 && r < S) {
      const int j = k - (r == 0 ? 0 : p.last_chunk[r - 1] + 1);
      if (j >= 0 && j < nch[r]) info = rank_of[r] | (j << 10);
    }
    kinfo[k] = info;
  }
  __syncthreads();
  // wq[q] = work of the chains of ranks < q (exclusive prefix of len_q * H); S <= 4 * 256
  {
    int v[4], sum = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = 4 * tid + u;
      v[u] = q < S ? len_q[q] * H : 0;
      sum += v[u];
    }
    part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int o = tid >= off ? part[tid - off] : 0;
      __syncthreads();
      part[tid] += o;
      __syncthreads();
    }
    int run = part[tid] - sum;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = 4 * tid + u;
      if (q < S) wq[q] = run;
      run += v[u];
    }
    if (tid == 255) wq[S] = part[255];
    __syncthreads();
  }
  const int total = wq[S], nchain = S * H;
  __shared__ int wcut[kXcds + 1];
  if (tid <= kXcds) {
    // run x starts at the first chain whose work-before reaches x * total / 8
    const int target = int((int64_t(tid) * total + kXcds - 1) / kXcds);
    int lo = 0, hi = S;   // last rank with wq <= target
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (wq[mid] <= target) lo = mid;
      else hi = mid - 1;
    }
    int c = nchain, w = total;   // the chain and the work before it
    if (lo < S) {
      const int t = len_q[lo] > 0 ? min(H, (target - wq[lo] + len_q[lo] - 1) / len_q[lo]) : 0;
      c = lo * H + t;
      w = wq[lo] + t * len_q[lo];
    }
    if (tid == 0) c = 0, w = 0;
    if (tid == kXcds) c = nchain, w = total;
    cut[tid] = c;
    wcut[tid] = w;
  }
  __syncthreads();
  // one (chunk, head) item per thread and step
  const int nitem = p.C * H;
  for (int idx = tid; idx < nitem; idx += nt) {
    const int k = idx / H, h = idx - k * H;
    const int info = kinfo[k];
    if (info < 0) continue;
    const int j = info >> 10;
    const int c = (info & 1023) * H + h;
    int x = 0;
    while (x + 1 < kXcds && c >= cut[x + 1]) ++x;
    const int a = cut[x], b = cut[x + 1];
    // first rank whose chains have fewer than j chunks: chains a .. e-1 have at least j
    int lo = 0, hi = S;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (len_q[mid] >= j) lo = mid + 1;
      else hi = mid;
    }
    int e = lo * H, we = wq[lo];
    if (e <= a) e = a, we = wcut[x];
    if (e >= b) e = b, we = wcut[x + 1];
    // row j of the run starts at sum over the run of min(length, j)
    const int64_t slot = int64_t(j) * (e - a) + (wcut[x + 1] - we) + (c - a);
    const int64_t id = slot * kXcds + x;
    if (id < p.chain_grid) p.items[id] = k * H + h;
  }
}

// delta = clamp(softplus(dt + bias)) and the chunk-local inclusive cumsum c of delta*A of
// one head, one wavefront: four tokens per lane, a lane-local prefix, a wave scan.  Written
// to the workspace as [C][H][2][CS] (c then delta); positions at or past the chunk end hold
// delta = 0 and c = c_last, the flat continuation the march relies on.
template <typename T>
__device__ __forceinline__ void load_dt4(const PrefillParams& p, int cs0, int L, int h, int lane,
                                         float (&raw)[4]) {
  const T* dtp = static_cast<const T*>(p.dt);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int tok = 4 * lane + t;
    const int row = tok < L ? tok : L - 1;
    raw[t] = to_f32(dtp[int64_t(cs0 + row) * p.dt_st + h]);
  }
}

template <int CS>
__device__ __forceinline__ void cumsum_head(const PrefillParams& p, int k, int cs0, int L, int h,
                                            int lane, const float (&raw)[4]) {
  static_assert(CS <= 256 && CS % 4 == 0, "chunk size");
  const float Ah = p.A[h], bias = p.prep.bias_of(h);
  float d[4], c[4];
  float run = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    d[t] = 4 * lane + t < L ? p.prep.apply(raw[t], bias) : 0.f;
    run += d[t] * Ah;
    c[t] = run;
  }
  const float incl = wave_inclusive_scan(run);
  const float base = incl - run;
#pragma unroll
  for (int t = 0; t < 4; ++t) c[t] += base;
  if (4 * lane < CS) {
    float* dst = p.dcw + (int64_t(k) * p.H + h) * (2 * CS) + 4 * lane;
    *reinterpret_cast<float4_v*>(dst) = float4_v{c[0], c[1], c[2], c[3]};
    *reinterpret_cast<float4_v*>(dst + CS) = float4_v{d[0], d[1], d[2], d[3]};
  }
  if (p.dA_cumsum_out) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (4 * lane + t < L) p.dA_cumsum_out[int64_t(h) * p.T + cs0 + 4 * lane + t] = c[t];
  }
}

// ---------------------------------------------------------------------------------------
// k_chunk_prep: per (chunk, group) the cumsum of delta*A of the group's heads (above), and
// B^T and the C.B^T blocks the y tiles need, both in the input dtype and in MFMA-fragment
// order (one fragment = 64 lanes x 8 values, 1 KB in bf16), so a wavefront fetches a
// fragment with one contiguous load.
//   B^T fragment (n-tile nt, 32-token step ss): lane (kg, li) holds B[s = 32 ss + 8 kg + j]
//     [n = 16 nt + li]; stored at ((chunk * G + g) * TN + nt) * NSTEP + ss.
//   C.B^T fragment (row tile i, block b <= i/2): lane (kg, li) holds (C_l . B_s) for
//     l = 16 i + li, s = 32 b + 8 kg + j; stored at (chunk * G + g) * NF + cb_frag_base(i) + b.
//   C fragment (row tile i, 32-wide dstate step kk): lane (kg, li) holds C[l = 16 i + li]
//     [n = 32 kk + 8 kg + j] (zero past dstate); stored at ((chunk * G + g) * NT + i) * KN + kk.
// Rows past the chunk end are zero.  Each (chunk, group) is split over gridDim.z
// workgroups (prep_split): more of them when there are few chunks, one when there are many,
// since every workgroup of a (chunk, group) stages the whole B chunk.
// ---------------------------------------------------------------------------------------
inline int prep_split(int chunks_x_groups) {
  const int z = (512 + chunks_x_groups - 1) / chunks_x_groups;
  return z < 1 ? 1 : (z > 8 ? 8 : z);
}

template <typename T, int N, int CS>
__global__ __launch_bounds__(256) void k_chunk_prep(PrefillParams p) {
  using O = Ops<T>;
  using lds_t = typename O::lds_t;
  using frag = typename O::frag;
  constexpr int NW = 4;
  constexpr int NP = N < 32 ? 32 : N;    // dstate padded to the MFMA K of 32
  constexpr int RSB = NP + O::kPad;
  constexpr int KN = NP / 32, NT = CS / 16, NSTEP = CS / 32, TN = N / 16;
  constexpr int NF = cb_frag_base(NT);
  constexpr int TLS = 36;                 // row stride of the per-wave 16 x 32 staging tile
  __shared__ __attribute__((aligned(16))) lds_t Bs[CS * RSB];
  __shared__ __attribute__((aligned(16))) float tl[NW][16 * TLS];

  const int k = blockIdx.x, g = blockIdx.y, z = blockIdx.z, tid = threadIdx.x;
  const int zs = gridDim.z;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  if (k == p.C) {
    // the grid's extra column: one workgroup orders the sequences (and the chain's work
    // items) beside the chunks' workgroups, with its B tile as scratch
    if (g == 0 && z == 0 && p.S <= kOrderMaxSeqs) {
      static_assert(sizeof(tl) >= 2 * kOrderMaxSeqs * sizeof(int), "order scratch");
      int* nch = reinterpret_cast<int*>(&tl[0][0]);
      sequence_order(p, nch, nch + kOrderMaxSeqs);
      if constexpr (sizeof(Bs) >= (2 * (kOrderMaxSeqs + 1) + kChainOrderMaxChunks) * sizeof(int)) {
        int* scratch = reinterpret_cast<int*>(Bs);
        if (p.items) chain_items(p, nch, nch + kOrderMaxSeqs, scratch, scratch + kOrderMaxSeqs + 1,
                                 scratch + 2 * (kOrderMaxSeqs + 1));
      }
    }
    return;
  }
  // the chain kernel's publication flags of this chunk start cleared
  if (p.chain_flag && z == 0) {
    const int n = (p.H / p.G) * kChainWaves;
    for (int i = tid; i < n; i += 256)
      p.chain_flag[(int64_t(k) * p.H + g * (p.H / p.G)) * kChainWaves + i] = 0;
  }
  int cs0, L, r;
  const bool bounds_ok = chunk_bounds(p, k, CS, cs0, L, r);
  // the all cache mode: the pool slot that receives this chunk's end state when the chunk
  // closes a cache block (-1: none; at a sequence's last chunk the final write takes its
  // place when there is one)
  if (p.blk_slot && g == 0 && z == 0 && tid == 0) {
    int slot = -1;
    if (bounds_ok) {
      const int col = block_end_col(p, r, p.cu_seqlens[r], cs0, cs0 + L, true);
      if (col >= 0 && !(k == p.last_chunk[r] && p.write_final)) slot = pool_slot(p, r, col, true);
    }
    p.blk_slot[k] = slot;
  }
  if (!bounds_ok) {
    if (tid == 0 && g == 0 && z == 0) raise_flag(p.flag, SSD_DEVERR_CHUNK_RANGE);
    return;
  }
  // the chunk's B rows: every request first, into registers
  constexpr int NBI = CS * (NP / 8) / 256;
  static_assert(CS * (NP / 8) % 256 == 0, "B staging");
  const T* bsrc = static_cast<const T*>(p.B) + int64_t(cs0) * p.bc_st + int64_t(g) * N;
  frag bv[NBI];
#pragma unroll
  for (int u = 0; u < NBI; ++u) {
    const int e = u * 256 + tid, s = e / (NP / 8), c8 = e % (NP / 8);
    bv[u] = O::gld8(bsrc + int64_t(s) * p.bc_st + 8 * c8, s < L && 8 * c8 < N);
  }
  // meanwhile the cumsum of this workgroup's share of the group's heads, one wavefront per
  // head, each head's dt requested one head ahead (the chain kernel forms its own)
  if (!p.chain_flag) {
    const int hpg = p.H / p.G, hz = (hpg + zs - 1) / zs;
    const int h0 = g * hpg + z * hz, h1 = min(g * hpg + hpg, h0 + hz);
    float raw[4], nxt[4];
    int h = h0 + wave;
    if (h < h1) load_dt4<T>(p, cs0, L, h, lane, nxt);
#pragma unroll 1
    for (; h < h1; h += 4) {
#pragma unroll
      for (int t = 0; t < 4; ++t) raw[t] = nxt[t];
      if (h + 4 < h1) load_dt4<T>(p, cs0, L, h + 4, lane, nxt);
      cumsum_head<CS>(p, k, cs0, L, h, lane, raw);
    }
  }
  // the C rows of this wave's first row tile, requested before the B rows are staged
  const int li = lane & 15, kg = lane >> 4;
  const T* csrc = static_cast<const T*>(p.Cm) + int64_t(cs0) * p.bc_st + int64_t(g) * N;
  const int NWT = NW * zs, NQ = (NT + NWT - 1) / NWT;
  auto tile_of = [&](int q) {   // row tiles w = z * NW + wave, then mirrored pairs
    const int w = z * NW + wave;
    return (q / 2) * 2 * NWT + ((q & 1) ? 2 * NWT - 1 - w : w);
  };
  frag cf[KN];
  auto load_c = [&](int q) {
    const int lrow = 16 * tile_of(q) + li;
#pragma unroll
    for (int kk = 0; kk < KN; ++kk)
      cf[kk] = O::gld8(csrc + int64_t(lrow) * p.bc_st + 32 * kk + 8 * kg,
                       lrow < L && 32 * kk + 8 * kg < N);
  };
  load_c(0);
#pragma unroll
  for (int u = 0; u < NBI; ++u) {
    const int e = u * 256 + tid, s = e / (NP / 8), c8 = e % (NP / 8);
    const frag& v = bv[u];
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<u32x4_v*>(&Bs[s * RSB + 8 * c8]) = u32x4_v{v.w[0], v.w[1], v.w[2], v.w[3]};
    } else {
      *reinterpret_cast<float4_v*>(&Bs[s * RSB + 8 * c8]) = float4_v{v.v[0], v.v[1], v.v[2], v.v[3]};
      *reinterpret_cast<float4_v*>(&Bs[s * RSB + 8 * c8 + 4]) = float4_v{v.v[4], v.v[5], v.v[6], v.v[7]};
    }
  }
  __syncthreads();

  // B^T fragments, this workgroup's share
  T* bt = static_cast<T*>(p.btw) + (int64_t(k) * p.G + g) * (int64_t(N) * CS);
  for (int e = z * 256 + tid; e < TN * NSTEP * 64; e += 256 * zs) {
    const int f = e >> 6, ln = e & 63;
    const int nt = f / NSTEP, ss = f % NSTEP, li = ln & 15, kg = ln >> 4;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = to_f32(Bs[(32 * ss + 8 * kg + j) * RSB + 16 * nt + li]);
    O::st8(bt + int64_t(e) * 8, O::from8(v));
  }

  // C.B^T fragments: each 16x16 tile is computed transposed (rows s, columns l) so lane
  // (kg, li) gets C_l . B_s for l = 16 i + li, s = 16 jt + 4 kg + rr; two tiles are regrouped
  // through LDS into the 8-consecutive-s fragment of one 32-token block.
  T* cb = static_cast<T*>(p.cbw) + (int64_t(k) * p.G + g) * (int64_t(NF) * 512);
  float* cb_dbg = p.cb_out ? p.cb_out + (int64_t(k) * p.G + g) * CS * CS : nullptr;
  float* tw = tl[wave];
  // row tiles of this workgroup (tile_of), the causal work balanced by mirrored pairs
#pragma unroll 1
  for (int q = 0; q < NQ; ++q) {
    const int i = tile_of(q);
    if (i >= NT) break;   // later tiles of this wave are larger still
    if (q > 0) load_c(q);
    const int lrow = 16 * i + li;
    T* cfo = static_cast<T*>(p.cfw) + ((int64_t(k) * p.G + g) * NT + i) * (KN * 512);
#pragma unroll
    for (int kk = 0; kk < KN; ++kk) O::st8(cfo + (kk * 64 + lane) * 8, cf[kk]);
#pragma unroll 1
    for (int b = 0; b <= i / 2; ++b) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int jt = 2 * b + half;
        f32x4_v acc = {0.f, 0.f, 0.f, 0.f};
        if (jt <= i) {
#pragma unroll
          for (int kk = 0; kk < KN; ++kk)
            acc = O::mma(O::ld8(&Bs[(16 * jt + li) * RSB + 32 * kk + 8 * kg]), cf[kk], acc);
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) tw[li * TLS + 16 * half + 4 * kg + rr] = acc[rr];
        if (cb_dbg && lrow < L && jt <= i) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            if (16 * jt + 4 * kg + rr <= lrow) cb_dbg[int64_t(lrow) * CS + 16 * jt + 4 * kg + rr] = acc[rr];
        }
      }
      wave_lds_sync();
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = tw[li * TLS + 8 * kg + j];
      O::st8(cb + (int64_t(cb_frag_base(i) + b) * 64 + lane) * 8, O::from8(v));
      wave_lds_sync();
    }
  }
}

// ---------------------------------------------------------------------------------------
// k_chunk_march: one workgroup (4 wavefronts) per (head, sequence, PW-column slice of the
// head dim) walks the sequence's chunks in order with its fp32 state rows in registers.
// For chunk k with incoming state H_in:
//   y_l   = exp(c_l) C_l . H_in[p, :] + sum_{s<=l} CB_{l,s} exp(c_l - c_s) delta_s x_s + D x_l
//   H_out = exp(c_last) H_in + sum_s delta_s exp(c_last - c_s) x_s B_s^T
// and H_out is the checkpoint written at the chunk end.  The intra-chunk sums are split
// at 32-token blocks b with reference r_b = 32b + 31: x is staged twice in LDS, raw (x^T)
// and as X~_s = exp(c_{r(s)} - c_s) delta_s x_s (X~^T).
//   * y, blocks entirely before the row's 32-token block: C.B^T fragments against X~, the
//     running sum rescaled by exp(c_{r_b} - c_{r_{b-1}}) per block and joined to row l with
//     exp(c_l - c_{r_last});
//   * y, the block holding the diagonal: exp(c_l - c_s) delta_s per element, causal mask,
//     raw x, and D on the diagonal (the skip connection D x_l);
//   * H_out: X~^T against B^T with the same running rescale, which ends at the chunk's
//     last token.
// Every factor is an exp of a non-positive cumsum difference (delta >= 0, A <= 0).
// y is computed transposed (rows p, columns l): a lane's result is 4 consecutive p of one
// token, stored straight from the accumulator.
// Work split: wave w owns the row tiles {w, 7-w} (+8 for the second half of a 256-token
// chunk), which balances the causal work, and the state n-tiles [w*TNW, (w+1)*TNW).
// ---------------------------------------------------------------------------------------
template <typename T, int P, int PW, int N, int CS>
struct MarchCfg {
  static constexpr int NW = 4, NTH = 256, NT = CS / 16, NSTEP = CS / 32;
  static constexpr int NP = N < 32 ? 32 : N;
  static constexpr int RSX = CS + Ops<T>::kPad, RSB = NP + Ops<T>::kPad;
  static constexpr int TPW = PW / 16, TN = N / 16, TNW = (TN + NW - 1) / NW, KN = NP / 32;
  static constexpr int NTQ = NT / NW;                 // row tiles per wave
  static constexpr int PT = NTQ < 2 ? NTQ : 2;        // row tiles processed together
  static constexpr int NPAIR = NTQ / PT;
  static constexpr int NG = PW / 8, NITEM = NG * CS / 4, NI = (NITEM + NTH - 1) / NTH;
  static constexpr int NF = cb_frag_base(NT);
  static_assert(NT % NW == 0 && NTQ <= 4, "row tiles");
  static_assert(PW % 16 == 0 && P % PW == 0 && PW <= 32, "head-dim slice");
};

// Per-thread registers of one chunk's staging: x rows of the thread's work items and the
// cumsum / delta of their four tokens.
template <typename T, int NI>
struct StageIn {
  typename Ops<T>::frag x[NI][4];
  float4_v c[NI], d[NI];
  float cref[NI];
};

struct ChunkLoc {
  int cs0, L;
};

// The march kernel's state slice (hreg: wave w holds n-tiles [w*TNW, (w+1)*TNW) of the
// slice's PW rows) to the pool slot whose slice starts at element e.
template <int PW, int N>
__device__ __forceinline__ void march_pool_store(const PrefillParams& p, int64_t e,
                                                 const f32x4_v (&hreg)[(N / 16 + 3) / 4][PW / 16],
                                                 int wave, int li, int kg) {
  constexpr int TN = N / 16, TNW = (TN + 3) / 4, TPW = PW / 16;
  // buffer stores: the slot in a descriptor, one lane offset, the tile offset in soffset
  const int esz = p.pool_kind ? 2 : 4;
  const BufRes b(static_cast<char*>(p.pool) + e * esz);
  const uint32_t lane_e = uint32_t(li * N + 4 * kg);
#pragma unroll
  for (int q = 0; q < TNW; ++q) {
    const int nt = wave * TNW + q;
    if (nt >= TN) continue;
#pragma unroll
    for (int pt = 0; pt < TPW; ++pt) {
      const f32x4_v v = hreg[q][pt];
      const uint32_t tile_e = uint32_t(pt * 16 * N + nt * 16);
      if (p.pool_kind == SSD_BF16)
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_v{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])},
                                              b.r, lane_e * 2, tile_e * 2, 0);
      else if (p.pool_kind == SSD_F16)
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_v{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])},
                                              b.r, lane_e * 2, tile_e * 2, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_v{__float_as_uint(v[0]), __float_as_uint(v[1]),
                                                       __float_as_uint(v[2]), __float_as_uint(v[3])},
                                               b.r, lane_e * 4, tile_e * 4, 0);
    }
  }
}

// Work item `it`: columns 8*g8 .. 8*g8+7 of the slice, tokens 4*sg .. 4*sg+3.
template <typename T, int P, int PW, int N, int CS>
__device__ __forceinline__ void march_load_stage(StageIn<T, MarchCfg<T, P, PW, N, CS>::NI>& st,
                                                 const PrefillParams& p, ChunkLoc c, int k,
                                                 int h, int p0) {
  using M = MarchCfg<T, P, PW, N, CS>;
  const BufRes xr(static_cast<const T*>(p.x) + int64_t(c.cs0) * p.x_st + int64_t(h) * P + p0);
  const uint32_t xrow_b = uint32_t(p.x_st * int64_t(sizeof(T)));
  const float* dc = p.dcw + (int64_t(k) * p.H + h) * (2 * CS);
#pragma unroll
  for (int u = 0; u < M::NI; ++u) {
    int it = u * M::NTH + int(threadIdx.x);
    it = it < M::NITEM ? it : 0;
    const int g8 = it % M::NG, s = 4 * (it / M::NG);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // unguarded: rows past the chunk end repeat its last row (their weight is zero)
      const int row = s + t < c.L ? s + t : c.L - 1;
      st.x[u][t] = buf_ld8<T>(xr, uint32_t(row) * xrow_b + uint32_t(g8) * 8 * sizeof(T), 0);
    }
    st.c[u] = *reinterpret_cast<const float4_v*>(dc + s);
    st.d[u] = *reinterpret_cast<const float4_v*>(dc + CS + s);
    st.cref[u] = dc[s | 31];
  }
}

#ifndef SSD_MARCH_WAVES_PER_EU
#define SSD_MARCH_WAVES_PER_EU 3
#endif
#ifndef SSD_MARCH_BT_RING
#define SSD_MARCH_BT_RING 4
#endif
#ifndef SSD_MARCH_CB_RING
#define SSD_MARCH_CB_RING 2
#endif
#ifndef SSD_MARCH_NEXT_BEFORE_STORE
#define SSD_MARCH_NEXT_BEFORE_STORE 0
#endif
#ifndef SSD_MARCH_EARLY_PAIR0
#define SSD_MARCH_EARLY_PAIR0 1
#endif
#ifndef SSD_MARCH_PAIR_UNROLL
#define SSD_MARCH_PAIR_UNROLL 2
#endif
// Three workgroups per CU (one wavefront of each on every SIMD) hide each other's
// latencies; that caps the registers at 512 / 3 per lane.
template <typename T, int P, int PW, int N, int CS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(SSD_MARCH_WAVES_PER_EU)))
void k_chunk_march(PrefillParams p) {
  using O = Ops<T>;
  using lds_t = typename O::lds_t;
  using frag = typename O::frag;
  using M = MarchCfg<T, P, PW, N, CS>;
  constexpr int NW = M::NW, NTH = M::NTH, NT = M::NT, NP = M::NP, NSTEP = M::NSTEP;
  constexpr int RSX = M::RSX, RSB = M::RSB;
  constexpr int TPW = M::TPW, TN = M::TN, TNW = M::TNW, KN = M::KN;
  constexpr int PT = M::PT, NPAIR = M::NPAIR, NF = M::NF;
  __shared__ __attribute__((aligned(16))) lds_t xT[PW * RSX];    // raw x^T (swizzled)
  __shared__ __attribute__((aligned(16))) lds_t xv[PW * RSX];    // X~^T (swizzled)
  __shared__ __attribute__((aligned(16))) lds_t Hs[PW * RSB];    // incoming state rows
  __shared__ __attribute__((aligned(16))) float s_c[CS];
  __shared__ __attribute__((aligned(16))) float s_d[CS];

  // work item of this workgroup (see march_grid): items are ordered by sequence (dispatch
  // order), group, head in group, head-dim slice
  constexpr int PS = P / PW;
  const int tid = threadIdx.x;
  const MarchGrid mg = march_grid(p.S, p.G, p.H, PS);
  const int xcd = blockIdx.x % kXcds, xslot = blockIdx.x / kXcds;
  const int item = (xcd + kXcds * (xslot / mg.bsize)) * mg.bsize + xslot % mg.bsize;
  if (item >= mg.items) return;
  const int hpg = p.H / p.G;
  const int p0 = (item % PS) * PW;
  const int hh = (item / PS) % hpg, gi = (item / (PS * hpg)) % p.G, ry = item / (PS * p.H);
  const int h = gi * hpg + hh;
  const int r = p.S <= kOrderMaxSeqs ? ld_meta(p.seq_ord, ry) : ry;
  if (r < 0 || r >= p.S) {   // the order array comes from this launch's first kernel
    if (tid == 0) raise_flag(p.flag, SSD_DEVERR_CHUNK_RANGE);
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, li = lane & 15, kg = lane >> 4;
  const uint32_t lane_b = uint32_t(lane) * 8 * sizeof(T);   // byte offset inside a fragment
  const int g = h / (p.H / p.G);

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
  // element offset of this workgroup's state slice in a pool slot (-1: none)
  const int64_t slice_e = (int64_t(h) * P + p0) * N;
  auto slot_e = [&](int slot) { return slot >= 0 ? int64_t(slot) * p.slot_stride + slice_e : int64_t(-1); };
  const int64_t src_e = slot_e(seq_slots(p, r, true, true, tid == 0).src);

  // the state slice, held transposed (the MFMA result layout of B^T X~): lane holds
  // H[p0 + pt*16 + li][nt*16 + 4*kg + rr], nt = wave*TNW + q, i.e. 4 consecutive n of one row
  f32x4_v hreg[TNW][TPW];
  const bool init = src_e >= 0 && p.has_init && p.has_init[r];
#pragma unroll
  for (int q = 0; q < TNW; ++q)
#pragma unroll
    for (int pt = 0; pt < TPW; ++pt) {
      const int nt = wave * TNW + q;
      hreg[q][pt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
      if (init && nt < TN) {
        const float4_v v = pool_ld4(p.pool, p.pool_kind, src_e + (pt * 16 + li) * N + nt * 16 + 4 * kg);
        hreg[q][pt] = f32x4_v{v.x, v.y, v.z, v.w};
      }
    }

  const float Dh = p.D ? p.D[h] : 0.f;

  StageIn<T, M::NI> st;
  ChunkLoc cur{ld_meta(p.cu_chunk, k0), ld_meta(p.cu_chunk, k0 + 1) - ld_meta(p.cu_chunk, k0)};
  march_load_stage<T, P, PW, N, CS>(st, p, cur, k0, h, p0);

  const int64_t grp = int64_t(g);
  for (int k = k0; k <= k1; ++k) {
    const int L = cur.L, cs0 = cur.cs0;
    const bool more = k < k1;
    ChunkLoc nxt = cur;
    if (more) {
      const int e0 = ld_meta(p.cu_chunk, k + 1), e1 = ld_meta(p.cu_chunk, k + 2);
      nxt = ChunkLoc{e0, e1 - e0};
    }
    __syncthreads();   // the previous chunk is done with every LDS buffer

    // B^T fragments of this wave's n-tiles (L2-resident) for the state update below: a
    // ring of BTR steps, the first BTR - 1 requested here
    const BufRes btr(static_cast<const T*>(p.btw) + (int64_t(k) * p.G + grp) * (int64_t(N) * CS));
    constexpr int BTR = SSD_MARCH_BT_RING < NSTEP ? SSD_MARCH_BT_RING : NSTEP;
    frag btf[BTR][TNW];
    auto load_bt = [&](int ss) {
#pragma unroll
      for (int q = 0; q < TNW; ++q) {
        const int nt = wave * TNW + q < TN ? wave * TNW + q : TN - 1;
        btf[ss % BTR][q] = ld_frag<T>(btr, nt * NSTEP + ss, lane_b);
      }
    };
#pragma unroll
    for (int ss = 0; ss < BTR - 1; ++ss) load_bt(ss);

    // incoming state as MFMA operand rows
#pragma unroll
    for (int q = 0; q < TNW; ++q) {
      const int nt = wave * TNW + q;
      if (TN % NW != 0 && nt >= TN) continue;
#pragma unroll
      for (int pt = 0; pt < TPW; ++pt) O::st4lds(&Hs[(pt * 16 + li) * RSB + nt * 16 + 4 * kg], hreg[q][pt]);
    }
    if constexpr (NP > N) {   // the padding columns of H must be zero for the K=32 MFMA
      for (int e = tid; e < PW * (NP - N); e += NTH)
        Hs[(e / (NP - N)) * RSB + N + e % (NP - N)] = O::cvt(0.f);
    }

    // staging: raw x^T and X~^T, cumsum and delta
#pragma unroll
    for (int u = 0; u < M::NI; ++u) {
      const int it = u * NTH + tid;
      if (it >= M::NITEM) break;
      const int g8 = it % M::NG, s = 4 * (it / M::NG);
      const float cv[4] = {st.c[u].x, st.c[u].y, st.c[u].z, st.c[u].w};
      const float dv[4] = {st.d[u].x, st.d[u].y, st.d[u].z, st.d[u].w};
      float v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = dv[t] * fast_exp(st.cref[u] - cv[t]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col = 8 * g8 + j;
        O::put4raw(&xT[col * RSX + xsw(col, s)], st.x[u], j);
        O::put4(&xv[col * RSX + xsw(col, s)], st.x[u], j, v);
      }
      if (g8 == 0) {
        *reinterpret_cast<float4_v*>(&s_c[s]) = st.c[u];
        *reinterpret_cast<float4_v*>(&s_d[s]) = st.d[u];
      }
    }
    __syncthreads();

    // the chunk's own state X~^T B^T with the running block rescale
    f32x4_v sacc[TNW][TPW];
#pragma unroll
    for (int q = 0; q < TNW; ++q)
#pragma unroll
      for (int pt = 0; pt < TPW; ++pt) sacc[q][pt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ss = 0; ss < NSTEP; ++ss) {
      if (ss + BTR - 1 < NSTEP) load_bt(ss + BTR - 1);
      if (ss > 0) {
        const float al = fast_exp(s_c[32 * ss + 31] - s_c[32 * ss - 1]);
#pragma unroll
        for (int q = 0; q < TNW; ++q)
#pragma unroll
          for (int pt = 0; pt < TPW; ++pt) sacc[q][pt] *= al;
      }
#pragma unroll
      for (int pt = 0; pt < TPW; ++pt) {
        const int pr = pt * 16 + li;
        const frag a = O::ld8(&xv[pr * RSX + xsw(pr, 32 * ss + 8 * kg)]);
#pragma unroll
        for (int q = 0; q < TNW; ++q)
          if (TN % NW == 0 || wave * TNW + q < TN) sacc[q][pt] = O::mma(btf[ss % BTR][q], a, sacc[q][pt]);
      }
    }
    // y^T is computed PT row tiles at a time (tiles 8*pr + w and 8*pr + 7 - w).  Each pair's
    // operand fragments are requested before the stores that precede its use: loads and
    // stores share one in-order completion counter, so a load issued behind a store would
    // also wait for the store.
    const BufRes cbr(static_cast<const T*>(p.cbw) + (int64_t(k) * p.G + grp) * (int64_t(NF) * 512));
    const BufRes cfr(static_cast<const T*>(p.cfw) + (int64_t(k) * p.G + grp) * (int64_t(NT) * KN * 512));
    T* ybase = static_cast<T*>(p.y) + int64_t(cs0) * p.y_st + int64_t(h) * P + p0;
    constexpr int CBR = SSD_MARCH_CB_RING;
    frag cf[PT][KN];      // C rows of the tiles as B operands (column l, contracted n)
    frag cbd[PT];         // the diagonal blocks' C.B^T fragments
    frag cbq[PT][CBR];    // the first CBR blocks before the diagonal, then a ring refilled
                          // CBR blocks ahead (clamped requests re-read the diagonal block)
    auto pair_tiles = [&](int pr, int* ti, int* bd) {
#pragma unroll
      for (int t = 0; t < PT; ++t) {
        ti[t] = __builtin_amdgcn_readfirstlane(8 * pr + (t ? 7 - wave : wave));
        bd[t] = ti[t] / 2;
      }
    };
    auto load_pair = [&](int pr) {
      int ti[PT], bd[PT];
      pair_tiles(pr, ti, bd);
#pragma unroll
      for (int t = 0; t < PT; ++t) {
#pragma unroll
        for (int kk = 0; kk < KN; ++kk) cf[t][kk] = ld_frag<T>(cfr, ti[t] * KN + kk, lane_b);
        cbd[t] = ld_frag<T>(cbr, cb_frag_base(ti[t]) + bd[t], lane_b);
#pragma unroll
        for (int j = 0; j < CBR; ++j)
          cbq[t][j] = ld_frag<T>(cbr, cb_frag_base(ti[t]) + (j < bd[t] ? j : bd[t]), lane_b);
      }
    };
#if SSD_MARCH_EARLY_PAIR0
    load_pair(0);
#endif

    // H_out = exp(c_last) H_in + S_k: the checkpoint at the chunk end
    const float dec = fast_exp(s_c[CS - 1]);
#pragma unroll
    for (int q = 0; q < TNW; ++q)
#pragma unroll
      for (int pt = 0; pt < TPW; ++pt) hreg[q][pt] = dec * hreg[q][pt] + sacc[q][pt];
    const int64_t sbase = (int64_t(k) * p.H + h) * (int64_t(P) * N) + int64_t(p0) * N;
    if (p.blk_slot) {   // the all cache mode: a chunk that closes a cache block
      const int slot = ld_meta(p.blk_slot, k);
      if (slot >= 0 && slot < p.num_slots) march_pool_store<PW, N>(p, slot_e(slot), hreg, wave, li, kg);
    }
    if (p.states) {
#pragma unroll
      for (int q = 0; q < TNW; ++q) {
        const int nt = wave * TNW + q;
        if (TN % NW != 0 && nt >= TN) continue;
#pragma unroll
        for (int pt = 0; pt < TPW; ++pt)
          st_f4(p.states + sbase + (pt * 16 + li) * N + nt * 16 + 4 * kg, hreg[q][pt]);
      }
    }
    if (p.local_states_out) {
#pragma unroll
      for (int q = 0; q < TNW; ++q) {
        const int nt = wave * TNW + q;
        if (TN % NW != 0 && nt >= TN) continue;
#pragma unroll
        for (int pt = 0; pt < TPW; ++pt)
          st_f4(p.local_states_out + sbase + (pt * 16 + li) * N + nt * 16 + 4 * kg, sacc[q][pt]);
      }
    }

#if !SSD_MARCH_EARLY_PAIR0
    load_pair(0);
#endif
#pragma unroll SSD_MARCH_PAIR_UNROLL
    for (int pr = 0; pr < NPAIR; ++pr) {
      int ti[PT], bd[PT];
      pair_tiles(pr, ti, bd);

      // inter-chunk term: exp(c_l) H_in[p, :] . C_l
      f32x4_v acc[PT][TPW];
#pragma unroll
      for (int t = 0; t < PT; ++t)
#pragma unroll
        for (int pt = 0; pt < TPW; ++pt) acc[t][pt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KN; ++kk)
#pragma unroll
        for (int pt = 0; pt < TPW; ++pt) {
          const frag hf = O::ld8(&Hs[(pt * 16 + li) * RSB + 32 * kk + 8 * kg]);
#pragma unroll
          for (int t = 0; t < PT; ++t) acc[t][pt] = O::mma(hf, cf[t][kk], acc[t][pt]);
        }
#pragma unroll
      for (int t = 0; t < PT; ++t) {
        const float e = fast_exp(s_c[16 * ti[t] + li]);
#pragma unroll
        for (int pt = 0; pt < TPW; ++pt) acc[t][pt] *= e;
      }
      // the next chunk's x rows and cumsum (the HBM stream), requested during the last pair
      // once its C fragments are consumed
      if (pr == NPAIR - 1 && more) march_load_stage<T, P, PW, N, CS>(st, p, nxt, k + 1, h, p0);

      // blocks entirely before each tile's diagonal block, with the running rescale
      const int bmax = bd[PT - 1] > bd[0] ? bd[PT - 1] : bd[0];
      if (bmax > 0) {
        f32x4_v acc2[PT][TPW];
#pragma unroll
        for (int t = 0; t < PT; ++t)
#pragma unroll
          for (int pt = 0; pt < TPW; ++pt) acc2[t][pt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < NT / 2 - 1; ++b) {
          if (b >= bmax) break;
          const float al = b > 0 ? fast_exp(s_c[32 * b + 31] - s_c[32 * b - 1]) : 1.f;
#pragma unroll
          for (int pt = 0; pt < TPW; ++pt) {
            const int prow = pt * 16 + li;
            const frag xf = O::ld8(&xv[prow * RSX + xsw(prow, 32 * b + 8 * kg)]);
#pragma unroll
            for (int t = 0; t < PT; ++t) {
              if (b < bd[t]) acc2[t][pt] = O::mma(xf, cbq[t][b % CBR], acc2[t][pt] * al);
            }
          }
#pragma unroll
          for (int t = 0; t < PT; ++t) {
            const int bn = b + CBR < bd[t] ? b + CBR : bd[t];
            cbq[t][b % CBR] = ld_frag<T>(cbr, cb_frag_base(ti[t]) + bn, lane_b);
          }
        }
#pragma unroll
        for (int t = 0; t < PT; ++t) {
          if (bd[t] == 0) continue;
          const float f = fast_exp(s_c[16 * ti[t] + li] - s_c[32 * bd[t] - 1]);
#pragma unroll
          for (int pt = 0; pt < TPW; ++pt) acc[t][pt] += f * acc2[t][pt];
        }
      }

      // the block holding the diagonal: exact decay per element, causal mask, D on the
      // diagonal
#pragma unroll
      for (int t = 0; t < PT; ++t) {
        const int s0 = 32 * bd[t], l = 16 * ti[t] + li;
        const float cl = s_c[l];
        const float4_v c0 = *reinterpret_cast<const float4_v*>(&s_c[s0 + 8 * kg]);
        const float4_v c1 = *reinterpret_cast<const float4_v*>(&s_c[s0 + 8 * kg + 4]);
        const float4_v d0 = *reinterpret_cast<const float4_v*>(&s_d[s0 + 8 * kg]);
        const float4_v d1 = *reinterpret_cast<const float4_v*>(&s_d[s0 + 8 * kg + 4]);
        const float cs8[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const float ds8[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
        float m[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int s = s0 + 8 * kg + j;
          const float v = O::val(cbd[t], j) * fast_exp(cl - cs8[j]) * ds8[j] + (s == l ? Dh : 0.f);
          m[j] = s <= l ? v : 0.f;
        }
        const frag mf = O::from8(m);
#pragma unroll
        for (int pt = 0; pt < TPW; ++pt) {
          const int prow = pt * 16 + li;
          acc[t][pt] = O::mma(O::ld8(&xT[prow * RSX + xsw(prow, s0 + 8 * kg)]), mf, acc[t][pt]);
        }
      }

#if SSD_MARCH_NEXT_BEFORE_STORE
      // the next pair's fragments go out before this pair's stores
      if (pr + 1 < NPAIR) load_pair(pr + 1);
#endif

      // y^T tile out: lane holds p = pt*16 + 4*kg + 0..3 of token l
#pragma unroll
      for (int t = 0; t < PT; ++t) store_yt<T, TPW>(ybase, p.y_st, 16 * ti[t] + li, L, kg, acc[t]);
#if !SSD_MARCH_NEXT_BEFORE_STORE
      if (pr + 1 < NPAIR) load_pair(pr + 1);
#endif
    }

    cur = nxt;
  }

  // final state back to the pool (a slot read at the start by this same workgroup, or a
  // later entry of the sequence)
  const int64_t fin_e = slot_e(seq_slots(p, r, false, true, false).fin);
  if (fin_e >= 0) march_pool_store<PW, N>(p, fin_e, hreg, wave, li, kg);
}

// ---------------------------------------------------------------------------------------
// k_chunk_chain: the chunks of one (sequence, head) as a chain of workgroups, one per
// (chunk, head), bf16 with P = 64.  The only serial dependency of the recurrence across
// chunks is the state, H_k = exp(c_last) H_{k-1} + S_k.  Each workgroup computes its chunk's
// own state S_k from its inputs alone, then takes H_{k-1} from its predecessor (the
// chunk-end checkpoint, read back from memory), forms and publishes H_k, and only then
// evaluates y with H_{k-1} as the incoming state.  The critical path per chunk is one
// checkpoint round trip; the heavy work of all chunks runs concurrently.
//
// Per chunk (4 wavefronts; wave w owns the state columns n of its n-tiles [2w, 2w+2) and
// the y row tiles {w, 7-w, 8+w, 15-w}), with only raw x^T staged in LDS and the per-token
// weights applied to the other MFMA operand in registers:
//   * S_k^T = (B^T o w) x with w_s = delta_s exp(c_last - c_s): one reference point, the
//     chunk end, so no rescaling;
//   * y, the blocks before the diagonal block: the C.B^T fragment, whose lane holds row l,
//     scaled per token by v_s exp(c_l - c_{r(s)}) = delta_s exp(c_l - c_s), where
//     v_s = delta_s exp(c_{r(s)} - c_s) is formed once per chunk (reference r(s): the end of
//     the token's 32-token block) and exp(c_l - c_{r(s)}) once per lane and block; both
//     factors are <= 1;
//   * y, the diagonal block: exact exp(c_l - c_s) delta_s per element, causal mask, D on
//     the diagonal; y^T leaves straight from the accumulators.
// Every shared fragment (B^T, C.B^T, C) feeds all four 16-row p-tiles of the head.
//
// Hand-off: each wave publishes its columns of H_k under a flag of its own (the successor's
// wave w reads exactly those columns), so the chain needs no workgroup barrier.  The
// publisher waits for its state stores to complete, then sets the flag; the cache policy of
// the stores and of the successor's loads is chosen as described at kCohDev.
//
// Dispatch order: k_chunk_prep's item table (chain_items) places every chain on one XCD and
// a workgroup's predecessor in an earlier row of that XCD.  Workgroups are dispatched in
// id order, so a waiting workgroup's predecessor is already resident or done; the wait is
// also bounded in time (about a second, then SSD_DEVERR_CHAIN_WAIT is raised and the
// workgroup goes on), so no metadata error can stall the device.
// ---------------------------------------------------------------------------------------

// A bf16 fragment with value j multiplied by v[j].
__device__ __forceinline__ Frag8 scale_frag(const Frag8& f, const float* v) {
  Frag8 r;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float lo = __uint_as_float(f.w[w] << 16), hi = __uint_as_float(f.w[w] & 0xffff0000u);
    r.w[w] = pack_bf16x2(lo * v[2 * w], hi * v[2 * w + 1]);
  }
  return r;
}

template <int N, int CS>
struct ChainCfg {
  static_assert(N % 128 == 0 && CS % 128 == 0, "the LDS swizzles need 128-element rows");
  static constexpr int P = 64, NW = kChainWaves, NTH = 64 * NW, NT = CS / 16, NSTEP = CS / 32;
  static constexpr int TP = 4, TN = N / 16, TNW = TN / NW, KN = N / 32;
  static constexpr int NTQ = NT / NW;                 // row tiles per wave
  static constexpr int NG = P / 8, NITEM = NG * CS / 4, NI = NITEM / NTH;
  static constexpr int NF = cb_frag_base(NT);
  static_assert(TN % NW == 0 && N % 32 == 0 && NT % NW == 0 && NITEM % NTH == 0, "shape");
  // delta and the cumsum are formed for one token per thread (token 64 * wave + lane)
  static_assert(CS <= 64 * NW, "one token per thread");
};

// The chunk's x rows.  Work item `it`: columns 8*g8 .. 8*g8+7, tokens 4*sg .. 4*sg+3.
template <int N, int CS, int NI>
__device__ __forceinline__ void chain_load_x(Frag8 (&x)[NI][4], const PrefillParams& p, ChunkLoc c,
                                             int h) {
  using M = ChainCfg<N, CS>;
  static_assert(NI == M::NI, "staging items");
  const BufRes xr(static_cast<const bf16_t*>(p.x) + int64_t(c.cs0) * p.x_st + int64_t(h) * M::P);
  const uint32_t xrow_b = uint32_t(p.x_st * int64_t(sizeof(bf16_t)));
#pragma unroll
  for (int u = 0; u < M::NI; ++u) {
    const int it = u * M::NTH + int(threadIdx.x);
    const int g8 = it % M::NG, s = 4 * (it / M::NG);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // unguarded: rows past the chunk end repeat its last row (their weight is zero)
      const int row = s + t < c.L ? s + t : c.L - 1;
      x[u][t] = buf_ld8<bf16_t>(xr, uint32_t(row) * xrow_b + uint32_t(g8) * 16, 0);
    }
  }
}

constexpr long long kChainWaitTicks = 100000000;   // ~1 s of the 100 MHz wall clock
// Cache policies of the published-state accesses.  Device-scope coherent (sc1) is the
// policy of device-scope relaxed atomics (the flags themselves use it): a store with it is
// performed for every CU once it completes, and a load with it observes such stores, in
// whichever L1 or L2 an older copy of the line may sit.
// Within one XCD the L2 is shared, so a plain store (complete once it is in L2) can stand
// in for the device-scope one: the publisher saves its wait for write-through stores (the
// L2 form).  The successor's load must then pass by its CU's L1 unless no L1 can hold an
// older copy of the line: a workgroup-scope load (sc0) may be served by the L1, and is used
// only for the checkpoint output, whose rows are written once and read once per launch
// (L1s start each launch invalidated); the two-deep workspace ring reuses its entries
// within a launch (chunk j+3 reads the entry chunk j+1 read, on the same XCD), and an
// all-cache-mode pool entry may be the one the sequence's first chunk read its initial
// state from, so those are read with device-scope loads, which pass by the L1 and take the
// line from the XCD's L2.  (The L2 does not keep the published line readable either way: a
// line allocated by stores alone is fetched from memory again on a read, merged with what
// the L2 holds; only a line filled from memory before it is written stays readable.)
// The publisher takes the L2 form whenever it has a successor: the successor's workgroup id
// is the same mod 8, and the XCD of workgroup id w is (w + rot) mod 8 with one rotation rot
// for the whole launch (measured: the rotation changes from launch to launch, 0 or 7 in
// eager launches and in graph replays, but never within one), so the two share an XCD.
// The publisher records its XCD and the form in the flag value.  A successor reads through
// its L2 only when the flag says the L2 form on its own XCD, and a state left in another
// XCD's L2 is reported (SSD_DEVERR_CHAIN_WAIT).  Neither side needs a cache flush or
// invalidate: the publisher waits for its stores to complete before the flag store, the
// successor issues its loads after it has seen the flag.
constexpr int kCohDev = 16;
constexpr int kCohWg = 1;
constexpr int kFlagLocal = 16;   // flag value - 1 = XCD id | kFlagLocal when kept in L2

__device__ __forceinline__ int xcd_id() {
  return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) & 15;   // HW_REG_XCC_ID[3:0]
}

// LDS tiles of the chain kernel, unpadded rows (52 KB in all, three workgroups per CU):
// x^T [p][s] with the 8-token (16-byte) groups XOR-ed with (p ^ p >> 3) & 15, so the
// staging writes (8 columns 8 apart per token group) and the fragment reads (16
// consecutive rows) both reach 16 different 16-byte bank groups; the state rows [p][n]
// with the 8-column groups XOR-ed with p & 15 (only p mod 16 matters, the p-tiles are 16
// rows).  Rows are a multiple of 128 elements long, so the XOR stays inside the row.
__device__ __forceinline__ int chain_xs(int p, int s) { return s ^ ((((p >> 3) ^ p) & 15) << 3); }
__device__ __forceinline__ int chain_hs(int pl, int n) { return n ^ ((pl & 15) << 3); }

// The state buffer a chain publishes H_k through: the checkpoint output when there is one,
// else (all cache mode, fp32 pool) the pool entry of the cache block chunk k closes, else a
// two-deep ring per (sequence, head) in the workspace (chunk j of a sequence uses entry
// j & 1; entry reuse is safe because chunk j+2 publishes only after chunk j+1 has read H_j).
__device__ __forceinline__ int chain_pool_pub(const PrefillParams& p, int k) {
  if (p.states || !p.blk_slot || p.pool_kind != SSD_F32) return -1;
  const int s = ld_meta(p.blk_slot, k);
  return s < p.num_slots ? s : -1;
}
__device__ __forceinline__ float* chain_state(const PrefillParams& p, int k, int h, int r, int j) {
  if (p.states) return p.states + (int64_t(k) * p.H + h) * int64_t(p.P) * p.N;
  const int s = chain_pool_pub(p, k);
  if (s >= 0) return static_cast<float*>(p.pool) + int64_t(s) * p.slot_stride + int64_t(h) * p.P * p.N;
  return p.hring + ((int64_t(r) * p.H + h) * 2 + (j & 1)) * int64_t(p.P) * p.N;
}

// Row tile q of wave w (tiles w and 2NW-1-w, then the same +2NW), and the most C.B^T
// fragments any wave needs for its q-th tile (its 32-token blocks 0 .. tile/2).
template <int NW>
__device__ __forceinline__ int chain_tile(int q, int w) {
  return 2 * NW * (q / 2) + ((q & 1) ? 2 * NW - 1 - w : w);
}
template <int NW>
constexpr int chain_ncb(int q) {
  return (2 * NW * (q / 2) + ((q & 1) ? 2 * NW - 1 : NW - 1)) / 2 + 1;
}

template <int N, int CS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void k_chunk_chain(PrefillParams p) {
  using T = bf16_t;
  using O = Ops<T>;
  using frag = Frag8;
  using M = ChainCfg<N, CS>;
  constexpr int P = M::P, NW = M::NW, NT = M::NT, NSTEP = M::NSTEP;
  constexpr int RSX = CS, RSB = N;
  constexpr int TP = M::TP, TNW = M::TNW, KN = M::KN, NTQ = M::NTQ;
  constexpr int NF = M::NF;
  constexpr int NCB = chain_ncb<NW>(NTQ - 1);     // C.B^T fragment buffer of one tile
  __shared__ __attribute__((aligned(16))) bf16_t xT[P * RSX];   // raw x^T (swizzled)
  __shared__ __attribute__((aligned(16))) bf16_t Hs[P * RSB];   // incoming state rows
  __shared__ __attribute__((aligned(16))) float s_c[CS];        // cumsum
  __shared__ __attribute__((aligned(16))) float s_d[CS];        // delta
  __shared__ __attribute__((aligned(16))) float s_v[CS];        // block-referenced weight
  __shared__ __attribute__((aligned(16))) float s_w[CS];        // chunk-end weight
  __shared__ float s_tot[NW];                                    // per-wave delta*A sums

  // (chunk, head) of this workgroup: from k_chunk_prep's item table, or (batches too large
  // to order) chunks in index order, which also puts every predecessor first, with the
  // heads spread over the XCDs
  const int tid = threadIdx.x;
  int k, h;
  if (p.items) {
    const int item = ld_meta(p.items, blockIdx.x);
    if (item < 0) return;
    k = item / p.H;
    h = item - k * p.H;
  } else {
    const int hx = (p.H + kXcds - 1) / kXcds;                  // heads per XCD and row
    const int row = blockIdx.x / (kXcds * hx), sl = blockIdx.x % (kXcds * hx);
    h = (sl % kXcds) * hx + sl / kXcds;
    if (h >= p.H || row >= p.C) return;
    k = row;
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, li = lane & 15, kg = lane >> 4;
  const uint32_t lane_b = uint32_t(lane) * 8 * sizeof(T);
  // one flag per (chunk, head, wave): wave w publishes (and its successor wave w reads)
  // the state columns n of its n-tiles, [w*TNW*16, (w+1)*TNW*16) of every row p
  int* const done = p.chain_flag;
  auto flag_of = [&](int kk) { return done + (int64_t(kk) * p.H + h) * NW + wave; };

  // the chunk, its sequence and its place in the sequence, all checked before any access
  bool ok = k >= 0 && k < p.C;
  int r = 0, cs0 = 0, L = 1, k0 = 0, k1 = 0;
  if (ok) {
    r = p.seq_idx[k];
    ok = r >= 0 && r < p.S;
  }
  if (ok) {
    k0 = r == 0 ? 0 : p.last_chunk[r - 1] + 1;
    k1 = p.last_chunk[r];
    cs0 = p.cu_chunk[k];
    const int cs1 = p.cu_chunk[k + 1];
    L = cs1 - cs0;
    const int t0 = p.cu_seqlens[r], t1 = p.cu_seqlens[r + 1];
    ok = k0 <= k && k <= k1 && k1 < p.C && L >= 1 && L <= CS && cs0 >= t0 && cs1 <= t1 &&
         t0 >= 0 && t1 <= p.T && (k != k0 || cs0 == t0) && (k != k1 || cs1 == t1);
  }
  if (!ok) {
    // publish anyway so that no successor waits for this workgroup
    if (tid == 0) raise_flag(p.flag, SSD_DEVERR_CHUNK_RANGE);
    if (lane == 0 && k >= 0 && k < p.C)
      __hip_atomic_store(flag_of(k), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const bool first = k == k0, last = k == k1;
  // pool slots: the initial state (first chunk), the final state (last chunk) and, in the
  // all cache mode, the entry of a cache block this chunk closes (-1: none)
  const SeqSlots ss = seq_slots(p, r, first, last, tid == 0 && (first || p.block_size > 0));
  int blk = p.blk_slot ? ld_meta(p.blk_slot, k) : -1;
  if (blk >= p.num_slots) blk = -1;
  // element offsets of this head's state in those slots (-1: none)
  auto slot_e = [&](int slot) {
    return slot >= 0 ? int64_t(slot) * p.slot_stride + int64_t(h) * P * N : int64_t(-1);
  };
  const int64_t src_e = slot_e(ss.src), fin_e = slot_e(ss.fin), blk_e = slot_e(blk);
  const int g = h / (p.H / p.G);
  const float Dh = p.D ? p.D[h] : 0.f;

  // every input of the chunk's own state at once: x rows, this wave's dt values (token
  // 64*wave + lane) and all of this wave's B^T fragments
  Frag8 xs[M::NI][4];
  const int tok = 64 * wave + lane;
  const float dt_raw = to_f32(static_cast<const T*>(p.dt)[int64_t(cs0 + (tok < L ? tok : L - 1)) * p.dt_st + h]);
  chain_load_x<N, CS, M::NI>(xs, p, ChunkLoc{cs0, L}, h);
  const BufRes btr(static_cast<const T*>(p.btw) + (int64_t(k) * p.G + g) * (int64_t(N) * CS));
  frag btf[NSTEP][TNW];
#pragma unroll
  for (int ss = 0; ss < NSTEP; ++ss)
#pragma unroll
    for (int q = 0; q < TNW; ++q) btf[ss][q] = ld_frag<T>(btr, (wave * TNW + q) * NSTEP + ss, lane_b);

  // delta = clamp(softplus(dt + bias)) and the chunk-local inclusive cumsum c of delta*A:
  // a scan inside each wave, then the earlier waves' sums (tokens at or past the chunk end
  // have delta = 0, so c stays flat there)
  const float dl = tok < L ? p.prep.apply(dt_raw, p.prep.bias_of(h)) : 0.f;
  const float incl = wave_inclusive_scan(dl * p.A[h]);
  if (lane == 63) s_tot[wave] = incl;

  // staging: raw x^T
#pragma unroll
  for (int u = 0; u < M::NI; ++u) {
    const int it = u * M::NTH + tid;
    const int g8 = it % M::NG, s = 4 * (it / M::NG);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = 8 * g8 + j;
      O::put4raw(&xT[col * RSX + chain_xs(col, s)], xs[u], j);
    }
  }
  __syncthreads();
  // cumsum, delta and the two token weights: v_s against the end of the token's 32-token
  // block, w_s against the chunk end
  {
    float base = 0.f, clast = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w < wave) base += s_tot[w];
      clast += s_tot[w];
    }
    const float c = incl + base;
    const float cref = __shfl(c, lane | 31, 64);
    if (tok < CS) {
      s_c[tok] = c;
      s_d[tok] = dl;
      s_v[tok] = dl * fast_exp(cref - c);
      s_w[tok] = dl * fast_exp(clast - c);
      if (p.dA_cumsum_out && tok < L) p.dA_cumsum_out[int64_t(h) * p.T + cs0 + tok] = c;
    }
  }
  __syncthreads();

  // the chunk's own state S^T = (B^T o w) x (one reference: the chunk end)
  f32x4_v sacc[TNW][TP];
#pragma unroll
  for (int q = 0; q < TNW; ++q)
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) sacc[q][pt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ss = 0; ss < NSTEP; ++ss) {
    const float4_v w0 = *reinterpret_cast<const float4_v*>(&s_w[32 * ss + 8 * kg]);
    const float4_v w1 = *reinterpret_cast<const float4_v*>(&s_w[32 * ss + 8 * kg + 4]);
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    frag a[TNW];
#pragma unroll
    for (int q = 0; q < TNW; ++q) a[q] = scale_frag(btf[ss][q], wv);
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) {
      const int pr = pt * 16 + li;
      const frag b = O::ld8(&xT[pr * RSX + chain_xs(pr, 32 * ss + 8 * kg)]);
#pragma unroll
      for (int q = 0; q < TNW; ++q) sacc[q][pt] = O::mma(a[q], b, sacc[q][pt]);
    }
  }
  if (p.local_states_out) {
    const int64_t sb = (int64_t(k) * p.H + h) * (int64_t(P) * N);
#pragma unroll
    for (int q = 0; q < TNW; ++q)
#pragma unroll
      for (int pt = 0; pt < TP; ++pt)
        st_f4(p.local_states_out + sb + (pt * 16 + li) * N + (wave * TNW + q) * 16 + 4 * kg, sacc[q][pt]);
  }

  // y^T operands, two row tiles in flight: C fragments and the tile's C.B^T fragments
  const BufRes cbr(static_cast<const T*>(p.cbw) + (int64_t(k) * p.G + g) * (int64_t(NF) * 512));
  const BufRes cfr(static_cast<const T*>(p.cfw) + (int64_t(k) * p.G + g) * (int64_t(NT) * KN * 512));
  frag cf[2][KN], cb[2][NCB];
  auto load_tile = [&](int q4) {
    const int i = __builtin_amdgcn_readfirstlane(chain_tile<NW>(q4, wave)), bd = i / 2;
#pragma unroll
    for (int kk = 0; kk < KN; ++kk) cf[q4 & 1][kk] = ld_frag<T>(cfr, i * KN + kk, lane_b);
#pragma unroll
    for (int j = 0; j < NCB; ++j)
      if (j < chain_ncb<NW>(q4)) cb[q4 & 1][j] = ld_frag<T>(cbr, cb_frag_base(i) + (j < bd ? j : bd), lane_b);
  };

  // the incoming state of this wave's columns: the pool slot (or zero) for a sequence's
  // first chunk, else what the predecessor's wave published
  const int my_xcd = xcd_id();
  const float* hin = nullptr;
  bool via_l2 = false;
  const bool from_pool = src_e >= 0 && p.has_init && p.has_init[r];
  if (!first) {
    int fv = 0;
    if (lane == 0) {
      const int* f = flag_of(k - 1);
      fv = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (fv == 0) {
        const long long t_start = wall_clock64();
        while ((fv = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == 0) {
          if (wall_clock64() - t_start > kChainWaitTicks) {
            raise_flag(p.flag, SSD_DEVERR_CHAIN_WAIT);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
    }
    asm volatile("" ::: "memory");
    const int e = __builtin_amdgcn_readfirstlane(fv) - 1;
    via_l2 = (e & kFlagLocal) && (e & 15) == my_xcd;
    if (!via_l2 && (e & kFlagLocal) && lane == 0) raise_flag(p.flag, SSD_DEVERR_CHAIN_WAIT);
    hin = chain_state(p, k - 1, h, r, k - 1 - k0);
  }
  // The state's rows move in the row layout: in the access (q, pt) of wave w, lane L holds
  // row pt*16 + L/4, columns (w*TNW + q)*16 + 4*(L%4) .. +3, so each four consecutive lanes
  // cover one contiguous 64-byte row segment (one address-unit pass per quad; the MFMA
  // accumulator layout, lane (li, kg) = row li, columns 4*kg.., takes four).
  const int rrow = lane >> 2, rcol = 4 * (lane & 3);
  auto roff = [&](int q, int pt) {   // element offset of this lane's four states
    return (pt * 16 + rrow) * N + (wave * TNW + q) * 16 + rcol;
  };
  f32x4_v hreg[TNW][TP];
  if (from_pool) {
    // a pool slot (fp32, bf16 or fp16), written before this launch
#pragma unroll
    for (int q = 0; q < TNW; ++q)
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        const float4_v v = pool_ld4(p.pool, p.pool_kind, src_e + roff(q, pt));
        hreg[q][pt] = f32x4_v{v.x, v.y, v.z, v.w};
      }
  } else if (hin) {
    // the predecessor's state: workgroup-scope loads after an L2-form publication on this
    // XCD into the checkpoint output, device-coherent ones otherwise (they pass by the L1,
    // which may hold an older copy of a reused ring or pool entry)
    const BufRes hb(hin);
    u32x4_v hv[TNW][TP];
    if (via_l2 && p.states) {
#pragma unroll
      for (int q = 0; q < TNW; ++q)
#pragma unroll
        for (int pt = 0; pt < TP; ++pt)
          hv[q][pt] = __builtin_amdgcn_raw_buffer_load_b128(hb.r, uint32_t(roff(q, pt)) * 4, 0, kCohWg);
    } else {
#pragma unroll
      for (int q = 0; q < TNW; ++q)
#pragma unroll
        for (int pt = 0; pt < TP; ++pt)
          hv[q][pt] = __builtin_amdgcn_raw_buffer_load_b128(hb.r, uint32_t(roff(q, pt)) * 4, 0, kCohDev);
    }
#pragma unroll
    for (int q = 0; q < TNW; ++q)
#pragma unroll
      for (int pt = 0; pt < TP; ++pt)
        hreg[q][pt] = f32x4_v{__uint_as_float(hv[q][pt].x), __uint_as_float(hv[q][pt].y),
                              __uint_as_float(hv[q][pt].z), __uint_as_float(hv[q][pt].w)};
  } else {
#pragma unroll
    for (int q = 0; q < TNW; ++q)
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) hreg[q][pt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  }
  load_tile(0);

  // H_k = exp(c_last) H_{k-1} + S_k for this wave's columns: stored (checkpoint, pool at the
  // sequence end), then, once the stores are complete, the wave's flag.  H_{k-1} goes to
  // LDS as the MFMA operand of the inter-chunk term.
#pragma unroll
  for (int q = 0; q < TNW; ++q)
#pragma unroll
    for (int pt = 0; pt < TP; ++pt)
      O::st4lds(&Hs[(pt * 16 + rrow) * RSB + chain_hs(rrow, (wave * TNW + q) * 16 + rcol)], hreg[q][pt]);
  {
    const float dec = fast_exp(s_c[CS - 1]);
    const BufRes hb(chain_state(p, k, h, r, k - k0));

    // the L2 form (plain stores, no wait for a write-through) whenever there is a
    // successor (on this XCD: same id mod 8, one rotation per launch)
    const bool keep_l2 = !last;
    // S_k into the row layout: lane L takes the accumulator values of lane (L%4)*16 + L/4
    const int src_b = ((lane & 3) * 16 + (lane >> 2)) * 4;
    f32x4_v hn[TNW][TP];
#pragma unroll
    for (int q = 0; q < TNW; ++q)
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        f32x4_v sr;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sr[e] = __int_as_float(__builtin_amdgcn_ds_bpermute(src_b, __float_as_int(sacc[q][pt][e])));
        hn[q][pt] = dec * hreg[q][pt] + sr;
      }
    auto hoff = [&](int q, int pt) { return uint32_t(roff(q, pt)) * 4; };
    auto hbits = [&](const f32x4_v& v) {
      return u32x4_v{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                     __float_as_uint(v[3])};
    };
    if (keep_l2) {
#pragma unroll
      for (int q = 0; q < TNW; ++q)
#pragma unroll
        for (int pt = 0; pt < TP; ++pt)
          __builtin_amdgcn_raw_buffer_store_b128(hbits(hn[q][pt]), hb.r, hoff(q, pt), 0, 0);
    } else if (p.states || !last) {
#pragma unroll
      for (int q = 0; q < TNW; ++q)
#pragma unroll
        for (int pt = 0; pt < TP; ++pt)
          __builtin_amdgcn_raw_buffer_store_b128(hbits(hn[q][pt]), hb.r, hoff(q, pt), 0, kCohDev);
    }
    auto to_pool = [&](int64_t e) {
#pragma unroll
      for (int q = 0; q < TNW; ++q)
#pragma unroll
        for (int pt = 0; pt < TP; ++pt)
          pool_st4(p.pool, p.pool_kind, e + hoff(q, pt) / 4, as_float4(hn[q][pt]));
    };
    if (fin_e >= 0) to_pool(fin_e);
    // the block entry, unless the publication above already went there
    if (blk_e >= 0 && (last || chain_pool_pub(p, k) < 0)) to_pool(blk_e);
    if (!last) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (lane == 0)
        __hip_atomic_store(flag_of(k), 1 + (my_xcd | (keep_l2 ? kFlagLocal : 0)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (NTQ > 1) load_tile(1);
  __syncthreads();   // H_{k-1} rows complete in LDS

  // y^T, one row tile at a time
  T* ybase = static_cast<T*>(p.y) + int64_t(cs0) * p.y_st + int64_t(h) * P;
#pragma unroll
  for (int q4 = 0; q4 < NTQ; ++q4) {
    const int i = __builtin_amdgcn_readfirstlane(chain_tile<NW>(q4, wave)), bd = i / 2;
    const int l = 16 * i + li;
    const frag* cfq = cf[q4 & 1];
    const frag* cbt = cb[q4 & 1];
    // inter-chunk term: exp(c_l) H_{k-1}[p, :] . C_l
    f32x4_v acc[TP];
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) acc[pt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KN; ++kk)
#pragma unroll
      for (int pt = 0; pt < TP; ++pt)
        acc[pt] = O::mma(O::ld8(&Hs[(pt * 16 + li) * RSB + chain_hs(li, 32 * kk + 8 * kg)]), cfq[kk], acc[pt]);
    {
      const float e = fast_exp(s_c[l]);
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) acc[pt] *= e;
    }
    // blocks entirely before the diagonal block: the C.B^T fragment (lane: row l) scaled
    // per token by v_s exp(c_l - c_{32b+31}) = delta_s exp(c_l - c_s), two factors <= 1
#pragma unroll
    for (int b = 0; b < chain_ncb<NW>(q4) - 1; ++b) {
      if (b >= bd) break;
      const float gb = fast_exp(s_c[l] - s_c[32 * b + 31]);
      const float4_v v0 = *reinterpret_cast<const float4_v*>(&s_v[32 * b + 8 * kg]);
      const float4_v v1 = *reinterpret_cast<const float4_v*>(&s_v[32 * b + 8 * kg + 4]);
      const float vv[8] = {v0.x * gb, v0.y * gb, v0.z * gb, v0.w * gb,
                           v1.x * gb, v1.y * gb, v1.z * gb, v1.w * gb};
      const frag cbs = scale_frag(cbt[b], vv);
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        const int prow = pt * 16 + li;
        acc[pt] = O::mma(O::ld8(&xT[prow * RSX + chain_xs(prow, 32 * b + 8 * kg)]), cbs, acc[pt]);
      }
    }
    // the block holding the diagonal: exact decay per element, causal mask, D on the
    // diagonal (its C.B^T fragment is entry bd, or the last loaded one when bd is smaller)
    {
      const int s0 = 32 * bd;
      const float cl = s_c[l];
      const float4_v c0 = *reinterpret_cast<const float4_v*>(&s_c[s0 + 8 * kg]);
      const float4_v c1 = *reinterpret_cast<const float4_v*>(&s_c[s0 + 8 * kg + 4]);
      const float4_v d0 = *reinterpret_cast<const float4_v*>(&s_d[s0 + 8 * kg]);
      const float4_v d1 = *reinterpret_cast<const float4_v*>(&s_d[s0 + 8 * kg + 4]);
      const float cs8[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      const float ds8[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
      frag cbd = cbt[0];
#pragma unroll
      for (int j = 1; j < chain_ncb<NW>(q4); ++j)
        if (j == bd) cbd = cbt[j];
      float m[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int s = s0 + 8 * kg + j;
        const float v = O::val(cbd, j) * fast_exp(cl - cs8[j]) * ds8[j] + (s == l ? Dh : 0.f);
        m[j] = s <= l ? v : 0.f;
      }
      const frag mf = O::from8(m);
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        const int prow = pt * 16 + li;
        acc[pt] = O::mma(O::ld8(&xT[prow * RSX + chain_xs(prow, s0 + 8 * kg)]), mf, acc[pt]);
      }
    }
    if (q4 + 2 < NTQ) load_tile(q4 + 2);
    store_yt<T, 2>(ybase, p.y_st, l, L, kg, acc);
    store_yt<T, 2>(ybase + 32, p.y_st, l, L, kg, acc + 2);
  }
}

// ---------------------------------------------------------------------------------------
// launch table (same order as kChunkedShapes)
// ---------------------------------------------------------------------------------------


template <typename T, int P, int N, int CS>
static hipError_t run_chunked(const PrefillParams& p, hipStream_t s, void* const* ev) {
  constexpr int PW = P >= 32 ? 32 : P;
  constexpr bool kChain = chain_supported(sizeof(T) == 2 ? SSD_BF16 : SSD_F32, P, N, CS);
  if (kChain && !p.chain_flag) return hipErrorInvalidValue;   // the plan gives it the buffers
  record_event(ev, 0, s);
  hipLaunchKernelGGL((k_chunk_prep<T, N, CS>), dim3(p.C + 1, p.G, prep_split(p.C * p.G)), dim3(256),
                     0, s, p);
  record_event(ev, 1, s);
  if constexpr (kChain) {
    hipLaunchKernelGGL((k_chunk_chain<N, CS>), dim3(p.chain_grid), dim3(64 * kChainWaves), 0, s, p);
  } else {
    const MarchGrid mg = march_grid(p.S, p.G, p.H, P / PW);
    hipLaunchKernelGGL((k_chunk_march<T, P, PW, N, CS>), dim3(mg.nblocks * mg.bsize), dim3(256), 0,
                       s, p);
  }
  record_event(ev, 2, s);
  return hipGetLastError();
}

typedef hipError_t (*RunFn)(const PrefillParams&, hipStream_t, void* const*);
static const RunFn kRun[] = {
    run_chunked<bf16_t, 64, 128, 256>, run_chunked<bf16_t, 64, 128, 128>,
    run_chunked<bf16_t, 64, 128, 64>,  run_chunked<bf16_t, 16, 16, 64>,
    run_chunked<float, 16, 16, 64>,    run_chunked<float, 64, 128, 64>,
    run_chunked<bf16_t, 16, 16, 256>,  run_chunked<float, 16, 16, 256>,
    run_chunked<float, 64, 128, 256>,
    run_chunked<bf16_t, 16, 128, 64>,  run_chunked<bf16_t, 16, 128, 256>,
    run_chunked<bf16_t, 64, 16, 64>,   run_chunked<bf16_t, 64, 16, 256>,
    run_chunked<float, 16, 128, 64>,   run_chunked<float, 16, 128, 256>,
    run_chunked<float, 64, 16, 64>,    run_chunked<float, 64, 16, 256>,
};

hipError_t launch_chunked_prefill(int variant, const PrefillParams& p, hipStream_t s,
                                  void* const* events) {
  if (variant < 0 || variant >= int(sizeof(kRun) / sizeof(kRun[0]))) return hipErrorInvalidValue;
  return kRun[variant](p, s, events);
}

}  // namespace ssd
