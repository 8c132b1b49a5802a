// ssd_decode.hip -- padded speculative decode state update (one workgroup per row x head).
//
// Decode is a sequential per-token update ("[vLLM] Mamba (SSM)", why-this-design item 2);
// rows padded with NULL_BLOCK_ID are skipped (CUDA Graph section) and the starting state is
// restored from column num_accepted-1 of the row's index list (item 4).
//
// Work split: one 256-thread workgroup owns the P x N fp32 state of one (row, head).  Each
// thread keeps ITERS float4 of it in registers: thread t holds columns n0 = 4*(t % NQ) ..
// n0+3 (NQ = N/4) of rows p = i*(256/NQ) + t/NQ.  One wave-wide float4 load therefore reads
// contiguous 1 KB of the slot (coalesced gather), and y[p] = sum_n h[p,n] C[n] is a
// reduction across the NQ lanes that share p.  The state is read once before any write
// (the source slot may be one of the destinations), then written after every token with
// non-temporal stores (the checkpoints are not re-read by this call).
#include "ssd_params.h"

namespace ssd {

// The pool slots of decode row r: `src` is read before any write, dst(j) receives the
// state after token j.  state_indices is [B_pad, ntok] (column j: token j's destination,
// column num_accepted-1: the source), or in the all cache mode [B_pad, idx_stride] with one
// token per row, source column block_idx_last_computed and destination column
// block_idx_last_scheduled.
struct DecodeRow {
  const int* idx;   // the row of state_indices
  int src;
  int one;          // the all cache mode's destination slot, else -1
  __device__ int dst(int j) const { return one >= 0 ? one : idx[j]; }
};

// 1: a live row; 0: a padding row (its first destination is null_block_id: nothing is read
// or written); -1: an invalid row (a column, slot or num_accepted out of range), skipped
// with the flag raised when `report`.
__device__ __forceinline__ int decode_row(const DecodeParams& p, int r, bool report,
                                          DecodeRow& row) {
  int err = 0;
  if (p.idx_stride > 0) {
    row.idx = p.idx + int64_t(r) * p.idx_stride;
    const int ls = p.blk_last_sched[r], lc = p.blk_last_comp[r];
    if (ls < 0 || ls >= p.idx_stride) {
      err = SSD_DEVERR_SLOT_RANGE;
    } else {
      row.one = row.idx[ls];
      if (row.one == p.null_id) return 0;
      if (lc < 0 || lc >= p.idx_stride) {
        err = SSD_DEVERR_SLOT_RANGE;
      } else {
        row.src = row.idx[lc];
        if (row.src < 0 || row.src >= p.num_slots || row.one < 0 || row.one >= p.num_slots)
          err = SSD_DEVERR_SLOT_RANGE;
      }
    }
  } else {
    row.idx = p.idx + int64_t(r) * p.ntok;
    row.one = -1;
    if (row.idx[0] == p.null_id) return 0;
    const int acc = p.num_acc ? p.num_acc[r] : 1;
    if (acc < 1 || acc > p.ntok) {
      err = SSD_DEVERR_ACCEPTED;
    } else {
      for (int j = 0; j < p.ntok; ++j) {
        const int s = row.idx[j];
        if (s < 0 || s >= p.num_slots) err = SSD_DEVERR_SLOT_RANGE;
      }
      row.src = row.idx[acc - 1];
    }
  }
  if (err) {
    if (report) raise_flag(p.flag, err);
    return -1;
  }
  return 1;
}

// States per lane of the decode kernel: 16 bytes of the pool per lane, i.e. 4 fp32 or 8 bf16.
template <typename S>
constexpr int decode_vec() { return sizeof(S) == 2 ? 8 : 4; }

template <typename T, typename S, int N, int ITERS>
__global__ __launch_bounds__(256) void k_state_update(DecodeParams p) {
  constexpr int V = decode_vec<S>();   // consecutive states n of one row p per lane
  constexpr int NQ = N / V;            // lanes per state row
  constexpr int RP = 256 / NQ;         // state rows covered per iteration
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int h = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const int ntok = p.ntok, P = p.P, H = p.H;
  DecodeRow row;
  if (decode_row(p, r, tid == 0, row) <= 0) return;   // padding or invalid: nothing touched

  // Gather the source state before any write; it is requested first so the state stream
  // is in flight while the small per-token inputs are staged.
  const int lane_q = tid % NQ, prow = tid / NQ;
  const int64_t head_off = int64_t(h) * P * N;
  const int64_t src = int64_t(row.src) * p.slot_stride + head_off;
  float st[ITERS][V];
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const int pr = i * RP + prow;
    const int64_t e = src + (pr < P ? pr : 0) * N + V * lane_q;
    if constexpr (V == 8) {
      PoolIO<S>::ld8(p.pool, e, st[i]);
    } else {
      const float4_v v = PoolIO<S>::ld4(p.pool, e);
      st[i][0] = v.x; st[i][1] = v.y; st[i][2] = v.z; st[i][3] = v.w;
    }
  }
  // Stage this row's token data for head h: x[ntok][P], B[ntok][N], C[ntok][N], delta.
  // B and C first: N is a multiple of 16, so their float4 reads stay 16-byte aligned.
  float* bs = lds;
  float* cs = bs + ntok * N;
  float* xs = cs + ntok * N;
  float* ys = xs + ntok * P;
  float* ds = ys + ntok * P;
  const int g = h / (H / p.G);
  const T* xg = static_cast<const T*>(p.x);
  const T* bg = static_cast<const T*>(p.B);
  const T* cg = static_cast<const T*>(p.Cm);
  const T* dg = static_cast<const T*>(p.dt);
  for (int e = tid; e < ntok * P; e += 256) {
    const int j = e / P, pp = e - j * P;
    xs[e] = Elem<T>::load(xg + ((int64_t(r) * ntok + j) * H + h) * P + pp);
  }
  for (int e = tid; e < ntok * N; e += 256) {
    const int j = e / N, n = e - j * N;
    const int64_t off = ((int64_t(r) * ntok + j) * p.G + g) * N + n;
    bs[e] = Elem<T>::load(bg + off);
    cs[e] = Elem<T>::load(cg + off);
  }
  if (tid < ntok) ds[tid] = p.prep(Elem<T>::load(dg + (int64_t(r) * ntok + tid) * H + h), h);

  __syncthreads();

  const float Ah = p.A[h];
  const float Dh = p.D ? p.D[h] : 0.f;
  for (int j = 0; j < ntok; ++j) {
    const float delta = ds[j];
    const float decay = fast_exp(delta * Ah);
    float bv[V], cv[V];
#pragma unroll
    for (int v4 = 0; v4 < V; v4 += 4) {
      const float4_v b4 = *reinterpret_cast<const float4_v*>(bs + j * N + V * lane_q + v4);
      const float4_v c4 = *reinterpret_cast<const float4_v*>(cs + j * N + V * lane_q + v4);
      bv[v4] = b4.x; bv[v4 + 1] = b4.y; bv[v4 + 2] = b4.z; bv[v4 + 3] = b4.w;
      cv[v4] = c4.x; cv[v4 + 1] = c4.y; cv[v4 + 2] = c4.z; cv[v4 + 3] = c4.w;
    }
    const int64_t dst = int64_t(row.dst(j)) * p.slot_stride + head_off;
    if constexpr (V == 8 && ITERS > 1 && ITERS <= NQ) {
      // 2-byte pool: the state rows first, each stored as soon as it is updated, then y[p]
      // = sum over the NQ lanes of a row group for all ITERS rows at once: halving
      // exchanges (lane bit NQ/2 picks the upper or lower half of the rows, then NQ/4 ...)
      // leave lane q with one row, i = q / (NQ / ITERS); plain exchanges finish its sum.
      // log2(NQ) cross-lane steps carry ITERS - 1 + log2(NQ / ITERS) values instead of
      // ITERS * log2(NQ) (measured: 167 -> 163 us at decode_spec; for an fp32 pool the
      // per-row form below is 1% faster).
      float part[ITERS], xpv[ITERS];
#pragma unroll
      for (int i = 0; i < ITERS; ++i) {
        const int pr = i * RP + prow;
        xpv[i] = pr < P ? xs[j * P + pr] : 0.f;
        const float dx = delta * xpv[i];
        part[i] = 0.f;
#pragma unroll
        for (int v = 0; v < V; ++v) {
          st[i][v] = decay * st[i][v] + dx * bv[v];
          part[i] += st[i][v] * cv[v];
        }
        if (pr < P) PoolIO<S>::st8_nt(p.pool, dst + pr * N + V * lane_q, st[i]);
      }
#pragma unroll
      for (int c = ITERS, o = NQ / 2; c > 1; c >>= 1, o >>= 1) {
        const bool up = lane_q & o;
#pragma unroll
        for (int k = 0; k < c / 2; ++k) {
          const float send = up ? part[k] : part[k + c / 2];
          const float keep = up ? part[k + c / 2] : part[k];
          part[k] = keep + __shfl_xor(send, o, 64);
        }
      }
#pragma unroll
      for (int o = NQ / ITERS / 2; o > 0; o >>= 1) part[0] += __shfl_xor(part[0], o, 64);
      const int i = lane_q / (NQ / ITERS), pr = i * RP + prow;
      float xp = xpv[0];
#pragma unroll
      for (int k = 1; k < ITERS; ++k)
        if (i == k) xp = xpv[k];
      if (lane_q % (NQ / ITERS) == 0 && pr < P) ys[j * P + pr] = part[0] + Dh * xp;
    } else {
#pragma unroll
      for (int i = 0; i < ITERS; ++i) {
        const int pr = i * RP + prow;
        const float xp = pr < P ? xs[j * P + pr] : 0.f;
        const float dx = delta * xp;
        float part = 0.f;
#pragma unroll
        for (int v = 0; v < V; ++v) {
          st[i][v] = decay * st[i][v] + dx * bv[v];
          part += st[i][v] * cv[v];
        }
#pragma unroll
        for (int off = NQ / 2; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
        if (pr < P) {
          if (lane_q == 0) ys[j * P + pr] = part + Dh * xp;
          const int64_t e = dst + pr * N + V * lane_q;
          if constexpr (V == 8) PoolIO<S>::st8_nt(p.pool, e, st[i]);
          else PoolIO<S>::st4_nt(p.pool, e, float4_v{st[i][0], st[i][1], st[i][2], st[i][3]});
        }
      }
    }
  }
  __syncthreads();
  T* yg = static_cast<T*>(p.y);
  for (int e = tid; e < ntok * P; e += 256) {
    const int j = e / P, pp = e - j * P;
    Elem<T>::store(yg + ((int64_t(r) * ntok + j) * H + h) * P + pp, ys[e]);
  }
}

template <typename T, typename S, int N>
static hipError_t launch_n(const DecodeParams& p, hipStream_t s, void* const* ev) {
  const int rows_per_iter = 256 / (N / decode_vec<S>());
  const int iters = (p.P + rows_per_iter - 1) / rows_per_iter;
  const dim3 grid(p.H, p.B_pad);
  const size_t lds = decode_lds_bytes(p.ntok, p.P, N);
  record_event(ev, 0, s);
  if (iters <= 1) hipLaunchKernelGGL((k_state_update<T, S, N, 1>), grid, dim3(256), lds, s, p);
  else if (iters <= 2) hipLaunchKernelGGL((k_state_update<T, S, N, 2>), grid, dim3(256), lds, s, p);
  else if (iters <= 4) hipLaunchKernelGGL((k_state_update<T, S, N, 4>), grid, dim3(256), lds, s, p);
  else if (iters <= 8) hipLaunchKernelGGL((k_state_update<T, S, N, 8>), grid, dim3(256), lds, s, p);
  else hipLaunchKernelGGL((k_state_update<T, S, N, 16>), grid, dim3(256), lds, s, p);
  record_event(ev, 1, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Mamba1 decode (diagonal A, P == 1, G == 1, N == 16): the same step with a decay
// exp(delta[c] A[c, n]) per channel c and state n.  Four adjacent lanes own one channel,
// four states each, so every state load and store of a wavefront is 1 KB contiguous in
// the slot; y is a 4-lane reduction.  B and C of the row's tokens are shared by every
// channel and staged in LDS.
// ---------------------------------------------------------------------------------------
constexpr int kDiagDecodeChannels = 64;   // channels per 256-thread workgroup

template <typename T, typename S>
__global__ __launch_bounds__(256) void k_state_update_diag(DecodeParams p) {
  constexpr int N = kDiagN, SPL = 4;
  constexpr int NBC = (kDecodeMaxTokens * 2 * N + 255) / 256;   // B/C elements per thread
  __shared__ __attribute__((aligned(16))) float s_bc[kDecodeMaxTokens][2][N];
  const int r = blockIdx.y, tid = threadIdx.x;
  const int c = blockIdx.x * kDiagDecodeChannels + tid / SPL, q = tid % SPL;
  const int ntok = p.ntok, H = p.H;
  DecodeRow row;
  if (decode_row(p, r, tid == 0 && blockIdx.x == 0, row) <= 0) return;   // padding or invalid
  // Every load of the step goes out before the first wait: the source state (read before
  // any write), A, the row's B and C (raw), and this channel's delta and x of every token
  // (raw).  Values are converted where they are used, so that no wait inside the token
  // loop also waits for a later load.
  const bool live = c < H;
  const int cc = live ? c : H - 1;
  float4_v h = PoolIO<S>::ld4(p.pool, int64_t(row.src) * p.slot_stride + int64_t(cc) * N + SPL * q);
  const float4_v a = *reinterpret_cast<const float4_v*>(p.A + int64_t(cc) * N + SPL * q);
  const T* bg = static_cast<const T*>(p.B);
  const T* cg = static_cast<const T*>(p.Cm);
  // (unconditional loads, positions past the row's tokens clamped to its last token; only
  // the LDS writes below are predicated, after every other load has gone out)
  T rbc[NBC];
#pragma unroll
  for (int u = 0; u < NBC; ++u) {
    const int e = u * 256 + tid;
    const int j = e / (2 * N), w = (e / N) & 1, n = e % N;
    rbc[u] = ((w ? cg : bg) + (int64_t(r) * ntok + min(j, ntok - 1)) * N)[n];
  }
  const T* xg = static_cast<const T*>(p.x);
  const T* dg = static_cast<const T*>(p.dt);
  // raw values one per register (a 16-bit value zero-extended), so that none is packed with
  // another before the token that uses it
  using Raw = typename std::conditional<sizeof(T) == 2, uint32_t, float>::type;
  Raw rd[kDecodeMaxTokens], rx[kDecodeMaxTokens];
#pragma unroll
  for (int j = 0; j < kDecodeMaxTokens; ++j) {
    if (j < ntok) {
      const int64_t tj = (int64_t(r) * ntok + j) * H + cc;
      rd[j] = dg[tj];
      rx[j] = xg[tj];
    }
  }
  const float bias = p.prep.bias_of(cc);
  const float Dc = p.D ? p.D[cc] : 0.f;
#pragma unroll
  for (int u = 0; u < NBC; ++u) {
    const int e = u * 256 + tid;
    const int j = e / (2 * N), w = (e / N) & 1, n = e % N;
    if (j < ntok) s_bc[j][w][n] = to_f32(rbc[u]);
  }
  __syncthreads();
  if (!live) return;   // whole 4-lane groups leave together

  const float A2[SPL] = {a.x * kLog2e, a.y * kLog2e, a.z * kLog2e, a.w * kLog2e};
  T* yg = static_cast<T*>(p.y);
#pragma unroll
  for (int j = 0; j < kDecodeMaxTokens; ++j) {
    if (j >= ntok) continue;
    const int64_t tj = (int64_t(r) * ntok + j) * H + c;
    const float delta = p.prep.apply(to_f32(T(rd[j])), bias);
    const float xv = to_f32(T(rx[j]));
    const float dx = delta * xv;
    const float4_v bv = *reinterpret_cast<const float4_v*>(&s_bc[j][0][SPL * q]);
    const float4_v cv = *reinterpret_cast<const float4_v*>(&s_bc[j][1][SPL * q]);
    h.x = __builtin_amdgcn_exp2f(delta * A2[0]) * h.x + dx * bv.x;
    h.y = __builtin_amdgcn_exp2f(delta * A2[1]) * h.y + dx * bv.y;
    h.z = __builtin_amdgcn_exp2f(delta * A2[2]) * h.z + dx * bv.z;
    h.w = __builtin_amdgcn_exp2f(delta * A2[3]) * h.w + dx * bv.w;
    float acc = cv.x * h.x + cv.y * h.y + cv.z * h.z + cv.w * h.w;
    // the channel's four lanes are one quad, all active: DPP quad permutations feed the adds
    acc += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, acc), 0xB1, 0xF, 0xF, true));
    acc += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, acc), 0x4E, 0xF, 0xF, true));
    if (q == 0) Elem<T>::store(yg + tj, acc + Dc * xv);
    const int dst = row.one >= 0 ? row.one : ld_meta(row.idx, j);   // wave-uniform: scalar
    PoolIO<S>::st4_nt(p.pool, int64_t(dst) * p.slot_stride + int64_t(c) * N + SPL * q, h);
  }
}

template <typename T, typename S>
static hipError_t launch_diag_update(const DecodeParams& p, hipStream_t s, void* const* ev) {
  const dim3 grid((p.H + kDiagDecodeChannels - 1) / kDiagDecodeChannels, p.B_pad);
  record_event(ev, 0, s);
  hipLaunchKernelGGL((k_state_update_diag<T, S>), grid, dim3(256), 0, s, p);
  record_event(ev, 1, s);
  return hipGetLastError();
}

template <typename T, typename S>
static hipError_t launch_t(const DecodeParams& p, hipStream_t s, void* const* ev) {
  if (p.diag) return launch_diag_update<T, S>(p, s, ev);
  switch (p.N) {
    case 16: return launch_n<T, S, 16>(p, s, ev);
    case 32: return launch_n<T, S, 32>(p, s, ev);
    case 64: return launch_n<T, S, 64>(p, s, ev);
    case 128: return launch_n<T, S, 128>(p, s, ev);
    default: return launch_n<T, S, 256>(p, s, ev);
  }
}

hipError_t launch_state_update(int in_dtype, const DecodeParams& p, hipStream_t s,
                               void* const* events) {
  if (in_dtype == SSD_BF16) {
    if (p.pool_kind == SSD_BF16) return launch_t<bf16_t, bf16_t>(p, s, events);
    if (p.pool_kind == SSD_F16) return launch_t<bf16_t, f16_t>(p, s, events);
    return launch_t<bf16_t, float>(p, s, events);
  }
  if (p.pool_kind == SSD_BF16) return launch_t<float, bf16_t>(p, s, events);
  if (p.pool_kind == SSD_F16) return launch_t<float, f16_t>(p, s, events);
  return launch_t<float, float>(p, s, events);
}

}  // namespace ssd
