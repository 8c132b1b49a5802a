// ssd_device.h -- device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef uint16_t bf16_t;  // raw bf16 bits in global memory and LDS
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_v;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_v;
typedef float float4_v __attribute__((ext_vector_type(4)));
typedef float float2_v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// exp(v) through the hardware base-2 exponential: exp(v) = 2^(v * log2(e)).
__device__ __forceinline__ float fast_exp(float v) {
  return __builtin_amdgcn_exp2f(v * kLog2e);
}

// softplus(v) = log(1 + e^v); for v > 20 the result equals v to < 2.1e-9 absolute.
__device__ __forceinline__ float softplus_f(float v) {
  return v > 20.f ? v : __logf(1.f + __expf(v));
}

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(uint32_t(v) << 16);
}

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

// Two fp32 -> packed pair of bf16 (low half = a), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_v v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// fp32 -> bf16, round to nearest even.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return bf16_t(pack_bf16x2(f, 0.f) & 0xffffu);
}

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v); }

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// Four consecutive pool states: fp32 in memory, or bf16 / fp16 (round to nearest even on
// store).
template <typename S> struct PoolIO;
template <> struct PoolIO<float> {
  static __device__ __forceinline__ float4_v ld4(const void* base, int64_t e) {
    return *reinterpret_cast<const float4_v*>(static_cast<const float*>(base) + e);
  }
  static __device__ __forceinline__ void st4(void* base, int64_t e, float4_v v) {
    *reinterpret_cast<float4_v*>(static_cast<float*>(base) + e) = v;
  }
  static __device__ __forceinline__ void st4_nt(void* base, int64_t e, float4_v v) {
    __builtin_nontemporal_store(v, reinterpret_cast<float4_v*>(static_cast<float*>(base) + e));
  }
};
template <> struct PoolIO<bf16_t> {
  static __device__ __forceinline__ float4_v ld4(const void* base, int64_t e) {
    const u32x2_v v = *reinterpret_cast<const u32x2_v*>(static_cast<const bf16_t*>(base) + e);
    return float4_v{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                    __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
  }
  static __device__ __forceinline__ void st4(void* base, int64_t e, float4_v v) {
    *reinterpret_cast<u32x2_v*>(static_cast<bf16_t*>(base) + e) =
        u32x2_v{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
  }
  static __device__ __forceinline__ void st4_nt(void* base, int64_t e, float4_v v) {
    __builtin_nontemporal_store(u32x2_v{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)},
                                reinterpret_cast<u32x2_v*>(static_cast<bf16_t*>(base) + e));
  }
  // eight consecutive states (16 bytes)
  static __device__ __forceinline__ void ld8(const void* base, int64_t e, float* v) {
    const u32x4_v w = *reinterpret_cast<const u32x4_v*>(static_cast<const bf16_t*>(base) + e);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(ws[i] << 16);
      v[2 * i + 1] = __uint_as_float(ws[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void st8_nt(void* base, int64_t e, const float* v) {
    __builtin_nontemporal_store(u32x4_v{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                        pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])},
                                reinterpret_cast<u32x4_v*>(static_cast<bf16_t*>(base) + e));
  }
};
// fp16 pool states: IEEE binary16, converted with round to nearest even.
typedef _Float16 f16_t;
typedef _Float16 f16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
  return float(__builtin_bit_cast(_Float16, uint16_t(bits & 0xffffu)));
}
// Two fp32 -> packed pair of fp16 (low half = a), round to nearest even, magnitudes past
// the fp16 range to infinity: one v_cvt_pk_f16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{a, b}, f16x2_v));
}
template <> struct PoolIO<f16_t> {
  static __device__ __forceinline__ float4_v ld4(const void* base, int64_t e) {
    const u32x2_v v = *reinterpret_cast<const u32x2_v*>(static_cast<const uint16_t*>(base) + e);
    return float4_v{f16_to_f32(v.x), f16_to_f32(v.x >> 16), f16_to_f32(v.y), f16_to_f32(v.y >> 16)};
  }
  static __device__ __forceinline__ void st4(void* base, int64_t e, float4_v v) {
    *reinterpret_cast<u32x2_v*>(static_cast<uint16_t*>(base) + e) =
        u32x2_v{pack_f16x2(v.x, v.y), pack_f16x2(v.z, v.w)};
  }
  static __device__ __forceinline__ void st4_nt(void* base, int64_t e, float4_v v) {
    __builtin_nontemporal_store(u32x2_v{pack_f16x2(v.x, v.y), pack_f16x2(v.z, v.w)},
                                reinterpret_cast<u32x2_v*>(static_cast<uint16_t*>(base) + e));
  }
  static __device__ __forceinline__ void ld8(const void* base, int64_t e, float* v) {
    const u32x4_v w = *reinterpret_cast<const u32x4_v*>(static_cast<const uint16_t*>(base) + e);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = f16_to_f32(ws[i]);
      v[2 * i + 1] = f16_to_f32(ws[i] >> 16);
    }
  }
  static __device__ __forceinline__ void st8_nt(void* base, int64_t e, const float* v) {
    __builtin_nontemporal_store(u32x4_v{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]),
                                        pack_f16x2(v[4], v[5]), pack_f16x2(v[6], v[7])},
                                reinterpret_cast<u32x4_v*>(static_cast<uint16_t*>(base) + e));
  }
};
__device__ __forceinline__ float4_v as_float4(f32x4_v v) { return float4_v{v[0], v[1], v[2], v[3]}; }
// The same with the pool dtype chosen at run time (kernels that touch the pool only at a
// sequence's first and last chunk); `kind` is the ABI's state_dtype (0 fp32, 1 bf16, 2 fp16).
__device__ __forceinline__ float4_v pool_ld4(const void* base, int kind, int64_t e) {
  if (kind == 1) return PoolIO<bf16_t>::ld4(base, e);
  if (kind == 2) return PoolIO<f16_t>::ld4(base, e);
  return PoolIO<float>::ld4(base, e);
}
__device__ __forceinline__ void pool_st4(void* base, int kind, int64_t e, float4_v v) {
  if (kind == 1) PoolIO<bf16_t>::st4(base, e, v);
  else if (kind == 2) PoolIO<f16_t>::st4(base, e, v);
  else PoolIO<float>::st4(base, e, v);
}

// delta from raw dt: + bias, optional softplus, clamp.
struct DtPrep {
  const float* bias;
  int softplus;
  float lo, hi;
  __device__ __forceinline__ float bias_of(int h) const { return bias ? bias[h] : 0.f; }
  // with the bias value already loaded (kernels that reuse one head's bias many times)
  __device__ __forceinline__ float apply(float raw, float b) const {
    float v = raw + b;
    if (softplus) v = softplus_f(v);
    return fminf(fmaxf(v, lo), hi);
  }
  __device__ __forceinline__ float operator()(float raw, int h) const {
    return apply(raw, bias_of(h));
  }
};

// Read-only metadata read through the constant address space: with a wave-uniform index
// this is a scalar load, which a wave does not have to drain its vector loads to use.
// Only for arrays no kernel of the launch writes.
typedef const __attribute__((address_space(4))) int32_t const_i32;
__device__ __forceinline__ int ld_meta(const int32_t* q, int i) {
  return ((const_i32*)q)[i];
}

// ---------------------------------------------------------------------------------------
// MFMA 16x16 tiles.  A 16x16 fp32 accumulator tile lives in f32x4_v per lane: lane L holds
// rows 4*(L/16)+r (r = 0..3) of column L%16.  An operand fragment is 8 values per lane:
// for the A operand lane L supplies row L%16, for the B operand column L%16, and the 8
// values fill the lane's 8 k-slots.  The contraction runs over all 32 (lane-group, slot)
// pairs, so any consistent assignment of the contracted index to k-slots is valid as long
// as A and B use the same one.
// ---------------------------------------------------------------------------------------
struct Frag8 {  // 8 operand values held as 4 packed bf16 pairs
  uint32_t w[4];
};

__device__ __forceinline__ f32x4_v mma_bf16(const Frag8& a, const Frag8& b, f32x4_v c) {
  bf16x8_v av, bv;
  __builtin_memcpy(&av, a.w, 16);
  __builtin_memcpy(&bv, b.w, 16);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}

struct Frag8f {  // 8 fp32 operand values (the fp32 path issues 8 K=4 instructions)
  float v[8];
};

__device__ __forceinline__ f32x4_v mma_f32(const Frag8f& a, const Frag8f& b, f32x4_v c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], c, 0, 0, 0);
  return c;
}

// ---------------------------------------------------------------------------------------
// Block-wide inclusive prefix sum of one float per thread (wave64 scans + LDS).
// `scratch` must hold blockDim.x / 64 floats.  All threads must call it.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float wave_inclusive_scan(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    float o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

__device__ __forceinline__ float block_inclusive_scan(float v, float* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_inclusive_scan(v);
  if (lane == 63) scratch[wave] = v;
  __syncthreads();
  float base = 0.f;
  for (int w = 0; w < wave; ++w) base += scratch[w];
  __syncthreads();
  return v + base;
}

__device__ __forceinline__ void raise_flag(int* flag, int bits) {
  if (flag) atomicOr(flag, bits);
}

}  // namespace ssd
