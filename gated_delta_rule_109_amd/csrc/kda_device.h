// Device-side helpers shared by the KDA kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_bits;  // bf16 as stored in memory

constexpr int kChunk = 16;      // tokens per chunk
constexpr int kWave = 64;       // CDNA wavefront width
constexpr float kLog2e = 1.4426950408889634f;

// ---- scalar conversions -----------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(bf16_bits b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
// Round-to-nearest-even fp32 -> bf16 (gfx950 has a hardware conversion).
__device__ __forceinline__ __bf16 f32_to_bf16(float x) { return (__bf16)x; }
__device__ __forceinline__ bf16_bits f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(bf16_bits, (__bf16)x);
}
__device__ __forceinline__ float bf16v_to_f32(__bf16 x) { return (float)x; }

// Element load/store for the two storage types of q, k, v and o.
template <typename T> struct Elem;
template <> struct Elem<bf16_bits> {
  static __device__ __forceinline__ float load(const bf16_bits* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(bf16_bits* p, float x) { *p = f32_to_bf16_bits(x); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float x) { *p = x; }
};

// Decay factor of one key channel: exp(clamp(g, g_min, 0)) (lower-bounded
// decay, at most 1).
__device__ __forceinline__ float gate_alpha(float g, float g_min) {
  g = fminf(fmaxf(g, g_min), 0.0f);
  return __builtin_amdgcn_exp2f(g * kLog2e);
}

// Front end (raw inputs; flag values as in kda.h):
// decay from a gate logit a: e^{-softplus(a)} = 1 / (1 + e^a), floored at
// alpha_min = e^{g_min}. Equal to exp(clamp(-softplus(a), g_min, 0)), since
// -softplus(a) < 0 and exp is monotone.
__device__ __forceinline__ float gate_alpha_logit(float a, float alpha_min) {
  return fmaxf(__builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a * kLog2e)), alpha_min);
}
// write strength from a logit b: sigmoid(b) = 1 / (1 + e^-b)
__device__ __forceinline__ float beta_logit(float b) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-b * kLog2e));
}
// 1 / sqrt(sum of squares + eps)
__device__ __forceinline__ float inv_norm(float sumsq, float eps) {
  return __builtin_amdgcn_rsqf(sumsq + eps);
}

// ---- bf16 operand packing -----------------------------------------------------
// Round-to-nearest-even fp32 -> bf16 of four values, as two packed
// conversions (v_cvt_pk_bf16_f32 takes a pair of values).
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) { return __builtin_convertvector(x, bf16x4); }
__device__ __forceinline__ f32x4 from_bf16x4(bf16x4 x) {
  f32x4 r;
  r[0] = (float)x[0]; r[1] = (float)x[1]; r[2] = (float)x[2]; r[3] = (float)x[3];
  return r;
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x4 lo_half(bf16x8 a) { return __builtin_shufflevector(a, a, 0, 1, 2, 3); }
__device__ __forceinline__ bf16x4 hi_half(bf16x8 a) { return __builtin_shufflevector(a, a, 4, 5, 6, 7); }

// Two-term bf16 split: x ~= hi + lo with hi = bf16(x), lo = bf16(x - hi).
// hi is widened back to fp32 from its packed pairs (element 2i in the low
// half of dword i, element 2i + 1 in the high half): a shift and a mask per
// pair of values, instead of a separate conversion per value.
__device__ __forceinline__ void split_bf16(f32x4 x, bf16x4& hi, bf16x4& lo) {
  hi = to_bf16x4(x);
  const uint2 p = __builtin_bit_cast(uint2, hi);
  f32x4 h;
  h[0] = __builtin_bit_cast(float, p.x << 16);
  h[1] = __builtin_bit_cast(float, p.x & 0xffff0000u);
  h[2] = __builtin_bit_cast(float, p.y << 16);
  h[3] = __builtin_bit_cast(float, p.y & 0xffff0000u);
  lo = to_bf16x4(x - h);
}

// ---- cross-lane -----------------------------------------------------------------
// The value of lane l ^ M (M a power of two below 64), for butterfly sums.
// M = 8: a DPP rotate by 8 inside 16-lane rows (a VALU operand modifier, no
// LDS crossbar); other M < 32: ds_swizzle in bitmask mode (xor M, no address
// operand); M = 32: ds_bpermute. All three give exactly lane l ^ M.
template <int M>
__device__ __forceinline__ float lane_xor(float x) {
  static_assert(M > 0 && M < 64 && (M & (M - 1)) == 0, "power of two below the wave width");
  if constexpr (M == 8) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
  } else if constexpr (M < 32) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), (M << 10) | 0x1F));
  } else {
    return __shfl_xor(x, M);
  }
}

// ---- MFMA -----------------------------------------------------------------------
// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16). Lane l holds
//   A[l%16][8*(l/16) + j], B[8*(l/16) + j][l%16] (j = 0..7),
//   D[4*(l/16) + i][l%16] (i = 0..3).
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---- LDS DMA ------------------------------------------------------------------------
// Each active lane copies `Bytes` bytes from its own global address to LDS at
// lds_base + lane * Bytes (lds_base must be wave-uniform). Completion is
// tracked by vmcnt only; wait_vmcnt<N>() must precede any LDS read of the data.
template <int Bytes>
__device__ __forceinline__ void dma_to_lds(const void* gsrc, void* lds_base) {
  static_assert(Bytes == 4 || Bytes == 16, "DMA lane size");
  auto* dst = (__attribute__((address_space(3))) void*)lds_base;
  if constexpr (Bytes == 16) __builtin_amdgcn_global_load_lds(gsrc, dst, 16, 0, 0);
  else __builtin_amdgcn_global_load_lds(gsrc, dst, 4, 0, 0);
}
// Waits until at most N vector-memory operations of this wave are outstanding.
// The memory clobber keeps the compiler from moving LDS reads above it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = A .. B-1, so
// that array indices derived from I are constants (keeps arrays in registers).
template <int A, int B, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (A < B) {
    f(std::integral_constant<int, A>{});
    static_for<A + 1, B>(f);
  }
}

// Workgroup barrier that does not drain outstanding vector-memory operations
// (__syncthreads() waits for vmcnt(0), which would cancel DMA prefetching).
// LDS operations of this wave complete first; the memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace kda
