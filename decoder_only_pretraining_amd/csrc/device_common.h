// Device helpers shared by the gfx950 kernels: element types, conversions,
// wavefront (64-lane) reductions and the MFMA fragment operations.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace gk {

constexpr int kWave = 64;

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return static_cast<bf16>(x); }

// Sum / max over the 64 lanes of a wavefront; every lane gets the result.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// ---------------------------------------------------------------------------
// MFMA fragments. A 32x32 output tile is accumulated over 16-wide slices of
// the contraction index. For one slice every lane holds 8 operand elements:
// lane l supplies row (l % 32) of the 32-row operand and the 8 contraction
// slots 8*(l/32) .. 8*(l/32)+7. The accumulator element e of lane l is
// output row 8*(e/4) + 4*(l/32) + (e%4), column l % 32.
//
// bf16: one v_mfma_f32_32x32x16_bf16 per slice.
// fp32: eight v_mfma_f32_32x32x2_f32; call j pairs slot j of both lane
//       halves, so the 16 slots are summed exactly as in the bf16 case.
// ---------------------------------------------------------------------------
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x4 lo, hi; };

__device__ __forceinline__ void frag_load(Frag<bf16>& f, const bf16* p) {
  f.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void frag_load(Frag<float>& f, const float* p) {
  f.lo = *reinterpret_cast<const f32x4*>(p);
  f.hi = *reinterpret_cast<const f32x4*>(p + 4);
}
__device__ __forceinline__ void frag_set(Frag<bf16>& f, int j, float x) { f.v[j] = static_cast<bf16>(x); }
__device__ __forceinline__ void frag_set(Frag<float>& f, int j, float x) {
  if (j < 4) f.lo[j] = x; else f.hi[j - 4] = x;
}
__device__ __forceinline__ void frag_zero(Frag<bf16>& f) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = static_cast<bf16>(0.0f);
}
__device__ __forceinline__ void frag_zero(Frag<float>& f) {
  f.lo = f32x4{0, 0, 0, 0};
  f.hi = f32x4{0, 0, 0, 0};
}

__device__ __forceinline__ void mfma(f32x16& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma(f32x16& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[j], b.lo[j], acc, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[j], b.hi[j], acc, 0, 0, 0);
}

// Per-tensor fp8 scale fmax / amax from the bit pattern of amax (fp32,
// correctly rounded); 1 when amax is 0 or not finite.
__device__ __forceinline__ float fp8_scale(uint32_t bits, float fmax) {
  const float a = __uint_as_float(bits);
  return (a > 0.0f && a <= 3.402823466e38f) ? __fdiv_rn(fmax, a) : 1.0f;
}

// Direct global->LDS copy, 16 bytes per lane (global_load_lds_dwordx4): lane
// l's bytes land at LDS byte address lds + 16 l, lds being uniform over the
// wavefront (it goes to M0). Written as inline assembly, not with the
// builtin: for the builtin the compiler records an LDS write that it cannot
// tell apart from the buffer being read, and puts a wait for every fill in
// flight (vmcnt(0)) before the next LDS read, which serialises the prefetch
// of the next stage with the reads of the current one. Here the compiler
// sees no LDS write, so the caller waits (vmcnt) and synchronises before the
// filled buffer is read. The copy has no register result.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// source: one 64-bit address per lane
__device__ __forceinline__ void lds_fill16(const void* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
// source: a base address uniform over the wavefront plus a 32-bit byte
// offset per lane
__device__ __forceinline__ void lds_fill16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// Output row (within a 32x32 tile) of accumulator element e for lane l.
__device__ __forceinline__ int acc_row(int e, int lane) { return (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3); }

}  // namespace gk
