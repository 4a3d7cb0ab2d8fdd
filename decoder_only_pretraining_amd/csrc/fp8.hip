// Dynamic per-tensor fp8 of the block linears ("Nanochat在nanoGPT之上的新增
// 功能", section 1 feature table: dynamic per-tensor fp8 with e4m3 / e5m2;
// "nanochat — 架构与原理", section 4: quantise and dequantise around each
// scaled matmul).
//
// A tensor X is quantised with s = fmax / amax(X), held in fp32 (s = 1 when
// amax is 0 or not finite): code = RNE(clamp(fp32(x * s), -fmax, fmax)) in
// the OCP e4m3 (fmax 448) or e5m2 (fmax 57344) format; the product of two
// quantised operands is rescaled by 1 / (s_a * s_b) in the GEMM epilogue.
// The gfx950 conversion instructions round to nearest-even but do not
// saturate, hence the explicit clamp.
//
// amax slots hold the bit pattern of max |x| as uint32: non-negative floats
// order like their bit patterns, so an integer atomic max reduces them.
#include "device_common.h"
#include "internal.h"

#include <algorithm>

namespace gk {

__device__ __forceinline__ int seg_of(const gpt::Segs& sg, int64_t pos) {
  int k = 0;
#pragma unroll
  for (int j = 0; j < 5; ++j)
    if (j < sg.n - 1 && pos >= sg.end[j]) k = j + 1;
  return k;
}

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* v) {
  if constexpr (sizeof(T) == 2) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = static_cast<float>(x[j]);
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a[j];
      v[4 + j] = b[j];
    }
  }
}

// Four codes, element j in byte j.
template <int FMT>
__device__ __forceinline__ uint32_t cvt4(const float* v, float s, float fmax) {
  float c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // saturate; a NaN input stays NaN (and converts to a NaN code)
    const float x = v[j] * s;
    c[j] = x > fmax ? fmax : (x < -fmax ? -fmax : x);
  }
  int w;
  if constexpr (FMT == gpt::FP8_E4M3) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c[0], c[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c[2], c[3], w, true);
  }
  return (uint32_t)w;
}

// max |x| per segment of (index mod period), atomically merged into the
// segments' amax slots. n is a multiple of 8 and every segment boundary too.
// Each block reduces through LDS and issues one atomic per segment: atomics
// on one address serialise, so their number is kept to the block count.
template <typename T>
__global__ __launch_bounds__(1024) void fp8_amax_kernel(const T* __restrict__ x, int64_t nv,
                                                       int64_t period, gpt::Segs sg,
                                                       uint32_t* __restrict__ amax) {
  __shared__ float red[6][16];
  float m[6] = {0, 0, 0, 0, 0, 0};
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  auto take = [&](int64_t v, const float* e) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(e[j]));
    const int k = sg.n > 1 ? seg_of(sg, (v * 8) % period) : 0;
#pragma unroll
    for (int j = 0; j < 6; ++j)
      if (j == k) m[j] = fmaxf(m[j], a);
  };
  // four vectors in flight per thread, then the remainder one at a time
  int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; v + 3 * stride < nv; v += 4 * stride) {
    float e[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8(x + (v + u * stride) * 8, e[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) take(v + u * stride, e[u]);
  }
  for (; v < nv; v += stride) {
    float e[8];
    load8(x + v * 8, e);
    take(v, e);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    if (j >= sg.n) break;
    const float w = wave_max(m[j]);
    if (lane == 0) red[j][wave] = w;
  }
  __syncthreads();
  if (threadIdx.x < sg.n) {
    const int j = threadIdx.x;
    float w = red[j][0];
#pragma unroll
    for (int q = 1; q < 16; ++q) w = fmaxf(w, red[j][q]);
    if (w > 0.0f) atomicMax(amax + sg.slot[j], __float_as_uint(w));
  }
}

// Quantise src [R][C] (row-major, C a multiple of 64). Writes the codes
// row-major to out [R][C] (if non-null) and transposed to outT [C][pitchT]
// (if non-null; rows R .. pitchT-1 of every column are written as zero).
// Segments run along rows (seg_rows) or along columns; each selects its own
// amax slot. Block tile: 128 rows x 64 columns; a thread loads 4 rows of one
// 8-column vector, packs the 4 row codes of each column into one dword and
// the block writes the transposed tile from LDS in 16-byte row pieces.
template <typename T, int FMT>
__global__ __launch_bounds__(256) void fp8_quant_kernel(
    const T* __restrict__ src, int64_t R, int64_t C, int seg_rows, gpt::Segs sg,
    const uint32_t* __restrict__ amax, float fmax, uint8_t* __restrict__ out,
    uint8_t* __restrict__ outT, int64_t pitchT) {
  constexpr int TP = 33;  // dword pitch of a transposed tile row: conflict-free packing writes
  __shared__ uint32_t tileT[64 * TP];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  const int64_t r0 = (int64_t)blockIdx.y * 128;
  const int cv = tid & 7, rg = tid >> 3;
  const int64_t c = c0 + cv * 8;
  const float s_col = seg_rows ? 1.0f : fp8_scale(amax[sg.slot[seg_of(sg, c)]], fmax);
  uint32_t packed[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) packed[j] = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = r0 + 4 * rg + i;
    if (r < R) {
      float v[8];
      load8(src + r * C + c, v);
      const float s = seg_rows ? fp8_scale(amax[sg.slot[seg_of(sg, r)]], fmax) : s_col;
      const uint32_t lo = cvt4<FMT>(v, s, fmax), hi = cvt4<FMT>(v + 4, s, fmax);
      if (out) *reinterpret_cast<uint2*>(out + r * C + c) = make_uint2(lo, hi);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        packed[j] |= ((lo >> (8 * j)) & 0xffu) << (8 * i);
        packed[4 + j] |= ((hi >> (8 * j)) & 0xffu) << (8 * i);
      }
    }
  }
  if (outT == nullptr) return;
#pragma unroll
  for (int j = 0; j < 8; ++j) tileT[(cv * 8 + j) * TP + rg] = packed[j];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int v = tid + i * 256;
    const int cc = v >> 3, rq = v & 7;
    const uint32_t* t = tileT + cc * TP + 4 * rq;
    *reinterpret_cast<uint4*>(outT + (c0 + cc) * pitchT + r0 + 16 * rq) =
        make_uint4(t[0], t[1], t[2], t[3]);
  }
}

}  // namespace gk

namespace gpt {
using namespace gk;

static float fmax_of(int fmt) { return fmt == FP8_E4M3 ? 448.0f : 57344.0f; }

void launch_fp8_amax(const void* x, bool bf16_src, int64_t n, int64_t period, const Segs& sg,
                     uint32_t* amax, hipStream_t s) {
  if (n <= 0) return;
  const int64_t nv = n / 8;
  // one 1024-thread block per CU at most: few atomics on the slots
  const unsigned blocks = (unsigned)std::min<int64_t>((nv + 1023) / 1024, 256);
  if (bf16_src)
    GK_LAUNCH(fp8_amax_kernel<bf16>, dim3(blocks), dim3(1024), 0, s,
                       static_cast<const bf16*>(x), nv, period, sg, amax);
  else
    GK_LAUNCH(fp8_amax_kernel<float>, dim3(blocks), dim3(1024), 0, s,
                       static_cast<const float*>(x), nv, period, sg, amax);
}

void launch_fp8_quant(const void* src, bool bf16_src, int64_t R, int64_t C, bool seg_rows,
                      const Segs& sg, const uint32_t* amax, int fmt, uint8_t* out, uint8_t* outT,
                      int64_t pitchT, hipStream_t s) {
  if (R <= 0 || C <= 0) return;
  const int64_t rows = outT ? pitchT : R;
  dim3 grid((unsigned)(C / 64), (unsigned)((rows + 127) / 128));
  const float fm = fmax_of(fmt);
#define GPT_QUANT(T, F)                                                                        \
  GK_LAUNCH((fp8_quant_kernel<T, F>), grid, dim3(256), 0, s, static_cast<const T*>(src), \
                     R, C, seg_rows ? 1 : 0, sg, amax, fm, out, outT, pitchT)
  if (bf16_src) {
    if (fmt == FP8_E4M3) GPT_QUANT(bf16, FP8_E4M3);
    else GPT_QUANT(bf16, FP8_E5M2);
  } else {
    if (fmt == FP8_E4M3) GPT_QUANT(float, FP8_E4M3);
    else GPT_QUANT(float, FP8_E5M2);
  }
#undef GPT_QUANT
}

}  // namespace gpt
