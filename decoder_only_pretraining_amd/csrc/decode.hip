// Decode attention over a KV cache: the newest token of each sequence
// attends its cached keys and values ("Nanochat在nanoGPT之上的新增功能",
// inference engine: pre-allocated KV cache; "nanochat — 架构与原理", section
// 5: flash attention with a KV cache), with the model's GQA head mapping and
// sliding window (additions page, notes on GQA and the sliding window).
//
// The work is reading the cache: per (sequence, KV head) 2 * n * D bf16
// values for n visible keys, shared by the G = H / Hk query heads of the
// group. The visible keys of a (sequence, KV head) are cut into chunks of
// kDecChunk = 128, one workgroup of 4 wavefronts each, which write their
// states (running maximum, exponential sum, weighted value sum per query
// head); a second kernel combines them in chunk order (a single chunk
// writes the output itself). Inside a workgroup, D/8 lanes hold one key (8
// elements each, one 16-byte load of K and one of V), so a wavefront step
// covers 64 / (D/8) keys; each wavefront takes 32 consecutive keys and
// issues all their loads before the first score, so the whole chunk is in
// flight at once (the kernel is bound by HBM latency as much as by
// bandwidth: every cache row is read once). Measured on the d12 decode
// workload: one workgroup of 16 wavefronts per (sequence, KV head), which
// needs no combine, ran 1.7x slower (a single CU's share of the cache
// streams at ~30 GB/s, so all CUs must take part); a last-workgroup-combines
// scheme needed device-scope fences, whose cache write-backs cost more than
// the combine kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "device_common.h"
#include "internal.h"

namespace gk {

constexpr int kDecChunk = 128;  // keys per workgroup
constexpr int kDecWaves = 4;    // wavefronts per workgroup (32 keys each)

__device__ __forceinline__ void merge_state(float& m, float& l, float* acc, float mo, float lo,
                                            const float* acco) {
  const float mn = fmaxf(m, mo);
  if (mn == -INFINITY) return;  // both empty
  const float c1 = exp2f(m - mn), c2 = exp2f(mo - mn);
  l = l * c1 + lo * c2;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = acc[e] * c1 + acco[e] * c2;
  m = mn;
}

// Scores are taken in log2 units (q pre-scaled by log2(e) / sqrt(D)).
// S == 1: out[b][h] is written; else the state of chunk c of head h goes to
// part[((b H + h) S + c)][D + 2] = (sum_s p_s v_s [D], max, sum_s p_s),
// p_s = 2^(score_s - max); a chunk with no visible key has max -inf.
template <int D, int G, int NW = kDecWaves>
__global__ __launch_bounds__(NW * 64) void decode_attn_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int32_t* __restrict__ seqlen, float* __restrict__ part, bf16* __restrict__ out, int H,
    int Hk, int Tmax, int window, int S, int chunk) {
  constexpr int LPK = D / 8, KPI = 64 / LPK, STEPS = 32 / KPI;
  __shared__ float red[NW][G][LPK][10];
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int sub = lane % LPK, slot = lane / LPK;
  const int t = min(max(seqlen[b], 1), Tmax) - 1;
  const int lo = window >= 0 ? max(0, t - window) : 0;
  const int c0 = lo + c * chunk, c1 = min(t + 1, c0 + chunk);
  const float qs = 1.4426950408889634f / sqrtf((float)D);
  float qv[G][8], m[G], l[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(q + ((size_t)b * H + j * G + g) * D + sub * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qv[g][e] = static_cast<float>(x[e]) * qs;
      acc[g][e] = 0.0f;
    }
    m[g] = -INFINITY;
    l[g] = 0.0f;
  }
  for (int r0 = c0; r0 < c1; r0 += NW * 32) {
    const int w0 = r0 + wv * 32 + slot;  // this lane's first key of the round
    bf16x8 kx[STEPS], vx[STEPS];
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
      const int s = w0 + i * KPI;
      const size_t row = ((size_t)b * Tmax + (s < c1 ? s : lo)) * Hk + j;
      kx[i] = *reinterpret_cast<const bf16x8*>(k + row * D + sub * 8);
      vx[i] = *reinterpret_cast<const bf16x8*>(v + row * D + sub * 8);
    }
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
      const bool ok = w0 + i * KPI < c1;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float dot = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) dot += qv[g][e] * static_cast<float>(kx[i][e]);
#pragma unroll
        for (int o = LPK / 2; o > 0; o >>= 1) dot += __shfl_xor(dot, o, kWave);
        if (ok) {
          const float mn = fmaxf(m[g], dot);
          const float corr = exp2f(m[g] - mn), p = exp2f(dot - mn);
          l[g] = l[g] * corr + p;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            acc[g][e] = acc[g][e] * corr + p * static_cast<float>(vx[i][e]);
          m[g] = mn;
        }
      }
    }
  }
  // the key slots of the wavefront (lanes sub, sub + LPK, ...)
#pragma unroll
  for (int o = LPK; o < 64; o <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], o, kWave), lo2 = __shfl_xor(l[g], o, kWave);
      float ao[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ao[e] = __shfl_xor(acc[g][e], o, kWave);
      merge_state(m[g], l[g], acc[g], mo, lo2, ao);
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      red[wv][g][sub][0] = m[g];
      red[wv][g][sub][1] = l[g];
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wv][g][sub][2 + e] = acc[g][e];
    }
  }
  __syncthreads();
  // the wavefronts, in order; thread (g, sub) finishes its 8 columns
  for (int i = threadIdx.x; i < G * LPK; i += NW * 64) {
    const int g = i / LPK, sb = i % LPK;
    float mm = red[0][g][sb][0], ll = red[0][g][sb][1], aa[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) aa[e] = red[0][g][sb][2 + e];
    for (int w = 1; w < NW; ++w)
      merge_state(mm, ll, aa, red[w][g][sb][0], red[w][g][sb][1], &red[w][g][sb][2]);
    const size_t bh = (size_t)b * H + j * G + g;
    if (S == 1) {  // every visible key was this workgroup's: ll >= 1
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = static_cast<bf16>(aa[e] / ll);
      *reinterpret_cast<bf16x8*>(out + bh * D + sb * 8) = o;
    } else {
      float* dst = part + (bh * S + c) * (D + 2);
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[sb * 8 + e] = aa[e];
      if (sb == 0) {
        dst[D] = mm;
        dst[D + 1] = ll;
      }
    }
  }
}

// out[b][h][:] from the S chunk states of (b, h): one pass rescaling to the
// running maximum, eight chunks' loads issued together; chunks past the
// visible keys (maximum -inf, sums 0) leave the state unchanged.
template <int D>
__global__ __launch_bounds__(D) void decode_attn_combine_kernel(const float* __restrict__ part,
                                                                bf16* __restrict__ out, int S) {
  const size_t bh = blockIdx.x;
  const float* p = part + bh * S * (D + 2);
  float M = -INFINITY, L = 0.0f, A = 0.0f;
  for (int c0 = 0; c0 < S; c0 += 8) {
    float mc[8], lc[8], ac[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float* pc = p + (size_t)min(c0 + i, S - 1) * (D + 2);
      mc[i] = c0 + i < S ? pc[D] : -INFINITY;
      lc[i] = pc[D + 1];
      ac[i] = pc[threadIdx.x];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (mc[i] != -INFINITY) {
        const float mn = fmaxf(M, mc[i]);
        const float s1 = exp2f(M - mn), s2 = exp2f(mc[i] - mn);
        L = L * s1 + lc[i] * s2;
        A = A * s1 + ac[i] * s2;
        M = mn;
      }
    }
  }
  out[bh * D + threadIdx.x] = static_cast<bf16>(A / L);
}

// KV-cache append: token i of sequence b (qkv row b * n_new + i) goes to
// position pos[b] + i; one thread per 16-byte vector of its k and v heads.
// Positions outside [0, Tmax) are skipped.
__global__ __launch_bounds__(256) void kv_cache_append_kernel(
    const bf16* __restrict__ qkv, const int32_t* __restrict__ pos, bf16* __restrict__ kc,
    bf16* __restrict__ vc, int B, int n_new, int H, int Hk, int D, int Tmax) {
  const int per_head = D / 8;
  const int64_t per_tok = (int64_t)2 * Hk * per_head;  // k vectors, then v vectors
  const int64_t total = (int64_t)B * n_new * per_tok;
  const int64_t row_w = (int64_t)(H + 2 * Hk) * D;
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < total;
       x += (int64_t)gridDim.x * 256) {
    const int64_t tokrow = x / per_tok;  // b * n_new + i
    const int r = (int)(x % per_tok);
    const int b = (int)(tokrow / n_new), i = (int)(tokrow % n_new);
    const int p = pos[b] + i;
    if (p < 0 || p >= Tmax) continue;
    const bool is_v = r >= Hk * per_head;
    const int rr = is_v ? r - Hk * per_head : r;  // head * per_head + vector
    const bf16x8 val = *reinterpret_cast<const bf16x8*>(
        qkv + tokrow * row_w + (int64_t)(H + (is_v ? Hk : 0)) * D + (int64_t)rr * 8);
    bf16* dst = is_v ? vc : kc;
    *reinterpret_cast<bf16x8*>(dst + ((int64_t)b * Tmax + p) * Hk * D + (int64_t)rr * 8) = val;
  }
}

}  // namespace gk

namespace gk {

// Scratch of the no-allocation entry point (gpt_decode_attn_noalloc): the
// chunk states of one call live in this file-scope device array instead of
// a caller's workspace. Each GPU the library runs on holds its own copy
// until the process ends. In host code `dec_scratch` names a host-side
// stand-in, never the device memory: its device address comes from
// hipGetSymbolAddress (decode_scratch below) and only that address is
// passed to kernels.
constexpr size_t kDecScratchBytes = (size_t)4 << 20;
static __device__ __attribute__((aligned(256))) float dec_scratch[kDecScratchBytes / sizeof(float)];

}  // namespace gk

namespace gpt {

size_t decode_scratch_capacity() { return gk::kDecScratchBytes; }

// Device address of the current GPU's copy of dec_scratch, looked up once
// per device (with that device current) and kept.
hipError_t decode_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(gk::dec_scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

// Chunks per (sequence, KV head) for the longest visible range.
int decode_splits(int Tmax, int window) {
  const int vis = window >= 0 ? std::min(Tmax, window + 1) : Tmax;
  return (vis + gk::kDecChunk - 1) / gk::kDecChunk;
}

size_t decode_workspace_bytes(int B, int H, int Hk, int D, int Tmax, int window) {
  const int S = decode_splits(Tmax, window);
  return S == 1 ? 0 : (size_t)B * H * S * (D + 2) * sizeof(float);
}

void launch_decode_attn(int B, int H, int Hk, int D, int Tmax, int window, const void* q,
                        const void* k, const void* v, const int32_t* seqlen, void* out,
                        void* workspace, hipStream_t s) {
  const int S = decode_splits(Tmax, window);
  const int chunk = gk::kDecChunk;
  const int G = H / Hk;
  const dim3 grid((unsigned)S, (unsigned)Hk, (unsigned)B);
  const bf16* qp = static_cast<const bf16*>(q);
  const bf16* kp = static_cast<const bf16*>(k);
  const bf16* vp = static_cast<const bf16*>(v);
  bf16* op = static_cast<bf16*>(out);
  float* part = static_cast<float*>(workspace);
#define DEC_P(DD, GG)                                                                        \
  GK_LAUNCH((gk::decode_attn_kernel<DD, GG>), grid, dim3(gk::kDecWaves * 64), 0, s,     \
                     qp, kp, vp, seqlen, part, op, H, Hk, Tmax, window, S, chunk)
#define DEC_G(DD)                      \
  switch (G) {                         \
    case 1: DEC_P(DD, 1); break;       \
    case 2: DEC_P(DD, 2); break;       \
    case 3: DEC_P(DD, 3); break;       \
    case 4: DEC_P(DD, 4); break;       \
    case 5: DEC_P(DD, 5); break;       \
    case 6: DEC_P(DD, 6); break;       \
    case 7: DEC_P(DD, 7); break;       \
    default: DEC_P(DD, 8); break;      \
  }
  if (D == 128) {
    DEC_G(128);
    if (S > 1)
      GK_LAUNCH(gk::decode_attn_combine_kernel<128>, dim3((unsigned)(B * H)), dim3(128),
                         0, s, part, op, S);
  } else {
    DEC_G(64);
    if (S > 1)
      GK_LAUNCH(gk::decode_attn_combine_kernel<64>, dim3((unsigned)(B * H)), dim3(64), 0,
                         s, part, op, S);
  }
#undef DEC_G
#undef DEC_P
}

void launch_kv_cache_append(int B, int n_new, int H, int Hk, int D, int Tmax, const void* qkv,
                            const int32_t* pos, void* k, void* v, hipStream_t s) {
  const int64_t total = (int64_t)B * n_new * 2 * Hk * (D / 8);
  const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
  GK_LAUNCH(gk::kv_cache_append_kernel, dim3(blocks), dim3(256), 0, s,
                     static_cast<const bf16*>(qkv), pos, static_cast<bf16*>(k),
                     static_cast<bf16*>(v), B, n_new, H, Hk, D, Tmax);
}

}  // namespace gpt
