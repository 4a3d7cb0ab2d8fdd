// Memory-bound kernels of the GPT step: weight cast, embedding gather and
// scatter, residual mix + RMSNorm (forward and backward), RoPE + QK-norm +
// value-embedding gate (forward and backward), softcap cross-entropy loss,
// and the small deterministic reductions for the lambda and gate weights.
//
// Row kernels give one 64-lane wavefront to one row of n_embd features and
// reduce with cross-lane shuffles; feature loads are 16-byte vectors.
#include "device_common.h"
#include "internal.h"

#include <mutex>

namespace gk {


// ------------------------------------------------------------ cast / zero
struct CastTable {
  gpt::CastSeg seg[128];
  int nseg;
};

__global__ __launch_bounds__(256) void cast_kernel(const float* __restrict__ src,
                                                   bf16* __restrict__ dst, CastTable t) {
  const gpt::CastSeg sg = t.seg[blockIdx.y];
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 8;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8; i < sg.n; i += stride) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(src + sg.off + i);
    const f32x4 b = *reinterpret_cast<const f32x4*>(src + sg.off + i + 4);
    bf16x8 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[j] = static_cast<bf16>(a[j]);
      o[j + 4] = static_cast<bf16>(b[j]);
    }
    *reinterpret_cast<bf16x8*>(dst + sg.off + i) = o;
  }
}

// Cast of weight matrices [rows][cols] (fp32, at offsets off[z]) to the
// compute-dtype mirror, plus a transposed mirror [cols][rows] for the
// products that contract over a weight's rows (input gradients). One 64 x 64
// tile per workgroup, transposed through LDS; both stores are 16 or 8 bytes
// per lane along rows of their own matrix.
struct CastTTable {
  int64_t off[64];
  int rows, cols;
};
__global__ __launch_bounds__(256) void cast_t_kernel(const float* __restrict__ src,
                                                     bf16* __restrict__ dst,
                                                     bf16* __restrict__ dstT, CastTTable t) {
  __shared__ float tile[64][65];
  const int tid = threadIdx.x;
  const int64_t off = t.off[blockIdx.z];
  const int R = t.rows, Cc = t.cols;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const float* a = src + off;
  // rows r0 + tid / 16 + 16 i, columns c0 + 4 (tid % 16) .. + 3
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = tid / 16 + 16 * i, c = (tid % 16) * 4;
    f32x4 v = {0, 0, 0, 0};
    if (r0 + r < R) {
      if (c0 + c + 3 < Cc) {
        v = *reinterpret_cast<const f32x4*>(a + (int64_t)(r0 + r) * Cc + c0 + c);
      } else {
        for (int j = 0; j < 4; ++j)
          if (c0 + c + j < Cc) v[j] = a[(int64_t)(r0 + r) * Cc + c0 + c + j];
      }
      bf16* o = dst + off + (int64_t)(r0 + r) * Cc + c0 + c;
      if (c0 + c + 3 < Cc) {
        bf16x4 w;
        for (int j = 0; j < 4; ++j) w[j] = static_cast<bf16>(v[j]);
        *reinterpret_cast<bf16x4*>(o) = w;
      } else {
        for (int j = 0; j < 4; ++j)
          if (c0 + c + j < Cc) o[j] = static_cast<bf16>(v[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) tile[r][c + j] = v[j];
  }
  __syncthreads();
  // transposed: rows c0 + tid / 8 + 32 i, columns r0 + 8 (tid % 8) .. + 7
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid / 8 + 32 * i, r = (tid % 8) * 8;
    if (c0 + c >= Cc) continue;
    bf16* o = dstT + off + (int64_t)(c0 + c) * R + r0 + r;
    if (r0 + r + 7 < R) {
      bf16x8 w;
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = static_cast<bf16>(tile[r + j][c]);
      *reinterpret_cast<bf16x8*>(o) = w;
    } else {
      for (int j = 0; j < 8; ++j)
        if (r0 + r + j < R) o[j] = static_cast<bf16>(tile[r + j][c]);
    }
  }
}

__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n4 = n / 4;
  for (int64_t j = i; j < n4; j += stride) reinterpret_cast<f32x4*>(p)[j] = f32x4{0, 0, 0, 0};
  for (int64_t j = n4 * 4 + i; j < n; j += stride) p[j] = 0.0f;
}

// cos / sin of t * theta^(-2i/D), evaluated in double precision.
__global__ void rope_table_kernel(float* __restrict__ cs, int T, int D, double theta) {
  const int h = D / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * h) return;
  const int t = (int)(idx / h), i = (int)(idx % h);
  const double inv = pow(theta, -2.0 * i / (double)D);
  const double phi = (double)t * inv;
  cs[idx] = (float)cos(phi);
  cs[(int64_t)T * h + idx] = (float)sin(phi);
}

// ------------------------------------------------------------ embedding
// Row `id` of a [V][W] table, or a row of zeros for an id outside [0, V):
// such ids violate the call's precondition, and every table access goes
// through here so that they never read outside the table (W <= 2048).
static __device__ __attribute__((aligned(16))) float g_zero_row[2048];
__device__ __forceinline__ const float* table_row(const float* tab, int32_t id, int V, int W) {
  return (uint32_t)id < (uint32_t)V ? tab + (int64_t)id * W : g_zero_row;
}

__global__ __launch_bounds__(256) void embed_kernel(const float* __restrict__ wte,
                                                    const int32_t* __restrict__ tok,
                                                    float* __restrict__ x0, int64_t N, int C, int V) {
  const int64_t n = blockIdx.x;
  const f32x4* s = reinterpret_cast<const f32x4*>(table_row(wte, tok[n], V, C));
  f32x4* o = reinterpret_cast<f32x4*>(x0 + n * C);
  for (int c = threadIdx.x; c < C / 4; c += blockDim.x) o[c] = s[c];
}

// ------------------------------------------------------------ Smear
// Smear at the embedding ("Nanochat在nanoGPT之上的新增功能", feature table
// row Smear and its note): x0[n] = e[n] + sigmoid(<e[n], w>) * e[n - 1] with
// e[n] = wte[tok[n]], for positions t = n mod T >= 1; x0[n] = e[n] at t = 0.
// One wavefront per row; the gate value (0 at t = 0) is kept for the
// backward.
template <int NC>
__global__ __launch_bounds__(256) void smear_embed_kernel(const float* __restrict__ wte,
                                                          const int32_t* __restrict__ tok,
                                                          const float* __restrict__ w,
                                                          float* __restrict__ x0,
                                                          float* __restrict__ sig, int64_t N,
                                                          int T, int C, int V) {
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const int C4 = C / 4;
  const bool has_prev = (n % T) != 0;  // uniform over the wavefront
  const f32x4* e = reinterpret_cast<const f32x4*>(table_row(wte, tok[n], V, C));
  f32x4* o = reinterpret_cast<f32x4*>(x0 + n * C);
  if (!has_prev) {
#pragma unroll
    for (int i = 0; i < NC; ++i)
      if (lane + i * 64 < C4) o[lane + i * 64] = e[lane + i * 64];
    if (lane == 0) sig[n] = 0.0f;
    return;
  }
  const f32x4* ep = reinterpret_cast<const f32x4*>(table_row(wte, tok[n - 1], V, C));
  f32x4 ev[NC], pv[NC];
  float dot = 0.0f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c4 = lane + i * 64;
    if (c4 < C4) {
      ev[i] = e[c4];
      pv[i] = ep[c4];
      const f32x4 wv = reinterpret_cast<const f32x4*>(w)[c4];
      dot += ev[i][0] * wv[0] + ev[i][1] * wv[1] + ev[i][2] * wv[2] + ev[i][3] * wv[3];
    }
  }
  dot = wave_sum(dot);
  const float g = 1.0f / (1.0f + expf(-dot));
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c4 = lane + i * 64;
    if (c4 < C4) o[c4] = ev[i] + g * pv[i];
  }
  if (lane == 0) sig[n] = g;
}

// Backward of the smear, from g = dL/dx0 [N][C]:
//   ge[n] = g[n] + sig[n+1] g[n+1]          (n+1 in the same sequence)
//             + dz[n] w,  dz[n] = sig[n] (1 - sig[n]) <g[n], e[n-1]>  (t >= 1)
//   g_w  += dz[n] e[n].
// A workgroup takes kSmearRows consecutive rows, 16 per wavefront in groups
// of 4 whose gradient and embedding rows are loaded together (row n needs
// g[n], g[n+1], e[n-1], e[n]: 5 + 5 row loads per group of 4). The g_w
// terms are summed in registers, then over the 4 wavefronts in LDS, and the
// workgroup writes its partial part[blockIdx][C]; the partials are added in
// workgroup order afterwards.
constexpr int kSmearRows = 64;
template <int NC>
__global__ __launch_bounds__(256) void smear_bwd_kernel(const float* __restrict__ g,
                                                        const float* __restrict__ wte,
                                                        const int32_t* __restrict__ tok,
                                                        const float* __restrict__ w,
                                                        const float* __restrict__ sig,
                                                        float* __restrict__ ge,
                                                        float* __restrict__ part, int64_t N,
                                                        int T, int C, int V) {
  constexpr int RG = 4, GROUPS = kSmearRows / 4 / RG;
  __shared__ f32x4 red[4][NC * 64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int C4 = C / 4;
  f32x4 wgt[NC], acc[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c4 = lane + i * 64;
    acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    wgt[i] = acc[i];
    if (c4 < C4) wgt[i] = reinterpret_cast<const f32x4*>(w)[c4];
  }
  const int64_t base = (int64_t)blockIdx.x * kSmearRows + wv * (kSmearRows / 4);
  for (int gi = 0; gi < GROUPS; ++gi) {
    const int64_t n0 = base + gi * RG;
    if (n0 >= N) break;  // uniform over the wavefront
    f32x4 G[RG + 1][NC], E[RG + 1][NC];  // G[j] = g[n0 + j], E[j] = e[n0 - 1 + j]
#pragma unroll
    for (int j = 0; j <= RG; ++j) {
      const int64_t n = n0 + j, m = n0 - 1 + j;
      const f32x4* gr = reinterpret_cast<const f32x4*>(g + (n < N ? n : 0) * C);
      const f32x4* er = reinterpret_cast<const f32x4*>(table_row(wte, tok[m >= 0 && m < N ? m : 0], V, C));
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int c4 = lane + i * 64;
        if (c4 < C4) {
          G[j][i] = gr[c4];
          E[j][i] = er[c4];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      const int64_t n = n0 + j;
      if (n < N) {
        const int t = (int)(n % T);
        f32x4 out[NC];
#pragma unroll
        for (int i = 0; i < NC; ++i) out[i] = G[j][i];
        if (t + 1 < T) {  // n + 1 < N: same sequence
          const float sn1 = sig[n + 1];
#pragma unroll
          for (int i = 0; i < NC; ++i) out[i] += sn1 * G[j + 1][i];
        }
        if (t > 0) {
          float dot = 0.0f;
#pragma unroll
          for (int i = 0; i < NC; ++i)
            if (lane + i * 64 < C4)
              dot += G[j][i][0] * E[j][i][0] + G[j][i][1] * E[j][i][1] +
                     G[j][i][2] * E[j][i][2] + G[j][i][3] * E[j][i][3];
          dot = wave_sum(dot);
          const float sn = sig[n];
          const float dz = sn * (1.0f - sn) * dot;
#pragma unroll
          for (int i = 0; i < NC; ++i) {
            out[i] += dz * wgt[i];
            acc[i] += dz * E[j + 1][i];
          }
        }
#pragma unroll
        for (int i = 0; i < NC; ++i) {
          const int c4 = lane + i * 64;
          if (c4 < C4) reinterpret_cast<f32x4*>(ge + n * C)[c4] = out[i];
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NC; ++i) red[wv][i * 64 + lane] = acc[i];
  __syncthreads();
  for (int c4 = threadIdx.x; c4 < C4; c4 += 256)
    reinterpret_cast<f32x4*>(part + (int64_t)blockIdx.x * C)[c4] =
        ((red[0][c4] + red[1][c4]) + red[2][c4]) + red[3][c4];
}

// The final norm's mix weights under Backout: out[0] = 1 (the stream),
// out[1] = -lambda (the cached stream).
__global__ void backout_weights_kernel(const float* __restrict__ lam, float* __restrict__ out) {
  if (threadIdx.x == 0) {
    out[0] = 1.0f;
    out[1] = -lam[0];
  }
}

// ------------------------------------------------------------ embedding-table gradients
// tab[tok[n]][:] += g[n][:] for the rows g of N positions. Frequent token
// ids would serialise per-position atomic adds on one table row, so the
// positions are cut into chunks of kChunk and, in each chunk, the first
// position holding an id (its leader) sums the rows of all the chunk's
// positions with that id, in position order, and makes the one atomic add
// per column. The links (leader flag, next position of the same id in the
// chunk) depend only on the tokens and are built once per call.
constexpr int kChunk = 128;

// link[n] = next position of tok[n]'s id in n's chunk (-1: none);
// link[N + n] = 1 if n is the first of its id in its chunk, else 0
__global__ __launch_bounds__(kChunk) void token_links_kernel(const int32_t* __restrict__ tok,
                                                             int64_t N, int32_t* __restrict__ link) {
  __shared__ int32_t ids[kChunk];
  const int t = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.x * kChunk;
  const int cnt = (int)min<int64_t>(kChunk, N - n0);
  ids[t] = t < cnt ? tok[n0 + t] : -1;
  __syncthreads();
  if (t >= cnt) return;
  const int my = ids[t];
  int first = 1, next = -1;
  for (int k = 0; k < t; ++k)
    if (ids[k] == my) {
      first = 0;
      break;
    }
  for (int k = t + 1; k < cnt; ++k)
    if (ids[k] == my) {
      next = k;
      break;
    }
  link[n0 + t] = next >= 0 ? (int32_t)(n0 + next) : -1;
  link[N + n0 + t] = first;
}

// One workgroup per (chunk, slice of CW columns): the chunk's rows of the
// slice are staged in LDS with every load in flight at once, the chunk's
// leaders are listed in position order (a ballot over the first 128
// threads), and the 256 / CW groups of threads take every (256 / CW)-th
// leader, each thread one column: its sum formed from LDS in position
// order, then one atomic add. (A single scan over all positions by every
// thread, and a workgroup per position walking the links in global
// memory, each spent their time waiting on dependent loads.)
template <int CW>
__global__ __launch_bounds__(256) void rows_to_table_kernel(const float* __restrict__ g, int W,
                                                            const int32_t* __restrict__ tok,
                                                            const int32_t* __restrict__ link,
                                                            int64_t N, float* __restrict__ tab,
                                                            int V) {
  static_assert(256 % CW == 0 && kChunk * CW / 4 % 256 == 0 && kChunk == 128,
                "whole vectors per thread; two wavefronts list the leaders");
  __shared__ __attribute__((aligned(16))) float rows[kChunk][CW];
  __shared__ int32_t ids[kChunk], nxt[kChunk], leaders[kChunk];
  __shared__ int nlead0, nlead;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t n0 = (int64_t)blockIdx.x * kChunk;
  const int cnt = (int)min<int64_t>(kChunk, N - n0);
  const int c0 = blockIdx.y * CW;
  int is_lead = 0;
  if (tid < cnt) {
    ids[tid] = tok[n0 + tid];
    const int32_t nx = link[n0 + tid];
    nxt[tid] = nx >= 0 ? (int32_t)(nx - n0) : -1;
    is_lead = link[N + n0 + tid];
  }
  constexpr int VPR = CW / 4, NV = kChunk * VPR / 256;  // 16-byte vectors per row, per thread
  f32x4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = tid + 256 * i, r = e / VPR, c4 = (e % VPR) * 4;
    if (r < cnt) v[i] = *reinterpret_cast<const f32x4*>(g + (n0 + r) * W + c0 + c4);
  }
  // leaders in position order: positions 0-63 are wavefront 0's lanes,
  // 64-127 wavefront 1's
  const uint64_t bal = __ballot(is_lead);
  const int below = __popcll(bal & ((1ull << lane) - 1ull));
  if (tid == 63) nlead0 = __popcll(bal);
  __syncthreads();
  if (tid < 128 && is_lead) leaders[(tid < 64 ? 0 : nlead0) + below] = tid;
  if (tid == 127) nlead = nlead0 + __popcll(bal);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = tid + 256 * i, r = e / VPR, c4 = (e % VPR) * 4;
    if (r < cnt) *reinterpret_cast<f32x4*>(&rows[r][c4]) = v[i];
  }
  __syncthreads();
  constexpr int GROUPS = 256 / CW;
  const int col = tid % CW, grp = tid / CW;
  for (int k = grp; k < nlead; k += GROUPS) {
    const int p = leaders[k];
    const int32_t id = ids[p];
    // an id outside [0, V) (and so its whole link chain) has no table row
    if ((uint32_t)id >= (uint32_t)V) continue;
    float acc = rows[p][col];
    for (int q = nxt[p]; q >= 0; q = nxt[q]) acc += rows[q][col];
    atomicAdd(tab + (int64_t)id * W + c0 + col, acc);
  }
}

// ------------------------------------------------------------ mix + RMSNorm
template <typename T>
__device__ __forceinline__ void store4(T* p, const f32x4& v);
template <>
__device__ __forceinline__ void store4<float>(float* p, const f32x4& v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, const f32x4& v) {
  bf16x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = static_cast<bf16>(v[j]);
  *reinterpret_cast<bf16x4*>(p) = o;
}
template <typename T>
__device__ __forceinline__ f32x4 load4(const T* p);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
template <>
__device__ __forceinline__ f32x4 load4<bf16>(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{static_cast<float>(v[0]), static_cast<float>(v[1]), static_cast<float>(v[2]),
               static_cast<float>(v[3])};
}
__device__ __forceinline__ f32x4 round4(const f32x4& v, float) { return v; }
__device__ __forceinline__ f32x4 round4(const f32x4& v, bf16) {
  f32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = static_cast<float>(static_cast<bf16>(v[j]));
  return r;
}

// One wavefront per row. With gate weights (STAGED) the workgroup first
// stages them in LDS (hk x C floats, dynamic) and its NT / 64 wavefronts
// then take rows in a grid-stride loop, so the weights are read from L2
// once per workgroup rather than once per row. Up to 64 KB of weights the
// workgroups have 256 threads; larger ones (up to the device's LDS per
// workgroup) have 1024, one workgroup per CU sharing one copy.
template <typename T, int NC, bool STAGED = false, int NT = 256>
__global__ __launch_bounds__(NT) void mix_norm_kernel(
    const float* __restrict__ x, const float* __restrict__ x0, const float* __restrict__ lam_r,
    const float* __restrict__ lam_0, float* __restrict__ xin_out, T* __restrict__ y,
    float* __restrict__ r_out, const float* __restrict__ wg, float* __restrict__ a, int64_t N,
    int C, int hk, float eps) {
  extern __shared__ f32x4 wgs[];  // hk * C / 4 vectors, with gate weights only
  const int lane = threadIdx.x & 63;
  const int C4 = C / 4;
  constexpr int RW = NT / 64;  // rows in flight per workgroup
  if (STAGED) {
    for (int i = threadIdx.x; i < hk * C4; i += NT) wgs[i] = reinterpret_cast<const f32x4*>(wg)[i];
    __syncthreads();
  }
  const f32x4* wsrc = STAGED ? wgs : reinterpret_cast<const f32x4*>(wg);
  const float lr = x0 ? lam_r[0] : 1.0f, l0 = x0 ? lam_0[0] : 0.0f;
  for (int64_t n = (int64_t)blockIdx.x * RW + (threadIdx.x >> 6); n < N;
       n += (int64_t)gridDim.x * RW) {
    f32x4 v[NC];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c4 = lane + i * 64;
      if (c4 < C4) {
        f32x4 xv = reinterpret_cast<const f32x4*>(x + n * C)[c4];
        if (x0) {
          const f32x4 zv = reinterpret_cast<const f32x4*>(x0 + n * C)[c4];
          xv = lr * xv + l0 * zv;
          if (xin_out) reinterpret_cast<f32x4*>(xin_out + n * C)[c4] = xv;
        }
        v[i] = xv;
        ss += xv[0] * xv[0] + xv[1] * xv[1] + xv[2] * xv[2] + xv[3] * xv[3];
      }
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)C + eps);
    if (lane == 0) r_out[n] = r;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c4 = lane + i * 64;
      if (c4 < C4) {
        v[i] = round4(v[i] * r, T{});
        store4<T>(y + n * C + c4 * 4, v[i]);
      }
    }
    if (wg) {  // gate logits from the rounded norm output, four KV heads at a time
      for (int j0 = 0; j0 < hk; j0 += 4) {
        float dot[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = min(j0 + q, hk - 1);  // past hk: a valid row, result unused
          dot[q] = 0.0f;
#pragma unroll
          for (int i = 0; i < NC; ++i) {
            const int c4 = lane + i * 64;
            if (c4 < C4) {
              const f32x4 w = wsrc[j * C4 + c4];
              dot[q] += v[i][0] * w[0] + v[i][1] * w[1] + v[i][2] * w[2] + v[i][3] * w[3];
            }
          }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1)
#pragma unroll
          for (int q = 0; q < 4; ++q) dot[q] += __shfl_xor(dot[q], o, kWave);
        if (lane == 0)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (j0 + q < hk) a[n * hk + j0 + q] = dot[q];
      }
    }
  }
}

// ------------------------------------------------------------ norm backward
// g_in -> g w.r.t. the norm input: r * (g - y * mean(g * y)), with the norm
// output y recomputed in fp32 from the fp32 norm input, so the result is
// orthogonal to that input to fp32 precision (the lambda gradients are
// projections on it).
template <int NC>
__global__ __launch_bounds__(256) void norm_bwd_kernel(gpt::NormBwdArgs p, int64_t N, int C,
                                                       int hk) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t n = (int64_t)blockIdx.x * 4 + wv;
  const int C4 = C / 4;
  __shared__ float part[4][2];
  float s_lr = 0.0f, s_l0 = 0.0f;
  const bool norm1 = p.mode == gpt::NB_NORM1;
  if (n < N) {
    f32x4 g[NC], yv[NC];
    const float r = p.r[n];
    const float lr = norm1 ? p.lam_r[0] : 1.0f;
    const float l0 = norm1 ? p.lam_0[0] : 0.0f;
    float dot = 0.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c4 = lane + i * 64;
      if (c4 < C4) g[i] = reinterpret_cast<const f32x4*>(p.gin + n * C)[c4];
    }
    if (norm1 && p.ga) {  // the value-embedding gate's share: g += sum_j ga[j] * wg[j]
      for (int j0 = 0; j0 < hk; j0 += 4) {  // four KV heads' loads at a time
        float gj[4];
        f32x4 w[4][NC];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = min(j0 + q, hk - 1);  // past hk: a valid row, not used
          gj[q] = p.ga[n * hk + j];
#pragma unroll
          for (int i = 0; i < NC; ++i) {
            const int c4 = lane + i * 64;
            if (c4 < C4) w[q][i] = reinterpret_cast<const f32x4*>(p.wg + (int64_t)j * C)[c4];
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (j0 + q < hk) {
#pragma unroll
            for (int i = 0; i < NC; ++i) {
              const int c4 = lane + i * 64;
              if (c4 < C4) g[i] += gj[q] * w[q][i];
            }
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c4 = lane + i * 64;
      if (c4 < C4) {
        const f32x4 gv = g[i];
        f32x4 src;
        if (norm1)
          src = lr * reinterpret_cast<const f32x4*>(p.x + n * C)[c4] +
                l0 * reinterpret_cast<const f32x4*>(p.x0 + n * C)[c4];
        else
          src = reinterpret_cast<const f32x4*>(p.ysrc + n * C)[c4];
        yv[i] = src * r;
        dot += gv[0] * yv[i][0] + gv[1] * yv[i][1] + gv[2] * yv[i][2] + gv[3] * yv[i][3];
      }
    }
    dot = wave_sum(dot) / (float)C;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c4 = lane + i * 64;
      if (c4 < C4) {
        f32x4 gx = r * (g[i] - yv[i] * dot);
        if (p.mode != gpt::NB_FINAL && !p.gx_first)
          gx += reinterpret_cast<const f32x4*>(p.gx + n * C)[c4];
        if (norm1) {
          // gx is now the gradient w.r.t. xin = lr * x + l0 * x0
          const f32x4 xv = reinterpret_cast<const f32x4*>(p.x + n * C)[c4];
          const f32x4 zv = reinterpret_cast<const f32x4*>(p.x0 + n * C)[c4];
          s_lr += gx[0] * xv[0] + gx[1] * xv[1] + gx[2] * xv[2] + gx[3] * xv[3];
          s_l0 += gx[0] * zv[0] + gx[1] * zv[1] + gx[2] * zv[2] + gx[3] * zv[3];
          f32x4 gr = lr * gx;  // w.r.t. the block input x
          if (p.gadd) gr += reinterpret_cast<const f32x4*>(p.gadd + n * C)[c4];
          f32x4 g0 = l0 * gx;
          if (p.last_layer0) g0 += gr;
          if (!p.gx0_first) g0 += reinterpret_cast<const f32x4*>(p.gx0 + n * C)[c4];
          reinterpret_cast<f32x4*>(p.gx0 + n * C)[c4] = g0;
          gx = gr;
        }
        if (!(norm1 && p.last_layer0)) {
          reinterpret_cast<f32x4*>(p.gx + n * C)[c4] = gx;
          if (p.gxc) {
            if (p.gxc_bf16)
              store4<bf16>(static_cast<bf16*>(p.gxc) + n * C + c4 * 4, gx);
            else
              store4<float>(static_cast<float*>(p.gxc) + n * C + c4 * 4, gx);
          }
        }
      }
    }
    if (norm1) {
      s_lr = wave_sum(s_lr);
      s_l0 = wave_sum(s_l0);
    }
  }
  if (norm1) {
    if (lane == 0) {
      part[wv][0] = s_lr;
      part[wv][1] = s_l0;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      p.lam_part[blockIdx.x * 2 + 0] = part[0][0] + part[1][0] + part[2][0] + part[3][0];
      p.lam_part[blockIdx.x * 2 + 1] = part[0][1] + part[1][1] + part[2][1] + part[3][1];
    }
  }
}

// Per-layer lambda gradients: fixed-order sums of the per-block partials;
// workgroup l takes layer l (partials at part + l * stride, outputs g_lr[l],
// g_l0[l]).
__global__ __launch_bounds__(256) void lambda_finalize_kernel(const float* __restrict__ part_all,
                                                              int nblk, int64_t stride,
                                                              float* g_lr_all, float* g_l0_all,
                                                              int accumulate, float scale) {
  __shared__ double red[2][256];
  const float* part = part_all + (int64_t)blockIdx.x * stride;
  float* g_lr = g_lr_all ? g_lr_all + blockIdx.x : nullptr;
  float* g_l0 = g_l0_all + blockIdx.x;
  double a = 0.0, b = 0.0;
  for (int i = threadIdx.x; i < nblk; i += 256) {
    a += part[2 * i];
    b += part[2 * i + 1];
  }
  red[0][threadIdx.x] = a;
  red[1][threadIdx.x] = b;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      red[0][threadIdx.x] += red[0][threadIdx.x + s];
      red[1][threadIdx.x] += red[1][threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float va = (float)(scale * red[0][0]), vb = (float)(scale * red[1][0]);
    if (g_lr) *g_lr = accumulate ? *g_lr + va : va;
    *g_l0 = accumulate ? *g_l0 + vb : vb;
  }
}

// Gate weight gradient g_Wg[j][c] = sum_n ga[n][j] * xn[n][c]. Block b sums
// the tokens [b * per, (b + 1) * per), per <= kVegPer: thread (phase,
// column group) owns 8 consecutive columns and every NP-th token of the
// range; the phases are then added in a fixed order and the block writes
// its partial. A second kernel adds the partials in block order. 32 tokens
// per block (d12: 512 blocks, two per CU) keep twice the loads in flight of
// 64-token blocks, whose threads walked their tokens in twice as many
// dependent rounds.
constexpr int kVegPer = 32;
// the smear partials (one per kSmearRows rows) fit the gate-weight partial buffer
static_assert(kSmearRows >= kVegPer, "smear partials exceed the veg partial rows");
template <typename T, int HK>
__global__ __launch_bounds__(256) void veg_partial_kernel(const float* __restrict__ ga,
                                                          const T* __restrict__ xn,
                                                          float* __restrict__ part, int64_t N,
                                                          int C, int hk, int64_t per) {
  __shared__ float red[256 * 8];
  __shared__ float gs[kVegPer * HK];  // the block's gate gradients, staged once
  const int CG = C / 8, NP = 256 / CG;  // column groups, token phases (C <= 2048)
  const int cg = threadIdx.x % CG, ph = threadIdx.x / CG;
  const int64_t lo = (int64_t)blockIdx.x * per, hi = lo + per < N ? lo + per : N;
  for (int64_t i = threadIdx.x; i < (hi - lo) * hk; i += 256) gs[i] = ga[lo * hk + i];
  __syncthreads();
  float acc[HK][8];
#pragma unroll
  for (int j = 0; j < HK; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;
  if (ph < NP) {
    // eight tokens' loads are issued before their products
    for (int64_t nb = lo + ph; nb < hi; nb += 8 * NP) {
      f32x4 xa[8], xb[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int64_t n = min(nb + q * NP, hi - 1);
        xa[q] = load4<T>(xn + n * C + cg * 8);
        xb[q] = load4<T>(xn + n * C + cg * 8 + 4);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int64_t n = nb + q * NP;
        if (n < hi) {
#pragma unroll
          for (int j = 0; j < HK; ++j) {
            if (j < hk) {
              const float g = gs[(n - lo) * hk + j];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                acc[j][e] += g * xa[q][e];
                acc[j][4 + e] += g * xb[q][e];
              }
            }
          }
        }
      }
    }
  }
  // fully unrolled with constant indices (no early exit), so acc stays in
  // registers; j < hk is uniform over the block
#pragma unroll
  for (int j = 0; j < HK; ++j) {
    if (j < hk) {
      if (NP == 1) {  // one token phase (C > 1024): nothing to add across threads
        if (ph == 0) {
          float* dst = part + ((int64_t)blockIdx.x * hk + j) * C + cg * 8;
          *reinterpret_cast<f32x4*>(dst) = f32x4{acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
          *reinterpret_cast<f32x4*>(dst + 4) = f32x4{acc[j][4], acc[j][5], acc[j][6], acc[j][7]};
        }
        continue;
      }
      __syncthreads();
      if (ph < NP) {
#pragma unroll
        for (int e = 0; e < 8; ++e) red[threadIdx.x * 8 + e] = acc[j][e];
      }
      __syncthreads();
      if (ph == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float v = acc[j][e];
          for (int q = 1; q < NP; ++q) v += red[(q * CG + cg) * 8 + e];
          part[((int64_t)blockIdx.x * hk + j) * C + cg * 8 + e] = v;
        }
      }
    }
  }
}

// Block b adds the partials of outputs 64b .. 64b+63: wavefront w takes the
// splits w, w + 4, ..., then the four sums are added in wavefront order.
__global__ __launch_bounds__(256) void veg_finalize_kernel(const float* __restrict__ part,
                                                           float* __restrict__ g, int n, int splits,
                                                           int accumulate) {
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + lane;
  float s = 0.0f;
  if (i < n) {
#pragma unroll 16
    for (int sp = w; sp < splits; sp += 4) s += part[(int64_t)sp * n + i];
  }
  red[w][lane] = s;
  __syncthreads();
  if (w == 0 && i < n) {
    const float v = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
    g[i] = accumulate ? g[i] + v : v;
  }
}

// ------------------------------------------------------------ RoPE + QK-norm + VE
// Tasks: every (token, q or k head) pair, then (value-embedding layers) every
// (token, v head) pair. A task belongs to LP = D/8 consecutive lanes; lane q
// of it owns elements 4q .. 4q+3 and D/2 + 4q .. D/2 + 4q + 3, i.e. the
// rotation pairs (p, p + D/2) for p = 4q .. 4q+3, and the group reduces
// with LP-lane shuffles. Head slots 0..H-1 of a token's row are q heads,
// H..H+Hk-1 k heads, H+Hk..H+2Hk-1 v heads.
template <int LP>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = LP / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float dot4(const f32x4& a, const f32x4& b) {
  return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

// y = rope(x) (pairs rotated by t * theta_p), then y * r with
// r = 1 / sqrt(mean(y^2) + eps), saved for the backward; v += sigmoid(a) * ve.
template <typename T, int D>
__global__ __launch_bounds__(256) void rope_fwd_kernel(T* __restrict__ qkv, float* __restrict__ rqk,
                                                       const float* __restrict__ cs,
                                                       const float* __restrict__ a,
                                                       const float* __restrict__ ve,
                                                       const int32_t* __restrict__ tok, int64_t N,
                                                       int T_, int H, int Hk, int Qkv, float eps,
                                                       int V) {
  constexpr int H2 = D / 2, LP = D / 8;
  const int q = threadIdx.x % LP;
  const int64_t task = (int64_t)blockIdx.x * (256 / LP) + threadIdx.x / LP;
  const int R = H + Hk;
  const int64_t nrot = N * R;
  if (task < nrot) {
    const int64_t n = task / R;
    const int sl = (int)(task % R), t = (int)(n % T_);
    T* hp = qkv + n * Qkv + sl * D;  // k heads follow the q heads contiguously
    const f32x4 x1 = load4<T>(hp + 4 * q), x2 = load4<T>(hp + H2 + 4 * q);
    const f32x4 c = *reinterpret_cast<const f32x4*>(cs + (int64_t)t * H2 + 4 * q);
    const f32x4 sn = *reinterpret_cast<const f32x4*>(cs + ((int64_t)T_ + t) * H2 + 4 * q);
    const f32x4 y1 = x1 * c - x2 * sn, y2 = x1 * sn + x2 * c;
    const float ss = group_sum<LP>(dot4(y1, y1) + dot4(y2, y2));
    const float r = 1.0f / sqrtf(ss / (float)D + eps);
    store4<T>(hp + 4 * q, y1 * r);
    store4<T>(hp + H2 + 4 * q, y2 * r);
    if (q == 0) rqk[n * R + sl] = r;
  } else if (ve && task - nrot < N * Hk) {
    const int64_t n = (task - nrot) / Hk;
    const int j = (int)((task - nrot) % Hk);
    T* vp = qkv + n * Qkv + (R + j) * D;
    const float g = 1.0f / (1.0f + __expf(-a[n * Hk + j]));
    const float* er = table_row(ve, tok[n], V, Hk * D) + j * D;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int o = half * H2 + 4 * q;
      store4<T>(vp + o, load4<T>(vp + o) + g * *reinterpret_cast<const f32x4*>(er + o));
    }
  }
}

// In place on the q / k / v gradient rows: through the QK-norm
// (r * (g - y * mean(g * y)), y the saved normalised output) and the inverse
// rotation; for v heads of value-embedding layers the per-position rows of
// the table gradient and the gate logit's gradient.
template <typename T, int D>
__global__ __launch_bounds__(256) void rope_bwd_kernel(
    T* __restrict__ gqkv, const T* __restrict__ qkv, const float* __restrict__ rqk,
    const float* __restrict__ cs, const float* __restrict__ a, const float* __restrict__ ve,
    float* __restrict__ rows, float* __restrict__ ga, const int32_t* __restrict__ tok, int64_t N,
    int T_, int H, int Hk, int Qkv, int V) {
  constexpr int H2 = D / 2, LP = D / 8;
  const int q = threadIdx.x % LP;
  const int64_t task = (int64_t)blockIdx.x * (256 / LP) + threadIdx.x / LP;
  const int R = H + Hk;
  const int64_t nrot = N * R;
  if (task < nrot) {
    const int64_t n = task / R;
    const int sl = (int)(task % R), t = (int)(n % T_);
    T* gp = gqkv + n * Qkv + sl * D;
    const T* yp = qkv + n * Qkv + sl * D;
    const f32x4 g1 = load4<T>(gp + 4 * q), g2 = load4<T>(gp + H2 + 4 * q);
    const f32x4 y1 = load4<T>(yp + 4 * q), y2 = load4<T>(yp + H2 + 4 * q);
    const float dot = group_sum<LP>(dot4(g1, y1) + dot4(g2, y2)) / (float)D;
    const float r = rqk[n * R + sl];
    const f32x4 a1 = r * (g1 - y1 * dot), a2 = r * (g2 - y2 * dot);
    const f32x4 c = *reinterpret_cast<const f32x4*>(cs + (int64_t)t * H2 + 4 * q);
    const f32x4 sn = *reinterpret_cast<const f32x4*>(cs + ((int64_t)T_ + t) * H2 + 4 * q);
    store4<T>(gp + 4 * q, a1 * c + a2 * sn);
    store4<T>(gp + H2 + 4 * q, a2 * c - a1 * sn);
  } else if (ve && task - nrot < N * Hk) {
    const int64_t n = (task - nrot) / Hk;
    const int j = (int)((task - nrot) % Hk);
    const T* gp = gqkv + n * Qkv + (R + j) * D;
    const float g = 1.0f / (1.0f + __expf(-a[n * Hk + j]));
    const float* vrow = table_row(ve, tok[n], V, Hk * D) + j * D;
    // position n's row of the table gradient (added to the table per token
    // id by rows_to_table_kernel)
    float* rp = rows + n * Hk * D + j * D;
    float dot = 0.0f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int o = 4 * q + e * H2;
      const f32x4 gv = load4<T>(gp + o);
      dot += dot4(gv, *reinterpret_cast<const f32x4*>(vrow + o));
      *reinterpret_cast<f32x4*>(rp + o) = g * gv;
    }
    dot = group_sum<LP>(dot);
    if (q == 0) ga[n * Hk + j] = g * (1.0f - g) * dot;
  }
}

// ------------------------------------------------------------ loss
// 1 / n_valid (scalars[0]) from the targets; one block.
__global__ __launch_bounds__(1024) void count_valid_kernel(const int32_t* __restrict__ tgt,
                                                           float* __restrict__ scalars, int64_t N,
                                                           int V) {
  __shared__ int s_cnt[1024];
  int cnt = 0;
  // a target counts iff it lies in [0, V): -1 (and, off the precondition,
  // any other id outside the vocabulary) is ignored
  for (int64_t n = threadIdx.x; n < N; n += 1024) cnt += (uint32_t)tgt[n] < (uint32_t)V ? 1 : 0;
  s_cnt[threadIdx.x] = cnt;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if (threadIdx.x < s) s_cnt[threadIdx.x] += s_cnt[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) scalars[0] = 1.0f / (float)(s_cnt[0] > 0 ? s_cnt[0] : 1);
}

// One workgroup per token. Its softcapped logits c (|c| <= cap) are read
// once: rowsum = sum_v exp(c_v - cap) in a fixed order (per-thread sums,
// then the four wavefronts'), loss_n = cap + log(rowsum) - c[y] (0 if
// ignored). With `grad`, the row is then replaced in place by the gradient
// of the mean loss w.r.t. the raw logits z:
//   (exp(c - cap) / rowsum - [v == y]) * (1 - (c / cap)^2) / n_valid.
// |c| <= cap, so exp(c - cap) in [e^(-2 cap), 1] needs no running maximum.
// The first RC 16-byte vectors per thread stay in registers between the
// two passes; the rest of a longer row is read again.
template <typename T>
struct Vec16;
template <>
struct Vec16<bf16> {
  using type = bf16x8;
  static constexpr int n = 8;
};
template <>
struct Vec16<float> {
  using type = f32x4;
  static constexpr int n = 4;
};

template <typename T, int RC>
__global__ __launch_bounds__(256) void ce_rows_kernel(T* __restrict__ logits,
                                                      const int32_t* __restrict__ tgt,
                                                      const float* __restrict__ scalars,
                                                      float* __restrict__ lossrow, int V, float cap,
                                                      int grad) {
  using VT = typename Vec16<T>::type;
  constexpr int VEC = Vec16<T>::n;
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t n = blockIdx.x;
  T* row = logits + n * V;
  const int nvec = V / VEC;
  const int y = tgt[n];
  const bool valid = (uint32_t)y < (uint32_t)V;  // ignored: -1, or off-precondition ids
  const float cy = valid ? static_cast<float>(row[y]) : 0.0f;  // read before the row is rewritten
  VT c[RC];
#pragma unroll
  for (int r = 0; r < RC; ++r) {
    const int v = tid + r * 256;
    if (v < nvec) c[r] = reinterpret_cast<const VT*>(row)[v];
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < RC; ++r) {
    const int v = tid + r * 256;
    if (v < nvec) {
#pragma unroll
      for (int j = 0; j < VEC; ++j) s += __expf(static_cast<float>(c[r][j]) - cap);
    }
  }
  for (int v = tid + RC * 256; v < nvec; v += 256) {
    const VT x = reinterpret_cast<const VT*>(row)[v];
#pragma unroll
    for (int j = 0; j < VEC; ++j) s += __expf(static_cast<float>(x[j]) - cap);
  }
  s = wave_sum(s);
  if (lane == 0) red[wv] = s;
  __syncthreads();
  s = (red[0] + red[1]) + (red[2] + red[3]);
  if (tid == 0) lossrow[n] = valid ? cap + logf(s) - cy : 0.0f;
  if (!grad) return;
  const float inv = valid ? 1.0f / s : 0.0f, inv_nv = scalars[0], icap = 1.0f / cap;
  auto gradv = [&](VT x, int v) {
    VT o;
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      const float cv = static_cast<float>(x[j]);
      float p = __expf(cv - cap) * inv;
      if (v * VEC + j == y) p -= 1.0f;
      const float q = cv * icap;
      o[j] = static_cast<T>(p * (1.0f - q * q) * inv_nv);
    }
    reinterpret_cast<VT*>(row)[v] = o;
  };
#pragma unroll
  for (int r = 0; r < RC; ++r) {
    const int v = tid + r * 256;
    if (v < nvec) gradv(c[r], v);
  }
  for (int v = tid + RC * 256; v < nvec; v += 256) gradv(reinterpret_cast<const VT*>(row)[v], v);
}

// Mean over valid tokens: fixed-order reduction in double.
__global__ __launch_bounds__(1024) void loss_kernel(const float* __restrict__ lossrow,
                                                    const float* __restrict__ scalars,
                                                    float* __restrict__ loss, int64_t N) {
  __shared__ double s_loss[1024];
  double acc = 0.0;
  for (int64_t n = threadIdx.x; n < N; n += 1024) acc += lossrow[n];
  s_loss[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if (threadIdx.x < s) s_loss[threadIdx.x] += s_loss[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = (float)(s_loss[0] * (double)scalars[0]);
}

}  // namespace gk

namespace gpt {
using namespace gk;

static unsigned blocks_for(int64_t n, int per) {
  int64_t b = (n + per - 1) / per;
  if (b > 65535 * 16) b = 65535 * 16;
  return (unsigned)(b < 1 ? 1 : b);
}

void launch_cast(const float* src, void* dst, const std::vector<CastSeg>& segs, hipStream_t s) {
  for (size_t base = 0; base < segs.size(); base += 128) {
    CastTable t{};
    t.nseg = (int)std::min<size_t>(128, segs.size() - base);
    int64_t mx = 0;
    for (int i = 0; i < t.nseg; ++i) {
      t.seg[i] = segs[base + i];
      mx = std::max(mx, t.seg[i].n);
    }
    dim3 grid(std::min<unsigned>(blocks_for(mx, 256 * 8), 1024), t.nseg);
    GK_LAUNCH(cast_kernel, grid, dim3(256), 0, s, src, static_cast<bf16*>(dst), t);
  }
}

void launch_cast_t(const float* src, void* dst, void* dstT, const std::vector<int64_t>& offs,
                   int rows, int cols, hipStream_t s) {
  for (size_t base = 0; base < offs.size(); base += 64) {
    CastTTable t{};
    const int n = (int)std::min<size_t>(64, offs.size() - base);
    for (int i = 0; i < n; ++i) t.off[i] = offs[base + i];
    t.rows = rows;
    t.cols = cols;
    dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64), (unsigned)n);
    GK_LAUNCH(cast_t_kernel, grid, dim3(256), 0, s, src, static_cast<bf16*>(dst),
                       static_cast<bf16*>(dstT), t);
  }
}

void launch_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  GK_LAUNCH(zero_kernel, dim3(std::min<unsigned>(blocks_for(n, 256 * 4), 8192)),
                     dim3(256), 0, s, p, n);
}

void launch_rope_table(float* cs, int T, int D, float theta, hipStream_t s) {
  const int64_t n = (int64_t)T * (D / 2);
  GK_LAUNCH(rope_table_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, s, cs, T, D,
                     (double)theta);
}

// ------------------------------------------------------------ debug checks
__global__ __launch_bounds__(1024) void check_ids_kernel(const int32_t* __restrict__ tok,
                                                         const int32_t* __restrict__ tgt,
                                                         int64_t N, int V, uint32_t* out) {
  __shared__ uint32_t s_bad[2][16];
  uint32_t bt = 0, by = 0;
  for (int64_t n = threadIdx.x; n < N; n += 1024) {
    bt += (uint32_t)tok[n] >= (uint32_t)V ? 1u : 0u;
    const int32_t y = tgt[n];
    by += (y < -1 || y >= V) ? 1u : 0u;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    bt += __shfl_xor(bt, o, 64);
    by += __shfl_xor(by, o, 64);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_bad[0][w] = bt;
    s_bad[1][w] = by;
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    uint32_t t = 0;
    for (int k = 0; k < 16; ++k) t += s_bad[threadIdx.x][k];
    out[threadIdx.x] = t;
  }
}

__global__ __launch_bounds__(256) void check_finite_kernel(const float* __restrict__ x, int64_t n,
                                                           uint32_t* flag) {
  uint32_t bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    bad |= (__float_as_uint(x[i]) & 0x7f800000u) == 0x7f800000u ? 1u : 0u;
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flag, 1u);
}

void launch_check_ids(const int32_t* tok, const int32_t* tgt, int64_t N, int V, uint32_t* out,
                      hipStream_t s) {
  GK_LAUNCH(check_ids_kernel, dim3(1), dim3(1024), 0, s, tok, tgt, N, V, out);
}

void launch_check_finite(const float* x, int64_t n, uint32_t* flag, hipStream_t s) {
  const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 8192);
  GK_LAUNCH(check_finite_kernel, dim3(blocks), dim3(256), 0, s, x, n, flag);
}

void launch_embed(const float* wte, const int32_t* tok, float* x0, int64_t N, int C, int V,
                  hipStream_t s) {
  GK_LAUNCH(embed_kernel, dim3((unsigned)N), dim3(256), 0, s, wte, tok, x0, N, C, V);
}

// LDS bytes a workgroup may allocate on the current device (looked up once
// per device; 64 KB if the query fails).
static int max_lds_per_block() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 65536;
  std::lock_guard<std::mutex> lk(mu);
  if (!cached[dev]) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        v < 65536)
      v = 65536;
    cached[dev] = v;
  }
  return cached[dev];
}

template <typename T, int NC>
static void mix_norm_nc(const Dims& d, const float* x, const float* x0, const float* lam_r,
                        const float* lam_0, float* xin_out, void* y, float* r, const float* wg,
                        float* a, hipStream_t s) {
  const int64_t rows4 = (d.N + 3) / 4;
  const size_t lds = (size_t)d.Hk * d.C * 4;
  if (wg && lds <= 65536) {  // fewer workgroups, each staging the gate weights once
    GK_LAUNCH((mix_norm_kernel<T, NC, true>), dim3((unsigned)std::min<int64_t>(rows4, 1024)),
              dim3(256), lds, s, x, x0, lam_r, lam_0, xin_out, static_cast<T*>(y), r, wg, a, d.N,
              d.C, d.Hk, d.eps);
    return;
  }
  if (wg && lds <= (size_t)max_lds_per_block()) {  // one 1024-thread workgroup per CU
    GK_LAUNCH((mix_norm_kernel<T, NC, true, 1024>),
              dim3((unsigned)std::min<int64_t>((d.N + 15) / 16, 256)), dim3(1024), lds, s, x, x0,
              lam_r, lam_0, xin_out, static_cast<T*>(y), r, wg, a, d.N, d.C, d.Hk, d.eps);
    return;
  }
  GK_LAUNCH((mix_norm_kernel<T, NC, false>), dim3((unsigned)rows4), dim3(256), 0, s, x, x0, lam_r,
            lam_0, xin_out, static_cast<T*>(y), r, wg, a, d.N, d.C, d.Hk, d.eps);
}

void launch_mix_norm(const Dims& d, const float* x, const float* x0, const float* lam_r,
                     const float* lam_0, float* xin_out, void* y, float* r, const float* wg,
                     float* a, hipStream_t s) {
#define MN_CALL(T, NC) mix_norm_nc<T, NC>(d, x, x0, lam_r, lam_0, xin_out, y, r, wg, a, s)
  const int nc = (d.C + 255) / 256;
  if (d.bf16) {
    switch (nc) {
      case 1: MN_CALL(bf16, 1); break;
      case 2: MN_CALL(bf16, 2); break;
      case 3: MN_CALL(bf16, 3); break;
      case 4: MN_CALL(bf16, 4); break;
      case 5: MN_CALL(bf16, 5); break;
      case 6: MN_CALL(bf16, 6); break;
      case 7: MN_CALL(bf16, 7); break;
      default: MN_CALL(bf16, 8); break;
    }
  } else {
    switch (nc) {
      case 1: MN_CALL(float, 1); break;
      case 2: MN_CALL(float, 2); break;
      case 3: MN_CALL(float, 3); break;
      case 4: MN_CALL(float, 4); break;
      case 5: MN_CALL(float, 5); break;
      case 6: MN_CALL(float, 6); break;
      case 7: MN_CALL(float, 7); break;
      default: MN_CALL(float, 8); break;
    }
  }
#undef MN_CALL
}

void launch_norm_bwd(const Dims& d, const NormBwdArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((d.N + 3) / 4));
  NormBwdArgs b = a;
  b.gxc_bf16 = d.bf16 ? 1 : 0;
#define NB_CALL(NC) GK_LAUNCH(norm_bwd_kernel<NC>, grid, dim3(256), 0, s, b, d.N, d.C, d.Hk)
  switch ((d.C + 255) / 256) {
    case 1: NB_CALL(1); break;
    case 2: NB_CALL(2); break;
    case 3: NB_CALL(3); break;
    case 4: NB_CALL(4); break;
    case 5: NB_CALL(5); break;
    case 6: NB_CALL(6); break;
    case 7: NB_CALL(7); break;
    default: NB_CALL(8); break;
  }
#undef NB_CALL
}

void launch_lambda_finalize(const Dims& d, const float* lam_part, int nblk, float* g_lr,
                            float* g_l0, hipStream_t s, int layers, float scale) {
  GK_LAUNCH(lambda_finalize_kernel, dim3((unsigned)layers), dim3(256), 0, s, lam_part,
                     nblk, (int64_t)nblk * 2, g_lr, g_l0, d.accumulate ? 1 : 0, scale);
}

void launch_smear_embed(const Dims& d, const float* wte, const int32_t* tok, const float* w,
                        float* x0, float* sig, hipStream_t s) {
  const dim3 grid((unsigned)((d.N + 3) / 4));
  const int nc = (d.C + 255) / 256;
#define SM_CALL(NC)                                                                             \
  GK_LAUNCH(smear_embed_kernel<NC>, grid, dim3(256), 0, s, wte, tok, w, x0, sig, d.N, \
                     d.T, d.C, d.V)
  if (nc <= 1) SM_CALL(1);
  else if (nc == 2) SM_CALL(2);
  else if (nc == 3) SM_CALL(3);
  else if (nc <= 4) SM_CALL(4);
  else if (nc <= 6) SM_CALL(6);
  else SM_CALL(8);
#undef SM_CALL
}

void launch_smear_bwd(const Dims& d, const float* g, const float* wte, const int32_t* tok,
                      const float* w, const float* sig, float* ge, float* part, float* gw,
                      hipStream_t s) {
  const int nblk = smear_blocks(d.N);
  const dim3 grid((unsigned)nblk);
  const int nc = (d.C + 255) / 256;
#define SB_CALL(NC)                                                                               \
  GK_LAUNCH(smear_bwd_kernel<NC>, grid, dim3(256), 0, s, g, wte, tok, w, sig, ge, part, \
                     d.N, d.T, d.C, d.V)
  if (nc <= 1) SB_CALL(1);
  else if (nc == 2) SB_CALL(2);
  else if (nc == 3) SB_CALL(3);
  else if (nc <= 4) SB_CALL(4);
  else if (nc <= 6) SB_CALL(6);
  else SB_CALL(8);
#undef SB_CALL
  GK_LAUNCH(veg_finalize_kernel, dim3((unsigned)((d.C + 63) / 64)), dim3(256), 0, s,
                     part, gw, d.C, nblk, d.accumulate ? 1 : 0);
}

int smear_blocks(int64_t N) { return (int)((N + kSmearRows - 1) / kSmearRows); }

void launch_backout_weights(const float* lam, float* out, hipStream_t s) {
  GK_LAUNCH(backout_weights_kernel, dim3(1), dim3(64), 0, s, lam, out);
}

int veg_splits(int64_t N) { return (int)std::max<int64_t>(256, (N + kVegPer - 1) / kVegPer); }

void launch_veg_wgrad(const Dims& d, const float* ga, const void* xn, float* part, int splits,
                      float* gwg, hipStream_t s) {
  const int64_t per = (d.N + splits - 1) / splits;  // <= kVegPer with splits = veg_splits(N)
#define GPT_VEG(TY, HK)                                                                            \
  GK_LAUNCH((veg_partial_kernel<TY, HK>), dim3((unsigned)splits), dim3(256), 0, s, ga,    \
                     static_cast<const TY*>(xn), part, d.N, d.C, d.Hk, per)
  if (d.bf16) {
    if (d.Hk <= 4) GPT_VEG(bf16, 4);
    else if (d.Hk <= 8) GPT_VEG(bf16, 8);
    else GPT_VEG(bf16, 16);
  } else {
    if (d.Hk <= 4) GPT_VEG(float, 4);
    else if (d.Hk <= 8) GPT_VEG(float, 8);
    else GPT_VEG(float, 16);
  }
#undef GPT_VEG
  const int n = d.C * d.Hk;
  GK_LAUNCH(veg_finalize_kernel, dim3((unsigned)((n + 63) / 64)), dim3(256), 0, s, part,
                     gwg, n, splits, d.accumulate ? 1 : 0);
}

static unsigned rope_blocks(const Dims& d, bool ve) {
  const int64_t tasks = d.N * (d.H + d.Hk + (ve ? d.Hk : 0));
  return (unsigned)((tasks + 256 / (d.D / 8) - 1) / (256 / (d.D / 8)));
}

void launch_rope_qk_ve_fwd(const Dims& d, void* qkv, float* rqk, const float* cs, const float* a,
                           const float* ve_table, const int32_t* tok, hipStream_t s) {
  const dim3 grid(rope_blocks(d, ve_table != nullptr));
#define GPT_ROPE_F(TY, DD)                                                                        \
  GK_LAUNCH((rope_fwd_kernel<TY, DD>), grid, dim3(256), 0, s, static_cast<TY*>(qkv), rqk, \
                     cs, a, ve_table, tok, d.N, d.T, d.H, d.Hk, d.Qkv, d.eps, d.V)
  if (d.bf16) {
    if (d.D == 128) GPT_ROPE_F(bf16, 128);
    else GPT_ROPE_F(bf16, 64);
  } else {
    if (d.D == 128) GPT_ROPE_F(float, 128);
    else GPT_ROPE_F(float, 64);
  }
#undef GPT_ROPE_F
}

void launch_rope_qk_ve_bwd(const Dims& d, void* gqkv, const void* qkv, const float* rqk,
                           const float* cs, const float* a, const float* ve_table,
                           float* gve_rows, float* ga, const int32_t* tok, hipStream_t s) {
  const dim3 grid(rope_blocks(d, ve_table != nullptr));
#define GPT_ROPE_B(TY, DD)                                                                          \
  GK_LAUNCH((rope_bwd_kernel<TY, DD>), grid, dim3(256), 0, s, static_cast<TY*>(gqkv),       \
                     static_cast<const TY*>(qkv), rqk, cs, a, ve_table, gve_rows, ga, tok, d.N,     \
                     d.T, d.H, d.Hk, d.Qkv, d.V)
  if (d.bf16) {
    if (d.D == 128) GPT_ROPE_B(bf16, 128);
    else GPT_ROPE_B(bf16, 64);
  } else {
    if (d.D == 128) GPT_ROPE_B(float, 128);
    else GPT_ROPE_B(float, 64);
  }
#undef GPT_ROPE_B
}

void launch_token_links(const int32_t* tok, int64_t N, int32_t* link, hipStream_t s) {
  GK_LAUNCH(token_links_kernel, dim3((unsigned)((N + kChunk - 1) / kChunk)), dim3(kChunk),
                     0, s, tok, N, link);
}

void launch_rows_to_table(const float* g, int W, const int32_t* tok, const int32_t* link,
                          int64_t N, float* tab, int V, hipStream_t s) {
  const unsigned chunks = (unsigned)((N + kChunk - 1) / kChunk);
  if (W % 128 == 0)
    GK_LAUNCH(rows_to_table_kernel<128>, dim3(chunks, (unsigned)(W / 128)), dim3(256), 0, s, g,
              W, tok, link, N, tab, V);
  else  // W is a multiple of 64
    GK_LAUNCH(rows_to_table_kernel<64>, dim3(chunks, (unsigned)(W / 64)), dim3(256), 0, s, g, W,
              tok, link, N, tab, V);
}

void launch_count_valid(const Dims& d, const int32_t* tgt, float* scalars, hipStream_t s) {
  GK_LAUNCH(count_valid_kernel, dim3(1), dim3(1024), 0, s, tgt, scalars, d.N, d.V);
}

void launch_loss(const Dims& d, void* logits, const int32_t* tgt, const float* scalars,
                 float* lossrow, float* loss, bool grad, hipStream_t s) {
  if (d.bf16)
    GK_LAUNCH((ce_rows_kernel<bf16, 16>), dim3((unsigned)d.N), dim3(256), 0, s,
                       static_cast<bf16*>(logits), tgt, scalars, lossrow, d.V, d.cap, grad ? 1 : 0);
  else
    GK_LAUNCH((ce_rows_kernel<float, 16>), dim3((unsigned)d.N), dim3(256), 0, s,
                       static_cast<float*>(logits), tgt, scalars, lossrow, d.V, d.cap, grad ? 1 : 0);
  GK_LAUNCH(loss_kernel, dim3(1), dim3(1024), 0, s, lossrow, scalars, loss, d.N);
}

}  // namespace gpt
