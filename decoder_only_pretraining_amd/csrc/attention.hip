// Causal GQA attention with a per-layer sliding window, forward and
// backward, on gfx950 MFMA.
//
// Layout: qkv is [N][(H + 2Hk) * D] (row n = b*T + t), q head h at column
// h*D, k head j at (H + j)*D, v head j at (H + Hk + j)*D. Key s is visible
// to query t iff s <= t and (full or t - s <= W).
//
// Forward (flash style): a workgroup owns 128 queries of one head (one
// wavefront per 32 queries) and walks the visible 64-key tiles, staged in
// LDS. Scores are formed transposed, S^T = K Q^T, so each lane owns one
// query column: the online-softmax statistics are per-lane scalars and the
// probabilities feed O^T += V^T P^T straight from the accumulator
// registers. Tiles wholly outside the window are never visited.
//
// Backward: delta = rowsum(dO * O); a key-major pass (one workgroup per 128
// keys of a KV head, looping over the query tiles that see them and over the
// query heads of its group) accumulates dK^T and dV^T in registers; a
// query-major pass recomputes S^T and dP^T and accumulates dQ^T. No atomics.
//
// Softmax works in base 2: the saved statistic is lse2 = log2(sum_s 2^(S*c))
// with c = log2(e) / sqrt(D), so P = 2^(S*c - lse2).
#include "device_common.h"
#include "internal.h"

namespace gk {

constexpr float kNegInf = -__builtin_huge_valf();

template <typename T, int ROWS, int D>
__device__ __forceinline__ void load_rows_lds(T (*lds)[D + 16 / sizeof(T)], const T* __restrict__ src,
                                              int64_t row0, int nvalid, int64_t ld, int tid) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int NV = ROWS * D / VEC / 256;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = tid + i * 256;
    const int r = v / (D / VEC), c = (v % (D / VEC)) * VEC;
    Frag<T> f;
    if (r < nvalid) {
      frag_load(f, src + (row0 + r) * ld + c);
    } else {
      frag_zero(f);
    }
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<bf16x8*>(&lds[r][c]) = f.v;
    } else {
      *reinterpret_cast<f32x4*>(&lds[r][c]) = f.lo;
    }
  }
}

// Per-lane query fragments for 32 query rows (B operand of K Q^T).
template <typename T, int D>
__device__ __forceinline__ void load_row_frags(Frag<T> (&f)[D / 16], const T* __restrict__ base,
                                               bool valid, int lane) {
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    if (valid)
      frag_load(f[kc], base + kc * 16 + (lane >> 5) * 8);
    else
      frag_zero(f[kc]);
  }
}

template <typename T>
__device__ __forceinline__ void store_col4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store_col4<bf16>(bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = static_cast<bf16>(a);
  v[1] = static_cast<bf16>(b);
  v[2] = static_cast<bf16>(c);
  v[3] = static_cast<bf16>(d);
  *reinterpret_cast<bf16x4*>(p) = v;
}
template <>
__device__ __forceinline__ void store_col4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// Fragment of an operand whose 32 rows run along the columns of an LDS tile
// T[row][col] and whose contraction slots run down the rows: lane l takes
// column col0 + l%32; slot jj (0..7) is row kbase + 8*(jj/4) + 4*(l/32) + jj%4
// (the slot order of the accumulator rows, so probabilities and score
// gradients feed MFMAs straight from the accumulators). bf16 uses two
// transposing LDS reads (ds_read_b64_tr_b16): in a 16-lane group, source lane
// 4q + a addresses T[k0 + q][m0 + 4a] and output lane i receives
// T[k0 .. k0+3][m0 + i].
template <int PITCH>
__device__ __forceinline__ void frag_down(Frag<bf16>& f, const bf16* lds, int kbase, int col0,
                                          int lane) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const int g16 = lane >> 4, L = lane & 15;
  const int k0 = kbase + (g16 >> 1) * 4 + (L >> 2);
  const int m = col0 + (g16 & 1) * 16 + (L & 3) * 4;
  const bf16* p = lds + k0 * PITCH + m;
  union {
    struct { v4i16 a, b; } s;
    bf16x8 v;
  } u;
  u.s.a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  u.s.b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 8 * PITCH));
  f.v = u.v;
}
template <int PITCH>
__device__ __forceinline__ void frag_down(Frag<float>& f, const float* lds, int kbase, int col0,
                                          int lane) {
#pragma unroll
  for (int jj = 0; jj < 8; ++jj)
    frag_set(f, jj, lds[(kbase + (jj >> 2) * 8 + (lane >> 5) * 4 + (jj & 3)) * PITCH + col0 +
                        (lane & 31)]);
}

// ------------------------------------------------------------ forward
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_fwd_kernel(const T* __restrict__ qkv, T* __restrict__ out,
                                                       float* __restrict__ lse2, int T_, int H,
                                                       int Hk, int W, int full, float c2) {
  constexpr int BQ = 128, BKV = 64, PAD = 16 / sizeof(T);
  __shared__ T Ks[BKV][D + PAD];
  __shared__ T Vs[BKV][D + PAD];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, hi = lane >> 5;
  const int qt = gridDim.x - 1 - blockIdx.x;  // longest rows first
  const int h = blockIdx.y, b = blockIdx.z;
  const int j = h / (H / Hk);
  const int Qkv = (H + 2 * Hk) * D;
  const int64_t rb = (int64_t)b * T_;
  const int t0 = qt * BQ, tw = t0 + wv * 32, t = tw + (lane & 31);

  Frag<T> qf[D / 16];
  load_row_frags<T, D>(qf, qkv + (rb + t) * Qkv + h * D, t < T_, lane);

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.0f;
  float m_i = kNegInf, l_i = 0.0f;

  const int lo = full ? 0 : max(0, t0 - W);
  const int hi_k = min(T_, t0 + BQ);
  const int w_lo = full ? 0 : max(0, tw - W), w_hi = min(T_, tw + 32);
  for (int s0 = (lo / BKV) * BKV; s0 < hi_k; s0 += BKV) {
    __syncthreads();
    load_rows_lds<T, BKV, D>(Ks, qkv + (H + j) * D, rb + s0, T_ - s0, Qkv, tid);
    load_rows_lds<T, BKV, D>(Vs, qkv + (H + Hk + j) * D, rb + s0, T_ - s0, Qkv, tid);
    __syncthreads();
    if (s0 >= w_hi || s0 + BKV <= w_lo) continue;
    f32x16 sacc[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[sb][e] = 0.0f;
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) {
        Frag<T> kf;
        frag_load(kf, &Ks[sb * 32 + (lane & 31)][kc * 16 + hi * 8]);
        mfma(sacc[sb], kf, qf[kc]);
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int s = s0 + sb * 32 + acc_row(e, lane);
        const bool vis = s <= t && (full || t - s <= W);
        const float v = vis ? sacc[sb][e] * c2 : kNegInf;
        sacc[sb][e] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_i, mx);
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = exp2f(m_i - m_use);
    float ps = 0.0f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2f(sacc[sb][e] - m_use);
        sacc[sb][e] = p;
        ps += p;
      }
    ps += __shfl_xor(ps, 32, 64);
    l_i = l_i * alpha + ps;
    m_i = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        Frag<T> pf;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) frag_set(pf, jj, sacc[sb][8 * c + jj]);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          Frag<T> vf;
          frag_down<D + PAD>(vf, &Vs[0][0], sb * 32 + 16 * c, db * 32, lane);
          mfma(o[db], vf, pf);
        }
      }
  }
  if (t < T_) {
    const float inv = 1.0f / l_i;
    T* op = out + (rb + t) * (H * D) + h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + g * 8 + hi * 4;
        store_col4<T>(op + d, o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                      o[db][4 * g + 3] * inv);
      }
    if (hi == 0) lse2[(rb + t) * H + h] = m_i + log2f(l_i);
  }
}

// ------------------------------------------------------------ delta
template <typename T>
__global__ __launch_bounds__(256) void attn_delta_kernel(const T* __restrict__ gO,
                                                         const T* __restrict__ O,
                                                         float* __restrict__ delta, int64_t NH,
                                                         int D) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (n, h) pair
  if (i >= NH) return;
  float s = 0.0f;
  for (int d = lane; d < D; d += 64) s += to_f(gO[i * D + d]) * to_f(O[i * D + d]);
  s = wave_sum(s);
  if (lane == 0) delta[i] = s;
}

// ------------------------------------------------------------ dK, dV
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_kv_kernel(
    const T* __restrict__ qkv, const T* __restrict__ gO, const float* __restrict__ lse2,
    const float* __restrict__ delta, T* __restrict__ gqkv, int T_, int H, int Hk, int W, int full,
    float c2, float scale) {
  constexpr int BK2 = 128, BQ2 = 64, PAD = 16 / sizeof(T);
  __shared__ T Qs[BQ2][D + PAD];
  __shared__ T dOs[BQ2][D + PAD];
  __shared__ float ls[BQ2], dl[BQ2];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, hi = lane >> 5;
  const int kt = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int G = H / Hk;
  const int Qkv = (H + 2 * Hk) * D, Cq = H * D;
  const int64_t rb = (int64_t)b * T_;
  const int s0 = kt * BK2, sw = s0 + wv * 32, s = sw + (lane & 31);

  Frag<T> kf[D / 16], vf[D / 16];
  load_row_frags<T, D>(kf, qkv + (rb + s) * Qkv + (H + j) * D, s < T_, lane);
  load_row_frags<T, D>(vf, qkv + (rb + s) * Qkv + (H + Hk + j) * D, s < T_, lane);

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dk[i][e] = 0.0f;
      dv[i][e] = 0.0f;
    }

  const int q_hi = full ? T_ : min(T_, s0 + BK2 + W);  // exclusive
  const int w_q_lo = sw, w_q_hi = full ? T_ : min(T_, sw + 32 + W);
  for (int hh = 0; hh < G; ++hh) {
    const int h = j * G + hh;
    for (int t0 = (s0 / BQ2) * BQ2; t0 < q_hi; t0 += BQ2) {
      __syncthreads();
      load_rows_lds<T, BQ2, D>(Qs, qkv + h * D, rb + t0, T_ - t0, Qkv, tid);
      load_rows_lds<T, BQ2, D>(dOs, gO + h * D, rb + t0, T_ - t0, Cq, tid);
      if (tid < BQ2) {
        const bool ok = t0 + tid < T_;
        ls[tid] = ok ? lse2[(rb + t0 + tid) * H + h] : 0.0f;
        dl[tid] = ok ? delta[(rb + t0 + tid) * H + h] : 0.0f;
      }
      __syncthreads();
      if (t0 >= w_q_hi || t0 + BQ2 <= w_q_lo) continue;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        f32x16 sa, dp;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          sa[e] = 0.0f;
          dp[e] = 0.0f;
        }
#pragma unroll
        for (int kc = 0; kc < D / 16; ++kc) {
          Frag<T> qa, da;
          frag_load(qa, &Qs[tb * 32 + (lane & 31)][kc * 16 + hi * 8]);
          frag_load(da, &dOs[tb * 32 + (lane & 31)][kc * 16 + hi * 8]);
          mfma(sa, qa, kf[kc]);
          mfma(dp, da, vf[kc]);
        }
        // rows t (local tb*32 + acc_row), column s
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int tl = tb * 32 + acc_row(e, lane);
          const int t = t0 + tl;
          const bool vis = t < T_ && s <= t && (full || t - s <= W);
          const float p = vis ? exp2f(sa[e] * c2 - ls[tl]) : 0.0f;
          sa[e] = p;
          dp[e] = p * (dp[e] - dl[tl]);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          Frag<T> pf, dsf;
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            frag_set(pf, jj, sa[8 * c + jj]);
            frag_set(dsf, jj, dp[8 * c + jj]);
          }
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            Frag<T> doT, qT;
            frag_down<D + PAD>(doT, &dOs[0][0], tb * 32 + 16 * c, db * 32, lane);
            frag_down<D + PAD>(qT, &Qs[0][0], tb * 32 + 16 * c, db * 32, lane);
            mfma(dv[db], doT, pf);
            mfma(dk[db], qT, dsf);
          }
        }
      }
    }
  }
  if (s < T_) {
    T* kp = gqkv + (rb + s) * Qkv + (H + j) * D;
    T* vp = gqkv + (rb + s) * Qkv + (H + Hk + j) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + g * 8 + hi * 4;
        store_col4<T>(kp + d, dk[db][4 * g] * scale, dk[db][4 * g + 1] * scale,
                      dk[db][4 * g + 2] * scale, dk[db][4 * g + 3] * scale);
        store_col4<T>(vp + d, dv[db][4 * g], dv[db][4 * g + 1], dv[db][4 * g + 2],
                      dv[db][4 * g + 3]);
      }
  }
}

// ------------------------------------------------------------ dQ
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_q_kernel(
    const T* __restrict__ qkv, const T* __restrict__ gO, const float* __restrict__ lse2,
    const float* __restrict__ delta, T* __restrict__ gqkv, int T_, int H, int Hk, int W, int full,
    float c2, float scale) {
  constexpr int BQ = 128, BKV = 64, PAD = 16 / sizeof(T);
  __shared__ T Ks[BKV][D + PAD];
  __shared__ T Vs[BKV][D + PAD];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, hi = lane >> 5;
  const int qt = gridDim.x - 1 - blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int j = h / (H / Hk);
  const int Qkv = (H + 2 * Hk) * D, Cq = H * D;
  const int64_t rb = (int64_t)b * T_;
  const int t0 = qt * BQ, tw = t0 + wv * 32, t = tw + (lane & 31);
  const bool tv = t < T_;

  Frag<T> qf[D / 16], df[D / 16];
  load_row_frags<T, D>(qf, qkv + (rb + t) * Qkv + h * D, tv, lane);
  load_row_frags<T, D>(df, gO + (rb + t) * Cq + h * D, tv, lane);
  const float lt = tv ? lse2[(rb + t) * H + h] : 0.0f;
  const float dt = tv ? delta[(rb + t) * H + h] : 0.0f;

  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[i][e] = 0.0f;

  const int lo = full ? 0 : max(0, t0 - W);
  const int hi_k = min(T_, t0 + BQ);
  const int w_lo = full ? 0 : max(0, tw - W), w_hi = min(T_, tw + 32);
  for (int s0 = (lo / BKV) * BKV; s0 < hi_k; s0 += BKV) {
    __syncthreads();
    load_rows_lds<T, BKV, D>(Ks, qkv + (H + j) * D, rb + s0, T_ - s0, Qkv, tid);
    load_rows_lds<T, BKV, D>(Vs, qkv + (H + Hk + j) * D, rb + s0, T_ - s0, Qkv, tid);
    __syncthreads();
    if (s0 >= w_hi || s0 + BKV <= w_lo) continue;
    f32x16 sa[2], dp[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sa[sb][e] = 0.0f;
        dp[sb][e] = 0.0f;
      }
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) {
        Frag<T> ka, va;
        frag_load(ka, &Ks[sb * 32 + (lane & 31)][kc * 16 + hi * 8]);
        frag_load(va, &Vs[sb * 32 + (lane & 31)][kc * 16 + hi * 8]);
        mfma(sa[sb], ka, qf[kc]);
        mfma(dp[sb], va, df[kc]);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int sidx = s0 + sb * 32 + acc_row(e, lane);
        const bool vis = tv && sidx <= t && (full || t - sidx <= W);
        const float p = vis ? exp2f(sa[sb][e] * c2 - lt) : 0.0f;
        dp[sb][e] = p * (dp[sb][e] - dt);
      }
    }
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        Frag<T> dsf;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) frag_set(dsf, jj, dp[sb][8 * c + jj]);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          Frag<T> kT;
          frag_down<D + PAD>(kT, &Ks[0][0], sb * 32 + 16 * c, db * 32, lane);
          mfma(dq[db], kT, dsf);
        }
      }
  }
  if (tv) {
    T* qp = gqkv + (rb + t) * Qkv + h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + g * 8 + hi * 4;
        store_col4<T>(qp + d, dq[db][4 * g] * scale, dq[db][4 * g + 1] * scale,
                      dq[db][4 * g + 2] * scale, dq[db][4 * g + 3] * scale);
      }
  }
}

template <typename T, int D>
void fwd(const gpt::Dims& d, bool full, const void* qkv, void* out, float* lse, hipStream_t s) {
  const float c2 = 1.4426950408889634f / sqrtf((float)D);
  dim3 grid((unsigned)((d.T + 127) / 128), d.H, d.B);
  hipLaunchKernelGGL((attn_fwd_kernel<T, D>), grid, dim3(256), 0, s, static_cast<const T*>(qkv),
                     static_cast<T*>(out), lse, d.T, d.H, d.Hk, d.W, full ? 1 : 0, c2);
}

template <typename T, int D>
void bwd(const gpt::Dims& d, bool full, const void* qkv, const void* gO, const float* lse,
         const float* delta, void* gqkv, hipStream_t s) {
  const float c2 = 1.4426950408889634f / sqrtf((float)D);
  const float scale = 1.0f / sqrtf((float)D);
  dim3 gkv((unsigned)((d.T + 127) / 128), d.Hk, d.B);
  hipLaunchKernelGGL((attn_bwd_kv_kernel<T, D>), gkv, dim3(256), 0, s, static_cast<const T*>(qkv),
                     static_cast<const T*>(gO), lse, delta, static_cast<T*>(gqkv), d.T, d.H, d.Hk,
                     d.W, full ? 1 : 0, c2, scale);
  dim3 gq((unsigned)((d.T + 127) / 128), d.H, d.B);
  hipLaunchKernelGGL((attn_bwd_q_kernel<T, D>), gq, dim3(256), 0, s, static_cast<const T*>(qkv),
                     static_cast<const T*>(gO), lse, delta, static_cast<T*>(gqkv), d.T, d.H, d.Hk,
                     d.W, full ? 1 : 0, c2, scale);
}

}  // namespace gk

namespace gpt {
using namespace gk;

void launch_attn_fwd(const Dims& d, bool full, const void* qkv, void* out, float* lse,
                     hipStream_t s) {
  if (d.bf16) {
    if (d.D == 128) fwd<bf16, 128>(d, full, qkv, out, lse, s);
    else fwd<bf16, 64>(d, full, qkv, out, lse, s);
  } else {
    if (d.D == 128) fwd<float, 128>(d, full, qkv, out, lse, s);
    else fwd<float, 64>(d, full, qkv, out, lse, s);
  }
}

void launch_attn_delta(const Dims& d, const void* gO, const void* O, float* delta, hipStream_t s) {
  const int64_t NH = d.N * d.H;
  dim3 grid((unsigned)((NH + 3) / 4));
  if (d.bf16)
    hipLaunchKernelGGL(attn_delta_kernel<bf16>, grid, dim3(256), 0, s, static_cast<const bf16*>(gO),
                       static_cast<const bf16*>(O), delta, NH, d.D);
  else
    hipLaunchKernelGGL(attn_delta_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(gO), static_cast<const float*>(O), delta, NH, d.D);
}

void launch_attn_bwd(const Dims& d, bool full, const void* qkv, const void* gO, const float* lse,
                     const float* delta, void* gqkv, hipStream_t s) {
  if (d.bf16) {
    if (d.D == 128) bwd<bf16, 128>(d, full, qkv, gO, lse, delta, gqkv, s);
    else bwd<bf16, 64>(d, full, qkv, gO, lse, delta, gqkv, s);
  } else {
    if (d.D == 128) bwd<float, 128>(d, full, qkv, gO, lse, delta, gqkv, s);
    else bwd<float, 64>(d, full, qkv, gO, lse, delta, gqkv, s);
  }
}

}  // namespace gpt
