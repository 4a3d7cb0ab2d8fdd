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
// with c = log2(e) / sqrt(D), so P = 2^(S*c - lse2). lse2 and delta are
// stored [batch][head][token], so a run of queries of one head is
// contiguous.
//
// All three kernels stream their tiles through two LDS buffers: the global
// loads of the next tile are in flight while the current tile's MFMAs run.
// Blocks of the score matrix that lie wholly inside the causal window skip
// the per-element mask.
#include "device_common.h"
#include "gemm_core.h"

#include <type_traits>
#include "internal.h"

namespace gk {

constexpr float kNegInf = -__builtin_huge_valf();

// 2^x with the hardware instruction (v_exp_f32, about 1 ulp; 2^-inf = 0).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

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

// A ROWS x D tile of head rows on its way from global memory (rows
// row0 .. row0 + ROWS - 1 of a matrix with row stride ld, rows past nvalid
// read as zero) to an LDS buffer with row pitch PITCH, held in registers in
// between so the global loads of the next tile overlap the current tile's
// MFMAs.
struct alignas(16) V16 {
  uint32_t w[4];
};
template <typename T, int ROWS, int D>
struct RowStage {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int NV = ROWS * D / VEC / 256;
  V16 v[NV];
  __device__ __forceinline__ void load(const T* __restrict__ src, int64_t row0, int nvalid,
                                       int64_t ld, int tid) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = tid + i * 256;
      const int r = idx / (D / VEC), c = (idx % (D / VEC)) * VEC;
      if (r < nvalid)
        v[i] = *reinterpret_cast<const V16*>(src + (row0 + r) * ld + c);
      else
        v[i] = V16{{0, 0, 0, 0}};
    }
  }
  template <int PITCH>
  __device__ __forceinline__ void store(T* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = tid + i * 256;
      const int r = idx / (D / VEC), c = (idx % (D / VEC)) * VEC;
      *reinterpret_cast<V16*>(lds + r * PITCH + c) = v[i];
    }
  }
};

// ------------------------------------------------------------ forward
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_fwd_kernel(const T* __restrict__ qkv, T* __restrict__ out,
                                                       float* __restrict__ lse2, int T_, int H,
                                                       int Hk, int W, int full, float c2) {
  constexpr int BQ = 128, BKV = 64, PAD = 16 / sizeof(T), P = D + PAD;
  __shared__ __attribute__((aligned(16))) T Ks[2][BKV * P];
  __shared__ __attribute__((aligned(16))) T Vs[2][BKV * P];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, hi = lane >> 5;
  const int qt = gridDim.x - 1 - blockIdx.x;  // longest rows first
  const int h = blockIdx.y, b = blockIdx.z;
  const int j = h / (H / Hk);
  const int Qkv = (H + 2 * Hk) * D;
  const int64_t rb = (int64_t)b * T_;
  const int t0 = qt * BQ, tw = t0 + wv * 32, t = tw + (lane & 31);
  const T* kbase = qkv + (H + j) * D;
  const T* vbase = qkv + (H + Hk + j) * D;

  Frag<T> qf[D / 16];
  load_row_frags<T, D>(qf, qkv + (rb + t) * Qkv + h * D, t < T_, lane);

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.0f;
  float m_i = kNegInf, l_i = 0.0f;

  const int first = ((full ? 0 : max(0, t0 - W)) / BKV) * BKV;
  const int hi_k = min(T_, t0 + BQ);
  const int ntile = (hi_k - first + BKV - 1) / BKV;
  const int w_lo = full ? 0 : max(0, tw - W), w_hi = min(T_, tw + 32);
  RowStage<T, BKV, D> kst, vst;
  kst.load(kbase, rb + first, T_ - first, Qkv, tid);
  vst.load(vbase, rb + first, T_ - first, Qkv, tid);
  kst.template store<P>(Ks[0], tid);
  vst.template store<P>(Vs[0], tid);
  __syncthreads();
  for (int it = 0; it < ntile; ++it) {
    const int s0 = first + it * BKV, cur = it & 1;
    const bool more = it + 1 < ntile;
    if (more) {
      kst.load(kbase, rb + s0 + BKV, T_ - s0 - BKV, Qkv, tid);
      vst.load(vbase, rb + s0 + BKV, T_ - s0 - BKV, Qkv, tid);
    }
    if (s0 < w_hi && s0 + BKV > w_lo) {
      // every key of the tile visible to every query of the wavefront
      const bool interior = (s0 + BKV - 1 <= tw) && (full || tw + 31 - s0 <= W);
      f32x16 sacc[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[sb][e] = 0.0f;
#pragma unroll
        for (int kc = 0; kc < D / 16; ++kc) {
          Frag<T> kf;
          frag_load(kf, &Ks[cur][(sb * 32 + (lane & 31)) * P + kc * 16 + hi * 8]);
          mfma(sacc[sb], kf, qf[kc]);
        }
      }
      float mx = kNegInf;
      if (interior) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            sacc[sb][e] *= c2;
            mx = fmaxf(mx, sacc[sb][e]);
          }
      } else {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int sidx = s0 + sb * 32 + acc_row(e, lane);
            const bool vis = sidx <= t && (full || t - sidx <= W);
            const float v = vis ? sacc[sb][e] * c2 : kNegInf;
            sacc[sb][e] = v;
            mx = fmaxf(mx, v);
          }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_i, mx);
      const float m_use = m_new == kNegInf ? 0.0f : m_new;
      const float alpha = exp2_fast(m_i - m_use);
      float ps = 0.0f;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = exp2_fast(sacc[sb][e] - m_use);
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
            frag_down<P>(vf, Vs[cur], sb * 32 + 16 * c, db * 32, lane);
            mfma(o[db], vf, pf);
          }
        }
    }
    if (more) {
      kst.template store<P>(Ks[cur ^ 1], tid);
      vst.template store<P>(Vs[cur ^ 1], tid);
    }
    __syncthreads();
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
    if (hi == 0) lse2[((int64_t)b * H + h) * T_ + t] = m_i + log2f(l_i);
  }
}

// ------------------------------------------------------------ forward, bf16
// A workgroup of 8 wavefronts owns 256 queries of one head, 32 per
// wavefront; two wavefronts share each SIMD so one's softmax arithmetic
// overlaps the other's MFMAs. K/V tiles of 64 keys stream into three LDS
// stages with direct global->LDS loads issued two tiles ahead by wavefronts
// 0-3. K is kept as a swizzled K-major tile [key][d]; V as [key][d + 32]
// for transposing fragment reads. The exponentials need no running max:
// q and k leave the QK-norm with RMS below 1, so |q.k| < D and every logit
// (base 2: c2 * q.k) lies within about +-m_fix = c2 * D * (1 + 2^-7), the
// margin covering the bf16 rounding of q and k. p = 2^(logit - m_fix) then
// lies in [2^(-2 m_fix), 1] up to that rounding (2^-33 for D = 128), far
// inside the normal range of fp32 and bf16, and the log2-sum-exp is
// m_fix + log2(sum p). Only tiles on the causal diagonal or
// the window edge compute a mask. The linear block id runs over (query
// tile, head, batch), latest (costliest) tiles first.
//
// BQ = 128, S = 2 (the sliding-window layers): 4 wavefronts, all of them
// loading, and two stages (72 KB of LDS), so two workgroups share a CU. A
// window layer's query tiles all cost about the same, and 256-query tiles
// (B H T / 256 of them, e.g. 384 at seq 2048, batch 8, 6 heads) would fill
// 1.5 rounds of the CUs; 128-query tiles fill 1.5 rounds of the 512 slots
// with half the work each.
template <int D, bool ALIGNED, int BQ = 256, int S = 3>
__global__ __launch_bounds__(2 * BQ) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_tiled_kernel(const bf16* __restrict__ qkv, bf16* __restrict__ out,
                           float* __restrict__ lse2, int T_, int H, int Hk, int W, int full,
                           float c2, int nq, int nb) {
  constexpr int BKV = 64;
  static_assert((BQ == 256 && S == 3) || (BQ == 128 && S == 2), "tile forms");
  using GK = TileGeom<BKV, D, true>;    // K tile: rows = keys, contraction = d
  using GV = TileGeom<D, BKV, false>;   // V tile: [key][d + 32]
  using LK = DirectLoader<BKV, D, true>;
  using LV = DirectLoader<D, BKV, false>;
  static_assert(LK::CHUNKS % 4 == 0 && LV::CHUNKS % 4 == 0, "whole chunks per loading wavefront");
  constexpr int PER_WAVE = LK::CHUNKS / 4 + LV::CHUNKS / 4;  // loads per loading wavefront per tile
  static_assert(PER_WAVE < 16, "vmcnt field");
  __shared__ __attribute__((aligned(16))) bf16 Ks[S][GK::ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 Vs[S][GV::ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, hi = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS fill addresses in SGPRs
  const bool loader = wv < 4;
  const int L = blockIdx.x;
  const int qt = nq - 1 - L / (H * nb);
  const int h = (L % (H * nb)) % H, b = (L % (H * nb)) / H;
  const int j = h / (H / Hk);
  const int Qkv = (H + 2 * Hk) * D;
  const int64_t rb = (int64_t)b * T_;
  const int t0 = qt * BQ, tw = t0 + wv * 32, t = tw + (lane & 31);
  const bf16* kbase = qkv + (H + j) * D;
  const bf16* vbase = qkv + (H + Hk + j) * D;

  Frag<bf16> qf[D / 16];
  load_row_frags<bf16, D>(qf, qkv + (rb + t) * Qkv + h * D, t < T_, lane);
  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.0f;
  const float m_fix = c2 * (float)D * (1.0f + 1.0f / 128.0f);
  float l_i = 0.0f;

  const int first = ((full ? 0 : max(0, t0 - W)) / BKV) * BKV;
  const int ntile = (min(T_, t0 + BQ) - first + BKV - 1) / BKV;
  const int w_lo = full ? 0 : max(0, tw - W), w_hi = min(T_, tw + 32);
  const unsigned wmax = full ? 0x7fffffffu : (unsigned)W;
  // ALIGNED (T a multiple of the key tile): every tile lies inside the
  // sequence and streams through precomputed offsets; otherwise the last
  // tile zero-fills its tail, so all go through the general path
  LK lk;
  LV lv;
  if (ALIGNED && loader) {
    lk.init(Qkv, 0, 1 << 30, wv, lane);
    lv.init(Qkv, 0, D, wv, lane);
  }
  auto issue = [&](int it) {
    if (!loader) return;
    const int64_t r0 = rb + first + (int64_t)it * BKV;
    if constexpr (ALIGNED) {
      lk.issue_fast(kbase + r0 * Qkv, Ks[it % S], wv);
      lv.issue_fast(vbase + r0 * Qkv, Vs[it % S], wv);
    } else {
      LK::issue(kbase, Qkv, r0, rb + T_, 0, D, Ks[it % S], wv, lane);
      LV::issue(vbase, Qkv, 0, D, r0, rb + T_, Vs[it % S], wv, lane);
    }
  };
#pragma unroll
  for (int it = 0; it < S - 1; ++it)
    if (it < ntile) issue(it);
  if (S == 3 && ntile > 1 && loader) __builtin_amdgcn_s_waitcnt(0x0f70 | PER_WAVE);  // tile 0 landed
  else __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  // One tile; the stage buffer CUR is a compile-time index so every LDS
  // address is a per-lane base plus an immediate offset.
  auto tile = [&](int it, auto cur_c) {
    constexpr int CUR = decltype(cur_c)::value;
    const int s0 = first + it * BKV;
    if (it + S - 1 < ntile) issue(it + S - 1);
    if (tw < T_ && s0 < w_hi && s0 + BKV > w_lo) {
      f32x16 sacc[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[sb][e] = 0.0f;
        Frag<bf16> kf[2];
        read_frag<BKV, D, true>(kf[0], Ks[CUR], sb * 32, 0, lane);
#pragma unroll
        for (int kc = 0; kc < D / 16; ++kc) {
          if (kc + 1 < D / 16) read_frag<BKV, D, true>(kf[(kc + 1) & 1], Ks[CUR], sb * 32, kc + 1, lane);
          mfma(sacc[sb], kf[kc & 1], qf[kc]);
        }
      }
      // all 64 keys visible to all 32 queries of the wavefront?
      const bool interior = (s0 + BKV - 1 <= tw) && (full || tw + 31 - s0 <= W);
      if (!interior) {
        asm volatile("" ::: "memory");  // keep the mask on its own branch
        // key s0 + sb*32 + r is visible iff 0 <= t - key <= W (unsigned compare)
        const int u = t - s0 - 4 * hi;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int r = sb * 32 + (e >> 2) * 8 + (e & 3);
            if ((unsigned)(u - r) > wmax) sacc[sb][e] = kNegInf;
          }
      }
      float ps0 = 0.0f, ps1 = 0.0f;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const float p0 = exp2_fast(fmaf(sacc[sb][e], c2, -m_fix));
          const float p1 = exp2_fast(fmaf(sacc[sb][e + 1], c2, -m_fix));
          sacc[sb][e] = p0;
          sacc[sb][e + 1] = p1;
          ps0 += p0;
          ps1 += p1;
        }
      float ps = ps0 + ps1;
      ps += __shfl_xor(ps, 32, 64);
      l_i += ps;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          Frag<bf16> pf;
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) frag_set(pf, jj, sacc[sb][8 * c + jj]);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            Frag<bf16> vf;
            frag_down<GV::PITCH>(vf, Vs[CUR], sb * 32 + 16 * c, db * 32, lane);
            mfma(o[db], vf, pf);
          }
        }
    }
    // tile it + 1 landed (with three stages tile it + 2 may still be in flight)
    if (S == 3 && it + S - 1 < ntile && loader) __builtin_amdgcn_s_waitcnt(0x0f70 | PER_WAVE);
    else __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
  };
  // the tile loop is unrolled by the stage count
  for (int it = 0; it < ntile; it += S) {
    tile(it, std::integral_constant<int, 0>{});
    if (it + 1 < ntile) tile(it + 1, std::integral_constant<int, 1>{});
    if constexpr (S == 3)
      if (it + 2 < ntile) tile(it + 2, std::integral_constant<int, 2>{});
  }
  if (t < T_) {
    const float inv = 1.0f / l_i;
    bf16* op = out + (rb + t) * (H * D) + h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + g * 8 + hi * 4;
        store_col4<bf16>(op + d, o[db][4 * g] * inv, o[db][4 * g + 1] * inv,
                         o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
      }
    if (hi == 0) lse2[((int64_t)b * H + h) * T_ + t] = m_fix + log2f(l_i);
  }
}

// ------------------------------------------------------------ delta
// delta = rowsum(dO * O) per (batch, head, token), stored in that order
// (token fastest). A row belongs to LP = D/8 lanes, 8 elements each.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_delta_kernel(const T* __restrict__ gO,
                                                         const T* __restrict__ O,
                                                         float* __restrict__ delta, int64_t NH,
                                                         int H, int T_) {
  constexpr int LP = D / 8;
  const int q = threadIdx.x % LP;
  const int64_t i = (int64_t)blockIdx.x * (256 / LP) + threadIdx.x / LP;
  if (i >= NH) return;
  const int64_t bh = i / T_, t = i % T_;
  const int64_t row = ((bh / H) * T_ + t) * H + bh % H;  // (n, h) row of gO and O
  const T* g = gO + row * D + 8 * q;
  const T* o = O + row * D + 8 * q;
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s += to_f(g[e]) * to_f(o[e]);
#pragma unroll
  for (int w = LP / 2; w > 0; w >>= 1) s += __shfl_xor(s, w, kWave);
  if (q == 0) delta[i] = s;
}

// ------------------------------------------------------------ dK, dV
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_kv_kernel(
    const T* __restrict__ qkv, const T* __restrict__ gO, const float* __restrict__ lse2,
    const float* __restrict__ delta, T* __restrict__ gqkv, int T_, int H, int Hk, int W, int full,
    float c2, float scale) {
  constexpr int BK2 = 128, BQ2 = 64, PAD = 16 / sizeof(T), P = D + PAD;
  __shared__ __attribute__((aligned(16))) T Qs[2][BQ2 * P];
  __shared__ __attribute__((aligned(16))) T dOs[2][BQ2 * P];
  __shared__ __attribute__((aligned(16))) float ls[2][BQ2], dl[2][BQ2];
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

  // (head, query tile) steps of this key tile, walked with a one-step prefetch
  const int q_first = (s0 / BQ2) * BQ2;
  const int q_hi = full ? T_ : min(T_, s0 + BK2 + W);  // exclusive
  const int nq = (q_hi - q_first + BQ2 - 1) / BQ2;
  const int nstep = G * nq;
  RowStage<T, BQ2, D> qst, dst;
  float st_l = 0.0f, st_d = 0.0f;
  auto fetch = [&](int step) {
    const int h = j * G + step / nq, t0 = q_first + (step % nq) * BQ2;
    qst.load(qkv + h * D, rb + t0, T_ - t0, Qkv, tid);
    dst.load(gO + h * D, rb + t0, T_ - t0, Cq, tid);
    if (tid < BQ2) {
      const bool ok = t0 + tid < T_;
      st_l = ok ? lse2[((int64_t)b * H + h) * T_ + t0 + tid] : 0.0f;
      st_d = ok ? delta[((int64_t)b * H + h) * T_ + t0 + tid] : 0.0f;
    }
  };
  auto put = [&](int buf) {
    qst.template store<P>(Qs[buf], tid);
    dst.template store<P>(dOs[buf], tid);
    if (tid < BQ2) {
      ls[buf][tid] = st_l;
      dl[buf][tid] = st_d;
    }
  };
  if (nstep > 0) {
    fetch(0);
    put(0);
  }
  __syncthreads();
  for (int step = 0; step < nstep; ++step) {
    const int cur = step & 1;
    const bool more = step + 1 < nstep;
    const int t0 = q_first + (step % nq) * BQ2;
    if (more) fetch(step + 1);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int tlo = t0 + tb * 32;
      // any (query, key) pair of this 32x32 block visible?
      if (!(tlo < T_ && tlo + 31 >= sw && (full || tlo - (sw + 31) <= W))) continue;
      const bool interior = tlo >= sw + 31 && (full || tlo + 31 - sw <= W) && tlo + 31 < T_;
      f32x16 sa, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sa[e] = 0.0f;
        dp[e] = 0.0f;
      }
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) {
        Frag<T> qa, da;
        frag_load(qa, &Qs[cur][(tb * 32 + (lane & 31)) * P + kc * 16 + hi * 8]);
        frag_load(da, &dOs[cur][(tb * 32 + (lane & 31)) * P + kc * 16 + hi * 8]);
        mfma(sa, qa, kf[kc]);
        mfma(dp, da, vf[kc]);
      }
      // accumulator rows t = tlo + 8*(e/4) + 4*hi + e%4: four consecutive
      // rows per group g = e/4, so their statistics load as one vector
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int tl = tb * 32 + g * 8 + hi * 4;
        const f32x4 lv = *reinterpret_cast<const f32x4*>(&ls[cur][tl]);
        const f32x4 dv4 = *reinterpret_cast<const f32x4*>(&dl[cur][tl]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 4 * g + r;
          bool vis = true;
          if (!interior) {
            const int tq = t0 + tl + r;
            vis = tq < T_ && s <= tq && (full || tq - s <= W);
          }
          const float p = vis ? exp2_fast(sa[e] * c2 - lv[r]) : 0.0f;
          sa[e] = p;
          dp[e] = p * (dp[e] - dv4[r]);
        }
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
          frag_down<P>(doT, dOs[cur], tb * 32 + 16 * c, db * 32, lane);
          frag_down<P>(qT, Qs[cur], tb * 32 + 16 * c, db * 32, lane);
          mfma(dv[db], doT, pf);
          mfma(dk[db], qT, dsf);
        }
      }
    }
    if (more) put(cur ^ 1);
    __syncthreads();
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
  constexpr int BQ = 128, BKV = 64, PAD = 16 / sizeof(T), P = D + PAD;
  __shared__ __attribute__((aligned(16))) T Ks[2][BKV * P];
  __shared__ __attribute__((aligned(16))) T Vs[2][BKV * P];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, hi = lane >> 5;
  const int qt = gridDim.x - 1 - blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int j = h / (H / Hk);
  const int Qkv = (H + 2 * Hk) * D, Cq = H * D;
  const int64_t rb = (int64_t)b * T_;
  const int t0 = qt * BQ, tw = t0 + wv * 32, t = tw + (lane & 31);
  const bool tv = t < T_;
  const T* kbase = qkv + (H + j) * D;
  const T* vbase = qkv + (H + Hk + j) * D;

  Frag<T> qf[D / 16], df[D / 16];
  load_row_frags<T, D>(qf, qkv + (rb + t) * Qkv + h * D, tv, lane);
  load_row_frags<T, D>(df, gO + (rb + t) * Cq + h * D, tv, lane);
  const float lt = tv ? lse2[((int64_t)b * H + h) * T_ + t] : 0.0f;
  const float dt = tv ? delta[((int64_t)b * H + h) * T_ + t] : 0.0f;

  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[i][e] = 0.0f;

  const int first = ((full ? 0 : max(0, t0 - W)) / BKV) * BKV;
  const int hi_k = min(T_, t0 + BQ);
  const int ntile = (hi_k - first + BKV - 1) / BKV;
  const int w_lo = full ? 0 : max(0, tw - W), w_hi = min(T_, tw + 32);
  RowStage<T, BKV, D> kst, vst;
  kst.load(kbase, rb + first, T_ - first, Qkv, tid);
  vst.load(vbase, rb + first, T_ - first, Qkv, tid);
  kst.template store<P>(Ks[0], tid);
  vst.template store<P>(Vs[0], tid);
  __syncthreads();
  for (int it = 0; it < ntile; ++it) {
    const int s0 = first + it * BKV, cur = it & 1;
    const bool more = it + 1 < ntile;
    if (more) {
      kst.load(kbase, rb + s0 + BKV, T_ - s0 - BKV, Qkv, tid);
      vst.load(vbase, rb + s0 + BKV, T_ - s0 - BKV, Qkv, tid);
    }
    if (s0 < w_hi && s0 + BKV > w_lo) {
      const bool interior = (s0 + BKV - 1 <= tw) && (full || tw + 31 - s0 <= W);
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
          frag_load(ka, &Ks[cur][(sb * 32 + (lane & 31)) * P + kc * 16 + hi * 8]);
          frag_load(va, &Vs[cur][(sb * 32 + (lane & 31)) * P + kc * 16 + hi * 8]);
          mfma(sa[sb], ka, qf[kc]);
          mfma(dp[sb], va, df[kc]);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          bool vis = tv;
          if (!interior) {
            const int sidx = s0 + sb * 32 + acc_row(e, lane);
            vis = tv && sidx <= t && (full || t - sidx <= W);
          }
          const float p = vis ? exp2_fast(sa[sb][e] * c2 - lt) : 0.0f;
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
            frag_down<P>(kT, Ks[cur], sb * 32 + 16 * c, db * 32, lane);
            mfma(dq[db], kT, dsf);
          }
        }
    }
    if (more) {
      kst.template store<P>(Ks[cur ^ 1], tid);
      vst.template store<P>(Vs[cur ^ 1], tid);
    }
    __syncthreads();
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

// ------------------------------------------------------------ backward, bf16
// Tiles read both by rows (8 consecutive columns of one row, 16 bytes per
// lane) and transposed (4 consecutive rows of one column, ds_read_b64_tr_b16)
// are kept with row pitch D + 32 and the 16-byte granules of row t XOR-
// permuted by (t >> 2) & 3. For a 16-lane row read (16 rows, one granule)
// the pitch spreads rows over four bank offsets and the permutation over
// the other four; for a 32-lane transposing read (4 rows, 4 granules of an
// aligned group) the rows fall 8 bank pairs apart and the permutation stays
// inside the group: neither pattern conflicts.
template <int ROWS, int D>
struct Dual {
  static constexpr int PITCH = D + 32;
  static constexpr int ELEMS = ROWS * PITCH;
  static constexpr int CHUNKS = ELEMS * 2 / 1024;
  static_assert(ELEMS * 2 % 1024 == 0 && CHUNKS % 4 == 0, "whole chunks per loading wavefront");
  __device__ __forceinline__ static int off(int t, int col) {
    return t * PITCH + ((((col >> 3) ^ ((t >> 2) & 3)) << 3) | (col & 7));
  }
  // Direct global->LDS fill by wavefronts 0-3: rows row0 .. row0 + ROWS - 1
  // of a matrix with row stride ld (rows at or past rows_end read as zero).
  __device__ __forceinline__ static void issue(const bf16* __restrict__ p, int64_t ld,
                                               int64_t row0, int64_t rows_end, bf16* lds,
                                               int wave, int lane) {
#pragma unroll
    for (int c = wave; c < CHUNKS; c += 4) {
      const int o = c * 1024 + lane * 16;
      const int t = o / (PITCH * 2), pg = (o % (PITCH * 2)) / 16;
      const int gi = pg ^ ((t >> 2) & 3);
      const bool ok = row0 + t < rows_end;
      const bf16* src = ok ? p + (row0 + t) * ld + gi * 8
                           : reinterpret_cast<const bf16*>(g_zero_page) + (lane & 15) * 8;
      if (gi < D / 8) lds_fill16(src, lds_addr(lds) + c * 1024);
    }
  }
  // Streaming form for tiles wholly inside the matrix: this lane's byte
  // offset from the tile's first element for each of its chunks (~0u for a
  // slot in the row padding), computed once; a fill is then one load per
  // chunk from a wavefront-uniform base.
  static constexpr int NJ = CHUNKS / 4;
  struct Offs {
    uint32_t o[NJ];
  };
  __device__ __forceinline__ static Offs offsets(int64_t ld, int wave, int lane) {
    Offs f;
#pragma unroll
    for (int q = 0; q < NJ; ++q) {
      const int o = (wave + 4 * q) * 1024 + lane * 16;
      const int t = o / (PITCH * 2), pg = (o % (PITCH * 2)) / 16;
      const int gi = pg ^ ((t >> 2) & 3);
      f.o[q] = gi < D / 8 ? (uint32_t)((t * ld + gi * 8) * 2) : ~0u;
    }
    return f;
  }
  __device__ __forceinline__ static void issue_fast(const bf16* tile, const Offs& f, bf16* lds,
                                                    int wave) {
#pragma unroll
    for (int q = 0; q < NJ; ++q)
      if (f.o[q] != ~0u) lds_fill16(tile, f.o[q], lds_addr(lds) + (wave + 4 * q) * 1024);
  }
  // Lane offsets (elements) of the two read patterns. For rows row0 a
  // multiple of 16 the permutation (t >> 2) & 3 depends on the lane alone,
  // and it changes only the low two bits of a granule index, so a read's
  // address is one of two lane offsets plus a constant: row fragments use
  // r[kc & 1] + 32 (kc / 2) + row0 PITCH, transposed fragments (kbase a
  // multiple of 16, col0 of 32) tr[0 or 1] + kbase PITCH + col0.
  struct Lane {
    int r[2], tr[2];
  };
  __device__ __forceinline__ static Lane lane_offsets(int lane) {
    Lane q;
    q.r[0] = off(lane & 31, (lane >> 5) * 8);
    q.r[1] = off(lane & 31, 16 + (lane >> 5) * 8);
    const int g16 = lane >> 4, L = lane & 15;
    const int k0 = (g16 >> 1) * 4 + (L >> 2), m = (g16 & 1) * 16 + (L & 3) * 4;
    q.tr[0] = off(k0, m);
    q.tr[1] = off(k0 + 8, m);
    return q;
  }
  __device__ __forceinline__ static void row_frag(Frag<bf16>& f, const bf16* lds, const Lane& q,
                                                  int row0, int kc) {
    f.v = *reinterpret_cast<const bf16x8*>(lds + q.r[kc & 1] + (kc >> 1) * 32 + row0 * PITCH);
  }
  __device__ __forceinline__ static void tr_frag(Frag<bf16>& f, const bf16* lds, const Lane& q,
                                                 int kbase, int col0) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    union {
      struct { v4i16 a, b; } s;
      bf16x8 v;
    } u;
    u.s.a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16*)(lds + q.tr[0] + kbase * PITCH + col0));
    u.s.b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16*)(lds + q.tr[1] + kbase * PITCH + col0));
    f.v = u.v;
  }
  // 32 rows from row0, contraction slice kc (lane l: row row0 + l%32,
  // columns 16 kc + 8 (l/32) .. +7)
  __device__ __forceinline__ static void row_frag(Frag<bf16>& f, const bf16* lds, int row0, int kc,
                                                  int lane) {
    f.v = *reinterpret_cast<const bf16x8*>(lds + off(row0 + (lane & 31), kc * 16 + (lane >> 5) * 8));
  }
  // columns col0 .. col0 + 31 as rows of the operand, contraction rows in the
  // accumulator slot order from kbase (see frag_down)
  __device__ __forceinline__ static void tr_frag(Frag<bf16>& f, const bf16* lds, int kbase, int col0,
                                                 int lane) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const int g16 = lane >> 4, L = lane & 15;
    const int k0 = kbase + (g16 >> 1) * 4 + (L >> 2);
    const int m = col0 + (g16 & 1) * 16 + (L & 3) * 4;
    union {
      struct { v4i16 a, b; } s;
      bf16x8 v;
    } u;
    u.s.a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds + off(k0, m)));
    u.s.b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds + off(k0 + 8, m)));
    f.v = u.v;
  }
};

// 64 floats of lse2 and of delta for query rows t0 .. t0 + 63 of one head,
// into st[0..63] and st[64..127]: 32 lanes of wavefront 0, 16 bytes each.
// Reads may run up to 63 floats past the head's row (the regions carry a
// 256-byte pad); those queries are masked.
__device__ __forceinline__ void stats_issue(const float* __restrict__ lse2,
                                            const float* __restrict__ delta, int64_t row,
                                            float* st, int lane) {
  if (lane < 32) {
    const float* src = (lane < 16 ? lse2 : delta) + row + (lane & 15) * 4;
    lds_fill16(src, lds_addr(st));
  }
}

// dK, dV: a workgroup of 8 wavefronts owns 256 keys of one KV head (32 per
// wavefront, K and V rows held as fragments) and walks the (query head of
// the group, 64-query tile) steps that see them; Q, dO and the softmax
// statistics stream through three LDS stages, two steps ahead.
template <int D, int NW, bool ALIGNED>
__global__ __launch_bounds__(64 * NW) void attn_bwd_kv_tiled_kernel(
    const bf16* __restrict__ qkv, const bf16* __restrict__ gO, const float* __restrict__ lse2,
    const float* __restrict__ delta, bf16* __restrict__ gqkv, int T_, int H, int Hk, int W,
    int full, float c2, float scale, int nkt, int nb) {
  constexpr int BK2 = 32 * NW, BQ2 = 64, S = 3;
  using DT = Dual<BQ2, D>;
  constexpr int PER_WAVE = 2 * DT::CHUNKS / 4;  // Q and dO loads per loading wavefront
  static_assert(PER_WAVE + 1 < 16, "vmcnt field");
  __shared__ __attribute__((aligned(16))) bf16 Qs[S][DT::ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 dOs[S][DT::ELEMS];
  __shared__ __attribute__((aligned(16))) float st[S][2 * BQ2];
  const int tid = threadIdx.x, lane = tid & 63, hi = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: branches and fill bases scalar
  const bool loader = wv < 4;
  const int L = blockIdx.x;
  const int kt = L / (Hk * nb);  // early keys are seen by the most queries: first
  const int j = (L % (Hk * nb)) % Hk, b = (L % (Hk * nb)) / Hk;
  const int G = H / Hk;
  const int Qkv = (H + 2 * Hk) * D, Cq = H * D;
  const int64_t rb = (int64_t)b * T_;
  const int s0 = kt * BK2, sw = s0 + wv * 32, s = sw + (lane & 31);

  const typename DT::Lane lo = DT::lane_offsets(lane);
  Frag<bf16> kf[D / 16], vf[D / 16];
  load_row_frags<bf16, D>(kf, qkv + (rb + s) * Qkv + (H + j) * D, s < T_, lane);
  load_row_frags<bf16, D>(vf, qkv + (rb + s) * Qkv + (H + Hk + j) * D, s < T_, lane);
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dk[i][e] = 0.0f;
      dv[i][e] = 0.0f;
    }
  const unsigned wmax = full ? 0x7fffffffu : (unsigned)W;
  const int q_first = (s0 / BQ2) * BQ2;
  const int q_hi = full ? T_ : min(T_, s0 + BK2 + W);  // exclusive
  const int nq = (q_hi - q_first + BQ2 - 1) / BQ2;
  const int nstep = G * nq;
  // T a multiple of 64: every query tile lies inside the sequence
  typename DT::Offs oq, od;
  if (ALIGNED && loader) {
    oq = DT::offsets(Qkv, wv, lane);
    od = DT::offsets(Cq, wv, lane);
  }
  auto issue = [&](int step) {
    if (!loader) return;
    const int h = j * G + step / nq, t0 = q_first + (step % nq) * BQ2;
    if constexpr (ALIGNED) {
      DT::issue_fast(qkv + (rb + t0) * Qkv + h * D, oq, Qs[step % S], wv);
      DT::issue_fast(gO + (rb + t0) * Cq + h * D, od, dOs[step % S], wv);
    } else {
      DT::issue(qkv + h * D, Qkv, rb + t0, rb + T_, Qs[step % S], wv, lane);
      DT::issue(gO + h * D, Cq, rb + t0, rb + T_, dOs[step % S], wv, lane);
    }
    if (wv == 0) stats_issue(lse2, delta, ((int64_t)b * H + h) * T_ + t0, st[step % S], lane);
  };
  // this wavefront's loads of one step
  auto wait_all_but_one = [&] {
    if (wv == 0) __builtin_amdgcn_s_waitcnt(0x0f70 | (PER_WAVE + 1));
    else if (loader) __builtin_amdgcn_s_waitcnt(0x0f70 | PER_WAVE);
    else __builtin_amdgcn_s_waitcnt(0x0f70);
  };
#pragma unroll
  for (int st0 = 0; st0 < S - 1; ++st0)
    if (st0 < nstep) issue(st0);
  if (nstep > 1) wait_all_but_one();
  else __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  auto step_fn = [&](int step, auto cur_c) {
    constexpr int CUR = decltype(cur_c)::value;
    const int t0 = q_first + (step % nq) * BQ2;
    if (step + S - 1 < nstep) issue(step + S - 1);
    // P and dS of the 32-query block tb from its scores and dP (in place)
    auto softgrad = [&](f32x16& sa, f32x16& dp, int tb) {
      // accumulator rows t = t0 + 32 tb + 8 (e/4) + 4 hi + e%4: four
      // consecutive rows per group g = e/4, so their statistics load as one
      // vector
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int tl = tb * 32 + g * 8 + hi * 4;
        const f32x4 lv = *reinterpret_cast<const f32x4*>(&st[CUR][tl]);
        const f32x4 dv4 = *reinterpret_cast<const f32x4*>(&st[CUR][BQ2 + tl]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 4 * g + r;
          const float p = exp2_fast(fmaf(sa[e], c2, -lv[r]));
          sa[e] = p;
          dp[e] = p * (dp[e] - dv4[r]);
        }
      }
    };
    // dV += P^T dO and dK += dS^T Q over the block's 32 queries
    auto accumulate = [&](const f32x16& sa, const f32x16& dp, int tb) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        Frag<bf16> pf, dsf;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          frag_set(pf, jj, sa[8 * c + jj]);
          frag_set(dsf, jj, dp[8 * c + jj]);
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          Frag<bf16> doT, qT;
          DT::tr_frag(doT, dOs[CUR], lo, tb * 32 + 16 * c, db * 32);
          DT::tr_frag(qT, Qs[CUR], lo, tb * 32 + 16 * c, db * 32);
          mfma(dv[db], doT, pf);
          mfma(dk[db], qT, dsf);
        }
      }
    };
    // any (query, key) pair of the step visible to this wavefront's keys?
    if (sw < T_ && t0 + 63 >= sw && (full || t0 - (sw + 31) <= W)) {
      // The scores and dP of the step's two 32-query blocks are formed
      // together: four independent accumulation chains, fragments read one
      // k-slice ahead. A block on the causal diagonal or the window edge is
      // masked on its own branch (a block with nothing visible is computed
      // and masked whole: it occurs only next to the diagonal or the edge).
      f32x16 sa[2], dp[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          sa[tb][e] = 0.0f;
          dp[tb][e] = 0.0f;
        }
      Frag<bf16> qa[2][2], da[2][2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        DT::row_frag(qa[0][tb], Qs[CUR], lo, tb * 32, 0);
        DT::row_frag(da[0][tb], dOs[CUR], lo, tb * 32, 0);
      }
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) {
        const int p = kc & 1;
        if (kc + 1 < D / 16) {
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            DT::row_frag(qa[p ^ 1][tb], Qs[CUR], lo, tb * 32, kc + 1);
            DT::row_frag(da[p ^ 1][tb], dOs[CUR], lo, tb * 32, kc + 1);
          }
        }
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          mfma(sa[tb], qa[p][tb], kf[kc]);
          mfma(dp[tb], da[p][tb], vf[kc]);
        }
      }
      auto mask = [&](int tb) {
        const int tlo = t0 + tb * 32;
        if (!(tlo >= sw + 31 && (full || tlo + 31 - sw <= W) && tlo + 31 < T_)) {
          asm volatile("" ::: "memory");  // keep the mask on its own branch
          // query tq = tlo + 8 (e/4) + 4 hi + e%4 sees key s iff tq < T and
          // 0 <= tq - s <= W
          const int u = tlo + 4 * hi - s;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int r = (e >> 2) * 8 + (e & 3);
            const bool vis = (unsigned)(u + r) <= wmax && tlo + 4 * hi + r < T_;
            if (!vis) {
              sa[tb][e] = 0.0f;
              dp[tb][e] = 0.0f;
            }
          }
        }
      };
      softgrad(sa[0], dp[0], 0);
      mask(0);
      // the second block's softmax gradient (VALU) is interleaved with the
      // first block's dK / dV products (MFMA): one wavefront per SIMD, so
      // only its own instruction stream can fill the MFMA shadow
      accumulate(sa[0], dp[0], 0);
      softgrad(sa[1], dp[1], 1);
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);  // VALU
      }
      mask(1);
      accumulate(sa[1], dp[1], 1);
    }
    if (step + S - 1 < nstep) wait_all_but_one();
    else __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
  };
  static_assert(S == 3, "the step loop is unrolled by the stage count");
  for (int step = 0; step < nstep; step += S) {
    step_fn(step, std::integral_constant<int, 0>{});
    if (step + 1 < nstep) step_fn(step + 1, std::integral_constant<int, 1>{});
    if (step + 2 < nstep) step_fn(step + 2, std::integral_constant<int, 2>{});
  }
  if (s < T_) {
    bf16* kp = gqkv + (rb + s) * Qkv + (H + j) * D;
    bf16* vp = gqkv + (rb + s) * Qkv + (H + Hk + j) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + g * 8 + hi * 4;
        store_col4<bf16>(kp + d, dk[db][4 * g] * scale, dk[db][4 * g + 1] * scale,
                         dk[db][4 * g + 2] * scale, dk[db][4 * g + 3] * scale);
        store_col4<bf16>(vp + d, dv[db][4 * g], dv[db][4 * g + 1], dv[db][4 * g + 2],
                         dv[db][4 * g + 3]);
      }
  }
}

// dK, dV with two workgroups per CU (T a multiple of 32): a workgroup of 4
// wavefronts owns 128 keys of one KV head, 32 per wavefront (its K rows held
// as fragments; the workgroup's V rows staged once in LDS, XOR-swizzled, and
// read by rows for dP), and walks the (query head of the group, 32-query
// tile) steps that see them; Q, dO and the softmax statistics stream through
// two LDS stages, one step ahead. Against attn_bwd_kv_tiled_kernel (64-query
// steps, K and V in registers, three stages) a wavefront needs at most 256
// registers and the workgroup 73 KB of LDS, so two workgroups share a CU
// and each SIMD runs two wavefronts: one's softmax-gradient arithmetic and
// LDS waits overlap the other's MFMAs. The arithmetic of a (query, key)
// pair is the same as in that kernel.
// LDS of one dK/dV workgroup: the V rows, two stages of Q and dO tiles and
// their statistics.
template <int D>
struct Kv2Lds {
  static constexpr int BK2 = 128, BQ2 = 32;
  static constexpr int QEL = BQ2 * Dual<64, D>::PITCH;
  static constexpr int V_BYTES = (TileGeom<BK2, D, true>::ELEMS * 2 + 15) / 16 * 16;
  static constexpr int Q_OFF = V_BYTES, DO_OFF = Q_OFF + 2 * QEL * 2, ST_OFF = DO_OFF + 2 * QEL * 2;
  static constexpr int BYTES = ST_OFF + 2 * 2 * BQ2 * 4;
};

// Workgroup L of the dK/dV pass (see attn_bwd_kv2_kernel), on the LDS `smem`.
template <int D>
__device__ __forceinline__ void attn_bwd_kv2_body(
    char* smem, int L, const bf16* __restrict__ qkv, const bf16* __restrict__ gO,
    const float* __restrict__ lse2, const float* __restrict__ delta, bf16* __restrict__ gqkv,
    int T_, int H, int Hk, int W, int full, float c2, float scale, int nb) {
  using LY = Kv2Lds<D>;
  constexpr int BK2 = LY::BK2, BQ2 = LY::BQ2;
  using DT = Dual<64, D>;                     // layout of the Q / dO tiles (32 of its rows)
  constexpr int PITCH = DT::PITCH, QEL = LY::QEL, QCH = QEL * 2 / 1024;
  static_assert(QEL * 2 % 1024 == 0, "whole 1 KiB chunks per tile");
  using LV = DirectLoader<BK2, D, true>;
  bf16* const Vs = reinterpret_cast<bf16*>(smem);
  bf16(*const Qs)[QEL] = reinterpret_cast<bf16(*)[QEL]>(smem + LY::Q_OFF);
  bf16(*const dOs)[QEL] = reinterpret_cast<bf16(*)[QEL]>(smem + LY::DO_OFF);
  float(*const st)[2 * BQ2] = reinterpret_cast<float(*)[2 * BQ2]>(smem + LY::ST_OFF);
  const int tid = threadIdx.x, lane = tid & 63, hi = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kt = L / (Hk * nb);  // early keys are seen by the most queries: first
  const int j = (L % (Hk * nb)) % Hk, b = (L % (Hk * nb)) / Hk;
  const int G = H / Hk;
  const int Qkv = (H + 2 * Hk) * D, Cq = H * D;
  const int64_t rb = (int64_t)b * T_;
  const int s0 = kt * BK2, sw = s0 + wv * 32, s = sw + (lane & 31);

  const typename DT::Lane lo = DT::lane_offsets(lane);
  Frag<bf16> kf[D / 16];
  load_row_frags<bf16, D>(kf, qkv + (rb + s) * Qkv + (H + j) * D, s < T_, lane);
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dk[i][e] = 0.0f;
      dv[i][e] = 0.0f;
    }
  const unsigned wmax = full ? 0x7fffffffu : (unsigned)W;
  const int q_hi = full ? T_ : min(T_, s0 + BK2 + W);  // exclusive; queries start at s0
  const int nq = (q_hi - s0 + BQ2 - 1) / BQ2;
  const int nstep = G * nq;
  // Fills of a 32-row tile into the Dual layout: the 1 KiB chunks are dealt
  // to the 4 wavefronts in turn (chunk wv + 4 q); each lane's byte offset
  // from the tile's first element is computed once per matrix (~0u: a slot
  // in the row padding), so a fill is one load per chunk from a
  // wavefront-uniform base. Every row lies inside the sequence.
  constexpr int NQC = (QCH + 3) / 4;
  auto tile_offs = [&](int64_t ld, uint32_t (&o)[NQC]) {
#pragma unroll
    for (int q = 0; q < NQC; ++q) {
      const int c = wv + 4 * q;
      const int ob = c * 1024 + lane * 16;
      const int t = ob / (PITCH * 2), pg = (ob % (PITCH * 2)) / 16;
      const int gi = pg ^ ((t >> 2) & 3);
      o[q] = (c < QCH && gi < D / 8) ? (uint32_t)((t * ld + gi * 8) * 2) : ~0u;
    }
  };
  uint32_t oq[NQC], od[NQC];
  tile_offs(Qkv, oq);
  tile_offs(Cq, od);
  auto fill_tile = [&](const bf16* tile, const uint32_t (&o)[NQC], bf16* lds) {
#pragma unroll
    for (int q = 0; q < NQC; ++q)
      if (o[q] != ~0u) lds_fill16(tile, o[q], lds_addr(lds) + (wv + 4 * q) * 1024);
  };
  // the step after (h, qi): the query tiles of one head, then the next head
  int ih = 0, iq = 0;  // head index in the group and query tile of the next fill
  auto issue = [&](int buf) {
    const int h = j * G + ih, t0 = s0 + iq * BQ2;
    fill_tile(qkv + (rb + t0) * Qkv + h * D, oq, Qs[buf]);
    fill_tile(gO + (rb + t0) * Cq + h * D, od, dOs[buf]);
    if (wv == 0 && lane < 16) {  // 32 floats of lse2, then 32 of delta
      const int64_t row = ((int64_t)b * H + h) * T_ + t0;
      const float* src = (lane < 8 ? lse2 : delta) + row + (lane & 7) * 4;
      lds_fill16(src, lds_addr(st[buf]) + lane * 16);
    }
    if (++iq == nq) {
      iq = 0;
      ++ih;
    }
  };
  LV::issue(qkv + (H + Hk + j) * D, Qkv, rb + s0, rb + T_, 0, D, Vs, wv, lane, 4);
  if (nstep > 0) issue(0);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  __syncthreads();
  int cq = 0;  // query tile of the current step
  auto step_fn = [&](int step, auto cur_c) {
    constexpr int CUR = decltype(cur_c)::value;
    const int t0 = s0 + cq * BQ2;
    if (++cq == nq) cq = 0;
    if (step + 1 < nstep) issue(CUR ^ 1);
    if (sw < T_ && t0 + 31 >= sw && (full || t0 - (sw + 31) <= W)) {
      // S = Q K^T and dP = dO V^T of the 32 queries x 32 keys, fragments
      // read one k-slice ahead
      f32x16 sa, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sa[e] = 0.0f;
        dp[e] = 0.0f;
      }
      Frag<bf16> qa[2], da[2], va[2];
      DT::row_frag(qa[0], Qs[CUR], lo, 0, 0);
      DT::row_frag(da[0], dOs[CUR], lo, 0, 0);
      read_frag<BK2, D, true>(va[0], Vs, wv * 32, 0, lane);
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) {
        const int p = kc & 1;
        if (kc + 1 < D / 16) {
          DT::row_frag(qa[p ^ 1], Qs[CUR], lo, 0, kc + 1);
          DT::row_frag(da[p ^ 1], dOs[CUR], lo, 0, kc + 1);
          read_frag<BK2, D, true>(va[p ^ 1], Vs, wv * 32, kc + 1, lane);
        }
        mfma(sa, qa[p], kf[kc]);
        mfma(dp, da[p], va[p]);
      }
      // P and dS in place: accumulator rows t0 + 8 (e/4) + 4 hi + e%4 are
      // queries, so each group of four reads one vector of statistics
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int tl = g * 8 + hi * 4;
        const f32x4 lv = *reinterpret_cast<const f32x4*>(&st[CUR][tl]);
        const f32x4 dv4 = *reinterpret_cast<const f32x4*>(&st[CUR][BQ2 + tl]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 4 * g + r;
          const float pr = exp2_fast(fmaf(sa[e], c2, -lv[r]));
          sa[e] = pr;
          dp[e] = pr * (dp[e] - dv4[r]);
        }
      }
      if (!(t0 >= sw + 31 && (full || t0 + 31 - sw <= W))) {
        asm volatile("" ::: "memory");  // keep the mask on its own branch
        // query t0 + 8 (e/4) + 4 hi + e%4 sees key s iff 0 <= t - s <= W
        const int u = t0 + 4 * hi - s;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = (e >> 2) * 8 + (e & 3);
          if ((unsigned)(u + r) > wmax) {
            sa[e] = 0.0f;
            dp[e] = 0.0f;
          }
        }
      }
      // dV += P^T dO and dK += dS^T Q over the 32 queries (two 16-query
      // slices in the accumulator's row order)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        Frag<bf16> pf, dsf;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          frag_set(pf, jj, sa[8 * c + jj]);
          frag_set(dsf, jj, dp[8 * c + jj]);
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          Frag<bf16> doT, qT;
          DT::tr_frag(doT, dOs[CUR], lo, 16 * c, db * 32);
          DT::tr_frag(qT, Qs[CUR], lo, 16 * c, db * 32);
          mfma(dv[db], doT, pf);
          mfma(dk[db], qT, dsf);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the next step's tiles landed
    __syncthreads();
  };
  for (int step = 0; step < nstep; step += 2) {
    step_fn(step, std::integral_constant<int, 0>{});
    if (step + 1 < nstep) step_fn(step + 1, std::integral_constant<int, 1>{});
  }
  if (s < T_) {
    bf16* kp = gqkv + (rb + s) * Qkv + (H + j) * D;
    bf16* vp = gqkv + (rb + s) * Qkv + (H + Hk + j) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + g * 8 + hi * 4;
        store_col4<bf16>(kp + d, dk[db][4 * g] * scale, dk[db][4 * g + 1] * scale,
                         dk[db][4 * g + 2] * scale, dk[db][4 * g + 3] * scale);
        store_col4<bf16>(vp + d, dv[db][4 * g], dv[db][4 * g + 1], dv[db][4 * g + 2],
                         dv[db][4 * g + 3]);
      }
  }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bwd_kv2_kernel(
    const bf16* __restrict__ qkv, const bf16* __restrict__ gO, const float* __restrict__ lse2,
    const float* __restrict__ delta, bf16* __restrict__ gqkv, int T_, int H, int Hk, int W,
    int full, float c2, float scale, int nb) {
  __shared__ __attribute__((aligned(16))) char smem[Kv2Lds<D>::BYTES];
  attn_bwd_kv2_body<D>(smem, (int)blockIdx.x, qkv, gO, lse2, delta, gqkv, T_, H, Hk, W, full, c2,
                       scale, nb);
}


// dQ: a workgroup of 8 wavefronts owns 256 queries of one head (32 per
// wavefront, Q and dO rows held as fragments) and walks the visible 64-key
// tiles; K (read by rows and transposed) and V (read by rows) stream
// through three LDS stages, two tiles ahead.
// LDS of one dQ workgroup: S stages of V and K tiles.
template <int D, int S>
struct QLds {
  static constexpr int BKV = 64;
  static constexpr int K_ELEMS = Dual<BKV, D>::ELEMS, V_ELEMS = TileGeom<BKV, D, true>::ELEMS;
  static constexpr int K_OFF = (S * V_ELEMS * 2 + 15) / 16 * 16;
  static constexpr int BYTES = K_OFF + S * K_ELEMS * 2;
};

// Workgroup L of the dQ pass (see attn_bwd_q_tiled_kernel), on the LDS `smem`.
template <int D, int NW, bool ALIGNED, int S>
__device__ __forceinline__ void attn_bwd_q_body(
    char* smem, int L, const bf16* __restrict__ qkv, const bf16* __restrict__ gO,
    const float* __restrict__ lse2, const float* __restrict__ delta, bf16* __restrict__ gqkv,
    int T_, int H, int Hk, int W, int full, float c2, float scale, int nq, int nb) {
  constexpr int BQ = 32 * NW, BKV = QLds<D, S>::BKV;
  static_assert(S == 2 || S == 3, "two or three stages");
  using DK = Dual<BKV, D>;
  using GV = TileGeom<BKV, D, true>;
  using LV = DirectLoader<BKV, D, true>;
  static_assert(LV::CHUNKS % 4 == 0, "whole chunks per loading wavefront");
  constexpr int PER_WAVE = DK::CHUNKS / 4 + LV::CHUNKS / 4;
  static_assert(PER_WAVE < 16, "vmcnt field");
  bf16(*const Vs)[GV::ELEMS] = reinterpret_cast<bf16(*)[GV::ELEMS]>(smem);
  bf16(*const Ks)[DK::ELEMS] = reinterpret_cast<bf16(*)[DK::ELEMS]>(smem + QLds<D, S>::K_OFF);
  const int tid = threadIdx.x, lane = tid & 63, hi = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS fill addresses in SGPRs
  const bool loader = wv < 4;
  const int qt = nq - 1 - L / (H * nb);
  const int h = (L % (H * nb)) % H, b = (L % (H * nb)) / H;
  const int j = h / (H / Hk);
  const int Qkv = (H + 2 * Hk) * D, Cq = H * D;
  const int64_t rb = (int64_t)b * T_;
  const int t0 = qt * BQ, tw = t0 + wv * 32, t = tw + (lane & 31);
  const bool tv = t < T_;
  const bf16* kbase = qkv + (H + j) * D;
  const bf16* vbase = qkv + (H + Hk + j) * D;

  const typename DK::Lane lo = DK::lane_offsets(lane);
  Frag<bf16> qf[D / 16], df[D / 16];
  load_row_frags<bf16, D>(qf, qkv + (rb + t) * Qkv + h * D, tv, lane);
  load_row_frags<bf16, D>(df, gO + (rb + t) * Cq + h * D, tv, lane);
  const float lt = tv ? lse2[((int64_t)b * H + h) * T_ + t] : 0.0f;
  const float dt = tv ? delta[((int64_t)b * H + h) * T_ + t] : 0.0f;
  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[i][e] = 0.0f;
  const unsigned wmax = full ? 0x7fffffffu : (unsigned)W;
  const int first = ((full ? 0 : max(0, t0 - W)) / BKV) * BKV;
  const int ntile = (min(T_, t0 + BQ) - first + BKV - 1) / BKV;
  const int w_lo = full ? 0 : max(0, tw - W), w_hi = min(T_, tw + 32);
  // T a multiple of 64: every key tile lies inside the sequence
  typename DK::Offs ok;
  LV lv;
  if (ALIGNED && loader) {
    ok = DK::offsets(Qkv, wv, lane);
    lv.init(Qkv, 0, 1 << 30, wv, lane);
  }
  auto issue = [&](int it) {
    if (!loader) return;
    const int64_t r0 = rb + first + (int64_t)it * BKV;
    if constexpr (ALIGNED) {
      DK::issue_fast(kbase + r0 * Qkv, ok, Ks[it % S], wv);
      lv.issue_fast(vbase + r0 * Qkv, Vs[it % S], wv);
    } else {
      DK::issue(kbase, Qkv, r0, rb + T_, Ks[it % S], wv, lane);
      LV::issue(vbase, Qkv, r0, rb + T_, 0, D, Vs[it % S], wv, lane);
    }
  };
#pragma unroll
  for (int it = 0; it < S - 1; ++it)
    if (it < ntile) issue(it);
  if (S == 3 && ntile > 1 && loader) __builtin_amdgcn_s_waitcnt(0x0f70 | PER_WAVE);
  else __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  auto tile = [&](int it, auto cur_c) {
    constexpr int CUR = decltype(cur_c)::value;
    const int s0 = first + it * BKV;
    if (it + S - 1 < ntile) issue(it + S - 1);
    if (tw < T_ && s0 < w_hi && s0 + BKV > w_lo) {
      const bool interior = (s0 + BKV - 1 <= tw) && (full || tw + 31 - s0 <= W);
      // The scores and dP of the tile's two 32-key blocks are formed
      // together: four independent accumulation chains, fragments read one
      // k-slice ahead.
      f32x16 sa[2], dp[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          sa[sb][e] = 0.0f;
          dp[sb][e] = 0.0f;
        }
      Frag<bf16> ka[2][2], va[2][2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        DK::row_frag(ka[0][sb], Ks[CUR], lo, sb * 32, 0);
        read_frag<BKV, D, true>(va[0][sb], Vs[CUR], sb * 32, 0, lane);
      }
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) {
        const int p = kc & 1;
        if (kc + 1 < D / 16) {
#pragma unroll
          for (int sb = 0; sb < 2; ++sb) {
            DK::row_frag(ka[p ^ 1][sb], Ks[CUR], lo, sb * 32, kc + 1);
            read_frag<BKV, D, true>(va[p ^ 1][sb], Vs[CUR], sb * 32, kc + 1, lane);
          }
        }
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          mfma(sa[sb], ka[p][sb], qf[kc]);
          mfma(dp[sb], va[p][sb], df[kc]);
        }
      }
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = exp2_fast(fmaf(sa[sb][e], c2, -lt));
          dp[sb][e] = p * (dp[sb][e] - dt);
        }
        if (!interior) {
          asm volatile("" ::: "memory");  // keep the mask on its own branch
          const int u = t - s0 - sb * 32 - 4 * hi;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int r = (e >> 2) * 8 + (e & 3);
            if ((unsigned)(u - r) > wmax) dp[sb][e] = 0.0f;
          }
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          Frag<bf16> dsf;
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) frag_set(dsf, jj, dp[sb][8 * c + jj]);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            Frag<bf16> kT;
            DK::tr_frag(kT, Ks[CUR], lo, sb * 32 + 16 * c, db * 32);
            mfma(dq[db], kT, dsf);
          }
        }
      }
    }
    if (S == 3 && it + S - 1 < ntile && loader) __builtin_amdgcn_s_waitcnt(0x0f70 | PER_WAVE);
    else __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
  };
  // the tile loop is unrolled by the stage count
  for (int it = 0; it < ntile; it += S) {
    tile(it, std::integral_constant<int, 0>{});
    if (it + 1 < ntile) tile(it + 1, std::integral_constant<int, 1>{});
    if constexpr (S == 3)
      if (it + 2 < ntile) tile(it + 2, std::integral_constant<int, 2 % S>{});
  }
  if (tv) {
    bf16* qp = gqkv + (rb + t) * Qkv + h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + g * 8 + hi * 4;
        store_col4<bf16>(qp + d, dq[db][4 * g] * scale, dq[db][4 * g + 1] * scale,
                         dq[db][4 * g + 2] * scale, dq[db][4 * g + 3] * scale);
      }
  }
}

template <int D, int NW, bool ALIGNED, int S>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(S == 2 ? 2 : 1, S == 2 ? 2 : 1))) void attn_bwd_q_tiled_kernel(
    const bf16* __restrict__ qkv, const bf16* __restrict__ gO, const float* __restrict__ lse2,
    const float* __restrict__ delta, bf16* __restrict__ gqkv, int T_, int H, int Hk, int W,
    int full, float c2, float scale, int nq, int nb) {
  __shared__ __attribute__((aligned(16))) char smem[QLds<D, S>::BYTES];
  attn_bwd_q_body<D, NW, ALIGNED, S>(smem, (int)blockIdx.x, qkv, gO, lse2, delta, gqkv, T_, H, Hk,
                                     W, full, c2, scale, nq, nb);
}

// Both backward passes in one launch (head_dim 128, T a multiple of 64):
// workgroups 0 .. nkv - 1 run the dK/dV pass, the rest the dQ pass. The two
// passes read the same inputs and write disjoint outputs, and both fit two
// workgroups per CU; in one grid the shorter dQ workgroups fill the CU slots
// the dK/dV workgroups leave (a d12 layer has 768 of each against 512
// slots, which as separate launches both end on a half-empty round).
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bwd_pair_kernel(
    const bf16* __restrict__ qkv, const bf16* __restrict__ gO, const float* __restrict__ lse2,
    const float* __restrict__ delta, bf16* __restrict__ gqkv, int T_, int H, int Hk, int W,
    int full, float c2, float scale, int nkv, int nq, int nb) {
  constexpr int BYTES = Kv2Lds<D>::BYTES > QLds<D, 2>::BYTES ? Kv2Lds<D>::BYTES : QLds<D, 2>::BYTES;
  __shared__ __attribute__((aligned(16))) char smem[BYTES];
  const int L = (int)blockIdx.x;
  if (L < nkv)
    attn_bwd_kv2_body<D>(smem, L, qkv, gO, lse2, delta, gqkv, T_, H, Hk, W, full, c2, scale, nb);
  else
    attn_bwd_q_body<D, 4, true, 2>(smem, L - nkv, qkv, gO, lse2, delta, gqkv, T_, H, Hk, W, full,
                                   c2, scale, nq, nb);
}


template <typename T, int D>
void fwd(const gpt::Dims& d, bool full, const void* qkv, void* out, float* lse, hipStream_t s) {
  const float c2 = 1.4426950408889634f / sqrtf((float)D);
  if constexpr (sizeof(T) == 2) {
    const int nq = (d.T + 255) / 256;
    if (!full && d.T % 64 == 0) {  // window layers: 128-query tiles
      const int nq2 = d.T / 128 + (d.T % 128 != 0);
      GK_LAUNCH((attn_fwd_tiled_kernel<D, true, 128, 2>), dim3((unsigned)(nq2 * d.H * d.B)),
                dim3(256), 0, s, static_cast<const bf16*>(qkv), static_cast<bf16*>(out), lse, d.T,
                d.H, d.Hk, d.W, 0, c2, nq2, d.B);
    } else if (d.T % 64 == 0)
      GK_LAUNCH((attn_fwd_tiled_kernel<D, true>), dim3((unsigned)(nq * d.H * d.B)),
                         dim3(512), 0, s, static_cast<const bf16*>(qkv), static_cast<bf16*>(out),
                         lse, d.T, d.H, d.Hk, d.W, full ? 1 : 0, c2, nq, d.B);
    else
      GK_LAUNCH((attn_fwd_tiled_kernel<D, false>), dim3((unsigned)(nq * d.H * d.B)),
                         dim3(512), 0, s, static_cast<const bf16*>(qkv), static_cast<bf16*>(out),
                         lse, d.T, d.H, d.Hk, d.W, full ? 1 : 0, c2, nq, d.B);
  } else {
    dim3 grid((unsigned)((d.T + 127) / 128), d.H, d.B);
    GK_LAUNCH((attn_fwd_kernel<T, D>), grid, dim3(256), 0, s, static_cast<const T*>(qkv),
                       static_cast<T*>(out), lse, d.T, d.H, d.Hk, d.W, full ? 1 : 0, c2);
  }
}

template <typename T, int D>
void bwd(const gpt::Dims& d, bool full, const void* qkv, const void* gO, const float* lse,
         const float* delta, void* gqkv, hipStream_t s) {
  const float c2 = 1.4426950408889634f / sqrtf((float)D);
  const float scale = 1.0f / sqrtf((float)D);
  if constexpr (sizeof(T) == 2) {
    // 4 wavefronts per workgroup. The dK/dV pass needs > 256 registers (one
    // wavefront per SIMD); the dQ pass fits 256 with two LDS stages when T is
    // a multiple of 64, so two of its workgroups share a CU.
    constexpr int NW = 4;
    const int nkt = (d.T + 32 * NW - 1) / (32 * NW), nq = (d.T + 32 * NW - 1) / (32 * NW);
#define GPT_ATTN_BWD(AL)                                                                          \
  GK_LAUNCH((attn_bwd_kv_tiled_kernel<D, NW, AL>), dim3((unsigned)(nkt * d.Hk * d.B)),    \
                     dim3(64 * NW), 0, s, static_cast<const bf16*>(qkv),                           \
                     static_cast<const bf16*>(gO), lse, delta, static_cast<bf16*>(gqkv), d.T, d.H, \
                     d.Hk, d.W, full ? 1 : 0, c2, scale, nkt, d.B);                                \
  GK_LAUNCH((attn_bwd_q_tiled_kernel<D, NW, AL, AL ? 2 : 3>), dim3((unsigned)(nq * d.H * d.B)), \
                     dim3(64 * NW), 0, s, static_cast<const bf16*>(qkv),                           \
                     static_cast<const bf16*>(gO), lse, delta, static_cast<bf16*>(gqkv), d.T, d.H, \
                     d.Hk, d.W, full ? 1 : 0, c2, scale, nq, d.B)
    if constexpr (D == 128) {
      if (d.T % 32 == 0) {
        const int nkt2 = (d.T + 127) / 128;
        const int nkv = nkt2 * d.Hk * d.B;
        if (d.T % 64 == 0) {
          GK_LAUNCH((attn_bwd_pair_kernel<D>), dim3((unsigned)(nkv + nq * d.H * d.B)), dim3(256), 0,
                    s, static_cast<const bf16*>(qkv), static_cast<const bf16*>(gO), lse, delta,
                    static_cast<bf16*>(gqkv), d.T, d.H, d.Hk, d.W, full ? 1 : 0, c2, scale, nkv,
                    nq, d.B);
          return;
        }
        GK_LAUNCH((attn_bwd_kv2_kernel<D>), dim3((unsigned)nkv), dim3(256), 0, s,
                  static_cast<const bf16*>(qkv), static_cast<const bf16*>(gO), lse, delta,
                  static_cast<bf16*>(gqkv), d.T, d.H, d.Hk, d.W, full ? 1 : 0, c2, scale, d.B);
        GK_LAUNCH((attn_bwd_q_tiled_kernel<D, NW, false, 3>), dim3((unsigned)(nq * d.H * d.B)),
                  dim3(64 * NW), 0, s, static_cast<const bf16*>(qkv),
                  static_cast<const bf16*>(gO), lse, delta, static_cast<bf16*>(gqkv), d.T, d.H,
                  d.Hk, d.W, full ? 1 : 0, c2, scale, nq, d.B);
        return;
      }
    }
    if (d.T % 64 == 0) {
      GPT_ATTN_BWD(true);
    } else {
      GPT_ATTN_BWD(false);
    }
#undef GPT_ATTN_BWD
    return;
  }
  dim3 gkv((unsigned)((d.T + 127) / 128), d.Hk, d.B);
  GK_LAUNCH((attn_bwd_kv_kernel<T, D>), gkv, dim3(256), 0, s, static_cast<const T*>(qkv),
                     static_cast<const T*>(gO), lse, delta, static_cast<T*>(gqkv), d.T, d.H, d.Hk,
                     d.W, full ? 1 : 0, c2, scale);
  dim3 gq((unsigned)((d.T + 127) / 128), d.H, d.B);
  GK_LAUNCH((attn_bwd_q_kernel<T, D>), gq, dim3(256), 0, s, static_cast<const T*>(qkv),
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
  const int per = 256 / (d.D / 8);
  dim3 grid((unsigned)((NH + per - 1) / per));
#define GPT_DELTA(TY, DD)                                                                         \
  GK_LAUNCH((attn_delta_kernel<TY, DD>), grid, dim3(256), 0, s, static_cast<const TY*>(gO), \
                     static_cast<const TY*>(O), delta, NH, d.H, d.T)
  if (d.bf16) {
    if (d.D == 128) GPT_DELTA(bf16, 128);
    else GPT_DELTA(bf16, 64);
  } else {
    if (d.D == 128) GPT_DELTA(float, 128);
    else GPT_DELTA(float, 64);
  }
#undef GPT_DELTA
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
