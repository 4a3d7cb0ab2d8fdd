// GEMM launchers of the GPT step: C[M][N] = sum_k A(m,k) * B(n,k) with fused
// operand prologues (ReLU^2, softcap cross-entropy gradient) and output
// epilogues (store, residual add, ReLU^2 backward, softcap + row sums,
// split-K atomic accumulation).
//
// bf16 products run on the tiled MFMA core in gemm_core.h. fp32 products
// (the small fp32 configuration) use the plain kernel below: each operand is
// either contraction-contiguous ("K-major": row m holds k) or output-
// contiguous ("MN-major": row k holds m); tiles are written to LDS in a
// [row][k] layout (MN-major operands transposed on the LDS write).
#include "device_common.h"
#include "gemm_core.h"
#include "internal.h"

#include <algorithm>
#include <cstdio>
#include <cstdlib>

namespace gk {

// ------------------------------------------------------------ prologues
// A prologue transforms each 8-element (bf16) or 4-element (fp32) operand
// vector after its global load; `vec<ALONG_K>` gets the coordinates of the
// vector's first element and whether the vector runs along the contraction
// index. init() runs once per thread before the first tile.
struct PreId {
  static constexpr bool kActive = false;
  __device__ void init() {}
  template <bool ALONG_K, int NE>
  __device__ void vec(float*, int64_t, int64_t) const {}
};
struct PreRelu2 {  // ReLU^2 of the MLP hidden pre-activation
  static constexpr bool kActive = true;
  __device__ void init() {}
  template <bool ALONG_K, int NE>
  __device__ void vec(float* v, int64_t, int64_t) const {
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      const float r = fmaxf(v[j], 0.0f);
      v[j] = r * r;
    }
  }
};
// ------------------------------------------------------------ epilogues
// value(m, n, acc): per-element transform in the accumulator layout;
// store4(m, n, v, cnt): write columns n .. n+cnt-1 of row m (cnt <= 4).
// at_split(s): the epilogue of K split s (split-K partials).
// Epilogues that read another operand split the write into aux(m, n, cnt),
// the load, and store4a(m, n, v, cnt, aux): the tiled kernel issues all
// loads of a slab before any store, so their latencies overlap.
// operator() is the element-wise form used by the fp32 kernel.
template <typename T>
__device__ __forceinline__ void put4(T* p, const f32x4& v, int cnt) {
  if (cnt == 4) {
    if constexpr (sizeof(T) == 2) {
      bf16x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = static_cast<bf16>(v[j]);
      *reinterpret_cast<bf16x4*>(p) = o;
    } else {
      *reinterpret_cast<f32x4*>(p) = v;
    }
  } else {
    for (int j = 0; j < cnt; ++j) p[j] = from_f<T>(v[j]);
  }
}
// Four consecutive elements as stored (bf16 stays bf16 until used, so a
// load in flight does not force a wait where it is issued).
template <typename T>
struct Raw4 {
  using type = f32x4;
};
template <>
struct Raw4<bf16> {
  using type = bf16x4;
};
template <typename T>
__device__ __forceinline__ typename Raw4<T>::type get4raw(const T* p, int cnt) {
  using R = typename Raw4<T>::type;
  if (cnt == 4) return *reinterpret_cast<const R*>(p);
  R r{};
  for (int j = 0; j < cnt; ++j) r[j] = p[j];
  return r;
}
__device__ __forceinline__ f32x4 to_f4(const f32x4& v) { return v; }
__device__ __forceinline__ f32x4 to_f4(const bf16x4& v) {
  return f32x4{static_cast<float>(v[0]), static_cast<float>(v[1]), static_cast<float>(v[2]),
               static_cast<float>(v[3])};
}
template <typename T>
__device__ __forceinline__ f32x4 get4(const T* p, int cnt) {
  if (cnt == 4) {
    if constexpr (sizeof(T) == 2) {
      const bf16x4 o = *reinterpret_cast<const bf16x4*>(p);
      return f32x4{static_cast<float>(o[0]), static_cast<float>(o[1]), static_cast<float>(o[2]),
                   static_cast<float>(o[3])};
    } else {
      return *reinterpret_cast<const f32x4*>(p);
    }
  }
  f32x4 r{0, 0, 0, 0};
  for (int j = 0; j < cnt; ++j) r[j] = to_f(p[j]);
  return r;
}

// sqrt of an activation: the hardware square root (about 1 ulp) for bf16
// activations, the correctly rounded one for fp32.
template <typename T>
__device__ __forceinline__ float sqrt_act(float x) {
  if constexpr (sizeof(T) == 2) return __builtin_amdgcn_sqrtf(x);
  else return sqrtf(x);
}

template <class Derived>
struct EpBase {
  using Aux = NoAux;
  // kAmax: the epilogue also returns max |stored value| of each store
  // (store4m / store4am) and the kernel merges the block's maximum into
  // *amax (when non-null) as the bits of a non-negative float
  static constexpr bool kAmax = false;
  // the epilogue of K split `split` (all splits write the same C by default)
  __device__ Derived at_split(int) const { return static_cast<const Derived&>(*this); }
  // the epilogue of batch entry `b` (batched launches only)
  __device__ Derived at_batch(int) const { return static_cast<const Derived&>(*this); }
  __device__ float value(int64_t, int64_t, float v) const { return v; }
  __device__ NoAux aux(int64_t, int64_t, int) const { return {}; }
  __device__ void store4a(int64_t m, int64_t n, f32x4 v, int cnt, const NoAux&) const {
    static_cast<const Derived&>(*this).store4(m, n, v, cnt);
  }
  __device__ void operator()(int64_t m, int64_t n, float acc) const {
    const Derived& d = static_cast<const Derived&>(*this);
    d.store4(m, n, f32x4{d.value(m, n, acc), 0, 0, 0}, 1);
  }
};

template <typename T>
struct EpStore : EpBase<EpStore<T>> {
  T* C;
  int64_t ldc;
  int64_t bstride;  // elements between the C of consecutive batch entries
  __device__ EpStore at_batch(int b) const {
    EpStore e = *this;
    e.C += (int64_t)b * bstride;
    return e;
  }
  __device__ void store4(int64_t m, int64_t n, f32x4 v, int cnt) const {
    put4<T>(C + m * ldc + n, v, cnt);
  }
};
struct EpF32 : EpBase<EpF32> {
  float* C;
  int64_t ldc;
  int accumulate;
  using Aux = f32x4;
  __device__ f32x4 aux(int64_t m, int64_t n, int cnt) const {
    return accumulate ? get4<float>(C + m * ldc + n, cnt) : f32x4{0, 0, 0, 0};
  }
  __device__ void store4a(int64_t m, int64_t n, f32x4 v, int cnt, const f32x4& old) const {
    put4<float>(C + m * ldc + n, v + old, cnt);
  }
  __device__ void store4(int64_t m, int64_t n, f32x4 v, int cnt) const {
    store4a(m, n, v, cnt, aux(m, n, cnt));
  }
};
struct EpPart : EpBase<EpPart> {  // split-K partials: split s writes C + s * stride
  float* C;
  int64_t ldc;
  int64_t stride;
  __device__ EpPart at_split(int split) const {
    EpPart e = *this;
    e.C += (int64_t)split * stride;
    return e;
  }
  __device__ void store4(int64_t m, int64_t n, f32x4 v, int cnt) const {
    put4<float>(C + m * ldc + n, v, cnt);
  }
};
struct EpResid : EpBase<EpResid> {  // C = R + acc (residual stream, fp32)
  const float* R;
  float* C;
  int64_t ldc;
  using Aux = f32x4;
  __device__ f32x4 aux(int64_t m, int64_t n, int cnt) const {
    return get4<float>(R + m * ldc + n, cnt);
  }
  __device__ void store4a(int64_t m, int64_t n, f32x4 v, int cnt, const f32x4& r) const {
    put4<float>(C + m * ldc + n, v + r, cnt);
  }
  __device__ void store4(int64_t m, int64_t n, f32x4 v, int cnt) const {
    store4a(m, n, v, cnt, aux(m, n, cnt));
  }
};
// C = alpha R + beta acc (R and C alike, same leading dimension); batched
// launches step R and C by bstride elements per entry
template <typename T>
struct EpLin : EpBase<EpLin<T>> {
  const T* R;
  T* C;
  int64_t ldc, bstride;
  float alpha, beta;
  using Aux = f32x4;
  __device__ EpLin at_batch(int b) const {
    EpLin e = *this;
    e.R += (int64_t)b * bstride;
    e.C += (int64_t)b * bstride;
    return e;
  }
  __device__ f32x4 aux(int64_t m, int64_t n, int cnt) const { return get4<T>(R + m * ldc + n, cnt); }
  __device__ void store4a(int64_t m, int64_t n, f32x4 v, int cnt, const f32x4& r) const {
    put4<T>(C + m * ldc + n, alpha * r + beta * v, cnt);
  }
  __device__ void store4(int64_t m, int64_t n, f32x4 v, int cnt) const {
    store4a(m, n, v, cnt, aux(m, n, cnt));
  }
};
template <typename T>
struct EpRelu2 : EpBase<EpRelu2<T>> {  // C = relu(acc)^2 (the MLP hidden activation h)
  static constexpr bool kStage32 = true;
  static constexpr bool kAmax = true;
  T* C;
  int64_t ldc;
  uint32_t* amax;  // max |C| (fp8 quantiser's amax slot), or null
  __device__ float store4m(int64_t m, int64_t n, f32x4 v, int cnt) const {
    f32x4 o;
    float mx = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float r = fmaxf(v[j], 0.0f);
      o[j] = r * r;
      if (j < cnt) mx = fmaxf(mx, o[j]);
    }
    put4<T>(C + m * ldc + n, o, cnt);
    return mx;
  }
  __device__ void store4(int64_t m, int64_t n, f32x4 v, int cnt) const { (void)store4m(m, n, v, cnt); }
  // the stored maximum: rounding to T is monotone, so max |round(o)| = round(max |o|)
  __device__ float amax_of(float mx) const { return static_cast<float>(from_f<T>(mx)); }
};
template <typename T>
struct EpRelu2Bwd : EpBase<EpRelu2Bwd<T>> {
  static constexpr bool kStage32 = true;
  // g_u = g_h * d/du relu(u)^2 = g_h * 2 relu(u), with relu(u) = sqrt(h)
  static constexpr bool kAmax = true;
  const T* H;
  T* C;
  int64_t ldc;
  uint32_t* amax;  // max |C| (fp8 quantiser's amax slot), or null
  using Aux = typename Raw4<T>::type;
  __device__ Aux aux(int64_t m, int64_t n, int cnt) const { return get4raw<T>(H + m * ldc + n, cnt); }
  __device__ float store4am(int64_t m, int64_t n, f32x4 v, int cnt, const Aux& hr) const {
    const f32x4 h = to_f4(hr);
    f32x4 o;
    float mx = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[j] = 2.0f * sqrt_act<T>(h[j]) * v[j];
      if (j < cnt) mx = fmaxf(mx, fabsf(o[j]));
    }
    put4<T>(C + m * ldc + n, o, cnt);
    return mx;
  }
  __device__ void store4a(int64_t m, int64_t n, f32x4 v, int cnt, const Aux& hr) const {
    (void)store4am(m, n, v, cnt, hr);
  }
  __device__ void store4(int64_t m, int64_t n, f32x4 v, int cnt) const {
    store4a(m, n, v, cnt, aux(m, n, cnt));
  }
  __device__ float amax_of(float mx) const { return static_cast<float>(from_f<T>(mx)); }
};
template <typename T>
struct EpSoftcap : EpBase<EpSoftcap<T>> {  // c = cap * tanh(z / cap)
  T* C;
  int64_t ldc;
  float cap;
  float k2;  // 2 log2(e) / cap
  __device__ float value(int64_t, int64_t, float z) const {
    if constexpr (sizeof(T) == 2) {
      // tanh(u) = 1 - 2 / (1 + e^(2u)) with the hardware exp2 and reciprocal
      // (about 1 ulp each): the absolute error of c, ~cap * 2^-23, is far
      // below the bf16 step of the stored value; saturates to +-cap
      const float e = __builtin_amdgcn_exp2f(z * k2);
      return cap - (2.0f * cap) * __builtin_amdgcn_rcpf(1.0f + e);
    } else {
      return cap * tanhf(z / cap);
    }
  }
  __device__ void store4(int64_t m, int64_t n, f32x4 v, int cnt) const {
    put4<T>(C + m * ldc + n, v, cnt);
  }
};

template <typename T>
EpStore<T> mk_store(void* C, int64_t ld) {
  EpStore<T> e;
  e.C = static_cast<T*>(C);
  e.ldc = ld;
  e.bstride = 0;
  return e;
}
inline EpF32 mk_f32(float* C, int64_t ld, int acc) {
  EpF32 e;
  e.C = C;
  e.ldc = ld;
  e.accumulate = acc;
  return e;
}
inline EpPart mk_part(float* part, int64_t M, int64_t N) {
  EpPart e;
  e.C = part;
  e.ldc = N;
  e.stride = M * N;
  return e;
}
inline EpResid mk_resid(const float* R, float* C, int64_t ld) {
  EpResid e;
  e.R = R;
  e.C = C;
  e.ldc = ld;
  return e;
}
template <typename T>
EpRelu2<T> mk_relu2(void* C, int64_t ld, uint32_t* amax = nullptr) {
  EpRelu2<T> e;
  e.C = static_cast<T*>(C);
  e.ldc = ld;
  e.amax = amax;
  return e;
}
template <typename T>
EpRelu2Bwd<T> mk_relu2bwd(const void* H, void* C, int64_t ld, uint32_t* amax = nullptr) {
  EpRelu2Bwd<T> e;
  e.H = static_cast<const T*>(H);
  e.C = static_cast<T*>(C);
  e.ldc = ld;
  e.amax = amax;
  return e;
}
template <typename T>
EpSoftcap<T> mk_softcap(void* C, int64_t ld, float cap) {
  EpSoftcap<T> e;
  e.C = static_cast<T*>(C);
  e.ldc = ld;
  e.cap = cap;
  e.k2 = 2.0f * 1.4426950408889634f / cap;
  return e;
}

// ------------------------------------------------------------ tile loader
struct alignas(16) Vec16 {
  uint32_t w[4];
};

template <typename T, int ROWS, int BK, bool KMAJ>
struct TileLoader {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int NV = ROWS * BK / VEC / 256;
  static_assert(NV >= 1, "tile too small for 256 threads");
  Vec16 raw[NV];
  bool ok[NV];

  __device__ void load(const T* __restrict__ p, int64_t ld, int64_t mn0, int64_t MN,
                       int64_t k0, int64_t K, int tid) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + i * 256;
      int64_t mn, k;
      if (KMAJ) {
        mn = mn0 + v / (BK / VEC);
        k = k0 + (v % (BK / VEC)) * VEC;
      } else {
        k = k0 + v / (ROWS / VEC);
        mn = mn0 + (v % (ROWS / VEC)) * VEC;
      }
      ok[i] = (mn < MN) && (k < K);
      if (ok[i]) {
        const T* src = KMAJ ? p + mn * ld + k : p + k * ld + mn;
        raw[i] = *reinterpret_cast<const Vec16*>(src);
      } else {
        raw[i] = Vec16{{0, 0, 0, 0}};
      }
    }
  }

  template <int LDK, class PRE>
  __device__ void store(T (*lds)[LDK], int64_t mn0, int64_t k0, int tid, const PRE& pre) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + i * 256;
      T* e = reinterpret_cast<T*>(&raw[i]);
      if (PRE::kActive && ok[i]) {
        int64_t mn, k;
        if (KMAJ) {
          mn = mn0 + v / (BK / VEC);
          k = k0 + (v % (BK / VEC)) * VEC;
        } else {
          k = k0 + v / (ROWS / VEC);
          mn = mn0 + (v % (ROWS / VEC)) * VEC;
        }
        float f[VEC];
#pragma unroll
        for (int j = 0; j < VEC; ++j) f[j] = to_f(e[j]);
        pre.template vec<KMAJ, VEC>(f, mn, k);
#pragma unroll
        for (int j = 0; j < VEC; ++j) e[j] = from_f<T>(f[j]);
      }
      if (KMAJ) {
        const int row = v / (BK / VEC), kk = (v % (BK / VEC)) * VEC;
        *reinterpret_cast<Vec16*>(&lds[row][kk]) = raw[i];
      } else {
        const int kk = v / (ROWS / VEC), row = (v % (ROWS / VEC)) * VEC;
#pragma unroll
        for (int j = 0; j < VEC; ++j) lds[row + j][kk] = e[j];
      }
    }
  }
};

// ------------------------------------------------------------ kernel
template <typename T, int BM, int BN, int BK, bool AK, bool BKM, class PA, class PB, class EP>
__global__ __launch_bounds__(256) void gemm_kernel(const T* __restrict__ A, int64_t lda,
                                                   const T* __restrict__ B, int64_t ldb,
                                                   int64_t M, int64_t N, int64_t K, PA pa,
                                                   PB pb, EP ep) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int LDK = BK + VEC;
  constexpr int TM = BM / 64, TN = BN / 64;
  __shared__ T As[2][BM][LDK];
  __shared__ T Bs[2][BN][LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int64_t m0 = (int64_t)blockIdx.y * BM;

  TileLoader<T, BM, BK, AK> la;
  TileLoader<T, BN, BK, BKM> lb;
  pa.init();
  pb.init();

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int64_t nk = (K + BK - 1) / BK;
  la.load(A, lda, m0, M, 0, K, tid);
  lb.load(B, ldb, n0, N, 0, K, tid);
  la.template store<LDK>(As[0], m0, 0, tid, pa);
  lb.template store<LDK>(Bs[0], n0, 0, tid, pb);
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(A, lda, m0, M, (kt + 1) * BK, K, tid);
      lb.load(B, ldb, n0, N, (kt + 1) * BK, K, tid);
    }
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      Frag<T> a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        frag_load(a[i], &As[cur][wm * (BM / 2) + i * 32 + (lane & 31)][ks * 16 + (lane >> 5) * 8]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        frag_load(b[j], &Bs[cur][wn * (BN / 2) + j * 32 + (lane & 31)][ks * 16 + (lane >> 5) * 8]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mfma(acc[i][j], a[i], b[j]);
    }
    if (more) {
      la.template store<LDK>(As[cur ^ 1], m0, (kt + 1) * BK, tid, pa);
      lb.template store<LDK>(Bs[cur ^ 1], n0, (kt + 1) * BK, tid, pb);
    }
    __syncthreads();
  }

  // epilogue
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t m = m0 + wm * (BM / 2) + i * 32 + acc_row(e, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wn * (BN / 2) + j * 32 + (lane & 31);
        if (m < M && n < N) ep(m, n, acc[i][j][e]);
      }
    }
  }
}

template <typename T, bool AK, bool BKM, class PA, class PB, class EP>
void run_f32(const void* A, int64_t lda, const void* B, int64_t ldb, int64_t M, int64_t N,
             int64_t K, PA pa, PB pb, EP ep, hipStream_t s) {
  constexpr int BM = 128, BN = 128, BK = 16;
  dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  GK_LAUNCH((gemm_kernel<T, BM, BN, BK, AK, BKM, PA, PB, EP>), grid, dim3(256), 0, s,
                     static_cast<const T*>(A), lda, static_cast<const T*>(B), ldb, M, N, K, pa,
                     pb, ep);
}

// ------------------------------------------------------------ bf16 dispatch
struct Tile {
  int bm, bn;
};

// Output tile for a product: the largest tile that still gives the 256 CUs
// at least one full wave of workgroups. Short contractions (K <= 1024) with
// 4 to 32 waves of 128 x 128 tiles take those instead: two such workgroups
// share a CU, so one's epilogue overlaps the other's main loop (measured on
// the d12 products with K = 768; the lm_head, with far more tiles, keeps
// the larger tile).
// bf16 products: among the 256-row tiles whose width divides N and that
// give at least one full wave (256 workgroups), the one with the fewest
// waves x tile area (a ragged last wave costs a whole wave); ties go to the
// wider tile. Measured on the d12 shapes (16384 rows, K = 768): N = 3072 runs
// 100 us as 256 x 256 against 111 as 128 x 128, N = 2304 85 us as 256 x 192
// (256 x 256 leaves a quarter wave) against 89, N = 768 35 us as 256 x 192.
// A tile plan's cost: rounds of 256 workgroups x tile area, 256 x 128 tiles
// priced 1.4x per area (they measured about that much slower per flop than
// the wider tiles: d20's 1280-column products, moved from 3 rounds of 256 x
// 256 to 5 of 256 x 128, made the step 5% slower). A tile must divide N,
// except that 256 x 256 tiles may overhang M and N while the padding stays
// under an eighth of the area (the 1664-wide d26 products).
static bool tile_fits(Tile t, int64_t M, int64_t N) {
  if (N % t.bn == 0) return true;
  const int64_t pm = (M + t.bm - 1) / t.bm * t.bm, pn = (N + t.bn - 1) / t.bn * t.bn;
  return t.bm == 256 && t.bn == 256 && pm * pn * 8 <= M * N * 9;
}
static int64_t tile_cost(Tile t, int64_t M, int64_t N) {
  const int64_t tiles = ((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
  return (tiles + 255) / 256 * t.bm * t.bn * (t.bn == 128 ? 7 : 5);
}

static Tile pick_tile_bf16(int64_t M, int64_t N, int64_t K) {
  auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  // 256 x 320 (fewer operand bytes per flop than 256 x 256) where it saves a
  // round: the d20 products with 1280 columns take 2 rounds instead of 2.5
  const Tile cand[4] = {{256, 256}, {256, 192}, {256, 320}, {256, 128}};
  Tile best{0, 0};
  int64_t best_cost = -1;
  for (const Tile& t : cand) {
    if (!tile_fits(t, M, N) || tiles(t.bm, t.bn) < 256) continue;
    const int64_t cost = tile_cost(t, M, N);
    if (best_cost < 0 || cost < best_cost) best = t, best_cost = cost;
  }
  if (best_cost >= 0) return best;
  (void)K;
  if (tiles(256, 128) >= 256) return {256, 128};
  return {128, 128};
}

// fp8 products: 128 x 128 for short contractions with 4-32 waves of such
// tiles, else the largest 256-row tile with enough tiles (measured on the
// d26 shapes before the bf16 rule above).
static Tile pick_tile(int64_t M, int64_t N, int64_t K) {
  auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  if (K <= 1024 && tiles(128, 128) >= 1024 && tiles(128, 128) <= 8192) return {128, 128};
  // otherwise the bf16 rule: the 256-row tile with the least rounds x area
  // (256 x 128 at 1.4x per area; 256 x 256 may overhang by up to an eighth,
  // e.g. the d26 products with 1664 columns: 2 rounds of 256 x 256 against 4
  // of 256 x 128)
  const Tile cand[3] = {{256, 256}, {256, 192}, {256, 128}};
  Tile best{0, 0};
  int64_t best_cost = -1;
  for (const Tile& t : cand) {
    if (!tile_fits(t, M, N) || tiles(t.bm, t.bn) < 256) continue;
    const int64_t cost = tile_cost(t, M, N);
    if (best_cost < 0 || cost < best_cost) best = t, best_cost = cost;
  }
  if (best_cost >= 0) return best;
  if (tiles(256, 128) >= 256) return {256, 128};
  return {128, 128};
}

// Tile for a weight gradient. With a full wave of 256 x 256 tiles or more
// the product runs unsplit and the tile with the fewest tile-area x waves
// wins (the lm_head gradient: 2 waves of 256 x 192 beat 1.5 of 256 x 256).
// Otherwise split-K fills the machine: 256 x 256 where the shape has at
// least 16 of them, else 256 x 192 with as many, 256 x 256 overhanging the
// edges (below), 256 x 128 with at least 16, else 128 x 128 (the 768 x 768
// gradient: 256 x 128 x 14 splits on the token-major K-major kernel beat
// 128 x 128 x 14 splits on the register-staged one, d12 +0.3%; on the
// register-staged kernel it had been the other way round, 41 vs 36 us).
static Tile pick_tile_wgrad(int64_t M, int64_t N) {
  auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  if (tiles(256, 256) >= 256) {
    const Tile cand[3] = {{256, 256}, {256, 192}, {256, 128}};
    Tile best = cand[0];
    int64_t best_cost = -1;
    for (const Tile& t : cand) {
      if (!tile_fits(t, M, N)) continue;
      const int64_t cost = tile_cost(t, M, N);
      if (best_cost < 0 || cost < best_cost) best = t, best_cost = cost;
    }
    return best;
  }
  if (M % 256 == 0 && N % 256 == 0 && tiles(256, 256) >= 16) return {256, 256};
  if (N % 192 == 0 && tiles(256, 192) >= 16) return {256, 192};
  // ragged edges: 256 x 256 tiles while their padding costs at most an
  // eighth of the area (the d26 gradients with 1664-wide sides: 4992 x 1664
  // pads 10.5%, 6656 x 1664 7.7%), the narrower tile being the slower one
  if (tiles(256, 256) >= 16 && tiles(256, 256) * 65536 * 8 <= M * N * 9) return {256, 256};
  if (tiles(256, 128) >= 16) return {256, 128};
  return {128, 128};
}

// ------------------------------------------------------------ split-K
// Long contractions over few output tiles are split along K for about one
// workgroup per CU (256; two for 128 x 128 tiles, which fit two to a CU).
// Each split writes its own fp32 partial of C and
// splitk_reduce_kernel adds the partials in split order, so the result does
// not depend on the order the workgroups run in. Chunks are multiples of
// `unit` and at least `min_chunk` long.
struct KSplit {
  int64_t chunk, splits;
};
static KSplit plan_split(int64_t tiles, int64_t K, int64_t unit, int64_t min_chunk,
                         int64_t target = 256) {
  const int64_t want = std::max<int64_t>(1, (target + tiles / 2) / tiles);
  int64_t chunk = std::max<int64_t>((K + want - 1) / want, min_chunk);
  chunk = std::min<int64_t>((chunk + unit - 1) / unit * unit, (K + unit - 1) / unit * unit);
  return {chunk, (K + chunk - 1) / chunk};
}
static int64_t tile_count(Tile t, int64_t M, int64_t N) {
  return ((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
}

// C (+)= sum over s of part[s], s ascending; n4 = M * N / 4 vectors.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int64_t splits, int64_t n4,
                                                            float* __restrict__ C,
                                                            int accumulate) {
  const f32x4* P = reinterpret_cast<const f32x4*>(part);
  f32x4* Cv = reinterpret_cast<f32x4*>(C);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * 256) {
    f32x4 v = accumulate ? Cv[i] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
    for (int64_t sp = 0; sp < splits; ++sp) v += P[sp * n4 + i];
    Cv[i] = v;
  }
}

static void splitk_reduce(const float* part, int64_t splits, int64_t M, int64_t N, float* C,
                          bool accumulate, hipStream_t s) {
  const int64_t n4 = M * N / 4;  // N is a multiple of 64
  const unsigned blocks = (unsigned)std::min<int64_t>((n4 + 255) / 256, 4096);
  GK_LAUNCH(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, part, splits, n4, C,
                     accumulate ? 1 : 0);
}

// The partial region is sized by the plan from the *_part_bytes functions
// (and the entry point checks that before enqueueing anything); a product
// that would still need more is not launched: the call's launch state
// records an error, so no later launch is enqueued and the entry point
// returns GPT_E_HIP.
static bool check_part(int64_t need, int64_t cap) {
  if (need <= cap) return true;
  ::gpt::launch_state().err = hipErrorInvalidValue;
  return false;
}

// Epilogues that fit 256 registers with 256 x 320 tiles (all but ReLU²).
template <class EP>
struct WideEp : std::true_type {};
template <typename T>
struct WideEp<EpRelu2<T>> : std::false_type {};
template <typename T>
struct WideEp<EpRelu2Bwd<T>> : std::false_type {};

// Products with 256-row tiles run 8 wavefronts per workgroup (two per SIMD,
// measured 4-10% faster than 4 on the d12 products); the others 4.
template <int BM, int BN, bool AK, bool BKM, class PA, class PB, class EP>
void launch_bf16(const void* A, int64_t lda, const void* B, int64_t ldb, int64_t M, int64_t N,
                 int64_t K, int64_t kchunk, PA pa, PB pb, EP ep, hipStream_t s, int batch = 1,
                 int64_t sA = 0, int64_t sB = 0) {
  // 256 x 320 tiles exist only on the K-major kernel, and not for the ReLU²
  // epilogues (with their 160-column wavefront tiles those exceed 256
  // registers); anything else takes 256 x 256 tiles instead
  if constexpr (BN == 320 && !(AK && BKM && !PA::kActive && !PB::kActive && WideEp<EP>::value)) {
    launch_bf16<256, 256, AK, BKM>(A, lda, B, ldb, M, N, K, kchunk, pa, pb, ep, s, batch, sA, sB);
  } else {
  if constexpr (BN == 320) {
    if (K % 64 != 0 || (kchunk < K && kchunk % 64 != 0)) {
      launch_bf16<256, 256, AK, BKM>(A, lda, B, ldb, M, N, K, kchunk, pa, pb, ep, s, batch, sA, sB);
      return;
    }
  }
  const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
  const int splits = K > 0 && kchunk > 0 ? (int)((K + kchunk - 1) / kchunk) : 1;
  // padded to a multiple of 8: see the kernel's tile order; y: batch entries
  dim3 grid((unsigned)((tm * tn * splits + 7) / 8 * 8), (unsigned)batch);
  if constexpr (BM == 256 && AK && BKM && !PA::kActive && !PB::kActive) {
    if (K % 64 == 0 && (splits == 1 || kchunk % 64 == 0)) {
      GK_LAUNCH((gemm_kmaj_kernel<BN, EP>), grid, dim3(512), 0, s,
                         static_cast<const bf16*>(A), lda, static_cast<const bf16*>(B), ldb, M, N,
                         K, splits == 1 ? K : kchunk, tm, tn, ep, sA, sB);
      return;
    }
  }
  // both operands token-major (the weight gradients): the same kernel with
  // padded row-major stages and transposing fragment reads; the direct fills
  // move 16 aligned bytes along M or N
  if constexpr (BM == 256 && BN != 320 && !AK && !BKM && !PA::kActive && !PB::kActive) {
    const bool aligned16 = ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) & 15) == 0;
    if (K % 64 == 0 && (splits == 1 || kchunk % 64 == 0) && M >= 8 && N >= 8 && M % 8 == 0 &&
        N % 8 == 0 && lda % 8 == 0 && ldb % 8 == 0 && sA % 8 == 0 && sB % 8 == 0 && aligned16) {
      GK_LAUNCH((gemm_kmaj_kernel<BN, EP, 0, NoDeq, true>), grid, dim3(512), 0, s,
                static_cast<const bf16*>(A), lda, static_cast<const bf16*>(B), ldb, M, N, K,
                splits == 1 ? K : kchunk, tm, tn, ep, sA, sB);
      return;
    }
  }
  constexpr int NW = BM == 256 ? 8 : 4;
  if constexpr (BN != 320)
  GK_LAUNCH((gemm_bf16_kernel<BM, BN, 64, AK, BKM, 0, PA, PB, EP, NoDeq, NW>), grid,
                     dim3(64 * NW), 0, s, static_cast<const bf16*>(A), lda,
                     static_cast<const bf16*>(B), ldb, M, N, K, kchunk, tm, tn, pa, pb, ep, NoDeq{},
                     sA, sB);
  }
}

template <bool AK, bool BKM, class PA, class PB, class EP>
void run_bf16(Tile t, const void* A, int64_t lda, const void* B, int64_t ldb, int64_t M, int64_t N,
              int64_t K, int64_t kchunk, PA pa, PB pb, EP ep, hipStream_t s, int batch = 1,
              int64_t sA = 0, int64_t sB = 0) {
  if (t.bm == 256 && t.bn == 256)
    launch_bf16<256, 256, AK, BKM>(A, lda, B, ldb, M, N, K, kchunk, pa, pb, ep, s, batch, sA, sB);
  else if (t.bm == 256 && t.bn == 320)
    launch_bf16<256, 320, AK, BKM>(A, lda, B, ldb, M, N, K, kchunk, pa, pb, ep, s, batch, sA, sB);
  else if (t.bm == 256 && t.bn == 192)
    launch_bf16<256, 192, AK, BKM>(A, lda, B, ldb, M, N, K, kchunk, pa, pb, ep, s, batch, sA, sB);
  else if (t.bm == 256 && t.bn == 128)
    launch_bf16<256, 128, AK, BKM>(A, lda, B, ldb, M, N, K, kchunk, pa, pb, ep, s, batch, sA, sB);
  else
    launch_bf16<128, 128, AK, BKM>(A, lda, B, ldb, M, N, K, kchunk, pa, pb, ep, s, batch, sA, sB);
}

// Tile of a batched product: the bf16 rule applied to the whole batch's
// tile count (a batch of small products fills the machine together).
static Tile pick_tile_batched(int batch, int64_t M, int64_t N) {
  auto tiles = [&](int bm, int bn) { return batch * ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  if (N % 256 == 0 && tiles(256, 256) >= 256) return {256, 256};
  if (N % 192 == 0 && tiles(256, 192) >= 256) return {256, 192};
  if (tiles(256, 128) >= 256) return {256, 128};
  return {128, 128};
}

// ------------------------------------------------------------ fp8 dispatch
// fp8 operands go through the same kernel as 2-byte units (a pair of codes
// per unit), so K, the leading dimensions and the K chunk are halved.
template <int BM, int BN, int MODE, class EP>
void launch_f8(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, int64_t M, int64_t N,
               int64_t K, int64_t kchunk, EP ep, const Deq8& dq, hipStream_t s) {
  const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
  const int64_t Kp = K / 2, kc = kchunk / 2;
  const int splits = Kp > 0 && kc > 0 ? (int)((Kp + kc - 1) / kc) : 1;
  dim3 grid((unsigned)((tm * tn * splits + 7) / 8 * 8));  // padded: see the kernel's tile order
  // The K-major kernel's fp8 mode (8 wavefronts, direct fills); its 256-
  // column epilogues stage 8 rows per pass, so those that read an fp32
  // operand fit its 256 registers too.
  constexpr bool kKmaj = BM == 256;
  if constexpr (kKmaj) {
    if (Kp % 64 == 0 && (splits == 1 || kc % 64 == 0)) {
      GK_LAUNCH((gemm_kmaj_kernel<BN, EP, MODE, Deq8>), grid, dim3(512), 0, s,
                reinterpret_cast<const bf16*>(A), lda / 2, reinterpret_cast<const bf16*>(B),
                ldb / 2, M, N, Kp, splits == 1 ? Kp : kc, tm, tn, ep, (int64_t)0, (int64_t)0, dq);
      return;
    }
  }
  GK_LAUNCH((gemm_bf16_kernel<BM, BN, 64, true, true, MODE, PreId, PreId, EP, Deq8>), grid,
                     dim3(256), 0, s, reinterpret_cast<const bf16*>(A), lda / 2,
                     reinterpret_cast<const bf16*>(B), ldb / 2, M, N, Kp, kc, tm, tn, PreId{},
                     PreId{}, ep, dq, (int64_t)0, (int64_t)0);
}

// The K-major kernel with scales cut along K (one unsplit launch; K and the
// segment ends multiples of 128 codes, checked by the caller).
template <int BN, int MODE>
void launch_f8_kseg(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, int64_t M,
                    int64_t N, int64_t K, EpF32 ep, const Deq8K& dq, hipStream_t s) {
  const int tm = (int)((M + 255) / 256), tn = (int)((N + BN - 1) / BN);
  GK_LAUNCH((gemm_kmaj_kernel<BN, EpF32, MODE, Deq8K>), dim3((unsigned)((tm * tn + 7) / 8 * 8)),
            dim3(512), 0, s, reinterpret_cast<const bf16*>(A), lda / 2,
            reinterpret_cast<const bf16*>(B), ldb / 2, M, N, K / 2, K / 2, tm, tn, ep, (int64_t)0,
            (int64_t)0, dq);
}

template <int MODE, class EP>
void run_f8(Tile t, const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, int64_t M,
            int64_t N, int64_t K, int64_t kchunk, EP ep, const Deq8& dq, hipStream_t s) {
  if (t.bm == 256 && t.bn == 256)
    launch_f8<256, 256, MODE>(A, lda, B, ldb, M, N, K, kchunk, ep, dq, s);
  else if (t.bm == 256 && t.bn == 192)
    launch_f8<256, 192, MODE>(A, lda, B, ldb, M, N, K, kchunk, ep, dq, s);
  else if (t.bm == 256 && t.bn == 128)
    launch_f8<256, 128, MODE>(A, lda, B, ldb, M, N, K, kchunk, ep, dq, s);
  else
    launch_f8<128, 128, MODE>(A, lda, B, ldb, M, N, K, kchunk, ep, dq, s);
}

}  // namespace gk

namespace gpt {
using namespace gk;

static Deq8 to_deq(const Fp8Deq& q) {
  Deq8 d{};
  d.amax = q.amax;
  d.axis = q.axis;
  d.nseg = q.nseg;
  d.end[0] = q.end[0];
  d.end[1] = q.end[1];
  for (int i = 0; i < 3; ++i) {
    d.sa[i] = q.sa[i < q.nseg ? i : 0];
    d.sb[i] = q.sb[i < q.nseg ? i : 0];
  }
  d.fa = q.fa == FP8_E4M3 ? 448.0f : 57344.0f;
  d.fb = q.fb == FP8_E4M3 ? 448.0f : 57344.0f;
  return d;
}

// MODE of an fp8 product: 1 for e4m3 x e4m3 (forward), 2 for e5m2 x e4m3
// (gradient products).
#define GPT_F8_DISPATCH(dq, call1, call2) \
  do {                                     \
    if ((dq).fa == FP8_E5M2) call2;        \
    else call1;                            \
  } while (0)

void gemm8_store(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                 const uint8_t* B, int64_t ldb, const Fp8Deq& dq, void* C, hipStream_t s) {
  const Tile t = pick_tile(M, N, K);
  const Deq8 q = to_deq(dq);
  GPT_F8_DISPATCH(dq, (run_f8<1>(t, A, lda, B, ldb, M, N, K, K, mk_store<bf16>(C, N), q, s)),
                  (run_f8<2>(t, A, lda, B, ldb, M, N, K, K, mk_store<bf16>(C, N), q, s)));
}

void gemm8_resid(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                 const uint8_t* B, int64_t ldb, const Fp8Deq& dq, const float* R, float* C,
                 hipStream_t s) {
  run_f8<1>(pick_tile(M, N, K), A, lda, B, ldb, M, N, K, K, mk_resid(R, C, N), to_deq(dq), s);
}

void gemm8_relu2(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                 const uint8_t* B, int64_t ldb, const Fp8Deq& dq, void* C, uint32_t* amax_c,
                 hipStream_t s) {
  run_f8<1>(pick_tile(M, N, K), A, lda, B, ldb, M, N, K, K, mk_relu2<bf16>(C, N, amax_c),
            to_deq(dq), s);
}

void gemm8_relu2bwd(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                    const uint8_t* B, int64_t ldb, const Fp8Deq& dq, const void* H, void* C,
                    uint32_t* amax_c, hipStream_t s) {
  run_f8<2>(pick_tile(M, N, K), A, lda, B, ldb, M, N, K, K, mk_relu2bwd<bf16>(H, C, N, amax_c),
            to_deq(dq), s);
}

void gemm8_f32(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
               const uint8_t* B, int64_t ldb, const Fp8Deq& dq, float* C, bool accumulate,
               hipStream_t s) {
  run_f8<2>(pick_tile(M, N, K), A, lda, B, ldb, M, N, K, K, mk_f32(C, N, accumulate ? 1 : 0),
            to_deq(dq), s);
}

// An fp8 product with scales that change along K (the q, k and v segments
// of the attention input gradient's contraction, each with its own
// output-gradient and weight scale): one launch of the K-major kernel,
// which rescales its accumulators where a segment ends, when the tile is
// 256 rows, not 256 columns (those fp32 epilogues run on the 4-wavefront
// kernel), K and the segment ends are multiples of 128 codes; otherwise one
// accumulating product per segment.
SplitSum gemm8_product(bool wgrad, int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                       const uint8_t* B, int64_t ldb, const Fp8Deq& dq, float* C, bool accumulate,
                       float* part, int64_t part_cap, hipStream_t s);

static bool f8_kseg_fused(int64_t M, int64_t N, int64_t K, const Fp8Deq& dq) {
  const Tile t = pick_tile(M, N, K);
  if (t.bm != 256 || (t.bn != 256 && t.bn != 192 && t.bn != 128) || K % 128) return false;
  for (int i = 0; i + 1 < dq.nseg; ++i)
    if (dq.end[i] % 128 || dq.end[i] > K) return false;
  return true;
}

void gemm8_f32_kseg(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                    const uint8_t* B, int64_t ldb, const Fp8Deq& dq, float* C, bool accumulate,
                    hipStream_t s) {
  if (f8_kseg_fused(M, N, K, dq)) {
    Deq8K q;
    static_cast<Deq8&>(q) = to_deq(dq);
    q.axis = 2;
    const EpF32 ep = mk_f32(C, N, accumulate ? 1 : 0);
    const Tile t = pick_tile(M, N, K);
    if (t.bn == 256)
      GPT_F8_DISPATCH(dq, (launch_f8_kseg<256, 1>(A, lda, B, ldb, M, N, K, ep, q, s)),
                      (launch_f8_kseg<256, 2>(A, lda, B, ldb, M, N, K, ep, q, s)));
    else if (t.bn == 192)
      GPT_F8_DISPATCH(dq, (launch_f8_kseg<192, 1>(A, lda, B, ldb, M, N, K, ep, q, s)),
                      (launch_f8_kseg<192, 2>(A, lda, B, ldb, M, N, K, ep, q, s)));
    else
      GPT_F8_DISPATCH(dq, (launch_f8_kseg<128, 1>(A, lda, B, ldb, M, N, K, ep, q, s)),
                      (launch_f8_kseg<128, 2>(A, lda, B, ldb, M, N, K, ep, q, s)));
    return;
  }
  int64_t k0 = 0;
  bool first = true;
  for (int i = 0; i < dq.nseg; ++i) {
    const int64_t k1 = i + 1 < dq.nseg ? std::min<int64_t>(dq.end[i], K) : K;
    if (k1 > k0) {
      Fp8Deq one = dq;
      one.axis = 0;
      one.nseg = 1;
      one.sa[0] = dq.sa[i];
      one.sb[0] = dq.sb[i];
      gemm8_product(false, M, N, k1 - k0, A + k0, lda, B + k0, ldb, one, C, accumulate || !first,
                    nullptr, 0, s);
      first = false;
    }
    k0 = std::max(k0, k1);
  }
}

// An fp8 product with an fp32 output on the step's code paths: the plain
// product (format of A picks e4m3 x e4m3 or e5m2 x e4m3), or the
// weight-gradient product (split-K partials, then the fixed-order sum).
SplitSum gemm8_product(bool wgrad, int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                       const uint8_t* B, int64_t ldb, const Fp8Deq& dq, float* C, bool accumulate,
                       float* part, int64_t part_cap, hipStream_t s);

static int64_t wgrad_target(Tile t) { return t.bm == 128 ? 512 : 256; }

// K splits of an fp8 weight gradient (K in codes, chunks multiples of 128):
// the count s in 1..8 with the least modelled time, where a split product
// takes ceil(tiles * s / 256) waves of one workgroup per CU, each as long as
// its chunk, and every split beyond one adds an fp32 partial of C written
// and read back. Work is priced in MFMA flops at ~40% of a CU's fp8 rate
// (7.8 TFLOP/s, as measured in these products) against partial bytes at
// ~5 TB/s of HBM: 1.56 flops per byte. (A 6656 x 1664 gradient over 16,384
// tokens: 338 tiles of 256 x 128 take 2 waves unsplit, 4 waves of a third
// of K in 3 splits.)
static KSplit f8_wgrad_split(int64_t M, int64_t N, int64_t K) {
  const Tile t = pick_tile_wgrad(M, N);
  const int64_t tiles = tile_count(t, M, N);
  const int64_t units = (K + 127) / 128;
  KSplit best{K, 1};
  double best_cost = -1.0;
  for (int64_t sp = 1; sp <= 8 && sp <= units; ++sp) {
    const int64_t chunk = (units + sp - 1) / sp * 128;
    const int64_t splits = (K + chunk - 1) / chunk;
    if (splits != sp) continue;
    const double waves = (double)((tiles * splits + 255) / 256);
    double cost = waves * (double)chunk * t.bm * t.bn * 2.0;
    if (splits > 1) cost += 1.56 * (double)splits * M * N * 8.0;
    if (best_cost < 0 || cost < best_cost) best = KSplit{splits > 1 ? chunk : K, splits}, best_cost = cost;
  }
  return best;
}
int64_t part_bytes_f8_wgrad(int64_t M, int64_t N, int64_t K) {
  const KSplit ks = f8_wgrad_split(M, N, K);
  return ks.splits > 1 ? ks.splits * M * N * 4 : 0;
}

SplitSum gemm8_wgrad(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                     const uint8_t* B, int64_t ldb, const Fp8Deq& dq, float* C, bool accumulate,
                     float* part, int64_t part_cap, hipStream_t s) {
  const Tile t = pick_tile_wgrad(M, N);
  const KSplit ks = f8_wgrad_split(M, N, K);
  const Deq8 q = to_deq(dq);
  if (ks.splits == 1) {
    run_f8<2>(t, A, lda, B, ldb, M, N, K, K, mk_f32(C, N, accumulate ? 1 : 0), q, s);
    return SplitSum{};
  }
  if (!check_part(part_bytes_f8_wgrad(M, N, K), part_cap)) return SplitSum{};
  run_f8<2>(t, A, lda, B, ldb, M, N, K, ks.chunk, mk_part(part, M, N), q, s);
  return SplitSum{part, ks.splits, M, N, C, accumulate};
}

SplitSum gemm8_product(bool wgrad, int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                       const uint8_t* B, int64_t ldb, const Fp8Deq& dq, float* C, bool accumulate,
                       float* part, int64_t part_cap, hipStream_t s) {
  if (wgrad) return gemm8_wgrad(M, N, K, A, lda, B, ldb, dq, C, accumulate, part, part_cap, s);
  const Tile t = pick_tile(M, N, K);
  const Deq8 q = to_deq(dq);
  const EpF32 ep = mk_f32(C, N, accumulate ? 1 : 0);
  GPT_F8_DISPATCH(dq, (run_f8<1>(t, A, lda, B, ldb, M, N, K, K, ep, q, s)),
                  (run_f8<2>(t, A, lda, B, ldb, M, N, K, K, ep, q, s)));
  return SplitSum{};
}

void gemm_nt_store(const Dims& d, int64_t M, int N, int K, const void* A, const void* B,
                   void* C, hipStream_t s) {
  if (d.bf16)
    run_bf16<true, true>(pick_tile_bf16(M, N, K), A, K, B, K, M, N, K, K, PreId{}, PreId{},
                         mk_store<bf16>(C, N), s);
  else
    run_f32<float, true, true>(A, K, B, K, M, N, K, PreId{}, PreId{},
                               mk_store<float>(C, N), s);
}

void gemm_nt_resid(const Dims& d, int64_t M, int N, int K, const void* A, const void* B,
                   const float* R, float* C, hipStream_t s) {
  if (d.bf16)
    run_bf16<true, true>(pick_tile_bf16(M, N, K), A, K, B, K, M, N, K, K, PreId{}, PreId{},
                         mk_resid(R, C, N), s);
  else
    run_f32<float, true, true>(A, K, B, K, M, N, K, PreId{}, PreId{}, mk_resid(R, C, N), s);
}

void gemm_nt_relu2(const Dims& d, int64_t M, int N, int K, const void* A, const void* B, void* C,
                   hipStream_t s) {
  if (d.bf16)
    run_bf16<true, true>(pick_tile_bf16(M, N, K), A, K, B, K, M, N, K, K, PreId{}, PreId{},
                         mk_relu2<bf16>(C, N), s);
  else
    run_f32<float, true, true>(A, K, B, K, M, N, K, PreId{}, PreId{}, mk_relu2<float>(C, N), s);
}

void gemm_nt_softcap(const Dims& d, int64_t M, int N, int K, const void* A, const void* B,
                     void* C, hipStream_t s) {
  if (d.bf16)
    run_bf16<true, true>(pick_tile_bf16(M, N, K), A, K, B, K, M, N, K, K, PreId{}, PreId{},
                         mk_softcap<bf16>(C, N, d.cap), s);
  else
    run_f32<float, true, true>(A, K, B, K, M, N, K, PreId{}, PreId{},
                               mk_softcap<float>(C, N, d.cap), s);
}

void gemm_nn_store(const Dims& d, int64_t M, int N, int K, const void* A, const void* B,
                   void* C, hipStream_t s, const void* Bt) {
  if (d.bf16 && Bt)
    run_bf16<true, true>(pick_tile_bf16(M, N, K), A, K, Bt, K, M, N, K, K, PreId{}, PreId{},
                         mk_store<bf16>(C, N), s);
  else if (d.bf16)
    run_bf16<true, false>(pick_tile_bf16(M, N, K), A, K, B, N, M, N, K, K, PreId{}, PreId{},
                          mk_store<bf16>(C, N), s);
  else
    run_f32<float, true, false>(A, K, B, N, M, N, K, PreId{}, PreId{},
                                mk_store<float>(C, N), s);
}

void gemm_nn_f32(const Dims& d, int64_t M, int N, int K, const void* A, const void* B,
                 float* C, hipStream_t s, const void* Bt) {
  if (d.bf16 && Bt)
    run_bf16<true, true>(pick_tile_bf16(M, N, K), A, K, Bt, K, M, N, K, K, PreId{}, PreId{},
                         mk_f32(C, N, 0), s);
  else if (d.bf16)
    run_bf16<true, false>(pick_tile_bf16(M, N, K), A, K, B, N, M, N, K, K, PreId{}, PreId{},
                          mk_f32(C, N, 0), s);
  else
    run_f32<float, true, false>(A, K, B, N, M, N, K, PreId{}, PreId{}, mk_f32(C, N, 0), s);
}

void gemm_nn_relu2bwd(const Dims& d, int64_t M, int N, int K, const void* A, const void* B,
                      const void* U, void* C, hipStream_t s, const void* Bt) {
  if (d.bf16 && Bt)
    run_bf16<true, true>(pick_tile_bf16(M, N, K), A, K, Bt, K, M, N, K, K, PreId{}, PreId{},
                         mk_relu2bwd<bf16>(U, C, N), s);
  else if (d.bf16)
    run_bf16<true, false>(pick_tile_bf16(M, N, K), A, K, B, N, M, N, K, K, PreId{}, PreId{},
                          mk_relu2bwd<bf16>(U, C, N), s);
  else
    run_f32<float, true, false>(
        A, K, B, N, M, N, K, PreId{}, PreId{},
        mk_relu2bwd<float>(U, C, N), s);
}

static KSplit nn_split(int64_t M, int64_t N, int64_t K) {
  return plan_split(tile_count(pick_tile_bf16(M, N, K), M, N), K, 64, 4096);
}
int64_t part_bytes_nn_splitk(const Dims& d, int64_t M, int64_t N, int64_t K) {
  if (!d.bf16) return 0;
  const KSplit ks = nn_split(M, N, K);
  return ks.splits > 1 ? ks.splits * M * N * 4 : 0;
}

SplitSum gemm_nn_f32_splitk(const Dims& d, int64_t M, int N, int K, const void* A,
                            const void* B, float* C, float* part, int64_t part_cap,
                            hipStream_t s, const void* Bt) {
  if (d.bf16) {
    const Tile t = pick_tile_bf16(M, N, K);
    const KSplit ks = nn_split(M, N, K);
    const int64_t chunk = ks.splits == 1 ? K : ks.chunk;
    if (ks.splits > 1 && !check_part(part_bytes_nn_splitk(d, M, N, K), part_cap)) return SplitSum{};
    if (Bt) {
      if (ks.splits == 1)
        run_bf16<true, true>(t, A, K, Bt, K, M, N, K, chunk, PreId{}, PreId{}, mk_f32(C, N, 0), s);
      else
        run_bf16<true, true>(t, A, K, Bt, K, M, N, K, chunk, PreId{}, PreId{}, mk_part(part, M, N),
                             s);
    } else {
      if (ks.splits == 1)
        run_bf16<true, false>(t, A, K, B, N, M, N, K, chunk, PreId{}, PreId{}, mk_f32(C, N, 0), s);
      else
        run_bf16<true, false>(t, A, K, B, N, M, N, K, chunk, PreId{}, PreId{}, mk_part(part, M, N),
                              s);
    }
    if (ks.splits == 1) return SplitSum{};
    return SplitSum{part, ks.splits, M, N, C, false};
  }
  run_f32<float, true, false>(A, K, B, N, M, N, K, PreId{}, PreId{}, mk_f32(C, N, 0), s);
  return SplitSum{};
}

// K splits of a bf16 weight gradient (chunks multiples of 64, at least 512
// long): the count s with the least modelled time, where the split product
// takes ceil(tiles * s / slots) rounds of workgroups (slots: 256, or 512 for
// 128 x 128 tiles, two to a CU), each as long as its chunk, and every split
// beyond one adds an fp32 partial of C written and read back. Work is priced
// in MFMA flops per CU (~3.9 TFLOP/s in these products) against partial
// bytes at ~5 TB/s of HBM: 0.8 flops per byte. Rounding 256 / tiles to the
// nearest count instead can spill a few workgroups into a second round (a
// 1280 x 768 gradient over 32,768 tokens: 13 splits of 20 tiles = 260
// workgroups; 5120 x 1280: 3 splits of 100 tiles = 300).
static KSplit tn_split(int64_t M, int64_t N, int64_t K) {
  const Tile t = pick_tile_wgrad(M, N);
  const int64_t tiles = tile_count(t, M, N), slots = wgrad_target(t);
  const int64_t units = (K + 63) / 64;
  KSplit best{K, 1};
  double best_cost = -1.0;
  for (int64_t sp = 1; sp <= 64 && sp <= units; ++sp) {
    const int64_t chunk = (units + sp - 1) / sp * 64;
    if (sp > 1 && chunk < 512) break;
    const int64_t splits = (K + chunk - 1) / chunk;
    if (splits != sp) continue;
    const double rounds = (double)((tiles * splits + slots - 1) / slots);
    double cost = rounds * (double)chunk * t.bm * t.bn * 2.0 * ((double)slots / 256.0);
    if (splits > 1) cost += 0.8 * (double)splits * M * N * 8.0;
    if (best_cost < 0 || cost < best_cost) best = KSplit{splits > 1 ? chunk : K, splits}, best_cost = cost;
  }
  return best;
}
int64_t part_bytes_tn_wgrad(const Dims& d, int64_t M, int64_t N, int64_t K) {
  if (!d.bf16) return 0;
  const KSplit ks = tn_split(M, N, K);
  return ks.splits > 1 ? ks.splits * M * N * 4 : 0;
}

SplitSum gemm_tn_wgrad(const Dims& d, int M, int N, int64_t K, const void* A, const void* B,
                       float* C, bool accumulate, float* part, int64_t part_cap, hipStream_t s) {
  if (d.bf16) {
    const Tile t = pick_tile_wgrad(M, N);
    const KSplit ks = tn_split(M, N, K);
    if (ks.splits == 1) {  // one split: plain (accumulating) stores
      run_bf16<false, false>(t, A, M, B, N, M, N, K, K, PreId{}, PreId{},
                             mk_f32(C, N, accumulate ? 1 : 0), s);
      return SplitSum{};
    }
    if (!check_part(part_bytes_tn_wgrad(d, M, N, K), part_cap)) return SplitSum{};
    run_bf16<false, false>(t, A, M, B, N, M, N, K, ks.chunk, PreId{}, PreId{},
                           mk_part(part, M, N), s);
    return SplitSum{part, ks.splits, M, N, C, accumulate};
  }
  run_f32<float, false, false>(A, M, B, N, M, N, K, PreId{}, PreId{},
                               mk_f32(C, N, accumulate ? 1 : 0), s);
  return SplitSum{};
}

void splitk_sum(const SplitSum& r, hipStream_t s) {
  if (r.splits > 1) splitk_reduce(r.part, r.splits, r.M, r.N, r.C, r.accumulate, s);
}

}  // namespace gpt

namespace gpt {
using namespace gk;

void gemm_nt_store_batched(const Dims& d, int batch, int64_t M, int N, int K, const void* A,
                           int64_t sA, const void* B, int64_t sB, void* C, int64_t sC,
                           hipStream_t s) {
  if (d.bf16) {
    EpStore<bf16> ep = mk_store<bf16>(C, N);
    ep.bstride = sC;
    run_bf16<true, true>(pick_tile_batched(batch, M, N), A, K, B, K, M, N, K, K, PreId{},
                         PreId{}, ep, s, batch, sA, sB);
  } else {
    const size_t A4 = 4;
    for (int b = 0; b < batch; ++b)
      gemm_nt_store(d, M, N, K, static_cast<const char*>(A) + b * sA * A4,
                    static_cast<const char*>(B) + b * sB * A4, static_cast<char*>(C) + b * sC * A4,
                    s);
  }
}

void gemm_nn_store_batched(const Dims& d, int batch, int64_t M, int N, int K, const void* A,
                           int64_t sA, const void* B, int64_t sB, void* C, int64_t sC,
                           hipStream_t s) {
  if (d.bf16) {
    EpStore<bf16> ep = mk_store<bf16>(C, N);
    ep.bstride = sC;
    run_bf16<true, false>(pick_tile_batched(batch, M, N), A, K, B, N, M, N, K, K, PreId{},
                          PreId{}, ep, s, batch, sA, sB);
  } else {
    const size_t A4 = 4;
    for (int b = 0; b < batch; ++b)
      gemm_nn_store(d, M, N, K, static_cast<const char*>(A) + b * sA * A4,
                    static_cast<const char*>(B) + b * sB * A4, static_cast<char*>(C) + b * sC * A4,
                    s);
  }
}

}  // namespace gpt

namespace gpt {
using namespace gk;

template <typename T>
static EpLin<T> mk_lin(const void* R, void* C, int64_t ld, int64_t bstride, float alpha,
                       float beta) {
  EpLin<T> e;
  e.R = static_cast<const T*>(R);
  e.C = static_cast<T*>(C);
  e.ldc = ld;
  e.bstride = bstride;
  e.alpha = alpha;
  e.beta = beta;
  return e;
}

void gemm_lin_batched(const Dims& d, bool nn, int batch, int64_t M, int N, int K, const void* A,
                      int64_t sA, const void* B, int64_t sB, const void* R, void* C, int64_t sC,
                      float alpha, float beta, hipStream_t s) {
  if (d.bf16) {
    const EpLin<bf16> ep = mk_lin<bf16>(R, C, N, sC, alpha, beta);
    if (nn)
      run_bf16<true, false>(pick_tile_batched(batch, M, N), A, K, B, N, M, N, K, K, PreId{},
                            PreId{}, ep, s, batch, sA, sB);
    else
      run_bf16<true, true>(pick_tile_batched(batch, M, N), A, K, B, K, M, N, K, K, PreId{},
                           PreId{}, ep, s, batch, sA, sB);
    return;
  }
  for (int b = 0; b < batch; ++b) {  // fp32: one product per entry
    const float* Ab = static_cast<const float*>(A) + b * sA;
    const float* Bb = static_cast<const float*>(B) + b * sB;
    const EpLin<float> ep = mk_lin<float>(static_cast<const float*>(R) + b * sC,
                                          static_cast<float*>(C) + b * sC, N, 0, alpha, beta);
    if (nn)
      run_f32<float, true, false>(Ab, K, Bb, N, M, N, K, PreId{}, PreId{}, ep, s);
    else
      run_f32<float, true, true>(Ab, K, Bb, K, M, N, K, PreId{}, PreId{}, ep, s);
  }
}

}  // namespace gpt
