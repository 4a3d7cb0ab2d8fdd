// Tiled MFMA GEMM for gfx950: C[M][N] = sum_k A(m,k) * B(n,k), fp32
// accumulation, with fused operand prologues and output epilogues.
//
// Each operand is either contraction-contiguous ("K-major": row m holds k)
// or output-contiguous ("MN-major": row k holds m). Global tiles are read
// with 16-byte vector loads along the contiguous axis and written to LDS in
// a [row][k] layout (MN-major operands are transposed on the LDS write), so
// the MFMA fragment read is one 16-byte LDS load per lane for every layout.
// Two LDS stages: the global loads of tile k+1 are issued before the MFMAs
// of tile k.
#include "device_common.h"
#include "internal.h"

namespace gk {

// ------------------------------------------------------------ prologues
struct PreId {
  static constexpr bool kActive = false;
  __device__ float operator()(float v, int64_t, int64_t) const { return v; }
};
struct PreRelu2 {  // ReLU^2 of the MLP hidden pre-activation
  static constexpr bool kActive = true;
  __device__ float operator()(float v, int64_t, int64_t) const {
    float r = fmaxf(v, 0.0f);
    return r * r;
  }
};
// Gradient of mean cross-entropy through the tanh softcap, from a stored
// softcapped logit c: (exp(c - cap) / rowsum - [v == y]) * (1 - (c/cap)^2) / n_valid.
// |c| <= cap, so exp(c - cap) never overflows and the row sums of
// exp(c - cap) need no running maximum.
struct PreCE {
  static constexpr bool kActive = true;
  const float* inv_rowsum;
  const int32_t* tgt;
  const float* inv_nvalid;
  float cap;
  int token_is_mn;  // 1: operand rows are tokens; 0: operand rows are vocab ids
  __device__ float operator()(float c, int64_t mn, int64_t k) const {
    const int64_t n = token_is_mn ? mn : k;
    const int64_t v = token_is_mn ? k : mn;
    const int y = tgt[n];
    if (y < 0) return 0.0f;
    float p = __expf(c - cap) * inv_rowsum[n];
    if (v == y) p -= 1.0f;
    const float q = c / cap;
    return p * (1.0f - q * q) * inv_nvalid[0];
  }
};

// ------------------------------------------------------------ epilogues
template <typename T>
struct EpStore {
  static constexpr bool kRowSum = false;
  T* C;
  int64_t ldc;
  __device__ float operator()(int64_t m, int64_t n, float v) const {
    C[m * ldc + n] = from_f<T>(v);
    return 0.0f;
  }
};
struct EpF32 {
  static constexpr bool kRowSum = false;
  float* C;
  int64_t ldc;
  int accumulate;
  __device__ float operator()(int64_t m, int64_t n, float v) const {
    float* p = C + m * ldc + n;
    *p = accumulate ? *p + v : v;
    return 0.0f;
  }
};
struct EpResid {  // C = R + acc (residual stream, fp32)
  static constexpr bool kRowSum = false;
  const float* R;
  float* C;
  int64_t ldc;
  __device__ float operator()(int64_t m, int64_t n, float v) const {
    C[m * ldc + n] = R[m * ldc + n] + v;
    return 0.0f;
  }
};
template <typename T>
struct EpRelu2Bwd {  // C = acc * d/du relu(u)^2 = acc * 2 max(u, 0)
  static constexpr bool kRowSum = false;
  const T* U;
  T* C;
  int64_t ldc;
  __device__ float operator()(int64_t m, int64_t n, float v) const {
    const float u = to_f(U[m * ldc + n]);
    C[m * ldc + n] = from_f<T>(u > 0.0f ? 2.0f * u * v : 0.0f);
    return 0.0f;
  }
};
template <typename T>
struct EpSoftcap {  // c = cap * tanh(z / cap), stored; row sums of exp(c - cap)
  static constexpr bool kRowSum = true;
  T* C;
  int64_t ldc;
  float cap;
  float* rowsum;
  __device__ float operator()(int64_t m, int64_t n, float v) const {
    const T c = from_f<T>(cap * tanhf(v / cap));
    C[m * ldc + n] = c;
    return __expf(to_f(c) - cap);
  }
};

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
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          int64_t mn, k;
          if (KMAJ) {
            mn = mn0 + v / (BK / VEC);
            k = k0 + (v % (BK / VEC)) * VEC + j;
          } else {
            k = k0 + v / (ROWS / VEC);
            mn = mn0 + (v % (ROWS / VEC)) * VEC + j;
          }
          e[j] = from_f<T>(pre(to_f(e[j]), mn, k));
        }
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
                                                   PB pb, EP ep, float* rowsum) {
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
      float rs = 0.0f;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wn * (BN / 2) + j * 32 + (lane & 31);
        if (m < M && n < N) rs += ep(m, n, acc[i][j][e]);
      }
      if (EP::kRowSum) {
        rs = half_sum(rs);
        if ((lane & 31) == 0 && m < M) atomicAdd(rowsum + m, rs);
      }
    }
  }
}

template <typename T, bool AK, bool BKM, class PA, class PB, class EP>
void run(const void* A, int64_t lda, const void* B, int64_t ldb, int64_t M, int64_t N,
         int64_t K, PA pa, PB pb, EP ep, float* rowsum, hipStream_t s) {
  constexpr int BM = 128, BN = 128, BK = sizeof(T) == 2 ? 32 : 16;
  dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, BK, AK, BKM, PA, PB, EP>), grid, dim3(256), 0, s,
                     static_cast<const T*>(A), lda, static_cast<const T*>(B), ldb, M, N, K, pa,
                     pb, ep, rowsum);
}

}  // namespace gk

namespace gpt {
using namespace gk;

#define DISPATCH_T(d, ...)        \
  if ((d).bf16) {                 \
    using T = bf16;               \
    __VA_ARGS__;                  \
  } else {                        \
    using T = float;              \
    __VA_ARGS__;                  \
  }

void gemm_nt_store(const Dims& d, int64_t M, int N, int K, const void* A, const void* B,
                   void* C, hipStream_t s) {
  DISPATCH_T(d, (run<T, true, true>(A, K, B, K, M, N, K, PreId{}, PreId{},
                                    EpStore<T>{static_cast<T*>(C), N}, nullptr, s)));
}

void gemm_nt_resid(const Dims& d, int64_t M, int N, int K, const void* A, const void* B,
                   const float* R, float* C, bool relu2_a, hipStream_t s) {
  if (relu2_a) {
    DISPATCH_T(d, (run<T, true, true>(A, K, B, K, M, N, K, PreRelu2{}, PreId{},
                                      EpResid{R, C, N}, nullptr, s)));
  } else {
    DISPATCH_T(d, (run<T, true, true>(A, K, B, K, M, N, K, PreId{}, PreId{},
                                      EpResid{R, C, N}, nullptr, s)));
  }
}

void gemm_nt_softcap(const Dims& d, int64_t M, int N, int K, const void* A, const void* B,
                     void* C, float* rowsum, hipStream_t s) {
  DISPATCH_T(d, (run<T, true, true>(A, K, B, K, M, N, K, PreId{}, PreId{},
                                    EpSoftcap<T>{static_cast<T*>(C), N, d.cap, rowsum}, rowsum,
                                    s)));
}

void gemm_nn_store(const Dims& d, int64_t M, int N, int K, const void* A, const void* B,
                   void* C, hipStream_t s) {
  DISPATCH_T(d, (run<T, true, false>(A, K, B, N, M, N, K, PreId{}, PreId{},
                                     EpStore<T>{static_cast<T*>(C), N}, nullptr, s)));
}

void gemm_nn_f32(const Dims& d, int64_t M, int N, int K, const void* A, const void* B,
                 float* C, hipStream_t s) {
  DISPATCH_T(d, (run<T, true, false>(A, K, B, N, M, N, K, PreId{}, PreId{}, EpF32{C, N, 0},
                                     nullptr, s)));
}

void gemm_nn_relu2bwd(const Dims& d, int64_t M, int N, int K, const void* A, const void* B,
                      const void* U, void* C, hipStream_t s) {
  DISPATCH_T(d, (run<T, true, false>(
                    A, K, B, N, M, N, K, PreId{}, PreId{},
                    EpRelu2Bwd<T>{static_cast<const T*>(U), static_cast<T*>(C), N}, nullptr, s)));
}

void gemm_nn_ce(const Dims& d, int64_t M, int N, int K, const void* logits, const void* B,
                const float* inv_rowsum, const int32_t* tgt, const float* inv_nvalid, float* C,
                hipStream_t s) {
  PreCE pre{inv_rowsum, tgt, inv_nvalid, d.cap, 1};
  DISPATCH_T(d, (run<T, true, false>(logits, K, B, N, M, N, K, pre, PreId{}, EpF32{C, N, 0},
                                     nullptr, s)));
}

void gemm_tn_wgrad(const Dims& d, int M, int N, int64_t K, const void* A, const void* B,
                   float* C, bool accumulate, bool relu2_b, hipStream_t s) {
  if (relu2_b) {
    DISPATCH_T(d, (run<T, false, false>(A, M, B, N, M, N, K, PreId{}, PreRelu2{},
                                        EpF32{C, N, accumulate ? 1 : 0}, nullptr, s)));
  } else {
    DISPATCH_T(d, (run<T, false, false>(A, M, B, N, M, N, K, PreId{}, PreId{},
                                        EpF32{C, N, accumulate ? 1 : 0}, nullptr, s)));
  }
}

void gemm_tn_wgrad_ce(const Dims& d, int M, int N, int64_t K, const void* logits, const void* B,
                      const float* inv_rowsum, const int32_t* tgt, const float* inv_nvalid,
                      float* C, bool accumulate, hipStream_t s) {
  PreCE pre{inv_rowsum, tgt, inv_nvalid, d.cap, 0};
  DISPATCH_T(d, (run<T, false, false>(logits, M, B, N, M, N, K, pre, PreId{},
                                      EpF32{C, N, accumulate ? 1 : 0}, nullptr, s)));
}

}  // namespace gpt
