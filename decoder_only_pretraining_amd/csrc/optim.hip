// MuonAdamW optimizer step ("NanoChat基础训练报告", optimizer block;
// "Nanochat在nanoGPT之上的新增功能", feature table row on the optimizer and the
// notes on Muon): Muon (momentum, then Newton-Schulz orthogonalisation) on
// the six block linears of every layer, AdamW on everything else.
//
// AdamW is one HBM-bound pass per tensor (p, g, m, v read, p, m, v written).
// Muon runs per group of equal-shaped matrices: a momentum pass that also sums the squares of the
// update in fixed-order workgroup partials, a single-workgroup sum giving
// 1 / (||u||_F + 1e-7), a pass writing X = u / ||u|| in the compute dtype
// in the wide orientation (rows <= cols; tall matrices transposed), then
// per Newton-Schulz step three products on the GEMM core: A = X X^T, then
// b A + c A A and a X + (b A + c A A) X, the linear combinations formed in
// the product epilogues (A is symmetric, so it serves as its own
// transpose), and a last pass applying
// p <- p (1 - lr wd) - lr sqrt(max(1, rows / cols)) X. One product of a
// block matrix is small (768 x 768 x 768 at d12 fills 36 of 256 CUs), so
// the matrices of equal shape (in the wide orientation) run as one group:
// every pass above is one launch over up to 64 matrices (a table of their
// offsets; the products are batched GEMMs).
#include <hip/hip_runtime.h>

#include <cmath>
#include <utility>

#include "device_common.h"
#include "internal.h"

namespace gk {

// four elements per thread and iteration (16-byte aligned tensors whose
// length is a multiple of 4)
__global__ __launch_bounds__(256) void adamw4_kernel(float* __restrict__ p,
                                                     const float* __restrict__ g,
                                                     float* __restrict__ m, float* __restrict__ v,
                                                     int64_t n4, float lr, float b1, float b2,
                                                     float eps, float c1, float c2) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const f32x4 gi = reinterpret_cast<const f32x4*>(g)[i];
    f32x4 mi = reinterpret_cast<f32x4*>(m)[i], vi = reinterpret_cast<f32x4*>(v)[i];
    f32x4 pi = reinterpret_cast<f32x4*>(p)[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mi[e] = b1 * mi[e] + (1.0f - b1) * gi[e];
      vi[e] = b2 * vi[e] + (1.0f - b2) * gi[e] * gi[e];
      pi[e] -= lr * (mi[e] / c1) / (sqrtf(vi[e] / c2) + eps);
    }
    reinterpret_cast<f32x4*>(m)[i] = mi;
    reinterpret_cast<f32x4*>(v)[i] = vi;
    reinterpret_cast<f32x4*>(p)[i] = pi;
  }
}

__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ p,
                                                    const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v,
                                                    int64_t n, float lr, float b1, float b2,
                                                    float eps, float c1, float c2) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float gi = g[i];
    const float mi = b1 * m[i] + (1.0f - b1) * gi;
    const float vi = b2 * v[i] + (1.0f - b2) * gi * gi;
    m[i] = mi;
    v[i] = vi;
    p[i] -= lr * (mi / c1) / (sqrtf(vi / c2) + eps);
  }
}

// The Muon matrices of one group share their wide shape r x k (r <= k);
// entry y of a launch's table is a matrix: its element offset in params /
// grads / the momentum buffer and whether it is stored tall (k x r).
constexpr int kMaxMats = 64;   // matrices per batched launch
constexpr int kMomBlocks = 64;  // momentum-pass workgroups per matrix
struct MatTable {
  int64_t off[kMaxMats];
  int32_t tall[kMaxMats];
};

// buf <- mu buf + g; per-workgroup partial sums of u^2 (u = g + mu buf,
// Nesterov, or buf) in a fixed order: part[y][blockIdx.x].
__global__ __launch_bounds__(256) void muon_momentum_kernel(const float* __restrict__ g0,
                                                            float* __restrict__ buf0,
                                                            MatTable T, int64_t n, float mu,
                                                            int nesterov,
                                                            float* __restrict__ part) {
  __shared__ float red[256];
  const float* g = g0 + T.off[blockIdx.y];
  float* buf = buf0 + T.off[blockIdx.y];
  float ss = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float gi = g[i];
    const float b = mu * buf[i] + gi;
    buf[i] = b;
    const float u = nesterov ? gi + mu * b : b;
    ss += u * u;
  }
  red[threadIdx.x] = ss;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.y * gridDim.x + blockIdx.x] = red[0];
}

// scal[y] = 1 / (sqrt(sum of matrix y's partials) + 1e-7), one workgroup each
__global__ __launch_bounds__(64) void muon_norm_kernel(const float* __restrict__ part,
                                                       float* __restrict__ scal) {
  double s = part[blockIdx.x * kMomBlocks + threadIdx.x];  // kMomBlocks == 64 lanes
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
  if (threadIdx.x == 0) scal[blockIdx.x] = (float)(1.0 / (sqrt(s) + 1e-7));
}

// X[y] = u * scal[y] in the wide orientation [r][k] (a tall matrix, stored
// [k][r], is transposed); u recomputed from g and the updated buffer.
template <typename T>
__global__ __launch_bounds__(256) void muon_to_x_kernel(const float* __restrict__ g0,
                                                        const float* __restrict__ buf0,
                                                        MatTable Tb, int r, int k, float mu,
                                                        int nesterov,
                                                        const float* __restrict__ scal,
                                                        T* __restrict__ X0) {
  const int y = blockIdx.y;
  const float* g = g0 + Tb.off[y];
  const float* buf = buf0 + Tb.off[y];
  T* X = X0 + (int64_t)y * r * k;
  const float inv = scal[y];
  if (Tb.tall[y]) {  // stored [k][r]: 64 x 64 tiles through LDS, both sides coalesced
    __shared__ float tile[64][65];
    const int tr = r / 64, tk = k / 64;  // r and k are multiples of 64
    for (int t = blockIdx.x; t < tr * tk; t += gridDim.x) {
      const int a0 = (t / tr) * 64, c0 = (t % tr) * 64;  // stored rows a0.., cols c0..
      for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int64_t i = (int64_t)(a0 + e / 64) * r + c0 + e % 64;
        tile[e / 64][e % 64] = (nesterov ? g[i] + mu * buf[i] : buf[i]) * inv;
      }
      __syncthreads();
      for (int e = threadIdx.x; e < 64 * 64; e += 256)  // X row c0 + e / 64, col a0 + e % 64
        X[(int64_t)(c0 + e / 64) * k + a0 + e % 64] = from_f<T>(tile[e % 64][e / 64]);
      __syncthreads();
    }
    return;
  }
  for (int a = blockIdx.x; a < r; a += gridDim.x)  // stored [r][k], row by row
    for (int c = threadIdx.x; c < k; c += 256) {
      const int64_t i = (int64_t)a * k + c;
      const float u = nesterov ? g[i] + mu * buf[i] : buf[i];
      X[i] = from_f<T>(u * inv);
    }
}

// p <- p * decay - lr * sqrt(max(1, rows / cols)) * X[y] (back in p's layout)
template <typename T>
__global__ __launch_bounds__(256) void muon_apply_kernel(float* __restrict__ p0,
                                                         const T* __restrict__ X0, MatTable Tb,
                                                         int r, int k, float decay, float lr) {
  const int y = blockIdx.y;
  float* p = p0 + Tb.off[y];
  const T* X = X0 + (int64_t)y * r * k;
  if (Tb.tall[y]) {  // p stored [k][r], X [r][k]: 64 x 64 tiles through LDS
    __shared__ float tile[64][65];
    const float step = lr * sqrtf((float)k / (float)r);
    const int tr = r / 64, tk = k / 64;
    for (int t = blockIdx.x; t < tr * tk; t += gridDim.x) {
      const int a0 = (t / tr) * 64, c0 = (t % tr) * 64;
      for (int e = threadIdx.x; e < 64 * 64; e += 256)  // X rows c0.., cols a0..
        tile[e / 64][e % 64] = to_f(X[(int64_t)(c0 + e / 64) * k + a0 + e % 64]);
      __syncthreads();
      for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int64_t i = (int64_t)(a0 + e / 64) * r + c0 + e % 64;
        p[i] = p[i] * decay - step * tile[e % 64][e / 64];
      }
      __syncthreads();
    }
    return;
  }
  for (int a = blockIdx.x; a < r; a += gridDim.x)
    for (int c = threadIdx.x; c < k; c += 256) {
      const int64_t i = (int64_t)a * k + c;
      p[i] = p[i] * decay - lr * to_f(X[i]);
    }
}

}  // namespace gk

namespace gpt {

static unsigned ew_blocks(int64_t n) {
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 4096));
}

std::vector<MuonGroup> muon_groups(const gpt_config& c) {
  std::vector<MuonGroup> out;
  for (const auto& t : param_layout(c)) {
    const size_t dot = t.name.find('.');
    if (dot == std::string::npos) continue;
    const std::string leaf = t.name.substr(dot + 1);
    if (!(leaf == "q" || leaf == "k" || leaf == "v" || leaf == "o" || leaf == "fc" || leaf == "mp"))
      continue;
    const int r = (int)std::min(t.rows, t.cols), k = (int)std::max(t.rows, t.cols);
    auto it = std::find_if(out.begin(), out.end(),
                           [&](const MuonGroup& g) { return g.r == r && g.k == k; });
    if (it == out.end()) {
      out.push_back(MuonGroup{r, k, {}, {}});
      it = out.end() - 1;
    }
    it->off.push_back(t.offset);
    it->tall.push_back(t.rows > t.cols ? 1 : 0);
  }
  return out;
}

OptimPlan make_optim_plan(const gpt_config& c) {
  const Dims d = make_dims(c);
  const size_t A = (size_t)d.act_bytes;
  size_t xb = 0, ab = 0;
  for (const auto& g : muon_groups(c)) {
    const size_t nm = std::min<size_t>(g.off.size(), gk::kMaxMats);
    xb = std::max(xb, nm * g.r * g.k * A);
    ab = std::max(ab, nm * g.r * g.r * A);
  }
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  OptimPlan o{};
  size_t off = 0;
  o.part = off;
  off += al((size_t)gk::kMaxMats * gk::kMomBlocks * 4);
  o.scal = off;
  off += al((size_t)gk::kMaxMats * 4);
  o.x = off;
  off += al(xb);
  o.y = off;
  off += al(xb);
  o.a = off;
  off += al(ab);
  o.aa = off;
  off += al(ab);
  o.total = off;
  return o;
}

void launch_adamw(float* p, const float* g, float* m, float* v, int64_t n, float lr, float b1,
                  float b2, float eps, int step, hipStream_t s) {
  const float c1 = 1.0f - std::pow(b1, (float)step), c2 = 1.0f - std::pow(b2, (float)step);
  const bool vec = n % 4 == 0 && ((uintptr_t)p | (uintptr_t)g | (uintptr_t)m | (uintptr_t)v) % 16 == 0;
  if (vec)
    GK_LAUNCH(gk::adamw4_kernel, dim3(ew_blocks(n / 4)), dim3(256), 0, s, p, g, m, v,
                       n / 4, lr, b1, b2, eps, c1, c2);
  else
    GK_LAUNCH(gk::adamw_kernel, dim3(ew_blocks(n)), dim3(256), 0, s, p, g, m, v, n, lr,
                       b1, b2, eps, c1, c2);
}

template <typename T>
static void muon_chunk(const Dims& d, const OptimPlan& o, char* ws, const gk::MatTable& tb,
                       int nm, int r, int k, float* params, const float* grads, float* buf,
                       float lr, float wd, float mu, int nesterov, float a, float b, float c,
                       int steps, hipStream_t s) {
  float* part = reinterpret_cast<float*>(ws + o.part);
  float* scal = reinterpret_cast<float*>(ws + o.scal);
  T* X = reinterpret_cast<T*>(ws + o.x);
  T* Y = reinterpret_cast<T*>(ws + o.y);
  T* Am = reinterpret_cast<T*>(ws + o.a);
  T* AA = reinterpret_cast<T*>(ws + o.aa);
  const int64_t n = (int64_t)r * k, nr = (int64_t)r * r;
  const unsigned per = (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 64));
  GK_LAUNCH(gk::muon_momentum_kernel, dim3(gk::kMomBlocks, nm), dim3(256), 0, s, grads,
                     buf, tb, n, mu, nesterov, part);
  GK_LAUNCH(gk::muon_norm_kernel, dim3(nm), dim3(64), 0, s, part, scal);
  GK_LAUNCH(gk::muon_to_x_kernel<T>, dim3(per, nm), dim3(256), 0, s, grads, buf, tb, r, k,
                     mu, nesterov, scal, X);
  for (int it = 0; it < steps; ++it) {
    gemm_nt_store_batched(d, nm, r, r, k, X, n, X, n, Am, nr, s);  // A = X X^T
    // Bm = b A + c A A (A symmetric: its own transpose), into AA
    gemm_lin_batched(d, false, nm, r, r, r, Am, nr, Am, nr, Am, AA, nr, b, c, s);
    // a X + Bm X, into Y; Y is the next X
    gemm_lin_batched(d, true, nm, r, k, r, AA, nr, X, n, X, Y, n, a, 1.0f, s);
    std::swap(X, Y);
  }
  GK_LAUNCH(gk::muon_apply_kernel<T>, dim3(per, nm), dim3(256), 0, s, params, X, tb, r,
                     k, 1.0f - lr * wd, lr);
}

void launch_muon_groups(const Dims& d, const std::vector<MuonGroup>& groups, const OptimPlan& o,
                        void* workspace, float* params, const float* grads, float* buf, float lr,
                        float wd, float mu, int nesterov, float a, float b, float c, int steps,
                        hipStream_t s) {
  char* ws = static_cast<char*>(workspace);
  for (const auto& g : groups) {
    for (size_t i0 = 0; i0 < g.off.size(); i0 += gk::kMaxMats) {
      const int nm = (int)std::min<size_t>(gk::kMaxMats, g.off.size() - i0);
      gk::MatTable tb{};
      for (int y = 0; y < nm; ++y) {
        tb.off[y] = g.off[i0 + y];
        tb.tall[y] = g.tall[i0 + y];
      }
      if (d.bf16)
        muon_chunk<bf16>(d, o, ws, tb, nm, g.r, g.k, params, grads, buf, lr, wd, mu, nesterov, a,
                         b, c, steps, s);
      else
        muon_chunk<float>(d, o, ws, tb, nm, g.r, g.k, params, grads, buf, lr, wd, mu, nesterov,
                          a, b, c, steps, s);
    }
  }
}

}  // namespace gpt
