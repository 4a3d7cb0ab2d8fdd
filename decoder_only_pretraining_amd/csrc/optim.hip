// MuonAdamW optimizer step ("NanoChat基础训练报告", optimizer block;
// "Nanochat在nanoGPT之上的新增功能", feature table row on the optimizer and the
// notes on Muon): Muon (momentum, then Newton-Schulz orthogonalisation) on
// the six block linears of every layer, AdamW on everything else.
//
// AdamW is one HBM-bound pass per tensor (p, g, m, v read, p, m, v written).
// Muon runs per matrix: a momentum pass that also sums the squares of the
// update in fixed-order workgroup partials, a single-workgroup sum giving
// 1 / (||u||_F + 1e-7), a pass writing X = u / ||u|| in the compute dtype
// in the wide orientation (rows <= cols; tall matrices transposed), then
// per Newton-Schulz step three products on the GEMM core (A = X X^T,
// A A, (b A + c A A) X, A being symmetric so it serves as its own
// transpose) and two element-wise passes, and a last pass applying
// p <- p (1 - lr wd) - lr sqrt(max(1, rows / cols)) X. The block matrices
// are small products (768 x 768 x 768 at d12 fills 36 of 256 CUs), so the
// matrices are spread over kOptStreams side streams, each with its own set
// of buffers, forked from and joined back to the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>

#include "device_common.h"
#include "internal.h"

namespace gk {

constexpr int kOptBlocks = 512;  // partial sums of the momentum pass

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

// buf <- mu buf + g; partial sums of u^2, u = g + mu buf (Nesterov) or buf,
// one per workgroup (grid-stride, then a fixed-order reduction in LDS).
__global__ __launch_bounds__(256) void muon_momentum_kernel(const float* __restrict__ g,
                                                            float* __restrict__ buf, int64_t n,
                                                            float mu, int nesterov,
                                                            float* __restrict__ part) {
  __shared__ float red[256];
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
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

// scal[0] = 1 / (sqrt(sum of the partials) + 1e-7)
__global__ __launch_bounds__(256) void muon_norm_kernel(const float* __restrict__ part, int n,
                                                        float* __restrict__ scal) {
  __shared__ double red[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) s += part[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) scal[0] = (float)(1.0 / (sqrt(red[0]) + 1e-7));
}

// X = u * scal[0] in the wide orientation: X [rows][cols] or, transposed,
// X [cols][rows]; u recomputed from g and the updated buffer.
template <typename T>
__global__ __launch_bounds__(256) void muon_to_x_kernel(const float* __restrict__ g,
                                                        const float* __restrict__ buf, int rows,
                                                        int cols, float mu, int nesterov,
                                                        int transpose,
                                                        const float* __restrict__ scal,
                                                        T* __restrict__ X) {
  const int64_t n = (int64_t)rows * cols;
  const float inv = scal[0];
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float u = nesterov ? g[i] + mu * buf[i] : buf[i];
    const int64_t r = i / cols, c = i % cols;
    X[transpose ? c * rows + r : i] = from_f<T>(u * inv);
  }
}

// y = alpha * y + beta * x (element-wise, compute dtype)
template <typename T>
__global__ __launch_bounds__(256) void axpby_kernel(T* __restrict__ y, const T* __restrict__ x,
                                                    int64_t n, float alpha, float beta) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    y[i] = from_f<T>(alpha * to_f(y[i]) + beta * to_f(x[i]));
}

// p <- p * decay - step * X (X in the wide orientation, see muon_to_x_kernel)
template <typename T>
__global__ __launch_bounds__(256) void muon_apply_kernel(float* __restrict__ p,
                                                         const T* __restrict__ X, int rows,
                                                         int cols, int transpose, float decay,
                                                         float step) {
  const int64_t n = (int64_t)rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / cols, c = i % cols;
    p[i] = p[i] * decay - step * to_f(X[transpose ? c * rows + r : i]);
  }
}

}  // namespace gk

namespace gpt {

static unsigned ew_blocks(int64_t n) {
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 4096));
}

OptimPlan make_optim_plan(const Dims& d) {
  // one buffer set per side stream
  OptimPlan o{};
  const int64_t mats[4][2] = {{d.Cq, d.C}, {d.Ckv, d.C}, {d.C, d.Cq}, {d.F, d.C}};
  int64_t max_rc = (int64_t)d.C * d.F, max_r = 0;
  for (const auto& m : mats) {
    max_rc = std::max(max_rc, m[0] * m[1]);
    max_r = std::max(max_r, std::min(m[0], m[1]));
  }
  const size_t A = (size_t)d.act_bytes;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t off = 0;
  o.part = off;
  off += al((size_t)gk::kOptBlocks * 4 + 64);
  o.x = off;
  off += al((size_t)max_rc * A);
  o.y = off;
  off += al((size_t)max_rc * A);
  o.a = off;
  off += al((size_t)max_r * max_r * A);
  o.aa = off;
  off += al((size_t)max_r * max_r * A);
  o.set_bytes = off;
  o.sets = kOptStreams;
  o.total = off * kOptStreams;
  return o;
}

void launch_adamw(float* p, const float* g, float* m, float* v, int64_t n, float lr, float b1,
                  float b2, float eps, int step, hipStream_t s) {
  const float c1 = 1.0f - std::pow(b1, (float)step), c2 = 1.0f - std::pow(b2, (float)step);
  hipLaunchKernelGGL(gk::adamw_kernel, dim3(ew_blocks(n)), dim3(256), 0, s, p, g, m, v, n, lr, b1,
                     b2, eps, c1, c2);
}

template <typename T>
static void muon_typed(const Dims& d, const OptimPlan& o, char* ws, float* p, const float* g,
                       float* buf, int rows, int cols, float lr, float wd, float mu, int nesterov,
                       float a, float b, float c, int steps, hipStream_t s) {
  const int64_t n = (int64_t)rows * cols;
  float* part = reinterpret_cast<float*>(ws + o.part);
  float* scal = part + gk::kOptBlocks;
  T* X = reinterpret_cast<T*>(ws + o.x);
  T* Y = reinterpret_cast<T*>(ws + o.y);
  T* Am = reinterpret_cast<T*>(ws + o.a);
  T* AA = reinterpret_cast<T*>(ws + o.aa);
  const int tr = rows > cols ? 1 : 0;
  const int r = tr ? cols : rows, k = tr ? rows : cols;  // X is [r][k], r <= k
  hipLaunchKernelGGL(gk::muon_momentum_kernel, dim3(gk::kOptBlocks), dim3(256), 0, s, g, buf, n,
                     mu, nesterov, part);
  hipLaunchKernelGGL(gk::muon_norm_kernel, dim3(1), dim3(256), 0, s, part, gk::kOptBlocks, scal);
  hipLaunchKernelGGL(gk::muon_to_x_kernel<T>, dim3(ew_blocks(n)), dim3(256), 0, s, g, buf, rows,
                     cols, mu, nesterov, tr, scal, X);
  for (int it = 0; it < steps; ++it) {
    gemm_nt_store(d, r, r, k, X, X, Am, s);   // A = X X^T
    gemm_nt_store(d, r, r, r, Am, Am, AA, s); // A A (A symmetric)
    hipLaunchKernelGGL(gk::axpby_kernel<T>, dim3(ew_blocks((int64_t)r * r)), dim3(256), 0, s, Am,
                       AA, (int64_t)r * r, b, c);  // B = b A + c A A
    gemm_nn_store(d, r, k, r, Am, X, Y, s);   // Y = B X
    hipLaunchKernelGGL(gk::axpby_kernel<T>, dim3(ew_blocks(n)), dim3(256), 0, s, X, Y, n, a,
                       1.0f);                  // X = a X + Y
  }
  const float scale = std::sqrt(std::max(1.0f, (float)rows / (float)cols));
  hipLaunchKernelGGL(gk::muon_apply_kernel<T>, dim3(ew_blocks(n)), dim3(256), 0, s, p, X, rows,
                     cols, tr, 1.0f - lr * wd, lr * scale);
}

void launch_muon(const Dims& d, const OptimPlan& o, void* workspace, float* p, const float* g,
                 float* buf, int rows, int cols, float lr, float wd, float mu, int nesterov,
                 float a, float b, float c, int steps, hipStream_t s) {
  char* ws = static_cast<char*>(workspace);
  if (d.bf16)
    muon_typed<bf16>(d, o, ws, p, g, buf, rows, cols, lr, wd, mu, nesterov, a, b, c, steps, s);
  else
    muon_typed<float>(d, o, ws, p, g, buf, rows, cols, lr, wd, mu, nesterov, a, b, c, steps, s);
}

}  // namespace gpt
