// Internal interfaces of the gfx950 GPT step library: derived sizes, the
// parameter layout, the workspace plan and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "gpt_step.h"

namespace gpt {

// ------------------------------------------------------------ launches
// Every kernel launch of an entry point goes through GK_LAUNCH, which keeps
// per-thread bookkeeping for the current call: the first launch error
// (hipGetLastError right after the launch) is recorded and every later
// launch of the call is skipped, so nothing is enqueued after a failure.
// Test support (gpt_debug_launches): a launch index at which a failure is
// injected instead of launching, and a dry run that counts the launch
// sequence without launching anything.
struct LaunchState {
  hipError_t err = hipSuccess;  // first error of the current call
  bool injected = false;        // err came from the fault-injection switch
  int64_t issued = 0;           // launches issued (or counted, in a dry run)
  int64_t fail_at = -1;         // inject a failure at this launch index (< 0: never)
  bool dry = false;             // count launches, launch nothing
};
LaunchState& launch_state();
// start of an entry point call: clears the error and the count
void launch_reset();
// before a launch: false if it must be skipped (earlier error, injected
// failure, dry run)
bool launch_begin();
// after a launch: record hipGetLastError
void launch_end();

#define GK_LAUNCH(...)                      \
  do {                                       \
    if (::gpt::launch_begin()) {             \
      hipLaunchKernelGGL(__VA_ARGS__);       \
      ::gpt::launch_end();                   \
    }                                        \
  } while (0)

struct Dims {
  int L, C, H, Hk, D, F, V, T, B, W;
  int64_t N;        // tokens per call = B * T
  int Cq, Ckv, Qkv; // H*D, Hk*D, Cq + 2*Ckv
  int G;            // H / Hk
  bool bf16;        // compute dtype
  bool fp8;         // block linears in dynamic per-tensor fp8
  int act_bytes;    // 2 (bf16) or 4 (fp32)
  float theta, eps, cap;
  bool accumulate;
  bool smear;       // Smear at the embedding (GPT_F_SMEAR)
  bool backout;     // Backout before the final norm (GPT_F_BACKOUT)
  int mid;          // Backout caches the stream entering this layer (L / 2)
  bool reuse_weights;  // GPT_F_REUSE_WEIGHTS: keep the workspace's bf16 weight mirrors
  bool check_finite;   // GPT_F_CHECK_FINITE
  bool check_inputs;   // GPT_F_CHECK_INPUTS
};

Dims make_dims(const gpt_config& c);
bool layer_full(int l, int L);
bool layer_ve(int l, int L);

struct TensorInfo {
  std::string name;
  int64_t offset, rows, cols;
};
std::vector<TensorInfo> param_layout(const gpt_config& c);

// Workspace plan: byte offsets of every region (all 256-byte aligned).
struct Plan {
  size_t wc;            // compute-dtype mirror of params (bf16 only)
  size_t wct;           // bf16 transposed mirror of the linear weights (same element
                        // offsets; a [rows][cols] weight is stored [cols][rows])
  size_t rope;          // fp32 cos [T][D/2], sin [T][D/2]
  size_t x;             // fp32 [(L+1)][N][C] residual stream per layer boundary
  size_t xin;           // fp32 [N][C] scratch
  // per layer, stride `layer_bytes`, starting at `layers`
  size_t layers, layer_bytes;
  size_t l_xn, l_r1, l_qkv, l_rqk, l_a, l_attn, l_lse, l_xmid, l_xn2, l_r2, l_u;
  size_t xf, rf, logits, lossrow, scalars;
  size_t part;           // split-K partials
  int64_t part_bytes;
  size_t gx, gxc, gx0, gu, gtmp, gO, gqkv, delta, ga, lam_part, veg_part;
  size_t vegrow;         // fp32 [N][Hk*D] per-position value-embedding gradient rows
  size_t tlink;          // int32 [2 N] token links of the embedding-table gradients
  size_t sgate;          // fp32 [N] Smear gate values (0 bytes without Smear)
  int lam_blocks, veg_splits;
  // fp8 linears only (0 bytes otherwise). Token-major code tensors that the
  // weight gradients contract over are stored transposed, [features][Np],
  // Np = N rounded up to 128, zero beyond N.
  int64_t Np;
  size_t amax;                // uint32 [16 L] amax slots
  size_t w8, w8_layer;        // per layer: qkv [Qkv][C], o [C][Cq], fc [F][C], mp [C][F]
  size_t w8t, w8t_layer;      // per layer: qkv^T [C][P(Qkv)], o^T [Cq][P(C)], fc^T [C][P(F)], mp^T [F][P(C)]
  size_t l_x8t, l_a8t, l_x28t, l_h8t;  // per layer: xn, attn, xn2, h codes, transposed
  size_t q8;                  // [N][max(C, Cq, F, Qkv)] row-major codes (scratch)
  size_t g8t;                 // [max(C, F, Qkv)][Np] transposed gradient codes (scratch)
  size_t total;
};
Plan make_plan(const Dims& d);

// ------------------------------------------------------------ launchers
// `act` pointers hold compute-dtype elements (bf16 or fp32 per d.bf16).

struct CastSeg {
  int64_t off, n;
};
void launch_cast(const float* src, void* dst, const std::vector<CastSeg>& segs, hipStream_t s);
// bf16 casts of the [rows][cols] fp32 matrices at offsets `offs` into dst and
// their transposes into dstT (same element offsets)
void launch_cast_t(const float* src, void* dst, void* dstT, const std::vector<int64_t>& offs,
                   int rows, int cols, hipStream_t s);
void launch_zero(float* p, int64_t n, hipStream_t s);
// Debug checks. check_ids: out[0] = number of token ids outside [0, V),
// out[1] = number of targets outside [-1, V) (one workgroup; writes both).
// check_finite: flag |= 1 if any of x[0 .. n) is NaN or infinite (flag must
// be zero before the first call).
void launch_check_ids(const int32_t* tok, const int32_t* tgt, int64_t N, int V, uint32_t* out,
                      hipStream_t s);
void launch_check_finite(const float* x, int64_t n, uint32_t* flag, hipStream_t s);
void launch_rope_table(float* cs, int T, int D, float theta, hipStream_t s);
void launch_embed(const float* wte, const int32_t* tok, float* x0, int64_t N, int C, int V,
                  hipStream_t s);
// Smear: x0[n] = e[n] + sigmoid(<e[n], w>) e[n-1] (t >= 1), e[n] = wte[tok[n]];
// the gate values go to sig (fp32 [N], 0 at t = 0).
void launch_smear_embed(const Dims& d, const float* wte, const int32_t* tok, const float* w,
                        float* x0, float* sig, hipStream_t s);
// Smear backward: ge (fp32 [N][C]) = dL/de from g = dL/dx0, and the gate
// weight gradient gw [C] (written, or added to with d.accumulate) through
// smear_blocks(N) fixed-order partials in part (fp32 [smear_blocks(N)][C]).
int smear_blocks(int64_t N);
void launch_smear_bwd(const Dims& d, const float* g, const float* wte, const int32_t* tok,
                      const float* w, const float* sig, float* ge, float* part, float* gw,
                      hipStream_t s);
// out[0] = 1, out[1] = -lam[0] (device scalars)
void launch_backout_weights(const float* lam, float* out, hipStream_t s);

// rows of x (fp32 [N][C]): if x0 != nullptr, xin = lr*x + l0*x0 (written to
// xin_out if non-null) else xin = x; y = rms(xin) (act), r (fp32 [N]).
// If wg != nullptr, a[n][j] = <y[n], wg[j]> for j < hk (fp32 [N][hk]).
void launch_mix_norm(const Dims& d, const float* x, const float* x0, const float* lam_r,
                     const float* lam_0, float* xin_out, void* y, float* r,
                     const float* wg, float* a, hipStream_t s);

void launch_rope_qk_ve_fwd(const Dims& d, void* qkv, float* rqk, const float* cs,
                           const float* a, const float* ve_table, const int32_t* tok,
                           hipStream_t s);
void launch_rope_qk_ve_bwd(const Dims& d, void* gqkv, const void* qkv, const float* rqk,
                           const float* cs, const float* a, const float* ve_table,
                           float* gve_rows, float* ga, const int32_t* tok, hipStream_t s);
// Embedding-table gradients tab[tok[n]][:] += g[n][:] over n < N (g [N][W]
// fp32): within each chunk of 128 positions the rows sharing a token id are
// summed in position order first, then one fp32 atomic add per (id,
// column). launch_token_links builds the per-call links (int32 [2 N]) from
// the tokens.
void launch_token_links(const int32_t* tok, int64_t N, int32_t* link, hipStream_t s);
void launch_rows_to_table(const float* g, int W, const int32_t* tok, const int32_t* link,
                          int64_t N, float* tab, int V, hipStream_t s);

void launch_attn_fwd(const Dims& d, bool full, const void* qkv, void* out, float* lse,
                     hipStream_t s);
void launch_attn_delta(const Dims& d, const void* gO, const void* O, float* delta, hipStream_t s);
void launch_attn_bwd(const Dims& d, bool full, const void* qkv, const void* gO,
                     const float* lse, const float* delta, void* gqkv, hipStream_t s);

// Norm backward modes.
enum NormBwdMode { NB_FINAL = 0, NB_NORM2 = 1, NB_NORM1 = 2 };
struct NormBwdArgs {
  int mode;
  const float* gin;     // fp32 [N][C] gradient w.r.t. the norm output
  const float* ysrc;    // fp32 [N][C] norm input (NB_FINAL, NB_NORM2); the norm
                        // output is recomputed as ysrc * r in fp32
  const float* r;       // fp32 [N]
  float* gx;            // fp32 [N][C] residual gradient (in/out)
  void* gxc;            // act [N][C] copy of the new gx (may be null)
  int gxc_bf16;         // set by the launcher
  // NB_NORM1 only
  const float* ga;      // fp32 [N][Hk] or null
  const float* wg;      // fp32 [Hk][C] or null
  const float* x;       // fp32 [N][C] block input (norm input = lr * x + l0 * x0)
  const float* x0;      // fp32 [N][C]
  const float* lam_r;   // device scalar
  const float* lam_0;
  float* gx0;           // fp32 [N][C]
  int gx0_first;        // gx0 = ... instead of +=
  int last_layer0;      // layer 0: add the final gx into gx0
  float* lam_part;      // fp32 [blocks][2]
  const float* gadd;    // fp32 [N][C] added to the gradient w.r.t. x, or null
  int gx_first;         // NB_NORM1: gx is written without reading it
};
void launch_norm_bwd(const Dims& d, const NormBwdArgs& a, hipStream_t s);

// The lambda gradients of `layers` layers: layer l's nblk partial pairs at
// lam_part + 2 l nblk, outputs scale * sums into g_lr[l] (skipped if g_lr is
// null) and g_l0[l].
void launch_lambda_finalize(const Dims& d, const float* lam_part, int nblk, float* g_lr,
                            float* g_l0, hipStream_t s, int layers, float scale = 1.0f);
// splits: veg_splits(N) (each split takes at most 64 tokens)
int veg_splits(int64_t N);
void launch_veg_wgrad(const Dims& d, const float* ga, const void* xn, float* part,
                      int splits, float* gwg, hipStream_t s);
// 1 / n_valid into scalars[0].
void launch_count_valid(const Dims& d, const int32_t* tgt, float* scalars, hipStream_t s);
// Softcap cross-entropy loss from the stored softcapped logits (row sums of
// exp(c - cap) in a fixed order, one workgroup per token); with `grad` the
// logits are overwritten in place by the logit gradient of the mean loss.
void launch_loss(const Dims& d, void* logits, const int32_t* tgt, const float* scalars,
                 float* lossrow, float* loss, bool grad, hipStream_t s);

// Decode attention over a KV cache (decode.hip): chunks per (sequence, KV
// head), workspace bytes (fp32 chunk states; 0 when there is one chunk), and
// the launch (q, out bf16 [B][H][D]; k, v bf16 [B][Tmax][Hk][D]; seqlen
// int32 [B], clamped to [1, Tmax]).
int decode_splits(int Tmax, int window);
size_t decode_workspace_bytes(int B, int H, int Hk, int D, int Tmax, int window);
// KV-cache append from fused QKV rows (bf16 [B * n_new][(H + 2Hk) D]) to
// positions pos[b] + i of the caches (bf16 [B][Tmax][Hk][D]).
void launch_kv_cache_append(int B, int n_new, int H, int Hk, int D, int Tmax, const void* qkv,
                            const int32_t* pos, void* k, void* v, hipStream_t s);
// The no-allocation variant's scratch: its capacity in bytes, and the
// current GPU's device address of it (looked up once per device).
size_t decode_scratch_capacity();
hipError_t decode_scratch(void** out);
void launch_decode_attn(int B, int H, int Hk, int D, int Tmax, int window, const void* q,
                        const void* k, const void* v, const int32_t* seqlen, void* out,
                        void* workspace, hipStream_t s);

// MuonAdamW (optim.hip). The Muon matrices grouped by their wide shape
// r x k (r <= k): element offsets and whether each is stored tall (k x r).
struct MuonGroup {
  int r, k;
  std::vector<int64_t> off;
  std::vector<int> tall;
};
std::vector<MuonGroup> muon_groups(const gpt_config& c);
// Workspace: per-matrix norm partials and scales, then X and Y [nm][r][k],
// A and A A [nm][r][r] (compute dtype) for the largest batch of a group.
struct OptimPlan {
  size_t part, scal, x, y, a, aa, total;
};
OptimPlan make_optim_plan(const gpt_config& c);
void launch_adamw(float* p, const float* g, float* m, float* v, int64_t n, float lr, float b1,
                  float b2, float eps, int step, hipStream_t s);
void launch_muon_groups(const Dims& d, const std::vector<MuonGroup>& groups, const OptimPlan& o,
                        void* workspace, float* params, const float* grads, float* buf, float lr,
                        float wd, float mu, int nesterov, float a, float b, float c, int steps,
                        hipStream_t s);

// ------------------------------------------------------------ GEMMs
// Shapes: C[M][N] = sum_k A(m,k) B(n,k).
// "nt": A [M][K], B [N][K] (both contraction-contiguous).
// "nn": A [M][K], B [K][N].
// "tn": A [K][M], B [K][N] (weight gradients: K = tokens).
void gemm_nt_store(const Dims& d, int64_t M, int N, int K, const void* A, const void* B,
                   void* C, hipStream_t s);
void gemm_nt_resid(const Dims& d, int64_t M, int N, int K, const void* A, const void* B,
                   const float* R, float* C, hipStream_t s);
// C = relu(A B^T)^2 (the MLP hidden activation)
void gemm_nt_relu2(const Dims& d, int64_t M, int N, int K, const void* A, const void* B, void* C,
                   hipStream_t s);
// Softcapped logits c = cap * tanh(A B^T / cap), stored in the activation type.
void gemm_nt_softcap(const Dims& d, int64_t M, int N, int K, const void* A, const void* B,
                     void* C, hipStream_t s);
// The nn products take an optional Bt = B^T ([N][K], bf16): with it the
// product runs with both operands K-major (direct LDS fills).
void gemm_nn_store(const Dims& d, int64_t M, int N, int K, const void* A, const void* B,
                   void* C, hipStream_t s, const void* Bt = nullptr);
// `batch` independent products in the compute dtype, operands and outputs
// sA / sB / sC elements apart: nt C_b = A_b B_b^T (A [M][K], B [N][K]);
// nn C_b = A_b B_b (A [M][K], B [K][N]).
void gemm_nt_store_batched(const Dims& d, int batch, int64_t M, int N, int K, const void* A,
                           int64_t sA, const void* B, int64_t sB, void* C, int64_t sC,
                           hipStream_t s);
void gemm_nn_store_batched(const Dims& d, int batch, int64_t M, int N, int K, const void* A,
                           int64_t sA, const void* B, int64_t sB, void* C, int64_t sC,
                           hipStream_t s);
// Batched C_b = alpha R_b + beta (A_b op(B_b)) with R_b, C_b [M][N] sC apart;
// op: B_b^T (B [N][K], nn = false) or B_b (B [K][N], nn = true).
void gemm_lin_batched(const Dims& d, bool nn, int batch, int64_t M, int N, int K, const void* A,
                      int64_t sA, const void* B, int64_t sB, const void* R, void* C, int64_t sC,
                      float alpha, float beta, hipStream_t s);
void gemm_nn_f32(const Dims& d, int64_t M, int N, int K, const void* A, const void* B,
                 float* C, hipStream_t s, const void* Bt = nullptr);
// C = (A B) * 2 sqrt(H): the MLP hidden gradient from h = relu(u)^2
void gemm_nn_relu2bwd(const Dims& d, int64_t M, int N, int K, const void* A, const void* B,
                      const void* H, void* C, hipStream_t s, const void* Bt = nullptr);
// Split-K products: each K split writes an fp32 partial of C into `part`
// (capacity part_cap bytes, at least what the matching *_part_bytes returns
// for the shape); the returned SplitSum, passed to splitk_sum, adds the
// partials into C in split order (nothing to do when the product ran
// unsplit and wrote C itself).
struct SplitSum {
  const float* part = nullptr;
  int64_t splits = 0, M = 0, N = 0;
  float* C = nullptr;
  bool accumulate = false;
};
void splitk_sum(const SplitSum& r, hipStream_t s);
// Like gemm_nn_f32 for a long contraction.
SplitSum gemm_nn_f32_splitk(const Dims& d, int64_t M, int N, int K, const void* A,
                            const void* B, float* C, float* part, int64_t part_cap,
                            hipStream_t s, const void* Bt = nullptr);
int64_t part_bytes_nn_splitk(const Dims& d, int64_t M, int64_t N, int64_t K);
// Weight gradients C[M][N] (+)= sum_k A[k][m] B[k][n].
SplitSum gemm_tn_wgrad(const Dims& d, int M, int N, int64_t K, const void* A, const void* B,
                       float* C, bool accumulate, float* part, int64_t part_cap, hipStream_t s);
int64_t part_bytes_tn_wgrad(const Dims& d, int64_t M, int64_t N, int64_t K);

// ------------------------------------------------------------ fp8 linears
// Per-tensor dynamic scaling: s = fmax / amax in fp32; codes are
// RNE(clamp(x * s)) in OCP e4m3 (forward operands) or e5m2 (output
// gradients). amax slots are uint32 bit patterns of max |x|.
enum Fp8Fmt { FP8_E4M3 = 0, FP8_E5M2 = 1 };

// Up to 6 consecutive segments of an index range, each with its own amax
// slot: segment i ends (exclusive) at end[i]; the last one is open-ended.
struct Segs {
  int n;
  int64_t end[6];
  int slot[6];
};
inline Segs one_seg(int slot) {
  Segs s{};
  s.n = 1;
  s.end[0] = INT64_MAX;
  s.slot[0] = slot;
  return s;
}

// amax of x (n elements, a multiple of 8; bf16 or fp32): the segment of an
// element is looked up from (index mod period) and every boundary is a
// multiple of 8.
void launch_fp8_amax(const void* x, bool bf16_src, int64_t n, int64_t period, const Segs& sg,
                     uint32_t* amax, hipStream_t s);
// Codes of src [R][C] (C a multiple of 64) row-major into out [R][C] and/or
// transposed into outT [C][pitchT] (pitchT a multiple of 128 and >= R; rows
// R .. pitchT-1 written as 0). Segments along rows (seg_rows) or columns.
void launch_fp8_quant(const void* src, bool bf16_src, int64_t R, int64_t C, bool seg_rows,
                      const Segs& sg, const uint32_t* amax, int fmt, uint8_t* out, uint8_t* outT,
                      int64_t pitchT, hipStream_t s);

// Dequantisation of an fp8 product: in segment i of the M or N index
// (axis 0 or 1) the sum of code products is multiplied by
// 1 / (s(amax[sa[i]], fa) * s(amax[sb[i]], fb)).
struct Fp8Deq {
  const uint32_t* amax;
  int axis;
  int nseg;
  int64_t end[3];
  int sa[3], sb[3];
  int fa, fb;
};

// fp8 products, both operands K-major: C[M][N] = sum_k A[m][k] B[n][k] with
// A [M][lda] and B [N][ldb] byte codes (K, lda, ldb multiples of 16).
void gemm8_store(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                 const uint8_t* B, int64_t ldb, const Fp8Deq& dq, void* C, hipStream_t s);
void gemm8_resid(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                 const uint8_t* B, int64_t ldb, const Fp8Deq& dq, const float* R, float* C,
                 hipStream_t s);
// The two activation products also merge max |C| (the stored bf16 values)
// into *amax_c when it is non-null: the amax the fp8 quantiser of C needs,
// without a separate pass over C.
void gemm8_relu2(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                 const uint8_t* B, int64_t ldb, const Fp8Deq& dq, void* C, uint32_t* amax_c,
                 hipStream_t s);
void gemm8_relu2bwd(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                    const uint8_t* B, int64_t ldb, const Fp8Deq& dq, const void* H, void* C,
                    uint32_t* amax_c, hipStream_t s);
// C (+)= the product (accumulate: add to C).
void gemm8_f32(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
               const uint8_t* B, int64_t ldb, const Fp8Deq& dq, float* C, bool accumulate,
               hipStream_t s);
// The same with scales that change along K (dq.axis 2: segments of the
// contraction cut at dq.end, in codes, multiples of 16): C (+)= sum over
// segments i of f_i * (A_i B_i^T).
void gemm8_f32_kseg(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                    const uint8_t* B, int64_t ldb, const Fp8Deq& dq, float* C, bool accumulate,
                    hipStream_t s);
// Weight gradient (K = tokens, split over workgroups when that fills the
// machine, partials as for gemm_tn_wgrad); C (+)= the product.
SplitSum gemm8_wgrad(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                     const uint8_t* B, int64_t ldb, const Fp8Deq& dq, float* C, bool accumulate,
                     float* part, int64_t part_cap, hipStream_t s);
int64_t part_bytes_f8_wgrad(int64_t M, int64_t N, int64_t K);
// One fp8 product with an fp32 output C [M][N] (+)= ... on the step's code
// paths: wgrad = the weight-gradient product (split-K partials in part,
// at least part_bytes_f8_wgrad(M, N, K) bytes); else the plain product with
// A's format from dq.fa. Returns the split sum still to be added
// (splitk_sum).
SplitSum gemm8_product(bool wgrad, int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                       const uint8_t* B, int64_t ldb, const Fp8Deq& dq, float* C, bool accumulate,
                       float* part, int64_t part_cap, hipStream_t s);

}  // namespace gpt
