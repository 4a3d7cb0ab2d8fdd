/*
 * gpt_step.h -- C ABI of the nanochat GPT forward+backward step on gfx950.
 *
 * One call computes the training loss of one batch and the gradient of every
 * parameter of the decoder-only GPT that these pages describe:
 *   - "Nanochat在nanoGPT之上的新增功能" (nanochat additions over nanoGPT),
 *     section 1 feature table and the notes under it: RoPE, parameter-free
 *     RMSNorm, ReLU^2 MLP, separate c_q/c_k/c_v/c_proj, GQA, QK-norm after
 *     RoPE, no bias, untied lm_head, no dropout, tanh softcap +-15, SSSL
 *     sliding windows (short = 1/4 context, last layer full), value
 *     embeddings v += gate * ve on alternating layers, per-layer
 *     resid / x0 lambdas, dynamic per-tensor fp8 linears;
 *   - "NanoChat基础训练报告" (d12 training report), architecture block: the
 *     d12 shape, bf16 training, value embeddings on odd layers;
 *   - "nanochat — 架构与原理" (architecture overview), section 4: the -1
 *     ignore index of the loss.
 *
 * Conventions shared by every entry point
 *   - Pointers marked (device) are HIP device pointers; (host) are host
 *     pointers. Every buffer is owned by the caller; the library allocates
 *     nothing and frees nothing.
 *   - Status: GPT_OK (0) or a negative gpt_status. Validation errors return
 *     before anything is enqueued. gpt_last_error() gives a per-thread text.
 *   - Device work is enqueued on `stream` (a hipStream_t passed as void*;
 *     NULL = the null stream) and the call returns without synchronising.
 */
#ifndef GPT_STEP_H
#define GPT_STEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GPT_ABI_VERSION 2

typedef enum gpt_status {
  GPT_OK = 0,
  GPT_E_INVAL = -1,        /* a config field, size or (checked) input is out of range */
  GPT_E_NULLPTR = -2,      /* a required pointer is NULL                     */
  GPT_E_ALIGN = -3,        /* a pointer breaks the alignment rule below      */
  GPT_E_WORKSPACE = -4,    /* workspace smaller than gpt_workspace_size      */
  GPT_E_UNSUPPORTED = -5,  /* valid model, but not built into this library   */
  GPT_E_HIP = -6,          /* the HIP runtime reported an error              */
  GPT_E_NONFINITE = -7     /* GPT_F_CHECK_FINITE: the loss or a gradient is not finite */
} gpt_status;

enum { GPT_DT_F32 = 0, GPT_DT_BF16 = 1 };

/* flags */
enum {
  GPT_F_ACCUMULATE = 1,    /* grads += new grads instead of grads = new grads */
  /* An RMSNorm of the token embedding before the first block. The pages
   * place RMSNorm only before attention, before the MLP and before lm_head
   * (nanochat additions page, feature table), so the library does not
   * build it: a config that sets this bit is GPT_E_UNSUPPORTED. */
  GPT_F_EMBED_NORM = 2,
  /* Debug checks, each reported after an internal hipStreamSynchronize of
   * `stream` (so the call is no longer asynchronous):
   * CHECK_FINITE: after the step, the loss (and with gpt_fwd_bwd every
   *   gradient) is checked on the device; GPT_E_NONFINITE if any is NaN or
   *   infinite (the outputs are written all the same).
   * CHECK_INPUTS: before anything else is enqueued, token ids are checked
   *   to lie in [0, vocab) and targets in [-1, vocab); GPT_E_INVAL if not,
   *   with nothing else enqueued. */
  GPT_F_CHECK_FINITE = 4,
  GPT_F_CHECK_INPUTS = 8,
  /* Model variants of the additions page (feature table rows Smear and
   * Backout, and the notes on them). Readings where the page is silent:
   * Smear: x0[b,t] = e[b,t] + sigmoid(<e[b,t], smear_gate>) * e[b,t-1] for
   *   t >= 1 and x0[b,0] = e[b,0], e = wte[tokens] (the gate is a bias-free
   *   linear map C -> 1 of the current token's embedding; x0 is the stream
   *   entering layer 0 and the one every block mixes in).
   * Backout: the final norm reads x - backout_lambda * x_mid, where x_mid
   *   is the residual stream entering layer n_layer / 2. */
  GPT_F_SMEAR = 16,
  GPT_F_BACKOUT = 32,
  /* The previous call on this workspace had the same params (same values,
   * e.g. the micro-batches of one optimizer step): its bf16 weight mirrors
   * in the workspace are reused instead of converted again from the fp32
   * params (fp8 weight codes are still made each call). Undefined results
   * if the params or the workspace changed since. */
  GPT_F_REUSE_WEIGHTS = 64,
  /* HIP-graph cache of gpt_fwd_bwd / gpt_fwd: the first call with a given
   * set of arguments (the config, every pointer, workspace_bytes, the
   * current device) captures its launch sequence on `stream` into a HIP
   * graph, which that call and every later call with the same arguments
   * replays with one hipGraphLaunch on their `stream` (so the host's
   * per-launch overhead and the gaps between launches go). Buffer contents
   * may change between calls; the pointers may not. `stream` must not be
   * the null stream; not with GPT_F_CHECK_FINITE or GPT_F_CHECK_INPUTS
   * (GPT_E_INVAL). Calls run eagerly (nothing captured or replayed) while
   * gpt_profile_begin is active and in a dry run. At most 64 graphs are
   * kept (the least recently used one is dropped after a device
   * synchronisation); gpt_graph_cache_clear drops them all. */
  GPT_F_GRAPH = 128
};

/*
 * Model and batch description. All sizes are element counts.
 *   n_embd = n_head * head_dim is not required (c_q/c_proj use n_head*head_dim).
 *   head_dim in {64, 128}; n_head % n_kv_head == 0; n_embd, mlp_hidden and
 *   vocab multiples of 64 (the additions page pads the vocabulary to a
 *   multiple of 64); 1 <= seq_len; 1 <= batch; 0 <= short_window.
 *   Layer l uses the full causal context iff l % 4 == 3 or l == n_layer-1,
 *   else the short window: key s is visible to query t iff
 *   0 <= t - s <= short_window. Layer l has a value embedding iff
 *   l % 2 == (n_layer - 1) % 2.
 */
typedef struct gpt_config {
  int32_t abi_version;     /* GPT_ABI_VERSION                                */
  int32_t n_layer;
  int32_t n_embd;          /* C                                              */
  int32_t n_head;          /* H                                              */
  int32_t n_kv_head;       /* Hk                                             */
  int32_t head_dim;        /* D                                              */
  int32_t mlp_hidden;      /* F                                              */
  int32_t vocab;           /* V                                              */
  int32_t seq_len;         /* T                                              */
  int32_t batch;           /* B                                              */
  int32_t short_window;    /* W                                              */
  int32_t compute_dtype;   /* GPT_DT_F32 | GPT_DT_BF16                       */
  int32_t fp8_linears;     /* 0 | 1: block linears in per-tensor fp8 (bf16 only) */
  int32_t flags;           /* GPT_F_*                                        */
  float rope_theta;        /* RoPE base, > 1                                 */
  float norm_eps;          /* RMSNorm epsilon (all norms), > 0               */
  float softcap;           /* logit cap c = softcap * tanh(z / softcap), > 0 */
} gpt_config;

/* GPT_ABI_VERSION of the loaded library. */
int gpt_abi_version(void);

/* Host only. GPT_OK if the library can run `cfg`, else the reason. */
int gpt_config_validate(const gpt_config* cfg);

/*
 * Host only. Canonical parameter layout: params and grads are flat fp32
 * arrays, row-major, no padding, tensors in this order:
 *   wte [V, C];
 *   per layer l: l.q [H*D, C], l.k [Hk*D, C], l.v [Hk*D, C], l.o [C, H*D],
 *                l.fc [F, C], l.mp [C, F], and on value-embedding layers
 *                l.ve [V, Hk*D], l.veg [Hk, C];
 *   lm_head [V, C]; with GPT_F_SMEAR smear_gate [1, C]; with GPT_F_BACKOUT
 *   backout_lambda [1]; resid_lambdas [L]; x0_lambdas [L].
 * Linear weights are [out, in] (y = x W^T). Names are "wte", "l3.q", ...
 * gpt_param_count: number of tensors and total element count.
 * gpt_param_info: tensor i's name (NUL-terminated, < 64 bytes), element
 * offset, rows and cols (cols = 1 for the lambda vectors and backout_lambda).
 */
int gpt_param_count(const gpt_config* cfg, int64_t* n_tensors, int64_t* n_elems);
int gpt_param_info(const gpt_config* cfg, int64_t i, char name[64],
                   int64_t* offset, int64_t* rows, int64_t* cols);

/* Host only. Window and value-embedding pattern of layer l (0/1 each). */
int gpt_layer_info(const gpt_config* cfg, int32_t l, int32_t* is_full, int32_t* has_ve);

/* Host only. Bytes of device workspace gpt_fwd_bwd needs for `cfg`. */
int gpt_workspace_size(const gpt_config* cfg, size_t* bytes);

/*
 * Host only. Where a named buffer lives inside the workspace, for inspection
 * after a synchronised call (contents are defined only for the forward
 * tensors below). Saved forward tensors:
 *   "x"    fp32 [N, C]   residual stream entering layer `layer`
 *                        (layer = n_layer: the stream before the final norm)
 *   "xn"   act  [N, C]   RMSNorm output feeding c_q/c_k/c_v
 *   "qkv"  act  [N, (H+2Hk)*D]  q, k after RoPE+QK-norm; v after the
 *                        value embedding; head-major columns
 *   "attn" act  [N, H*D] attention output
 *   "xmid" fp32 [N, C]   residual stream after the attention block
 *   "xn2"  act  [N, C]   RMSNorm output feeding the MLP
 *   "h"    act  [N, F]   MLP hidden activation relu(c_fc output)^2
 *   "xf"   act  [N, C]   final RMSNorm output
 *   "logits" act [N, V]  softcapped logits after gpt_fwd; after gpt_fwd_bwd
 *                        the gradient of the loss w.r.t. the raw logits
 * Scratch (layout only): "wc", "wct" (bf16 weight mirror and its per-matrix
 * transposes; 0 bytes for fp32), "rope", "xin", "rf", "lossrow", "scalars",
 * "gx", "gxc", "gx0", "gu", "gtmp", "gO", "gqkv", "delta", "ga", "lam_part",
 * "veg_part", "part" (split-K partials; 0 bytes when no product is split),
 * "vegrow" (per-position value-embedding gradient rows, fp32 [N, Hk*D]),
 * "tlink" (int32 [2N] token links of the embedding-table gradients),
 * "sgate" (fp32 [N] Smear gate values; 0 bytes without GPT_F_SMEAR);
 * per layer "r1", "rqk", "a", "lse", "r2". With fp8_linears = 1 also "amax", "w8", "w8t", "q8", "g8t" and per
 * layer "x8t", "a8t", "x28t", "h8t" (fp8 codes; 0 bytes otherwise).
 * All regions are disjoint. `layer` is ignored for global regions.
 * N = batch * seq_len, row n = b * seq_len + t; act = compute_dtype.
 * Returns the byte offset and size. GPT_E_INVAL for an unknown name/layer.
 */
int gpt_workspace_region(const gpt_config* cfg, const char* name, int32_t layer,
                         size_t* offset, size_t* bytes);

/*
 * Forward + backward of one batch.
 *   params    (device) fp32 [n_elems], canonical layout; read only.
 *   tokens    (device) int32 [batch, seq_len], ids in [0, vocab).
 *   targets   (device) int32 [batch, seq_len], ids in [0, vocab) or -1
 *             (ignored). The loss is the mean over non-ignored targets
 *             (0 if there are none).
 *   loss      (device) fp32 [1], written.
 *   grads     (device) fp32 [n_elems], canonical layout; overwritten, or
 *             added to with GPT_F_ACCUMULATE.
 *   workspace (device) >= gpt_workspace_size bytes; scratch, contents
 *             undefined after the call.
 * Alignment: params, grads and workspace 256-byte aligned; tokens, targets
 * and loss 4-byte aligned. Concurrent calls need distinct workspaces,
 * grads and loss buffers.
 * Ids out of range are a precondition violation, reported only with
 * GPT_F_CHECK_INPUTS; without it they never make a kernel touch memory
 * outside its buffers: a token id outside [0, vocab) embeds as a zero row
 * (no table row is read or receives a gradient), and a target outside
 * [0, vocab) is ignored like -1.
 * Errors: validation errors return before anything is enqueued; if a
 * kernel launch fails, no later launch of the call is enqueued and the call
 * returns GPT_E_HIP (detail in gpt_last_error).
 */
int gpt_fwd_bwd(const gpt_config* cfg, const float* params, const int32_t* tokens,
                const int32_t* targets, float* loss, float* grads,
                void* workspace, size_t workspace_bytes, void* stream);

/* Forward only: the loss (same arguments and rules, no grads). */
int gpt_fwd(const gpt_config* cfg, const float* params, const int32_t* tokens,
            const int32_t* targets, float* loss,
            void* workspace, size_t workspace_bytes, void* stream);

/*
 * The attention step of one layer on its own (the kernels gpt_fwd_bwd runs
 * for F5 and its backward), for tests of the step and for reuse: causal
 * GQA softmax attention with the layer's window ("Nanochat在nanoGPT之上的新增
 * 功能", feature table and notes: GQA, SSSL sliding window, last layer full):
 *   y[b,t,h] = sum_s softmax_s(q[b,t,h] . k[b,s,h'] / sqrt(D)) v[b,s,h'],
 * h' = h / (n_head / n_kv_head), over keys s <= t with (full or
 * t - s <= short_window). Sizes, window and dtype come from cfg (n_embd,
 * mlp_hidden, vocab, n_layer, flags and fp8_linears are not used).
 *   qkv   (device) act [batch * seq_len, (H + 2 Hk) * D]: q heads, k heads,
 *         v heads of each token (head-major columns), as the QK-norm and the
 *         value embedding leave them. bf16: q and k rows must have an RMS
 *         over head_dim of at most 1 (up to bf16 rounding), which the
 *         parameter-free QK-norm guarantees; the kernels take their softmax
 *         reference from that bound.
 *   out   (device) act [batch * seq_len, H * D], written (gpt_attn_fwd).
 *   lse2  (device) fp32 [batch, H, seq_len] + 64 elements of padding:
 *         log2 of each query's softmax denominator, written by
 *         gpt_attn_fwd, read by gpt_attn_bwd.
 *   g_out (device) act [batch * seq_len, H * D]: dL/dy.
 *   delta (device) fp32 [batch, H, seq_len] + 64 elements of padding:
 *         scratch, rowsum(g_out * out) per query.
 *   g_qkv (device) act [batch * seq_len, (H + 2 Hk) * D], written: dL/dq,
 *         dL/dk, dL/dv (k and v gradients summed over the query heads that
 *         share them).
 *   full  1: full causal context, 0: the short window.
 * act = the compute dtype; every pointer 16-byte aligned. Validation errors
 * return before anything is enqueued; the work is enqueued on `stream`.
 */
int gpt_attn_fwd(const gpt_config* cfg, int32_t full, const void* qkv, void* out, float* lse2,
                 void* stream);
int gpt_attn_bwd(const gpt_config* cfg, int32_t full, const void* qkv, const void* out,
                 const void* g_out, const float* lse2, float* delta, void* g_qkv, void* stream);

/*
 * Dynamic per-tensor fp8 quantisation of a row-major matrix: the operation
 * applied to every operand of the six block linears when fp8_linears = 1
 * (additions page, feature table: dynamic per-tensor fp8, e4m3 / e5m2;
 * overview page, section 4: quantise / dequantise around each scaled
 * matmul). amax = max |x| over the matrix; s = fmax / amax in fp32 (s = 1
 * if amax is 0 or not finite), fmax = 448 (e4m3) or 57344 (e5m2);
 * code = round-to-nearest-even of clamp(fp32(x * s), -fmax, fmax) in the
 * OCP encoding (sign, biased exponent, mantissa; e4m3 bias 7, e5m2 bias 15).
 *   src      (device) [rows, cols], fp32 (GPT_DT_F32) or bf16 (GPT_DT_BF16),
 *            16-byte aligned; cols a multiple of 64.
 *   fmt      0: e4m3, 1: e5m2.
 *   codes    (device) uint8 [rows, cols], written; may be NULL.
 *   codes_t  (device) uint8 [cols, pitch_t]: the transposed codes, written
 *            with zeros in columns rows .. pitch_t-1; may be NULL.
 *            pitch_t is a multiple of 128 and >= rows (ignored if NULL).
 *   amax     (device) uint32 [1]: the bit pattern of amax as fp32, written.
 * codes and codes_t 16-byte aligned. Enqueued on `stream`.
 */
int gpt_fp8_quantize(const void* src, int32_t src_dtype, int64_t rows, int64_t cols,
                     int32_t fmt, uint8_t* codes, uint8_t* codes_t, int64_t pitch_t,
                     uint32_t* amax, void* stream);

/*
 * One product of the fp8 block linears on given codes, with an fp32
 * output (test support: it pins the fp8 MFMA arithmetic apart from the
 * quantiser). "Nanochat在nanoGPT之上的新增功能", feature table: dynamic
 * per-tensor fp8, e4m3 / e5m2; "nanochat — 架构与原理", section 4: the
 * dequantisation after each scaled matmul.
 *   C[m][n] (+)= f(m, n) * sum_k a(A[m][k]) b(B[n][k])
 * with a, b the values of the byte codes (A in fmt_a, B in e4m3), both
 * operands K-major (A [M][lda], B [N][ldb]), and f = 1 / (s_a * s_b) of the
 * segment that (m, n) falls in: the segments cut the M (axis 0) or N
 * (axis 1) index at end[0] and end[1] (nseg of them), segment i takes the
 * amax slots slot_a[i] and slot_b[i] of `amax` (uint32 bit patterns of
 * fp32 amax values, as gpt_fp8_quantize writes them), and
 * s = fmax / amax in fp32 (1 if amax is 0 or not finite; fmax 448 for
 * e4m3, 57344 for e5m2). With axis 2 (wgrad = 0 only) the segments cut the
 * contraction instead (ends multiples of 16, at most K):
 *   C[m][n] (+)= sum over segments i of f_i * sum_{k in segment i} a b,
 * as the step's attention input gradient runs it (its q, k and v parts
 * carry their own scales); one launch that rescales its accumulators at
 * the segment ends when the tile plan allows (K and the ends multiples of
 * 128), else one product per segment.
 *   wgrad = 0: the product the step runs for forward and input-gradient
 *     linears; wgrad = 1: the weight-gradient product (K = tokens, split
 *     over workgroups with fp32 partials in `workspace`, then summed in a
 *     fixed order), which needs gpt_fp8_gemm_workspace bytes (0 for the
 *     plain product; workspace may then be NULL).
 *   C (device) fp32 [M][N], written (accumulate = 0) or added to.
 * K, lda, ldb multiples of 16 with lda, ldb >= K; N a multiple of 4;
 * A, B, C 16-byte aligned, amax 4, workspace 256. Validation errors return
 * before anything is enqueued; the work is enqueued on `stream`.
 */
typedef struct gpt_fp8_scales {
  int32_t axis;        /* 0: segments of M, 1: of N, 2: of K (wgrad = 0)   */
  int32_t nseg;        /* 1, 2 or 3                                         */
  int64_t end[2];      /* exclusive ends of segments 0 and 1 (ascending)    */
  int32_t slot_a[3];   /* amax slot of A in segment i                       */
  int32_t slot_b[3];   /* amax slot of B in segment i                       */
} gpt_fp8_scales;
int gpt_fp8_gemm_workspace(int32_t wgrad, int64_t M, int64_t N, int64_t K, size_t* bytes);
int gpt_fp8_gemm(int32_t wgrad, int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                 int32_t fmt_a, const uint8_t* B, int64_t ldb, const uint32_t* amax,
                 const gpt_fp8_scales* scales, int32_t accumulate, float* C, void* workspace,
                 size_t workspace_bytes, void* stream);

/*
 * The bf16 products of the step on their own, for element-wise tests of the
 * GEMM core (each runs the tiles, K-major or transposing operand paths and
 * split plan that the step uses for a product of that shape; the products
 * are the linear maps of the model, "Nanochat在nanoGPT之上的新增功能",
 * section 1 table: bias-free linears, untied lm_head):
 *   kind 0: C[M][N] = sum_k A[m][k] B[n][k]; A [M][K], B [N][K], both
 *           contraction-contiguous (the forward products, and the input
 *           gradients on the transposed weight copy);
 *   kind 1: the same product for a long contraction (the lm_head input
 *           gradient), split over K into fp32 partials added in split order
 *           when the plan splits it (gpt_bf16_gemm_workspace bytes);
 *   kind 2: C[M][N] (+)= sum_k A[k][m] B[k][n]; A [K][M], B [K][N] with K
 *           the tokens (the weight gradients), split over K as the step
 *           plans it, partials added in split order.
 *   A, B (device) bf16; C (device) fp32 [M][N], written (accumulate = 0) or,
 *   for kind 2 only, added to (accumulate = 1).
 * M >= 1 and N a multiple of 64; kinds 0 and 1: K a multiple of 64; kind 2:
 * M a multiple of 64, K >= 1. A, B, C 16-byte aligned, workspace 256 (may be
 * NULL when gpt_bf16_gemm_workspace reports 0). Validation errors return
 * before anything is enqueued; the work is enqueued on `stream`.
 */
int gpt_bf16_gemm_workspace(int32_t kind, int64_t M, int64_t N, int64_t K, size_t* bytes);
int gpt_bf16_gemm(int32_t kind, int64_t M, int64_t N, int64_t K, const void* A, const void* B,
                  int32_t accumulate, float* C, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * Decode attention over a KV cache: the attention step of generating one
 * token per sequence with a pre-allocated cache ("Nanochat在nanoGPT之上的新增
 * 功能", inference engine: KV cache, batch-1 prefill then the cache copied
 * per sample; "nanochat — 架构与原理", section 5: flash attention with a KV
 * cache). For sequence b the newest token sits at position
 * t = seqlen[b] - 1 (its k and v already written into the cache); query
 * head h reads KV head h / (n_head / n_kv_head) and attends the positions s
 * with max(0, t - window) <= s <= t (window = -1: 0 <= s <= t), with the
 * model's softmax(q k^T / sqrt(head_dim)) (additions page, notes on GQA
 * and the sliding window):
 *   out[b][h] = sum_s softmax_s(q[b][h] . k[b][s][h'] / sqrt(D)) v[b][s][h'].
 *   q        (device) bf16 [batch, n_head, head_dim] (after RoPE and QK-norm)
 *   k_cache, v_cache (device) bf16 [batch, max_len, n_kv_head, head_dim];
 *            rows at positions >= seqlen[b] are not read
 *   seqlen   (device) int32 [batch]; values are clamped to [1, max_len]
 *   out      (device) bf16 [batch, n_head, head_dim], written
 *   workspace (device) >= gpt_decode_attn_workspace bytes (may be NULL when
 *            that is 0): fp32 chunk states. The visible keys of each
 *            (sequence, KV head) are split into chunks of 128 positions
 *            whose states a second kernel combines in chunk order (one
 *            chunk, max_len or window + 1 <= 128: no workspace). Calls that
 *            share a workspace must not overlap.
 * head_dim 64 or 128; n_head a multiple of n_kv_head with at most 8 query
 * heads per KV head; window >= -1. q, caches and out 16-byte aligned,
 * seqlen 4, workspace 256. Validation errors return before anything is
 * enqueued; the work is enqueued on `stream`.
 */
int gpt_decode_attn_workspace(int32_t batch, int32_t n_head, int32_t n_kv_head, int32_t head_dim,
                              int32_t max_len, int32_t window, size_t* bytes);
int gpt_decode_attn(int32_t batch, int32_t n_head, int32_t n_kv_head, int32_t head_dim,
                    int32_t max_len, int32_t window, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* seqlen, void* out, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * gpt_decode_attn without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, rules and results as
 * gpt_decode_attn, minus the workspace: the chunk states live in a static
 * 4 MiB scratch array inside the library, one copy per GPU, held until the
 * process ends (its device address is looked up on the first call on each
 * device). Calls whose chunk states need more (gpt_decode_attn_workspace
 * above 4 MiB: batch * n_head * chunks above 8,065 at head_dim 128, above
 * 15,887 at head_dim 64; chunks = ceil(min(max_len, window + 1) / 128))
 * return GPT_E_WORKSPACE before anything is enqueued. The call allocates and frees nothing. Every call on a GPU
 * shares that GPU's scratch, so calls that overlap on one GPU (on
 * different streams, or from different threads) race; calls ordered on one
 * stream do not. Each call writes every chunk state it reads, so nothing
 * left by an earlier call is used.
 */
int gpt_decode_attn_noalloc(int32_t batch, int32_t n_head, int32_t n_kv_head, int32_t head_dim,
                            int32_t max_len, int32_t window, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* seqlen, void* out, void* stream);

/*
 * KV-cache append: writes the k and v rows of n_new tokens per sequence into
 * the caches gpt_decode_attn reads (prefill: the prompt's rows after a
 * forward; decode: the new token's). qkv holds one row per token, row
 * b * n_new + i for token i of sequence b, laid out as the model's fused
 * QKV product output: H query heads, then Hk key heads, then Hk value
 * heads, head_dim each (gpt_fwd leaves it, after RoPE, QK-norm and the
 * value embedding, in the per-layer workspace region "qkv").
 *   qkv      (device) bf16 [batch * n_new, (n_head + 2 n_kv_head) * head_dim]
 *   pos      (device) int32 [batch]: cache position of each sequence's first
 *            new token; token i goes to pos[b] + i, and rows falling outside
 *            [0, max_len) are not written
 *   k_cache, v_cache (device) bf16 [batch, max_len, n_kv_head, head_dim]
 * Same size rules as gpt_decode_attn (window not used); n_new >= 1. qkv and
 * caches 16-byte aligned, pos 4. Enqueued on `stream`.
 */
int gpt_kv_cache_append(int32_t batch, int32_t n_new, int32_t n_head, int32_t n_kv_head,
                        int32_t head_dim, int32_t max_len, const void* qkv, const int32_t* pos,
                        void* k_cache, void* v_cache, void* stream);

/*
 * MuonAdamW optimizer step ("NanoChat基础训练报告", optimizer block: Muon for
 * the matrices, AdamW for the rest; matrix rate 0.02, scalar 0.5, embedding
 * 0.3, unembedding 0.008, weight decay 0.28, a warmup / decay schedule;
 * "Nanochat在nanoGPT之上的新增功能", notes on Muon: momentum, then
 * Newton-Schulz orthogonalisation). The pages give neither the Newton-Schulz
 * coefficients nor the step count nor the Adam betas: they are fields here.
 * Groups (fixed by the library):
 *   Muon, rate lr_matrix: l.q, l.k, l.v, l.o, l.fc, l.mp of every layer;
 *     buf <- momentum buf + g; u = g + momentum buf (nesterov) or buf;
 *     X = u / (||u||_F + 1e-7), rows <= cols orientation (tall matrices
 *     transposed); ns_steps times X <- a X + (b A + c A^2) X, A = X X^T, in
 *     the compute dtype; p <- p (1 - lr weight_decay) - lr
 *     sqrt(max(1, rows / cols)) X.
 *   AdamW (no weight decay; bias-corrected with `step`): wte and l.ve at
 *     lr_embed, lm_head at lr_unembed, every other tensor (lambdas, l.veg,
 *     smear_gate, backout_lambda) at lr_scalar.
 * Every rate is multiplied by lr_mult (the caller's schedule).
 */
typedef struct gpt_optim_hparams {
  int32_t step;            /* 1, 2, ...: AdamW bias correction            */
  int32_t ns_steps;        /* Newton-Schulz iterations, [0, 100]           */
  int32_t nesterov;        /* 0 | 1                                        */
  float lr_matrix, lr_scalar, lr_embed, lr_unembed, lr_mult;
  float weight_decay;      /* Muon matrices                                */
  float beta1, beta2, eps; /* AdamW, betas in [0, 1)                       */
  float momentum;          /* Muon                                         */
  float ns_a, ns_b, ns_c;  /* Newton-Schulz coefficients                   */
} gpt_optim_hparams;

/* Host only. Bytes of device workspace gpt_optimizer_step needs. */
int gpt_optim_workspace_size(const gpt_config* cfg, size_t* bytes);

/*
 * One optimizer step, in place.
 *   params (device) fp32 [n_elems], canonical layout; updated.
 *   grads  (device) fp32 [n_elems]; read only.
 *   state  (device) fp32 [2 * n_elems]: first n_elems the AdamW first moment
 *          or the Muon momentum buffer, then the AdamW second moment; zero
 *          before step 1; updated.
 *   workspace (device) >= gpt_optim_workspace_size bytes; scratch.
 * params, grads, state and workspace 256-byte aligned. Validation errors
 * return before anything is enqueued; the work is enqueued on `stream`
 * (the Muon matrices of equal shape run as batched launches). Concurrent
 * calls need distinct workspaces.
 */
int gpt_optimizer_step(const gpt_config* cfg, const gpt_optim_hparams* hp, float* params,
                       const float* grads, float* state, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Host only; measurement support. After gpt_profile_begin(prefixes), every
 * kernel launch of gpt_fwd_bwd / gpt_fwd whose launch-site name starts with
 * one of the comma-separated `prefixes` is bracketed by two HIP events
 * recorded on the call's stream.
 * Site names: "embed.fwd", "gemm.qkv.fwd", "rope.fwd", "attn.fwd",
 * "gemm.o.fwd", "gemm.fc.fwd", "gemm.mp.fwd", "gemm.lm.fwd", "loss",
 * "gemm.lm.dgrad", "gemm.lm.wgrad", "gemm.mp.dgrad", "gemm.mp.wgrad",
 * "gemm.fc.dgrad", "gemm.fc.wgrad", "gemm.o.dgrad", "gemm.o.wgrad",
 * "attn.delta", "attn.bwd", "gemm.qkv.dgrad", "gemm.qkv.wgrad", "embed.bwd",
 * and with fp8 linears "fp8.weights" (weight amax + codes) and "fp8.quant"
 * (amax + codes of an activation or gradient).
 * gpt_profile_end waits for the recorded events, returns the summed
 * kernel time in milliseconds and the number of bracketed launches, and
 * stops recording. Process-wide state: not for concurrent callers. While
 * it is active, calls with GPT_F_GRAPH run eagerly.
 */
int gpt_profile_begin(const char* site_prefix);
int gpt_profile_end(double* total_ms, int64_t* launches);

/*
 * Host only; test support for the error path. For the calling thread's
 * later entry-point calls: fail_at >= 0 makes launch number fail_at
 * (0-based) of each call fail as if the HIP runtime had refused it (it is
 * not launched, nor is any later launch of the call, and the call returns
 * GPT_E_HIP); fail_at < 0 turns this off. dry_run = 1 counts the launch
 * sequence without launching anything (device pointers are then never
 * used, and the debug checks' synchronisations are skipped), so the host
 * logic of a call can run on a machine without a GPU. Both default to off.
 * gpt_debug_launch_count gives the number of launches the thread's last
 * entry-point call issued (counted, in a dry run).
 */
int gpt_debug_launches(int64_t fail_at, int32_t dry_run);
int gpt_debug_launch_count(int64_t* issued);

/* Drops every cached HIP graph (GPT_F_GRAPH) after synchronising the
 * device; host only. */
int gpt_graph_cache_clear(void);

/* Static text for a status code. */
const char* gpt_status_string(int status);

/* Per-thread detail of the last error ("" if none). */
const char* gpt_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GPT_STEP_H */
