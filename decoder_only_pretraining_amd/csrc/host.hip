// Host side of the GPT step library: config validation, the canonical
// parameter layout, the workspace plan, the launch sequence of one forward +
// backward pass, and the extern "C" entry points declared in gpt_step.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <initializer_list>
#include <map>
#include <mutex>

#include "internal.h"

namespace gpt {

static thread_local char g_err[512] = "";

static int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

// ---------------------------------------------------------------- launches
static thread_local LaunchState g_launch;
LaunchState& launch_state() { return g_launch; }
void launch_reset() {
  g_launch.err = hipSuccess;
  g_launch.injected = false;
  g_launch.issued = 0;
  if (!g_launch.dry) (void)hipGetLastError();  // drop an error left by earlier work
}
bool launch_begin() {
  LaunchState& st = g_launch;
  if (st.err != hipSuccess) return false;
  if (st.fail_at >= 0 && st.issued == st.fail_at) {
    st.err = hipErrorLaunchFailure;
    st.injected = true;
    return false;
  }
  ++st.issued;
  return !st.dry;
}
void launch_end() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess && g_launch.err == hipSuccess) g_launch.err = e;
}
// status of the current call's launches: GPT_OK or GPT_E_HIP with the detail
static int launch_status() {
  const LaunchState& st = g_launch;
  if (st.err == hipSuccess) return GPT_OK;
  if (st.injected)
    return fail(GPT_E_HIP, "HIP: injected launch failure at launch %lld (nothing later enqueued)",
                (long long)st.issued);
  return fail(GPT_E_HIP, "HIP: %s at launch %lld (nothing later enqueued)", hipGetErrorString(st.err),
              (long long)st.issued);
}

// ---------------------------------------------------------------- profiling
// When enabled, every launch whose site name starts with the chosen prefix is
// bracketed by two HIP events recorded on the launch stream. Events come from
// a pool that grows on demand and is reused across calls.
struct Profiler {
  std::mutex mu;
  bool on = false;
  std::string prefix;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
};
static Profiler g_prof;

// Does `name` start with one of the comma-separated prefixes?
static bool site_selected(const char* name) {
  const std::string& p = g_prof.prefix;
  size_t b = 0;
  while (b <= p.size()) {
    size_t e = p.find(',', b);
    if (e == std::string::npos) e = p.size();
    if (e > b && strncmp(name, p.c_str() + b, e - b) == 0) return true;
    b = e + 1;
  }
  return false;
}

template <class Fn>
static void site(const char* name, hipStream_t s, Fn&& fn) {
  if (g_prof.on && site_selected(name)) {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    while (g_prof.pool.size() < g_prof.used + 2) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) {
        fn();
        return;
      }
      g_prof.pool.push_back(e);
    }
    hipEvent_t a = g_prof.pool[g_prof.used], b = g_prof.pool[g_prof.used + 1];
    g_prof.used += 2;
    (void)hipEventRecord(a, s);
    fn();
    (void)hipEventRecord(b, s);
  } else {
    fn();
  }
}

// Sliding-window pattern: three short-window layers then one full layer,
// tiled over depth, with the last layer always full ("Nanochat在nanoGPT之上
// 的新增功能", notes on the sliding window).
bool layer_full(int l, int L) { return (l % 4 == 3) || (l == L - 1); }
// Value embeddings on every other layer, the last one included (same page,
// notes on value residuals).
bool layer_ve(int l, int L) { return (l % 2) == ((L - 1) % 2); }

Dims make_dims(const gpt_config& c) {
  Dims d{};
  d.L = c.n_layer;
  d.C = c.n_embd;
  d.H = c.n_head;
  d.Hk = c.n_kv_head;
  d.D = c.head_dim;
  d.F = c.mlp_hidden;
  d.V = c.vocab;
  d.T = c.seq_len;
  d.B = c.batch;
  d.W = c.short_window;
  d.N = (int64_t)c.batch * c.seq_len;
  d.Cq = d.H * d.D;
  d.Ckv = d.Hk * d.D;
  d.Qkv = d.Cq + 2 * d.Ckv;
  d.G = d.Hk > 0 ? d.H / d.Hk : 0;
  d.bf16 = c.compute_dtype == GPT_DT_BF16;
  d.fp8 = c.fp8_linears != 0;
  d.act_bytes = d.bf16 ? 2 : 4;
  d.theta = c.rope_theta;
  d.eps = c.norm_eps;
  d.cap = c.softcap;
  d.accumulate = (c.flags & GPT_F_ACCUMULATE) != 0;
  d.smear = (c.flags & GPT_F_SMEAR) != 0;
  d.backout = (c.flags & GPT_F_BACKOUT) != 0;
  d.mid = d.L / 2;
  d.reuse_weights = (c.flags & GPT_F_REUSE_WEIGHTS) != 0;
  d.check_finite = (c.flags & GPT_F_CHECK_FINITE) != 0;
  d.check_inputs = (c.flags & GPT_F_CHECK_INPUTS) != 0;
  return d;
}

static int validate(const gpt_config* c) {
  if (!c) return fail(GPT_E_NULLPTR, "config is NULL");
  if (c->abi_version != GPT_ABI_VERSION)
    return fail(GPT_E_INVAL, "abi_version %d != %d", c->abi_version, GPT_ABI_VERSION);
  if (c->n_layer < 1 || c->n_layer > 256) return fail(GPT_E_INVAL, "n_layer %d not in [1, 256]", c->n_layer);
  if (c->n_embd < 64 || c->n_embd > 2048 || c->n_embd % 64)
    return fail(GPT_E_INVAL, "n_embd %d: need a multiple of 64 in [64, 2048]", c->n_embd);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(GPT_E_INVAL, "head_dim %d: need 64 or 128", c->head_dim);
  if (c->n_head < 1 || c->n_kv_head < 1 || c->n_kv_head > 16 || c->n_head % c->n_kv_head)
    return fail(GPT_E_INVAL, "n_head %d / n_kv_head %d: need n_kv_head in [1, 16] dividing n_head",
                c->n_head, c->n_kv_head);
  if ((int64_t)c->n_head * c->head_dim > 16384) return fail(GPT_E_INVAL, "n_head * head_dim too large");
  if (c->mlp_hidden < 64 || c->mlp_hidden % 64 || c->mlp_hidden > 65536)
    return fail(GPT_E_INVAL, "mlp_hidden %d: need a multiple of 64 in [64, 65536]", c->mlp_hidden);
  if (c->vocab < 64 || c->vocab % 64 || c->vocab > (1 << 24))
    return fail(GPT_E_INVAL, "vocab %d: need a multiple of 64 in [64, 2^24]", c->vocab);
  if (c->seq_len < 1 || c->batch < 1) return fail(GPT_E_INVAL, "seq_len and batch must be >= 1");
  const int64_t N = (int64_t)c->seq_len * c->batch;
  if (N > (1 << 22)) return fail(GPT_E_INVAL, "batch * seq_len = %lld exceeds 2^22", (long long)N);
  if (c->short_window < 0) return fail(GPT_E_INVAL, "short_window %d < 0", c->short_window);
  if (c->compute_dtype != GPT_DT_F32 && c->compute_dtype != GPT_DT_BF16)
    return fail(GPT_E_INVAL, "compute_dtype %d unknown", c->compute_dtype);
  if (c->fp8_linears != 0 && c->fp8_linears != 1) return fail(GPT_E_INVAL, "fp8_linears must be 0 or 1");
  if (c->flags & ~(GPT_F_ACCUMULATE | GPT_F_EMBED_NORM | GPT_F_CHECK_FINITE | GPT_F_CHECK_INPUTS |
                   GPT_F_SMEAR | GPT_F_BACKOUT | GPT_F_REUSE_WEIGHTS | GPT_F_GRAPH))
    return fail(GPT_E_INVAL, "unknown flag bits 0x%x", c->flags);
  if (!(std::isfinite(c->rope_theta) && c->rope_theta > 1.0f))
    return fail(GPT_E_INVAL, "rope_theta must be finite and > 1");
  if (!(std::isfinite(c->norm_eps) && c->norm_eps > 0.0f)) return fail(GPT_E_INVAL, "norm_eps must be > 0");
  if (!(std::isfinite(c->softcap) && c->softcap > 0.0f)) return fail(GPT_E_INVAL, "softcap must be > 0");
  if (c->fp8_linears && c->compute_dtype != GPT_DT_BF16)
    return fail(GPT_E_INVAL, "fp8 linears need bf16 compute");
  if (c->flags & GPT_F_EMBED_NORM)
    return fail(GPT_E_UNSUPPORTED, "GPT_F_EMBED_NORM: no embedding norm is built into this library");
  return GPT_OK;
}

std::vector<TensorInfo> param_layout(const gpt_config& c) {
  const Dims d = make_dims(c);
  std::vector<TensorInfo> v;
  int64_t o = 0;
  auto add = [&](const std::string& name, int64_t r, int64_t cc) {
    v.push_back({name, o, r, cc});
    o += r * cc;
  };
  add("wte", d.V, d.C);
  for (int l = 0; l < d.L; ++l) {
    const std::string p = "l" + std::to_string(l) + ".";
    add(p + "q", d.Cq, d.C);
    add(p + "k", d.Ckv, d.C);
    add(p + "v", d.Ckv, d.C);
    add(p + "o", d.C, d.Cq);
    add(p + "fc", d.F, d.C);
    add(p + "mp", d.C, d.F);
    if (layer_ve(l, d.L)) {
      add(p + "ve", d.V, d.Ckv);
      add(p + "veg", d.Hk, d.C);
    }
  }
  add("lm_head", d.V, d.C);
  if (d.smear) add("smear_gate", 1, d.C);
  if (d.backout) add("backout_lambda", 1, 1);
  add("resid_lambdas", d.L, 1);
  add("x0_lambdas", d.L, 1);
  return v;
}

static size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

Plan make_plan(const Dims& d) {
  Plan p{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t r = o;
    o += al(bytes);
    return r;
  };
  const size_t N = (size_t)d.N, A = (size_t)d.act_bytes;
  int64_t n_elems = 0;
  {
    // total parameter count, same walk as param_layout
    n_elems = (int64_t)d.V * d.C * 2 + 2 * d.L + (d.smear ? d.C : 0) + (d.backout ? 1 : 0);
    for (int l = 0; l < d.L; ++l) {
      n_elems += (int64_t)d.Qkv * d.C + (int64_t)d.C * d.Cq + 2 * (int64_t)d.F * d.C;
      if (layer_ve(l, d.L)) n_elems += (int64_t)d.V * d.Ckv + (int64_t)d.Hk * d.C;
    }
  }
  p.wc = take(d.bf16 ? (size_t)n_elems * 2 : 0);
  p.wct = take(d.bf16 ? (size_t)n_elems * 2 : 0);
  p.rope = take((size_t)d.T * d.D * 4);
  p.x = take((size_t)(d.L + 1) * N * d.C * 4);
  p.xin = take(N * d.C * 4);
  // per-layer saved activations
  size_t lo = 0;
  auto ltake = [&](size_t bytes) {
    const size_t r = lo;
    lo += al(bytes);
    return r;
  };
  p.l_xn = ltake(N * d.C * A);
  p.l_r1 = ltake(N * 4);
  p.l_qkv = ltake(N * d.Qkv * A);
  p.l_rqk = ltake(N * (d.H + d.Hk) * 4);
  p.l_a = ltake(N * d.Hk * 4);
  p.l_attn = ltake(N * d.Cq * A);
  p.l_lse = ltake(N * d.H * 4 + 256);  // [B][H][T]; the pad covers 16-byte tile reads past T
  p.l_xmid = ltake(N * d.C * 4);
  p.l_xn2 = ltake(N * d.C * A);
  p.l_r2 = ltake(N * 4);
  p.l_u = ltake(N * d.F * A);
  if (d.fp8) {  // transposed activation codes for the weight gradients
    const size_t Np = (size_t)((d.N + 127) / 128 * 128);
    p.l_x8t = ltake(d.C * Np);
    p.l_a8t = ltake(d.Cq * Np);
    p.l_x28t = ltake(d.C * Np);
    p.l_h8t = ltake(d.F * Np);
  }
  p.layer_bytes = lo;
  p.layers = take(lo * d.L);
  p.xf = take(N * d.C * A);
  p.rf = take(N * 4);
  p.logits = take(N * d.V * A);
  p.lossrow = take(N * 4);
  p.scalars = take(256);
  p.gx = take(N * d.C * 4);
  p.gxc = take(N * d.C * A);
  p.gx0 = take(N * d.C * 4);
  p.gu = take(N * d.F * A);
  p.gtmp = take(N * d.C * 4);
  p.gO = take(N * d.Cq * A);
  p.gqkv = take(N * d.Qkv * A);
  p.delta = take(N * d.H * 4 + 256);  // [B][H][T], padded like lse
  p.ga = take(N * d.Hk * 4);
  p.lam_blocks = (int)((d.N + 3) / 4);
  // one slot per layer, and one for the final norm's mix under Backout
  p.lam_part = take((size_t)(d.L + (d.backout ? 1 : 0)) * p.lam_blocks * 2 * 4);
  p.veg_splits = veg_splits(d.N);
  p.veg_part = take((size_t)p.veg_splits * d.Hk * d.C * 4);
  p.vegrow = take(N * d.Ckv * 4);  // every model has a value-embedding layer (the last)
  p.tlink = take(2 * N * 4);
  p.sgate = take(d.smear ? N * 4 : 0);
  {  // split-K partials: the largest over the step's split products
    int64_t pb = std::max(part_bytes_nn_splitk(d, d.N, d.C, d.V),
                          part_bytes_tn_wgrad(d, d.V, d.C, d.N));
    const int64_t shapes[4][2] = {{d.Qkv, d.C}, {d.C, d.Cq}, {d.F, d.C}, {d.C, d.F}};
    for (const auto& mn : shapes) {
      pb = std::max(pb, part_bytes_tn_wgrad(d, mn[0], mn[1], d.N));
      if (d.fp8) pb = std::max(pb, part_bytes_f8_wgrad(mn[0], mn[1], (d.N + 15) / 16 * 16));
    }
    p.part_bytes = pb;
    p.part = take((size_t)pb);
  }
  if (d.fp8) {
    auto P128 = [](int64_t x) { return (size_t)((x + 127) / 128 * 128); };
    const size_t C = d.C, Cq = d.Cq, F = d.F, Qkv = d.Qkv;
    p.Np = (int64_t)P128(d.N);
    const size_t Np = (size_t)p.Np;
    p.amax = take((size_t)16 * d.L * 4);
    p.w8_layer = al(Qkv * C + C * Cq + F * C + C * F);
    p.w8 = take(p.w8_layer * d.L);
    p.w8t_layer = al(C * P128(Qkv) + Cq * P128(C) + C * P128(F) + F * P128(C));
    p.w8t = take(p.w8t_layer * d.L);
    const size_t wmax = std::max(std::max(C, Cq), std::max(F, Qkv));
    p.q8 = take(N * wmax);
    p.g8t = take(std::max(std::max(C, F), Qkv) * Np);
  }
  p.total = o;
  return p;
}

struct Offs {
  int64_t wte, lm, lr, l0, sm = -1, bo = -1;
  std::vector<int64_t> q, o, fc, mp, ve, veg;
};

static Offs offsets(const gpt_config& c) {
  Offs f;
  const int L = c.n_layer;
  f.q.assign(L, -1);
  f.o.assign(L, -1);
  f.fc.assign(L, -1);
  f.mp.assign(L, -1);
  f.ve.assign(L, -1);
  f.veg.assign(L, -1);
  for (const auto& t : param_layout(c)) {
    const std::string& n = t.name;
    if (n == "wte") f.wte = t.offset;
    else if (n == "lm_head") f.lm = t.offset;
    else if (n == "resid_lambdas") f.lr = t.offset;
    else if (n == "x0_lambdas") f.l0 = t.offset;
    else if (n == "smear_gate") f.sm = t.offset;
    else if (n == "backout_lambda") f.bo = t.offset;
    else {
      const size_t dot = n.find('.');
      const int l = std::stoi(n.substr(1, dot - 1));
      const std::string k = n.substr(dot + 1);
      if (k == "q") f.q[l] = t.offset;
      else if (k == "o") f.o[l] = t.offset;
      else if (k == "fc") f.fc[l] = t.offset;
      else if (k == "mp") f.mp[l] = t.offset;
      else if (k == "ve") f.ve[l] = t.offset;
      else if (k == "veg") f.veg[l] = t.offset;
    }
  }
  return f;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static int run(const gpt_config* cfg, const float* params, const int32_t* tokens,
               const int32_t* targets, float* loss, float* grads, void* workspace,
               size_t workspace_bytes, void* stream, bool backward) {
  g_err[0] = 0;
  int st = validate(cfg);
  if (st) return st;
  if (!params || !tokens || !targets || !loss || !workspace || (backward && !grads))
    return fail(GPT_E_NULLPTR, "a required pointer is NULL");
  if (!aligned(params, 256) || !aligned(workspace, 256) || (backward && !aligned(grads, 256)) ||
      !aligned(tokens, 4) || !aligned(targets, 4) || !aligned(loss, 4))
    return fail(GPT_E_ALIGN, "params/grads/workspace need 256-byte alignment, tokens/targets/loss 4");
  const Dims d = make_dims(*cfg);
  const Plan P = make_plan(d);
  if (workspace_bytes < P.total)
    return fail(GPT_E_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, P.total);
  const Offs F = offsets(*cfg);
  // the split-K partial region holds every split product of the step (a
  // shortfall would be a planning error of this library)
  {
    int64_t need = std::max(part_bytes_nn_splitk(d, d.N, d.C, d.V), part_bytes_tn_wgrad(d, d.V, d.C, d.N));
    const int64_t shapes[4][2] = {{d.Qkv, d.C}, {d.C, d.Cq}, {d.F, d.C}, {d.C, d.F}};
    for (const auto& mn : shapes) {
      need = std::max(need, part_bytes_tn_wgrad(d, mn[0], mn[1], d.N));
      if (d.fp8) need = std::max(need, part_bytes_f8_wgrad(mn[0], mn[1], (d.N + 15) / 16 * 16));
    }
    if (need > P.part_bytes)
      return fail(GPT_E_WORKSPACE, "internal: split-K partials need %lld bytes, the plan holds %lld",
                  (long long)need, (long long)P.part_bytes);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_reset();

  char* W = static_cast<char*>(workspace);
  // debug flags in the scalars region: [8], [9] id checks, [10] finiteness
  uint32_t* dbg = reinterpret_cast<uint32_t*>(W + P.scalars) + 8;
  // device values of the debug checks, after an internal synchronisation
  auto read_flags = [&](uint32_t* host, const uint32_t* dev, int n) -> int {
    if (launch_state().dry) {
      for (int i = 0; i < n; ++i) host[i] = 0;
      return GPT_OK;
    }
    int st2 = launch_status();
    if (st2) return st2;
    hipError_t e = hipMemcpyAsync(host, dev, n * sizeof(uint32_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(GPT_E_HIP, "HIP: %s (debug check)", hipGetErrorString(e));
    return GPT_OK;
  };
  if (d.check_inputs) {
    launch_check_ids(tokens, targets, d.N, d.V, dbg, s);
    uint32_t bad[2];
    const int st2 = read_flags(bad, dbg, 2);
    if (st2) return st2;
    if (bad[0] || bad[1])
      return fail(GPT_E_INVAL, "%u token ids outside [0, %d), %u targets outside [-1, %d)", bad[0],
                  d.V, bad[1], d.V);
  }
  const size_t A = (size_t)d.act_bytes;
  // compute-dtype weights: a mirror of params with the same element offsets
  const char* wc = d.bf16 ? W + P.wc : reinterpret_cast<const char*>(params);
  auto wmat = [&](int64_t off) { return static_cast<const void*>(wc + off * A); };
  // bf16: transposed copies of the linear weights, so the input-gradient
  // products run with both operands K-major (nullptr: not kept)
  auto wmatT = [&](int64_t off) -> const void* {
    return d.bf16 ? static_cast<const void*>(W + P.wct + off * 2) : nullptr;
  };
  if (d.bf16 && !d.reuse_weights) {
    std::vector<CastSeg> segs;
    for (int l = 0; l < d.L; ++l)
      if (F.veg[l] >= 0) segs.push_back({F.veg[l], (int64_t)d.Hk * d.C});
    if (!segs.empty()) launch_cast(params, W + P.wc, segs, s);
    if (!d.fp8) {
      std::vector<int64_t> q(d.L), o(d.L), fc(d.L), mp(d.L);
      for (int l = 0; l < d.L; ++l) q[l] = F.q[l], o[l] = F.o[l], fc[l] = F.fc[l], mp[l] = F.mp[l];
      launch_cast_t(params, W + P.wc, W + P.wct, q, d.Qkv, d.C, s);
      launch_cast_t(params, W + P.wc, W + P.wct, o, d.C, d.Cq, s);
      launch_cast_t(params, W + P.wc, W + P.wct, fc, d.F, d.C, s);
      launch_cast_t(params, W + P.wc, W + P.wct, mp, d.C, d.F, s);
    }
    launch_cast_t(params, W + P.wc, W + P.wct, {F.lm}, d.V, d.C, s);
  }
  float* cs = reinterpret_cast<float*>(W + P.rope);
  launch_rope_table(cs, d.T, d.D, d.theta, s);

  const size_t xstride = (size_t)d.N * d.C;
  auto X = [&](int l) { return reinterpret_cast<float*>(W + P.x) + (size_t)l * xstride; };
  auto LY = [&](int l, size_t off) { return W + P.layers + (size_t)l * P.layer_bytes + off; };
  auto LY8 = [&](int l, size_t off) { return reinterpret_cast<uint8_t*>(LY(l, off)); };
  float* xin = reinterpret_cast<float*>(W + P.xin);
  const int64_t N = d.N;

  // ---- fp8 linears: amax slots 16 l + {0..5: W q k v o fc mp; 6..9: inputs
  // xn, attn, xn2, h; 10..15: output gradients of mp, fc, o, q, k, v}
  uint32_t* amax = d.fp8 ? reinterpret_cast<uint32_t*>(W + P.amax) : nullptr;
  uint8_t* q8 = d.fp8 ? reinterpret_cast<uint8_t*>(W + P.q8) : nullptr;
  uint8_t* g8t = d.fp8 ? reinterpret_cast<uint8_t*>(W + P.g8t) : nullptr;
  const int64_t Np = P.Np, Nk = (N + 15) / 16 * 16;  // code pitch / K of token contractions
  auto P128 = [](int64_t x) { return (x + 127) / 128 * 128; };
  auto slot = [](int l, int k) { return 16 * l + k; };
  // per-layer fp8 weights: row-major for the forward, transposed for dgrad
  auto w8 = [&](int l, int which) {
    uint8_t* b = reinterpret_cast<uint8_t*>(W + P.w8 + (size_t)l * P.w8_layer);
    const int64_t C = d.C, Cq = d.Cq, Fh = d.F, Qkv = d.Qkv;
    const int64_t off[4] = {0, Qkv * C, Qkv * C + C * Cq, Qkv * C + C * Cq + Fh * C};
    return b + off[which];
  };
  auto w8t = [&](int l, int which) {
    uint8_t* b = reinterpret_cast<uint8_t*>(W + P.w8t + (size_t)l * P.w8t_layer);
    const int64_t C = d.C, Cq = d.Cq, Fh = d.F, Qkv = d.Qkv;
    const int64_t o1 = C * P128(Qkv), o2 = o1 + Cq * P128(C), o3 = o2 + C * P128(Fh);
    const int64_t off[4] = {0, o1, o2, o3};
    return b + off[which];
  };
  auto segs3 = [&](int64_t e0, int64_t e1, int s0, int s1, int s2) {
    Segs g{};
    g.n = 3;
    g.end[0] = e0;
    g.end[1] = e1;
    g.end[2] = INT64_MAX;
    g.slot[0] = s0;
    g.slot[1] = s1;
    g.slot[2] = s2;
    return g;
  };
  // dequantisation of a product: one segment, or three along `axis`
  auto deq1 = [&](int sa, int sb, int fa) {
    Fp8Deq q{};
    q.amax = amax;
    q.axis = 1;
    q.nseg = 1;
    q.sa[0] = sa;
    q.sb[0] = sb;
    q.fa = fa;
    q.fb = FP8_E4M3;
    return q;
  };
  auto deq3 = [&](int axis, int sa0, int sa1, int sa2, int sb0, int sb1, int sb2, int fa) {
    Fp8Deq q{};
    q.amax = amax;
    q.axis = axis;
    q.nseg = 3;
    q.end[0] = d.Cq;
    q.end[1] = d.Cq + d.Ckv;
    q.end[2] = INT64_MAX;
    q.sa[0] = sa0; q.sa[1] = sa1; q.sa[2] = sa2;
    q.sb[0] = sb0; q.sb[1] = sb1; q.sb[2] = sb2;
    q.fa = fa;
    q.fb = FP8_E4M3;
    return q;
  };
  // amax, then codes of a token-major tensor [N][cols]: row-major into q8,
  // transposed into outT (backward calls only)
  auto quant_tok = [&](const void* src, bool bf, int64_t cols, const Segs& sg, int fmt,
                       uint8_t* outT) {
    launch_fp8_amax(src, bf, N * cols, cols, sg, amax, s);
    launch_fp8_quant(src, bf, N, cols, false, sg, amax, fmt, q8, backward ? outT : nullptr, Np, s);
  };
  // codes of a tensor whose producer already merged its amax into the slot
  auto quant_only = [&](const void* src, int64_t cols, const Segs& sg, int fmt, uint8_t* outT) {
    launch_fp8_quant(src, true, N, cols, false, sg, amax, fmt, q8, backward ? outT : nullptr, Np, s);
  };
  if (d.fp8) {
    launch_zero(reinterpret_cast<float*>(amax), 16 * d.L, s);
    site("fp8.weights", s, [&] {
      for (int l = 0; l < d.L; ++l) {
        const int64_t C = d.C, Cq = d.Cq, Ckv = d.Ckv, Fh = d.F;
        Segs g{};
        g.n = 6;
        const int64_t ends[6] = {Cq * C, (Cq + Ckv) * C, (Cq + 2 * Ckv) * C,
                                 (Cq + 2 * Ckv) * C + C * Cq, (Cq + 2 * Ckv) * C + C * Cq + Fh * C,
                                 INT64_MAX};
        for (int k = 0; k < 6; ++k) {
          g.end[k] = ends[k];
          g.slot[k] = slot(l, k);
        }
        const int64_t n = F.mp[l] + C * Fh - F.q[l];
        launch_fp8_amax(params + F.q[l], false, n, n, g, amax, s);
        const Segs gq = segs3(Cq, Cq + Ckv, slot(l, 0), slot(l, 1), slot(l, 2));
        launch_fp8_quant(params + F.q[l], false, d.Qkv, C, true, gq, amax, FP8_E4M3, w8(l, 0),
                         backward ? w8t(l, 0) : nullptr, P128(d.Qkv), s);
        launch_fp8_quant(params + F.o[l], false, C, Cq, true, one_seg(slot(l, 3)), amax, FP8_E4M3,
                         w8(l, 1), backward ? w8t(l, 1) : nullptr, P128(C), s);
        launch_fp8_quant(params + F.fc[l], false, Fh, C, true, one_seg(slot(l, 4)), amax,
                         FP8_E4M3, w8(l, 2), backward ? w8t(l, 2) : nullptr, P128(Fh), s);
        launch_fp8_quant(params + F.mp[l], false, C, Fh, true, one_seg(slot(l, 5)), amax,
                         FP8_E4M3, w8(l, 3), backward ? w8t(l, 3) : nullptr, P128(C), s);
      }
    });
  }

  float* sgate = reinterpret_cast<float*>(W + P.sgate);
  site("embed.fwd", s, [&] {
    if (d.smear)
      launch_smear_embed(d, params + F.wte, tokens, params + F.sm, X(0), sgate, s);
    else
      launch_embed(params + F.wte, tokens, X(0), N, d.C, d.V, s);
  });
  for (int l = 0; l < d.L; ++l) {
    const bool ve = layer_ve(l, d.L), full = layer_full(l, d.L);
    void* xn = LY(l, P.l_xn);
    float* r1 = reinterpret_cast<float*>(LY(l, P.l_r1));
    void* qkv = LY(l, P.l_qkv);
    float* rqk = reinterpret_cast<float*>(LY(l, P.l_rqk));
    float* a = reinterpret_cast<float*>(LY(l, P.l_a));
    void* att = LY(l, P.l_attn);
    float* lse = reinterpret_cast<float*>(LY(l, P.l_lse));
    float* xmid = reinterpret_cast<float*>(LY(l, P.l_xmid));
    void* xn2 = LY(l, P.l_xn2);
    float* r2 = reinterpret_cast<float*>(LY(l, P.l_r2));
    void* u = LY(l, P.l_u);
    launch_mix_norm(d, X(l), X(0), params + F.lr + l, params + F.l0 + l, xin, xn, r1,
                    ve ? params + F.veg[l] : nullptr, ve ? a : nullptr, s);
    if (d.fp8) {
      site("fp8.quant", s, [&] { quant_tok(xn, true, d.C, one_seg(slot(l, 6)), FP8_E4M3, LY8(l, P.l_x8t)); });
      site("gemm.qkv.fwd", s, [&] {
        gemm8_store(N, d.Qkv, d.C, q8, d.C, w8(l, 0), d.C,
                    deq3(1, slot(l, 6), slot(l, 6), slot(l, 6), slot(l, 0), slot(l, 1), slot(l, 2),
                         FP8_E4M3), qkv, s);
      });
    } else {
      site("gemm.qkv.fwd", s, [&] { gemm_nt_store(d, N, d.Qkv, d.C, xn, wmat(F.q[l]), qkv, s); });
    }
    site("rope.fwd", s, [&] { launch_rope_qk_ve_fwd(d, qkv, rqk, cs, a, ve ? params + F.ve[l] : nullptr, tokens, s); });
    site("attn.fwd", s, [&] { launch_attn_fwd(d, full, qkv, att, lse, s); });
    if (d.fp8) {
      site("fp8.quant", s, [&] { quant_tok(att, true, d.Cq, one_seg(slot(l, 7)), FP8_E4M3, LY8(l, P.l_a8t)); });
      site("gemm.o.fwd", s, [&] {
        gemm8_resid(N, d.C, d.Cq, q8, d.Cq, w8(l, 1), d.Cq, deq1(slot(l, 7), slot(l, 3), FP8_E4M3),
                    xin, xmid, s);
      });
    } else {
      site("gemm.o.fwd", s, [&] { gemm_nt_resid(d, N, d.C, d.Cq, att, wmat(F.o[l]), xin, xmid, s); });
    }
    launch_mix_norm(d, xmid, nullptr, nullptr, nullptr, nullptr, xn2, r2, nullptr, nullptr, s);
    if (d.fp8) {
      site("fp8.quant", s, [&] { quant_tok(xn2, true, d.C, one_seg(slot(l, 8)), FP8_E4M3, LY8(l, P.l_x28t)); });
      site("gemm.fc.fwd", s, [&] {
        gemm8_relu2(N, d.F, d.C, q8, d.C, w8(l, 2), d.C, deq1(slot(l, 8), slot(l, 4), FP8_E4M3), u,
                    amax + slot(l, 9), s);
      });
      site("fp8.quant", s, [&] { quant_only(u, d.F, one_seg(slot(l, 9)), FP8_E4M3, LY8(l, P.l_h8t)); });
      site("gemm.mp.fwd", s, [&] {
        gemm8_resid(N, d.C, d.F, q8, d.F, w8(l, 3), d.F, deq1(slot(l, 9), slot(l, 5), FP8_E4M3),
                    xmid, X(l + 1), s);
      });
    } else {
      site("gemm.fc.fwd", s, [&] { gemm_nt_relu2(d, N, d.F, d.C, xn2, wmat(F.fc[l]), u, s); });
      site("gemm.mp.fwd", s, [&] { gemm_nt_resid(d, N, d.C, d.F, u, wmat(F.mp[l]), xmid, X(l + 1), s); });
    }
  }
  void* xf = W + P.xf;
  float* rf = reinterpret_cast<float*>(W + P.rf);
  void* logits = W + P.logits;
  float* lossrow = reinterpret_cast<float*>(W + P.lossrow);
  float* scalars = reinterpret_cast<float*>(W + P.scalars);
  // Backout: the final norm reads x - lambda * x_mid, a mix with weights
  // (1, -lambda) kept in scalars[4], scalars[5]
  float* bo_w = scalars + 4;
  if (d.backout) {
    launch_backout_weights(params + F.bo, bo_w, s);
    launch_mix_norm(d, X(d.L), X(d.mid), bo_w, bo_w + 1, nullptr, xf, rf, nullptr, nullptr, s);
  } else {
    launch_mix_norm(d, X(d.L), nullptr, nullptr, nullptr, nullptr, xf, rf, nullptr, nullptr, s);
  }
  launch_count_valid(d, targets, scalars, s);
  site("gemm.lm.fwd", s, [&] { gemm_nt_softcap(d, N, d.V, d.C, xf, wmat(F.lm), logits, s); });
  // the loss; in a backward call the logits become the logit gradient g_z
  site("loss", s, [&] { launch_loss(d, logits, targets, scalars, lossrow, loss, backward, s); });

  if (backward) {
    const bool acc = d.accumulate;
    if (!acc) {
      launch_zero(grads + F.wte, (int64_t)d.V * d.C, s);
      for (int l = 0; l < d.L; ++l)
        if (F.ve[l] >= 0) launch_zero(grads + F.ve[l], (int64_t)d.V * d.Ckv, s);
    }
    float* vegrow = reinterpret_cast<float*>(W + P.vegrow);
    int32_t* tlink = reinterpret_cast<int32_t*>(W + P.tlink);
    launch_token_links(tokens, N, tlink, s);
    float* gx = reinterpret_cast<float*>(W + P.gx);
    void* gxc = d.bf16 ? static_cast<void*>(W + P.gxc) : static_cast<void*>(gx);
    float* gx0 = reinterpret_cast<float*>(W + P.gx0);
    void* gu = W + P.gu;
    float* gtmp = reinterpret_cast<float*>(W + P.gtmp);
    void* gO = W + P.gO;
    void* gqkv = W + P.gqkv;
    float* delta = reinterpret_cast<float*>(W + P.delta);
    float* ga = reinterpret_cast<float*>(W + P.ga);
    float* lam_part = reinterpret_cast<float*>(W + P.lam_part);
    float* veg_part = reinterpret_cast<float*>(W + P.veg_part);

    float* part = reinterpret_cast<float*>(W + P.part);
    const int64_t pcap = P.part_bytes;
    SplitSum ssum;  // split-K partials still to be added into their gradient
    auto sum_splits = [&] { site("splitk.sum", s, [&] { splitk_sum(ssum, s); }); };
    site("gemm.lm.dgrad", s, [&] { ssum = gemm_nn_f32_splitk(d, N, d.C, d.V, logits, wmat(F.lm), gtmp, part, pcap, s, wmatT(F.lm)); });
    sum_splits();
    site("gemm.lm.wgrad", s, [&] { ssum = gemm_tn_wgrad(d, d.V, d.C, N, logits, xf, grads + F.lm, acc, part, pcap, s); });
    sum_splits();
    // Backout's share of the gradient w.r.t. x_mid, -lambda * g, is held in
    // the forward's xin scratch until the backward reaches layer d.mid
    float* gbo = reinterpret_cast<float*>(W + P.xin);
    NormBwdArgs nb{};
    nb.gin = gtmp;
    nb.r = rf;
    nb.gx = gx;
    nb.gxc = d.bf16 ? gxc : nullptr;
    if (d.backout) {  // the final norm as a mix of x and x_mid with weights (1, -lambda)
      nb.mode = NB_NORM1;
      nb.gx_first = 1;
      nb.x = X(d.L);
      nb.x0 = X(d.mid);
      nb.lam_r = bo_w;
      nb.lam_0 = bo_w + 1;
      nb.gx0 = gbo;
      nb.gx0_first = 1;
      nb.lam_part = lam_part + (size_t)d.L * P.lam_blocks * 2;
    } else {
      nb.mode = NB_FINAL;
      nb.ysrc = X(d.L);
    }
    launch_norm_bwd(d, nb, s);
    for (int l = d.L - 1; l >= 0; --l) {
      const bool ve = layer_ve(l, d.L), full = layer_full(l, d.L);
      const void* xn = LY(l, P.l_xn);
      const float* r1 = reinterpret_cast<const float*>(LY(l, P.l_r1));
      const void* qkv = LY(l, P.l_qkv);
      const float* rqk = reinterpret_cast<const float*>(LY(l, P.l_rqk));
      const float* a = reinterpret_cast<const float*>(LY(l, P.l_a));
      const void* att = LY(l, P.l_attn);
      const float* lse = reinterpret_cast<const float*>(LY(l, P.l_lse));
      const float* xmid = reinterpret_cast<const float*>(LY(l, P.l_xmid));
      const void* xn2 = LY(l, P.l_xn2);
      const float* r2 = reinterpret_cast<const float*>(LY(l, P.l_r2));
      const void* u = LY(l, P.l_u);
      // MLP
      if (d.fp8) {
        const int64_t C = d.C, Fh = d.F;
        site("fp8.quant", s, [&] { quant_tok(gxc, true, C, one_seg(slot(l, 10)), FP8_E5M2, g8t); });
        site("gemm.mp.dgrad", s, [&] {
          gemm8_relu2bwd(N, Fh, C, q8, C, w8t(l, 3), P128(C),
                         deq1(slot(l, 10), slot(l, 5), FP8_E5M2), u, gu, amax + slot(l, 11), s);
        });
        site("gemm.mp.wgrad", s, [&] {
          ssum = gemm8_wgrad(C, Fh, Nk, g8t, Np, LY8(l, P.l_h8t), Np,
                             deq1(slot(l, 10), slot(l, 9), FP8_E5M2), grads + F.mp[l], acc, part, pcap, s);
        });
        sum_splits();
        site("fp8.quant", s, [&] { quant_only(gu, Fh, one_seg(slot(l, 11)), FP8_E5M2, g8t); });
        site("gemm.fc.dgrad", s, [&] {
          gemm8_f32(N, C, Fh, q8, Fh, w8t(l, 2), P128(Fh), deq1(slot(l, 11), slot(l, 4), FP8_E5M2),
                    gtmp, false, s);
        });
        site("gemm.fc.wgrad", s, [&] {
          ssum = gemm8_wgrad(Fh, C, Nk, g8t, Np, LY8(l, P.l_x28t), Np,
                             deq1(slot(l, 11), slot(l, 8), FP8_E5M2), grads + F.fc[l], acc, part, pcap, s);
        });
        sum_splits();
      } else {
        site("gemm.mp.dgrad", s, [&] { gemm_nn_relu2bwd(d, N, d.F, d.C, gxc, wmat(F.mp[l]), u, gu, s, wmatT(F.mp[l])); });
        site("gemm.mp.wgrad", s, [&] { ssum = gemm_tn_wgrad(d, d.C, d.F, N, gxc, u, grads + F.mp[l], acc, part, pcap, s); });
        sum_splits();
        site("gemm.fc.dgrad", s, [&] { gemm_nn_f32(d, N, d.C, d.F, gu, wmat(F.fc[l]), gtmp, s, wmatT(F.fc[l])); });
        site("gemm.fc.wgrad", s, [&] { ssum = gemm_tn_wgrad(d, d.F, d.C, N, gu, xn2, grads + F.fc[l], acc, part, pcap, s); });
        sum_splits();
      }
      nb = NormBwdArgs{};
      nb.mode = NB_NORM2;
      nb.gin = gtmp;
      nb.ysrc = xmid;
      nb.r = r2;
      nb.gx = gx;
      nb.gxc = d.bf16 ? gxc : nullptr;
      launch_norm_bwd(d, nb, s);
      // attention
      if (d.fp8) {
        site("fp8.quant", s, [&] { quant_tok(gxc, true, d.C, one_seg(slot(l, 12)), FP8_E5M2, g8t); });
        site("gemm.o.dgrad", s, [&] {
          gemm8_store(N, d.Cq, d.C, q8, d.C, w8t(l, 1), P128(d.C),
                      deq1(slot(l, 12), slot(l, 3), FP8_E5M2), gO, s);
        });
        site("gemm.o.wgrad", s, [&] {
          ssum = gemm8_wgrad(d.C, d.Cq, Nk, g8t, Np, LY8(l, P.l_a8t), Np,
                             deq1(slot(l, 12), slot(l, 7), FP8_E5M2), grads + F.o[l], acc, part, pcap, s);
        });
        sum_splits();
      } else {
        site("gemm.o.dgrad", s, [&] { gemm_nn_store(d, N, d.Cq, d.C, gxc, wmat(F.o[l]), gO, s, wmatT(F.o[l])); });
        site("gemm.o.wgrad", s, [&] { ssum = gemm_tn_wgrad(d, d.C, d.Cq, N, gxc, att, grads + F.o[l], acc, part, pcap, s); });
        sum_splits();
      }
      site("attn.delta", s, [&] { launch_attn_delta(d, gO, att, delta, s); });
      site("attn.bwd", s, [&] { launch_attn_bwd(d, full, qkv, gO, lse, delta, gqkv, s); });
      launch_rope_qk_ve_bwd(d, gqkv, qkv, rqk, cs, a, ve ? params + F.ve[l] : nullptr,
                            ve ? vegrow : nullptr, ga, tokens, s);
      if (ve) launch_rows_to_table(vegrow, d.Ckv, tokens, tlink, N, grads + F.ve[l], d.V, s);
      if (d.fp8) {
        const int g0 = slot(l, 13), g1 = slot(l, 14), g2 = slot(l, 15);
        site("fp8.quant", s, [&] {
          quant_tok(gqkv, true, d.Qkv, segs3(d.Cq, d.Cq + d.Ckv, g0, g1, g2), FP8_E5M2, g8t);
        });
        // the q, k and v gradients carry their own scales along the
        // contraction (K segments)
        site("gemm.qkv.dgrad", s, [&] {
          gemm8_f32_kseg(N, d.C, d.Qkv, q8, d.Qkv, w8t(l, 0), P128(d.Qkv),
                         deq3(2, g0, g1, g2, slot(l, 0), slot(l, 1), slot(l, 2), FP8_E5M2), gtmp,
                         false, s);
        });
        site("gemm.qkv.wgrad", s, [&] {
          const int x = slot(l, 6);
          ssum = gemm8_wgrad(d.Qkv, d.C, Nk, g8t, Np, LY8(l, P.l_x8t), Np,
                             deq3(0, g0, g1, g2, x, x, x, FP8_E5M2), grads + F.q[l], acc, part, pcap, s);
        });
        sum_splits();
      } else {
        site("gemm.qkv.dgrad", s, [&] { gemm_nn_f32(d, N, d.C, d.Qkv, gqkv, wmat(F.q[l]), gtmp, s, wmatT(F.q[l])); });
        site("gemm.qkv.wgrad", s, [&] { ssum = gemm_tn_wgrad(d, d.Qkv, d.C, N, gqkv, xn, grads + F.q[l], acc, part, pcap, s); });
        sum_splits();
      }
      if (ve) launch_veg_wgrad(d, ga, xn, veg_part, P.veg_splits, grads + F.veg[l], s);
      nb = NormBwdArgs{};
      nb.mode = NB_NORM1;
      nb.gin = gtmp;
      nb.r = r1;
      nb.gx = gx;
      nb.gxc = d.bf16 ? gxc : nullptr;
      nb.ga = ve ? ga : nullptr;
      nb.wg = ve ? params + F.veg[l] : nullptr;
      nb.x = X(l);
      nb.x0 = X(0);
      nb.lam_r = params + F.lr + l;
      nb.lam_0 = params + F.l0 + l;
      nb.gx0 = gx0;
      nb.gx0_first = l == d.L - 1;
      nb.last_layer0 = l == 0;
      nb.lam_part = lam_part + (size_t)l * P.lam_blocks * 2;
      nb.gadd = d.backout && l == d.mid ? gbo : nullptr;
      launch_norm_bwd(d, nb, s);
    }
    site("embed.bwd", s, [&] {
      if (d.smear) {  // dL/dx0 -> dL/de (into gtmp) and the smear gate's gradient
        // its partials (smear_blocks(N) <= veg_splits rows of C) reuse veg_part
        launch_smear_bwd(d, gx0, params + F.wte, tokens, params + F.sm, sgate, gtmp, veg_part,
                         grads + F.sm, s);
        launch_rows_to_table(gtmp, d.C, tokens, tlink, N, grads + F.wte, d.V, s);
      } else {
        launch_rows_to_table(gx0, d.C, tokens, tlink, N, grads + F.wte, d.V, s);
      }
    });
    // every layer's lambda gradients in one launch (layer l's partials at
    // lam_part + l * 2 * lam_blocks)
    launch_lambda_finalize(d, lam_part, P.lam_blocks, grads + F.lr, grads + F.l0, s, d.L);
    // Backout: dL/dlambda = -sum g * x_mid (the second sum of the final mix's slot)
    if (d.backout)
      launch_lambda_finalize(d, lam_part + (size_t)d.L * P.lam_blocks * 2, P.lam_blocks, nullptr,
                             grads + F.bo, s, 1, -1.0f);
  }
  if (d.check_finite) {
    launch_zero(reinterpret_cast<float*>(dbg + 2), 1, s);
    launch_check_finite(loss, 1, dbg + 2, s);
    if (backward) {
      int64_t n_elems = 0;
      for (const auto& t : param_layout(*cfg)) n_elems = std::max(n_elems, t.offset + t.rows * t.cols);
      launch_check_finite(grads, n_elems, dbg + 2, s);
    }
    uint32_t bad = 0;
    const int st2 = read_flags(&bad, dbg + 2, 1);
    if (st2) return st2;
    if (bad)
      return fail(GPT_E_NONFINITE, backward ? "the loss or a gradient is NaN or infinite"
                                            : "the loss is NaN or infinite");
  }
  return launch_status();
}

// ---------------------------------------------------------------- graph cache
// GPT_F_GRAPH: one instantiated HIP graph per distinct argument set (the
// key holds the config and every pointer), least recently used dropped past
// kMaxGraphs.
struct GraphCache {
  std::mutex mu;
  std::map<std::string, hipGraphExec_t> exec;
  std::vector<std::string> lru;  // most recent last
};
static GraphCache g_graphs;
static constexpr size_t kMaxGraphs = 64;

static int graph_cache_clear() {
  std::lock_guard<std::mutex> lk(g_graphs.mu);
  if (g_graphs.exec.empty()) return GPT_OK;
  const hipError_t e = hipDeviceSynchronize();
  for (auto& kv : g_graphs.exec) (void)hipGraphExecDestroy(kv.second);
  g_graphs.exec.clear();
  g_graphs.lru.clear();
  if (e != hipSuccess) return fail(GPT_E_HIP, "HIP: %s (graph cache)", hipGetErrorString(e));
  return GPT_OK;
}

static int run_cached(const gpt_config* cfg, const float* params, const int32_t* tokens,
                      const int32_t* targets, float* loss, float* grads, void* workspace,
                      size_t workspace_bytes, void* stream, bool backward) {
  if (!cfg || !(cfg->flags & GPT_F_GRAPH) || launch_state().dry || g_prof.on)
    return run(cfg, params, tokens, targets, loss, grads, workspace, workspace_bytes, stream,
               backward);
  g_err[0] = 0;
  if (!stream) return fail(GPT_E_INVAL, "GPT_F_GRAPH needs a stream other than the null stream");
  if (cfg->flags & (GPT_F_CHECK_FINITE | GPT_F_CHECK_INPUTS))
    return fail(GPT_E_INVAL, "GPT_F_GRAPH cannot be combined with the debug checks");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GPT_E_HIP, "HIP: %s", hipGetErrorString(e));
  struct {
    gpt_config cfg;
    const void* ptr[7];
    size_t ws;
    int dev, backward;
  } key;
  std::memset(&key, 0, sizeof key);
  key.cfg = *cfg;
  const void* ptrs[7] = {params, tokens, targets, loss, grads, workspace, nullptr};
  for (int i = 0; i < 7; ++i) key.ptr[i] = ptrs[i];
  key.ws = workspace_bytes;
  key.dev = dev;
  key.backward = backward ? 1 : 0;
  const std::string k(reinterpret_cast<const char*>(&key), sizeof key);
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lk(g_graphs.mu);
  auto it = g_graphs.exec.find(k);
  if (it == g_graphs.exec.end()) {
    // capture: validation errors return before any launch, so the capture
    // is then empty and dropped
    e = hipStreamBeginCapture(s, hipStreamCaptureModeRelaxed);
    if (e != hipSuccess) return fail(GPT_E_HIP, "HIP: %s (begin capture)", hipGetErrorString(e));
    const int st = run(cfg, params, tokens, targets, loss, grads, workspace, workspace_bytes,
                       stream, backward);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(s, &graph);
    if (st) {
      if (graph) (void)hipGraphDestroy(graph);
      return st;
    }
    if (e != hipSuccess) return fail(GPT_E_HIP, "HIP: %s (end capture)", hipGetErrorString(e));
    hipGraphExec_t ex = nullptr;
    e = hipGraphInstantiate(&ex, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) return fail(GPT_E_HIP, "HIP: %s (instantiate)", hipGetErrorString(e));
    if (g_graphs.exec.size() >= kMaxGraphs) {  // drop the least recently used
      (void)hipDeviceSynchronize();
      (void)hipGraphExecDestroy(g_graphs.exec[g_graphs.lru.front()]);
      g_graphs.exec.erase(g_graphs.lru.front());
      g_graphs.lru.erase(g_graphs.lru.begin());
    }
    it = g_graphs.exec.emplace(k, ex).first;
  } else {
    g_graphs.lru.erase(std::find(g_graphs.lru.begin(), g_graphs.lru.end(), k));
  }
  g_graphs.lru.push_back(k);
  e = hipGraphLaunch(it->second, s);
  if (e != hipSuccess) return fail(GPT_E_HIP, "HIP: %s (graph launch)", hipGetErrorString(e));
  return GPT_OK;
}

}  // namespace gpt

using namespace gpt;

extern "C" {

int gpt_abi_version(void) { return GPT_ABI_VERSION; }

int gpt_config_validate(const gpt_config* cfg) {
  g_err[0] = 0;
  return validate(cfg);
}

int gpt_param_count(const gpt_config* cfg, int64_t* n_tensors, int64_t* n_elems) {
  g_err[0] = 0;
  int st = validate(cfg);
  if (st && st != GPT_E_UNSUPPORTED) return st;
  if (!n_tensors || !n_elems) return fail(GPT_E_NULLPTR, "output pointer is NULL");
  const auto v = param_layout(*cfg);
  *n_tensors = (int64_t)v.size();
  *n_elems = v.back().offset + v.back().rows * v.back().cols;
  return GPT_OK;
}

int gpt_param_info(const gpt_config* cfg, int64_t i, char name[64], int64_t* offset,
                   int64_t* rows, int64_t* cols) {
  g_err[0] = 0;
  int st = validate(cfg);
  if (st && st != GPT_E_UNSUPPORTED) return st;
  if (!name || !offset || !rows || !cols) return fail(GPT_E_NULLPTR, "output pointer is NULL");
  const auto v = param_layout(*cfg);
  if (i < 0 || i >= (int64_t)v.size()) return fail(GPT_E_INVAL, "tensor index %lld out of range", (long long)i);
  snprintf(name, 64, "%s", v[i].name.c_str());
  *offset = v[i].offset;
  *rows = v[i].rows;
  *cols = v[i].cols;
  return GPT_OK;
}

int gpt_layer_info(const gpt_config* cfg, int32_t l, int32_t* is_full, int32_t* has_ve) {
  g_err[0] = 0;
  int st = validate(cfg);
  if (st && st != GPT_E_UNSUPPORTED) return st;
  if (!is_full || !has_ve) return fail(GPT_E_NULLPTR, "output pointer is NULL");
  if (l < 0 || l >= cfg->n_layer) return fail(GPT_E_INVAL, "layer %d out of range", l);
  *is_full = layer_full(l, cfg->n_layer) ? 1 : 0;
  *has_ve = layer_ve(l, cfg->n_layer) ? 1 : 0;
  return GPT_OK;
}

int gpt_workspace_size(const gpt_config* cfg, size_t* bytes) {
  g_err[0] = 0;
  int st = validate(cfg);
  if (st) return st;
  if (!bytes) return fail(GPT_E_NULLPTR, "output pointer is NULL");
  *bytes = make_plan(make_dims(*cfg)).total;
  return GPT_OK;
}

int gpt_workspace_region(const gpt_config* cfg, const char* name, int32_t layer, size_t* offset,
                         size_t* bytes) {
  g_err[0] = 0;
  int st = validate(cfg);
  if (st) return st;
  if (!name || !offset || !bytes) return fail(GPT_E_NULLPTR, "pointer is NULL");
  const Dims d = make_dims(*cfg);
  const Plan P = make_plan(d);
  const size_t N = (size_t)d.N, A = (size_t)d.act_bytes, C = (size_t)d.C;
  const std::string n(name);
  struct R {
    const char* name;
    size_t off, bytes;
  };
  if (n == "x") {
    if (layer < 0 || layer > d.L) return fail(GPT_E_INVAL, "layer out of range");
    *offset = P.x + (size_t)layer * N * C * 4;
    *bytes = N * C * 4;
    return GPT_OK;
  }
  const R global[] = {
      {"wc", P.wc, d.bf16 ? (P.wct - P.wc) : 0}, {"wct", P.wct, d.bf16 ? (P.rope - P.wct) : 0},
      {"rope", P.rope, (size_t)d.T * d.D * 4},
      {"xin", P.xin, N * C * 4}, {"xf", P.xf, N * C * A}, {"rf", P.rf, N * 4},
      {"logits", P.logits, N * d.V * A}, {"lossrow", P.lossrow, N * 4},
      {"scalars", P.scalars, 256},
      {"gx", P.gx, N * C * 4}, {"gxc", P.gxc, N * C * A}, {"gx0", P.gx0, N * C * 4},
      {"gu", P.gu, N * d.F * A}, {"gtmp", P.gtmp, N * C * 4}, {"gO", P.gO, N * d.Cq * A},
      {"gqkv", P.gqkv, N * d.Qkv * A}, {"delta", P.delta, N * d.H * 4},
      {"ga", P.ga, N * d.Hk * 4}, {"lam_part", P.lam_part, (size_t)(d.L + (d.backout ? 1 : 0)) * P.lam_blocks * 8},
      {"veg_part", P.veg_part, (size_t)P.veg_splits * d.Hk * C * 4},
      {"vegrow", P.vegrow, N * (size_t)d.Ckv * 4}, {"tlink", P.tlink, 2 * N * 4},
      {"sgate", P.sgate, d.smear ? N * 4 : 0},
      {"part", P.part, (size_t)P.part_bytes},
      {"amax", P.amax, d.fp8 ? (size_t)16 * d.L * 4 : 0},
      {"w8", P.w8, d.fp8 ? P.w8_layer * d.L : 0},
      {"w8t", P.w8t, d.fp8 ? P.w8t_layer * d.L : 0},
      {"q8", P.q8, d.fp8 ? N * std::max(std::max(C, (size_t)d.Cq), std::max((size_t)d.F, (size_t)d.Qkv)) : 0},
      {"g8t", P.g8t, d.fp8 ? std::max(std::max(C, (size_t)d.F), (size_t)d.Qkv) * (size_t)P.Np : 0}};
  for (const R& r : global)
    if (n == r.name) {
      *offset = r.off;
      *bytes = r.bytes;
      return GPT_OK;
    }
  const R per_layer[] = {{"xn", P.l_xn, N * C * A},
                         {"r1", P.l_r1, N * 4},
                         {"qkv", P.l_qkv, N * d.Qkv * A},
                         {"rqk", P.l_rqk, N * (d.H + d.Hk) * 4},
                         {"a", P.l_a, N * d.Hk * 4},
                         {"attn", P.l_attn, N * d.Cq * A},
                         {"lse", P.l_lse, N * d.H * 4},
                         {"xmid", P.l_xmid, N * C * 4},
                         {"xn2", P.l_xn2, N * C * A},
                         {"r2", P.l_r2, N * 4},
                         {"h", P.l_u, N * d.F * A},
                         {"x8t", P.l_x8t, d.fp8 ? C * (size_t)P.Np : 0},
                         {"a8t", P.l_a8t, d.fp8 ? (size_t)d.Cq * P.Np : 0},
                         {"x28t", P.l_x28t, d.fp8 ? C * (size_t)P.Np : 0},
                         {"h8t", P.l_h8t, d.fp8 ? (size_t)d.F * P.Np : 0}};
  for (const R& r : per_layer)
    if (n == r.name) {
      if (layer < 0 || layer >= d.L) return fail(GPT_E_INVAL, "layer out of range");
      *offset = P.layers + (size_t)layer * P.layer_bytes + r.off;
      *bytes = r.bytes;
      return GPT_OK;
    }
  return fail(GPT_E_INVAL, "unknown region '%s'", name);
}

int gpt_fwd_bwd(const gpt_config* cfg, const float* params, const int32_t* tokens,
                const int32_t* targets, float* loss, float* grads, void* workspace,
                size_t workspace_bytes, void* stream) {
  return run_cached(cfg, params, tokens, targets, loss, grads, workspace, workspace_bytes, stream,
                    true);
}

int gpt_fwd(const gpt_config* cfg, const float* params, const int32_t* tokens,
            const int32_t* targets, float* loss, void* workspace, size_t workspace_bytes,
            void* stream) {
  return run_cached(cfg, params, tokens, targets, loss, nullptr, workspace, workspace_bytes, stream,
                    false);
}

int gpt_graph_cache_clear(void) {
  g_err[0] = 0;
  return graph_cache_clear();
}

static int attn_args(const gpt_config* cfg, int32_t full, std::initializer_list<const void*> ptrs) {
  int st = validate(cfg);
  if (st == GPT_E_UNSUPPORTED) st = GPT_OK;  // flags that only the full step reads
  if (st) return st;
  if (full != 0 && full != 1) return fail(GPT_E_INVAL, "full must be 0 or 1");
  for (const void* p : ptrs) {
    if (!p) return fail(GPT_E_NULLPTR, "a required pointer is NULL");
    if (!aligned(p, 16)) return fail(GPT_E_ALIGN, "every pointer needs 16-byte alignment");
  }
  return GPT_OK;
}

int gpt_attn_fwd(const gpt_config* cfg, int32_t full, const void* qkv, void* out, float* lse2,
                 void* stream) {
  g_err[0] = 0;
  const int st = attn_args(cfg, full, {qkv, out, lse2});
  if (st) return st;
  const Dims d = make_dims(*cfg);
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_reset();
  launch_attn_fwd(d, full != 0, qkv, out, lse2, s);
  return launch_status();
}

int gpt_attn_bwd(const gpt_config* cfg, int32_t full, const void* qkv, const void* out,
                 const void* g_out, const float* lse2, float* delta, void* g_qkv, void* stream) {
  g_err[0] = 0;
  const int st = attn_args(cfg, full, {qkv, out, g_out, lse2, delta, g_qkv});
  if (st) return st;
  const Dims d = make_dims(*cfg);
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_reset();
  launch_attn_delta(d, g_out, out, delta, s);
  launch_attn_bwd(d, full != 0, qkv, g_out, lse2, delta, g_qkv, s);
  return launch_status();
}

int gpt_fp8_quantize(const void* src, int32_t src_dtype, int64_t rows, int64_t cols,
                     int32_t fmt, uint8_t* codes, uint8_t* codes_t, int64_t pitch_t,
                     uint32_t* amax, void* stream) {
  g_err[0] = 0;
  if (!src || !amax) return fail(GPT_E_NULLPTR, "src and amax are required");
  if (src_dtype != GPT_DT_F32 && src_dtype != GPT_DT_BF16)
    return fail(GPT_E_INVAL, "src_dtype %d unknown", src_dtype);
  if (fmt != FP8_E4M3 && fmt != FP8_E5M2) return fail(GPT_E_INVAL, "fmt %d unknown", fmt);
  if (rows < 1 || cols < 64 || cols % 64 || rows > ((int64_t)1 << 31) || cols > (1 << 20))
    return fail(GPT_E_INVAL, "rows %lld / cols %lld: need rows >= 1, cols a multiple of 64",
                (long long)rows, (long long)cols);
  if (codes_t && (pitch_t < rows || pitch_t % 128))
    return fail(GPT_E_INVAL, "pitch_t %lld: need a multiple of 128 >= rows", (long long)pitch_t);
  if (!aligned(src, 16) || (codes && !aligned(codes, 16)) || (codes_t && !aligned(codes_t, 16)) ||
      !aligned(amax, 4))
    return fail(GPT_E_ALIGN, "src, codes, codes_t need 16-byte alignment, amax 4");
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_reset();
  const bool bf = src_dtype == GPT_DT_BF16;
  const Segs sg = one_seg(0);
  launch_zero(reinterpret_cast<float*>(amax), 1, s);
  launch_fp8_amax(src, bf, rows * cols, rows * cols, sg, amax, s);
  launch_fp8_quant(src, bf, rows, cols, false, sg, amax, fmt, codes, codes_t, pitch_t, s);
  return launch_status();
}

static int fp8_gemm_sizes(int32_t wgrad, int64_t M, int64_t N, int64_t K) {
  if (wgrad != 0 && wgrad != 1) return fail(GPT_E_INVAL, "wgrad must be 0 or 1");
  if (M < 1 || N < 1 || N % 4 || K < 16 || K % 16 || M > (1 << 24) || N > (1 << 24) ||
      K > ((int64_t)1 << 30))
    return fail(GPT_E_INVAL, "M %lld / N %lld / K %lld: need M >= 1, N a multiple of 4, K a multiple of 16",
                (long long)M, (long long)N, (long long)K);
  return GPT_OK;
}

int gpt_fp8_gemm_workspace(int32_t wgrad, int64_t M, int64_t N, int64_t K, size_t* bytes) {
  g_err[0] = 0;
  const int st = fp8_gemm_sizes(wgrad, M, N, K);
  if (st) return st;
  if (!bytes) return fail(GPT_E_NULLPTR, "output pointer is NULL");
  *bytes = wgrad ? (size_t)part_bytes_f8_wgrad(M, N, K) : 0;
  return GPT_OK;
}

int gpt_fp8_gemm(int32_t wgrad, int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                 int32_t fmt_a, const uint8_t* B, int64_t ldb, const uint32_t* amax,
                 const gpt_fp8_scales* sc, int32_t accumulate, float* C, void* workspace,
                 size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  int st = fp8_gemm_sizes(wgrad, M, N, K);
  if (st) return st;
  if (fmt_a != FP8_E4M3 && fmt_a != FP8_E5M2) return fail(GPT_E_INVAL, "fmt_a %d unknown", fmt_a);
  if (accumulate != 0 && accumulate != 1) return fail(GPT_E_INVAL, "accumulate must be 0 or 1");
  if (lda < K || ldb < K || lda % 16 || ldb % 16)
    return fail(GPT_E_INVAL, "lda %lld / ldb %lld: need multiples of 16, >= K", (long long)lda,
                (long long)ldb);
  if (!A || !B || !amax || !sc || !C) return fail(GPT_E_NULLPTR, "a required pointer is NULL");
  if (sc->axis < 0 || sc->axis > 2) return fail(GPT_E_INVAL, "scales.axis must be 0, 1 or 2");
  if (sc->nseg < 1 || sc->nseg > 3) return fail(GPT_E_INVAL, "scales.nseg must be 1, 2 or 3");
  if (sc->nseg == 3 && sc->end[1] < sc->end[0]) return fail(GPT_E_INVAL, "scales.end must ascend");
  if (sc->axis == 2) {
    if (wgrad) return fail(GPT_E_INVAL, "scales along K (axis 2) need wgrad = 0");
    for (int i = 0; i + 1 < sc->nseg; ++i)
      if (sc->end[i] < 0 || sc->end[i] > K || sc->end[i] % 16)
        return fail(GPT_E_INVAL, "scales.end[%d] = %lld: along K, need a multiple of 16 in [0, K]",
                    i, (long long)sc->end[i]);
  }
  for (int i = 0; i < sc->nseg; ++i)
    if (sc->slot_a[i] < 0 || sc->slot_b[i] < 0) return fail(GPT_E_INVAL, "amax slots must be >= 0");
  const size_t need = wgrad ? (size_t)part_bytes_f8_wgrad(M, N, K) : 0;
  if (need && !workspace) return fail(GPT_E_NULLPTR, "workspace is NULL");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(amax, 4) ||
      (need && !aligned(workspace, 256)))
    return fail(GPT_E_ALIGN, "A, B, C need 16-byte alignment, amax 4, workspace 256");
  if (workspace_bytes < need)
    return fail(GPT_E_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  Fp8Deq q{};
  q.amax = amax;
  q.axis = sc->axis;
  q.nseg = sc->nseg;
  q.end[0] = sc->nseg > 1 ? sc->end[0] : INT64_MAX;
  q.end[1] = sc->nseg > 2 ? sc->end[1] : INT64_MAX;
  q.end[2] = INT64_MAX;
  for (int i = 0; i < 3; ++i) {
    q.sa[i] = sc->slot_a[i < sc->nseg ? i : 0];
    q.sb[i] = sc->slot_b[i < sc->nseg ? i : 0];
  }
  q.fa = fmt_a;
  q.fb = FP8_E4M3;
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_reset();
  if (q.axis == 2) {
    gemm8_f32_kseg(M, N, K, A, lda, B, ldb, q, C, accumulate != 0, s);
    return launch_status();
  }
  const SplitSum r = gemm8_product(wgrad != 0, M, N, K, A, lda, B, ldb, q, C, accumulate != 0,
                                   static_cast<float*>(workspace), (int64_t)workspace_bytes, s);
  splitk_sum(r, s);
  return launch_status();
}

// The bf16 products of the step on their own: the K-major product of the
// forward and input-gradient GEMMs with an fp32 result, its split-K form for
// long contractions, and the weight-gradient product (split-K partials
// summed in split order), each with the tile and split plan the step uses.
static int bf16_gemm_sizes(int32_t kind, int64_t M, int64_t N, int64_t K) {
  if (kind < 0 || kind > 2) return fail(GPT_E_INVAL, "kind %d: need 0, 1 or 2", kind);
  if (M < 1 || M > (1 << 24) || N < 64 || N % 64 || N > (1 << 24))
    return fail(GPT_E_INVAL, "M %lld / N %lld: need M >= 1, N a multiple of 64", (long long)M,
                (long long)N);
  if (kind == 2) {
    if (M % 64 || K < 1 || K > ((int64_t)1 << 30))
      return fail(GPT_E_INVAL, "weight gradient M %lld / K %lld: need M a multiple of 64, K >= 1",
                  (long long)M, (long long)K);
  } else if (K < 64 || K % 64 || K > ((int64_t)1 << 30)) {
    return fail(GPT_E_INVAL, "K %lld: need a multiple of 64", (long long)K);
  }
  return GPT_OK;
}

static int64_t bf16_gemm_need(int32_t kind, int64_t M, int64_t N, int64_t K) {
  Dims d{};
  d.bf16 = true;
  if (kind == 1) return part_bytes_nn_splitk(d, M, N, K);
  if (kind == 2) return part_bytes_tn_wgrad(d, M, N, K);
  return 0;
}

int gpt_bf16_gemm_workspace(int32_t kind, int64_t M, int64_t N, int64_t K, size_t* bytes) {
  g_err[0] = 0;
  const int st = bf16_gemm_sizes(kind, M, N, K);
  if (st) return st;
  if (!bytes) return fail(GPT_E_NULLPTR, "output pointer is NULL");
  *bytes = (size_t)bf16_gemm_need(kind, M, N, K);
  return GPT_OK;
}

int gpt_bf16_gemm(int32_t kind, int64_t M, int64_t N, int64_t K, const void* A, const void* B,
                  int32_t accumulate, float* C, void* workspace, size_t workspace_bytes,
                  void* stream) {
  g_err[0] = 0;
  const int st = bf16_gemm_sizes(kind, M, N, K);
  if (st) return st;
  if (accumulate != 0 && accumulate != 1) return fail(GPT_E_INVAL, "accumulate must be 0 or 1");
  if (accumulate && kind != 2)
    return fail(GPT_E_INVAL, "accumulate: only the weight-gradient product (kind 2) adds into C");
  if (!A || !B || !C) return fail(GPT_E_NULLPTR, "a required pointer is NULL");
  const size_t need = (size_t)bf16_gemm_need(kind, M, N, K);
  if (need && !workspace) return fail(GPT_E_NULLPTR, "workspace is NULL");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16) || (need && !aligned(workspace, 256)))
    return fail(GPT_E_ALIGN, "A, B, C need 16-byte alignment, workspace 256");
  if (workspace_bytes < need)
    return fail(GPT_E_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  Dims d{};
  d.bf16 = true;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* part = static_cast<float*>(workspace);
  launch_reset();
  if (kind == 0) {
    gemm_nn_f32(d, M, (int)N, (int)K, A, nullptr, C, s, B);
  } else if (kind == 1) {
    splitk_sum(gemm_nn_f32_splitk(d, M, (int)N, (int)K, A, nullptr, C, part,
                                  (int64_t)workspace_bytes, s, B),
               s);
  } else {
    splitk_sum(gemm_tn_wgrad(d, (int)M, (int)N, K, A, B, C, accumulate != 0, part,
                             (int64_t)workspace_bytes, s),
               s);
  }
  return launch_status();
}

static int decode_validate(int32_t B, int32_t H, int32_t Hk, int32_t D, int32_t Tmax,
                           int32_t window) {
  if (B < 1 || B > 65535) return fail(GPT_E_INVAL, "batch %d not in [1, 65535]", B);
  if (D != 64 && D != 128) return fail(GPT_E_INVAL, "head_dim %d: need 64 or 128", D);
  if (H < 1 || Hk < 1 || H % Hk || H / Hk > 8 || Hk > 65535)
    return fail(GPT_E_INVAL, "n_head %d / n_kv_head %d: need n_kv_head dividing n_head, at most 8 "
                "query heads per KV head", H, Hk);
  if (Tmax < 1 || (int64_t)B * Tmax * Hk * D > ((int64_t)1 << 40))
    return fail(GPT_E_INVAL, "cache length %d out of range", Tmax);
  if (window < -1) return fail(GPT_E_INVAL, "window %d: need >= 0, or -1 for full context", window);
  return GPT_OK;
}

int gpt_decode_attn_workspace(int32_t batch, int32_t n_head, int32_t n_kv_head, int32_t head_dim,
                              int32_t max_len, int32_t window, size_t* bytes) {
  g_err[0] = 0;
  const int st = decode_validate(batch, n_head, n_kv_head, head_dim, max_len, window);
  if (st) return st;
  if (!bytes) return fail(GPT_E_NULLPTR, "output pointer is NULL");
  *bytes = decode_workspace_bytes(batch, n_head, n_kv_head, head_dim, max_len, window);
  return GPT_OK;
}

int gpt_decode_attn(int32_t batch, int32_t n_head, int32_t n_kv_head, int32_t head_dim,
                    int32_t max_len, int32_t window, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* seqlen, void* out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const int st = decode_validate(batch, n_head, n_kv_head, head_dim, max_len, window);
  if (st) return st;
  const size_t need = decode_workspace_bytes(batch, n_head, n_kv_head, head_dim, max_len, window);
  if (!q || !k_cache || !v_cache || !seqlen || !out || (need && !workspace))
    return fail(GPT_E_NULLPTR, "a required pointer is NULL");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(seqlen, 4) || !aligned(workspace, 256))
    return fail(GPT_E_ALIGN, "q, caches and out need 16-byte alignment, seqlen 4, workspace 256");
  if (workspace_bytes < need)
    return fail(GPT_E_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_reset();
  launch_decode_attn(batch, n_head, n_kv_head, head_dim, max_len, window, q, k_cache, v_cache,
                     seqlen, out, workspace, s);
  return launch_status();
}

int gpt_decode_attn_noalloc(int32_t batch, int32_t n_head, int32_t n_kv_head, int32_t head_dim,
                            int32_t max_len, int32_t window, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* seqlen, void* out, void* stream) {
  g_err[0] = 0;
  const int st = decode_validate(batch, n_head, n_kv_head, head_dim, max_len, window);
  if (st) return st;
  const size_t need = decode_workspace_bytes(batch, n_head, n_kv_head, head_dim, max_len, window);
  if (need > decode_scratch_capacity())
    return fail(GPT_E_WORKSPACE, "chunk states need %zu bytes; the static scratch holds %zu", need,
                decode_scratch_capacity());
  if (!q || !k_cache || !v_cache || !seqlen || !out)
    return fail(GPT_E_NULLPTR, "a required pointer is NULL");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(seqlen, 4))
    return fail(GPT_E_ALIGN, "q, caches and out need 16-byte alignment, seqlen 4");
  void* scratch = nullptr;
  if (need) {
    const hipError_t e = decode_scratch(&scratch);
    if (e != hipSuccess) return fail(GPT_E_HIP, "HIP: %s (scratch address)", hipGetErrorString(e));
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_reset();
  launch_decode_attn(batch, n_head, n_kv_head, head_dim, max_len, window, q, k_cache, v_cache,
                     seqlen, out, scratch, s);
  return launch_status();
}

int gpt_kv_cache_append(int32_t batch, int32_t n_new, int32_t n_head, int32_t n_kv_head,
                        int32_t head_dim, int32_t max_len, const void* qkv, const int32_t* pos,
                        void* k_cache, void* v_cache, void* stream) {
  g_err[0] = 0;
  const int st = decode_validate(batch, n_head, n_kv_head, head_dim, max_len, -1);
  if (st) return st;
  if (n_new < 1 || (int64_t)batch * n_new > ((int64_t)1 << 26))
    return fail(GPT_E_INVAL, "n_new %d: need >= 1 and batch * n_new <= 2^26", n_new);
  if (!qkv || !pos || !k_cache || !v_cache) return fail(GPT_E_NULLPTR, "a required pointer is NULL");
  if (!aligned(qkv, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(pos, 4))
    return fail(GPT_E_ALIGN, "qkv and caches need 16-byte alignment, pos 4");
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_reset();
  launch_kv_cache_append(batch, n_new, n_head, n_kv_head, head_dim, max_len, qkv, pos, k_cache,
                         v_cache, s);
  return launch_status();
}

int gpt_optim_workspace_size(const gpt_config* cfg, size_t* bytes) {
  g_err[0] = 0;
  const int st = validate(cfg);
  if (st) return st;
  if (!bytes) return fail(GPT_E_NULLPTR, "output pointer is NULL");
  *bytes = make_optim_plan(*cfg).total;
  return GPT_OK;
}

int gpt_optimizer_step(const gpt_config* cfg, const gpt_optim_hparams* hp, float* params,
                       const float* grads, float* state, void* workspace, size_t workspace_bytes,
                       void* stream) {
  g_err[0] = 0;
  const int st = validate(cfg);
  if (st) return st;
  if (!hp || !params || !grads || !state || !workspace)
    return fail(GPT_E_NULLPTR, "a required pointer is NULL");
  if (!aligned(params, 256) || !aligned(grads, 256) || !aligned(state, 256) ||
      !aligned(workspace, 256))
    return fail(GPT_E_ALIGN, "params, grads, state and workspace need 256-byte alignment");
  if (hp->step < 1 || hp->ns_steps < 0 || hp->ns_steps > 100 || (hp->nesterov != 0 && hp->nesterov != 1))
    return fail(GPT_E_INVAL, "step >= 1, ns_steps in [0, 100] and nesterov 0/1 required");
  const float fl[] = {hp->lr_matrix, hp->lr_scalar, hp->lr_embed, hp->lr_unembed, hp->lr_mult,
                      hp->weight_decay, hp->beta1, hp->beta2, hp->eps, hp->momentum,
                      hp->ns_a, hp->ns_b, hp->ns_c};
  for (float f : fl)
    if (!std::isfinite(f)) return fail(GPT_E_INVAL, "hyper-parameters must be finite");
  if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f && hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
    return fail(GPT_E_INVAL, "betas must lie in [0, 1)");
  const Dims d = make_dims(*cfg);
  const OptimPlan o = make_optim_plan(*cfg);
  if (workspace_bytes < o.total)
    return fail(GPT_E_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, o.total);
  int64_t n_elems = 0;
  const std::vector<TensorInfo> lay = param_layout(*cfg);
  for (const auto& t : lay) n_elems = std::max(n_elems, t.offset + t.rows * t.cols);
  float* m = state;
  float* v = state + n_elems;
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_reset();
  // Muon: the block matrices, batched by shape
  launch_muon_groups(d, muon_groups(*cfg), o, workspace, params, grads, m,
                     hp->lr_matrix * hp->lr_mult, hp->weight_decay, hp->momentum, hp->nesterov,
                     hp->ns_a, hp->ns_b, hp->ns_c, hp->ns_steps, s);
  // AdamW: every other tensor
  for (const auto& t : lay) {
    const std::string& n = t.name;
    const size_t dot = n.find('.');
    const std::string leaf = dot == std::string::npos ? n : n.substr(dot + 1);
    if (leaf == "q" || leaf == "k" || leaf == "v" || leaf == "o" || leaf == "fc" || leaf == "mp")
      continue;
    const float lr = n == "wte" || leaf == "ve" ? hp->lr_embed
                     : n == "lm_head"            ? hp->lr_unembed
                                                 : hp->lr_scalar;
    launch_adamw(params + t.offset, grads + t.offset, m + t.offset, v + t.offset,
                 t.rows * t.cols, lr * hp->lr_mult, hp->beta1, hp->beta2, hp->eps, hp->step, s);
  }
  return launch_status();
}

const char* gpt_status_string(int status) {
  switch (status) {
    case GPT_OK: return "ok";
    case GPT_E_INVAL: return "invalid argument";
    case GPT_E_NULLPTR: return "null pointer";
    case GPT_E_ALIGN: return "misaligned pointer";
    case GPT_E_WORKSPACE: return "workspace too small";
    case GPT_E_UNSUPPORTED: return "unsupported configuration";
    case GPT_E_HIP: return "HIP runtime error";
    case GPT_E_NONFINITE: return "non-finite loss or gradient";
    default: return "unknown status";
  }
}

const char* gpt_last_error(void) { return g_err; }

int gpt_debug_launches(int64_t fail_at, int32_t dry_run) {
  g_err[0] = 0;
  if (dry_run != 0 && dry_run != 1) return fail(GPT_E_INVAL, "dry_run must be 0 or 1");
  LaunchState& st = launch_state();
  st.fail_at = fail_at < 0 ? -1 : fail_at;
  st.dry = dry_run != 0;
  return GPT_OK;
}

int gpt_debug_launch_count(int64_t* issued) {
  // a query: the last call's error text is left as it is
  if (!issued) return fail(GPT_E_NULLPTR, "output pointer is NULL");
  *issued = launch_state().issued;
  return GPT_OK;
}

int gpt_profile_begin(const char* site_prefix) {
  g_err[0] = 0;
  if (!site_prefix) return fail(GPT_E_NULLPTR, "site_prefix is NULL");
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.prefix = site_prefix;
  g_prof.used = 0;
  g_prof.on = true;
  return GPT_OK;
}

int gpt_profile_end(double* total_ms, int64_t* launches) {
  g_err[0] = 0;
  if (!total_ms || !launches) return fail(GPT_E_NULLPTR, "output pointer is NULL");
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on = false;
  double ms = 0.0;
  for (size_t i = 0; i + 1 < g_prof.used; i += 2) {
    if (hipEventSynchronize(g_prof.pool[i + 1]) != hipSuccess)
      return fail(GPT_E_HIP, "hipEventSynchronize failed");
    float t = 0.0f;
    if (hipEventElapsedTime(&t, g_prof.pool[i], g_prof.pool[i + 1]) != hipSuccess)
      return fail(GPT_E_HIP, "hipEventElapsedTime failed");
    ms += t;
  }
  *total_ms = ms;
  *launches = (int64_t)(g_prof.used / 2);
  g_prof.used = 0;
  return GPT_OK;
}

}  // extern "C"
