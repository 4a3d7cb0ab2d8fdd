// Drives the host-only logic of the GPT step library (config validation,
// parameter layout, workspace plan and regions, argument checks, and the
// launch sequence of every entry point in dry-run mode) for a sanitizer
// build: host.hip compiled with AddressSanitizer and UndefinedBehavior-
// Sanitizer. No GPU is needed: dry runs launch nothing and fake device
// pointers are never dereferenced. Exit status 0 when every expectation
// holds; the sanitizers abort the process on the first report.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "gpt_step.h"

static int g_fail = 0;
#define EXPECT(c)                                                        \
  do {                                                                   \
    if (!(c)) {                                                          \
      std::fprintf(stderr, "expectation failed at line %d: %s\n", __LINE__, #c); \
      ++g_fail;                                                          \
    }                                                                    \
  } while (0)

static gpt_config make(int L, int C, int H, int Hk, int D, int F, int V, int T, int B, int W,
                       int dt, int fp8, int flags) {
  gpt_config c;
  std::memset(&c, 0, sizeof c);
  c.abi_version = GPT_ABI_VERSION;
  c.n_layer = L; c.n_embd = C; c.n_head = H; c.n_kv_head = Hk; c.head_dim = D;
  c.mlp_hidden = F; c.vocab = V; c.seq_len = T; c.batch = B; c.short_window = W;
  c.compute_dtype = dt; c.fp8_linears = fp8; c.flags = flags;
  c.rope_theta = 10000.0f; c.norm_eps = 1.0f / 8388608.0f; c.softcap = 15.0f;
  return c;
}

static const char* kRegions[] = {"wc", "wct", "rope", "xin", "xf", "rf", "logits", "lossrow",
                                 "scalars", "gx", "gxc", "gx0", "gu", "gtmp", "gO", "gqkv",
                                 "delta", "ga", "lam_part", "veg_part", "vegrow", "tlink",
                                 "sgate", "part", "amax", "w8", "w8t", "q8", "g8t", "x", "xn",
                                 "r1", "qkv", "rqk", "a", "attn", "lse", "xmid", "xn2", "r2",
                                 "h", "x8t", "a8t", "x28t", "h8t", "no-such-region", ""};

static void exercise(const gpt_config& c) {
  EXPECT(gpt_config_validate(&c) == GPT_OK);
  int64_t nt = 0, ne = 0;
  EXPECT(gpt_param_count(&c, &nt, &ne) == GPT_OK && nt > 0 && ne > 0);
  int64_t end = 0;
  for (int64_t i = -1; i <= nt; ++i) {
    char name[64];
    int64_t o = 0, r = 0, k = 0;
    const int st = gpt_param_info(&c, i, name, &o, &r, &k);
    if (i < 0 || i == nt) {
      EXPECT(st == GPT_E_INVAL);
      continue;
    }
    EXPECT(st == GPT_OK && o == end && std::strlen(name) < 64);
    end = o + r * k;
  }
  EXPECT(end == ne);
  for (int l = -1; l <= c.n_layer; ++l) {
    int32_t f = 0, v = 0;
    EXPECT((gpt_layer_info(&c, l, &f, &v) == GPT_OK) == (l >= 0 && l < c.n_layer));
  }
  size_t ws = 0;
  EXPECT(gpt_workspace_size(&c, &ws) == GPT_OK && ws > 0);
  for (const char* r : kRegions)
    for (int l = -1; l <= c.n_layer + 1; ++l) {
      size_t off = 0, nb = 0;
      if (gpt_workspace_region(&c, r, l, &off, &nb) == GPT_OK) EXPECT(off + nb <= ws);
    }
  // the launch sequence, dry
  void* p = reinterpret_cast<void*>(uintptr_t(1) << 20);
  const float* fp = static_cast<const float*>(p);
  const int32_t* ip = static_cast<const int32_t*>(p);
  EXPECT(gpt_debug_launches(-1, 1) == GPT_OK);
  EXPECT(gpt_fwd_bwd(&c, fp, ip, ip, (float*)p, (float*)p, p, ws, nullptr) == GPT_OK);
  int64_t n = 0;
  EXPECT(gpt_debug_launch_count(&n) == GPT_OK && n > 0);
  EXPECT(gpt_fwd(&c, fp, ip, ip, (float*)p, p, ws, nullptr) == GPT_OK);
  gpt_config dbg = c;
  dbg.flags |= GPT_F_CHECK_FINITE | GPT_F_CHECK_INPUTS;
  EXPECT(gpt_fwd_bwd(&dbg, fp, ip, ip, (float*)p, (float*)p, p, ws, nullptr) == GPT_OK);
  EXPECT(gpt_debug_launches(n / 2, 1) == GPT_OK);
  EXPECT(gpt_fwd_bwd(&c, fp, ip, ip, (float*)p, (float*)p, p, ws, nullptr) == GPT_E_HIP);
  EXPECT(gpt_debug_launch_count(&n) == GPT_OK);
  EXPECT(std::strstr(gpt_last_error(), "injected") != nullptr);
  EXPECT(gpt_debug_launches(-1, 1) == GPT_OK);
  // argument errors
  EXPECT(gpt_fwd_bwd(&c, nullptr, ip, ip, (float*)p, (float*)p, p, ws, nullptr) == GPT_E_NULLPTR);
  EXPECT(gpt_fwd_bwd(&c, fp + 1, ip, ip, (float*)p, (float*)p, p, ws, nullptr) == GPT_E_ALIGN);
  EXPECT(gpt_fwd_bwd(&c, fp, ip, ip, (float*)p, (float*)p, p, ws - 1, nullptr) == GPT_E_WORKSPACE);
  // optimizer
  size_t ows = 0;
  EXPECT(gpt_optim_workspace_size(&c, &ows) == GPT_OK);
  gpt_optim_hparams hp;
  std::memset(&hp, 0, sizeof hp);
  hp.step = 1; hp.ns_steps = 5; hp.nesterov = 1; hp.lr_matrix = 0.02f; hp.lr_scalar = 0.5f;
  hp.lr_embed = 0.3f; hp.lr_unembed = 0.008f; hp.lr_mult = 1.0f; hp.weight_decay = 0.28f;
  hp.beta1 = 0.9f; hp.beta2 = 0.999f; hp.eps = 1e-8f; hp.momentum = 0.95f;
  hp.ns_a = 3.4445f; hp.ns_b = -4.775f; hp.ns_c = 2.0315f;
  EXPECT(gpt_optimizer_step(&c, &hp, (float*)p, fp, (float*)p, p, ows, nullptr) == GPT_OK);
  hp.step = 0;
  EXPECT(gpt_optimizer_step(&c, &hp, (float*)p, fp, (float*)p, p, ows, nullptr) == GPT_E_INVAL);
  EXPECT(gpt_debug_launches(-1, 0) == GPT_OK);
}

int main() {
  std::vector<gpt_config> ok = {
      make(2, 128, 2, 2, 64, 512, 512, 64, 2, 16, GPT_DT_F32, 0, 0),
      make(2, 128, 2, 2, 64, 512, 512, 64, 2, 16, GPT_DT_F32, 0, GPT_F_SMEAR | GPT_F_BACKOUT),
      make(12, 768, 6, 6, 128, 3072, 32768, 2048, 8, 512, GPT_DT_BF16, 0, 0),
      make(12, 768, 6, 2, 128, 3072, 32768, 2048, 16, 512, GPT_DT_BF16, 0, GPT_F_ACCUMULATE),
      make(20, 1280, 10, 10, 128, 5120, 32768, 2048, 16, 512, GPT_DT_BF16, 0, 0),
      make(26, 1664, 13, 13, 128, 6656, 32768, 2048, 8, 512, GPT_DT_BF16, 1, 0),
      make(3, 768, 6, 2, 128, 3072, 1024, 77, 3, 19, GPT_DT_BF16, 1, GPT_F_SMEAR),
      make(1, 64, 1, 1, 64, 64, 64, 1, 1, 0, GPT_DT_BF16, 0, GPT_F_BACKOUT)};
  for (const auto& c : ok) exercise(c);
  // invalid configs and arguments
  const gpt_config base = ok[0];
  auto bad = [&](int st, gpt_config c) { EXPECT(gpt_config_validate(&c) == st); };
  gpt_config c = base; c.abi_version = 1; bad(GPT_E_INVAL, c);
  c = base; c.n_layer = 0; bad(GPT_E_INVAL, c);
  c = base; c.n_embd = 100; bad(GPT_E_INVAL, c);
  c = base; c.head_dim = 96; bad(GPT_E_INVAL, c);
  c = base; c.n_head = 3; c.n_kv_head = 2; bad(GPT_E_INVAL, c);
  c = base; c.vocab = 500; bad(GPT_E_INVAL, c);
  c = base; c.seq_len = 1 << 20; c.batch = 1 << 10; bad(GPT_E_INVAL, c);
  c = base; c.flags = 1 << 9; bad(GPT_E_INVAL, c);
  c = base; c.flags = GPT_F_EMBED_NORM; bad(GPT_E_UNSUPPORTED, c);
  c = base; c.softcap = 0.0f; bad(GPT_E_INVAL, c);
  c = base; c.norm_eps = -1.0f; bad(GPT_E_INVAL, c);
  c = base; c.fp8_linears = 1; bad(GPT_E_INVAL, c);
  EXPECT(gpt_config_validate(nullptr) == GPT_E_NULLPTR);
  size_t ws = 0;
  c = base; c.n_layer = -5;
  EXPECT(gpt_workspace_size(&c, &ws) == GPT_E_INVAL);
  EXPECT(gpt_workspace_size(&base, nullptr) == GPT_E_NULLPTR);
  // status strings, including unknown codes
  for (int s = -9; s <= 1; ++s) EXPECT(gpt_status_string(s) != nullptr);
  // fp8 quantiser and decode attention: validation and dry runs
  void* p = reinterpret_cast<void*>(uintptr_t(1) << 20);
  EXPECT(gpt_debug_launches(-1, 1) == GPT_OK);
  EXPECT(gpt_fp8_quantize(p, GPT_DT_BF16, 300, 128, 0, (uint8_t*)p, (uint8_t*)p, 384,
                          (uint32_t*)p, nullptr) == GPT_OK);
  EXPECT(gpt_fp8_quantize(p, GPT_DT_BF16, 300, 100, 0, (uint8_t*)p, nullptr, 0, (uint32_t*)p,
                          nullptr) == GPT_E_INVAL);
  size_t dws = 0;
  EXPECT(gpt_decode_attn_workspace(16, 6, 6, 128, 2048, -1, &dws) == GPT_OK && dws > 0);
  EXPECT(gpt_decode_attn(16, 6, 6, 128, 2048, -1, p, p, p, (const int32_t*)p, p, p, dws,
                         nullptr) == GPT_OK);
  EXPECT(gpt_decode_attn_workspace(16, 6, 4, 128, 2048, -1, &dws) == GPT_E_INVAL);
  EXPECT(gpt_kv_cache_append(4, 3, 6, 2, 128, 100, p, (const int32_t*)p, p, p, nullptr) == GPT_OK);
  EXPECT(gpt_decode_attn_noalloc(64, 16, 16, 128, 2048, -1, p, p, p, (const int32_t*)p, p,
                                 nullptr) == GPT_E_WORKSPACE);
  EXPECT(gpt_debug_launches(-1, 0) == GPT_OK);
  if (g_fail) {
    std::fprintf(stderr, "%d expectations failed\n", g_fail);
    return 1;
  }
  std::printf("host sanitizer driver: all checks passed\n");
  return 0;
}
