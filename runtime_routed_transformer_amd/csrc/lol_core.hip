// Host side of liblol_core: argument validation, workspace layout, the
// per-depth launch sequence of the routed core, flags and timing.
//
// The depth loop follows Algorithm 1 of the paper "Library of Layers (LoL)"
// (App. A), routed depths only: partition, window means, router per window,
// the chosen block on each window, gated blend.  All windows of a depth read
// s^(l-1) and the blend writes each token exactly once, after every kernel
// of the depth that reads s^(l-1) has run (review "Library of Layers:
// Routing Whole Transformer Blocks at Runtime", reader's Algorithm 1 and the
// note after it: means come from the unchanged depth input, the new states
// replace the old ones after all windows), so the residual stream is
// updated in place.
#include <math.h>
#include <stdio.h>

#include <mutex>
#include <vector>

#include "lol_internal.h"

namespace lol {
int max_slots();

namespace {

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

lol_status validate(const lol_core_config *c) {
  if (!c) return LOL_EINVAL;
  if (c->batch < 1 || c->n < 1 || c->d < 1 || c->n_heads < 1 || c->d_ffn < 1 || c->L < 1 ||
      c->D < 1 || c->W < 1 || c->S < 0)
    return LOL_EINVAL;
  if (c->mlp != LOL_MLP_SWIGLU && c->mlp != LOL_MLP_GELU) return LOL_EINVAL;
  if (c->dtype != LOL_FP32 && c->dtype != LOL_BF16) return LOL_EINVAL;
  if (!(c->rms_eps > 0.f) || !(c->rope_theta >= 0.f) || isinf(c->rope_theta)) return LOL_EINVAL;
  if (c->d % c->n_heads != 0) return LOL_EINVAL;
  const int dh = c->d / c->n_heads;
  if (dh != 32 && dh != 64) return LOL_EUNSUPPORTED;
  if (c->d % 64 != 0 || c->d_ffn % 64 != 0) return LOL_EUNSUPPORTED;
  if (c->dtype == LOL_BF16 && (c->d % 128 != 0 || c->d_ffn % 128 != 0)) return LOL_EUNSUPPORTED;
  if (c->L > kMaxExperts) return LOL_EUNSUPPORTED;
  const long long kmax = (c->n + (long long)c->W - 1) / c->W + 1;
  if ((long long)c->batch * kmax > max_slots()) return LOL_EUNSUPPORTED;
  if ((long long)c->batch * c->n >= (1LL << 30)) return LOL_EUNSUPPORTED;  // int32 row ids
  if (c->d > 16384) return LOL_EUNSUPPORTED;  // the router input is staged in 64 KiB of LDS
  return LOL_OK;
}


// gcd of the lengths of a depth's windows (first, full and last windows of
// the partition with offset delta): every expert's grouped row count is a
// multiple of it, which tells the GEMMs which M tile height leaves no
// partial tiles.
int window_length_gcd(int n, int W, int delta, int K) {
  auto gcd = [](int a, int b) { while (b) { const int t = a % b; a = b; b = t; } return a; };
  int g = 0;
  for (int k = 0; k < K; ++k) {
    const int start = k * W - delta > 0 ? k * W - delta : 0;
    const int end = (k + 1) * W - delta - 1 < n - 1 ? (k + 1) * W - delta - 1 : n - 1;
    g = gcd(g, end - start + 1);
  }
  return g;
}

Plan make_plan(const lol_core_config *c) {
  Plan p;
  p.cfg = *c;
  p.K_max = (c->n + c->W - 1) / c->W + 1;
  p.d_head = c->d / c->n_heads;
  p.T = c->batch * c->n;
  p.n_slots = c->batch * p.K_max;
  p.n_tokens = p.T;
  p.act_bytes = c->dtype == LOL_BF16 ? 2 : 4;
  return p;
}

// ---- timing instrumentation ----
}  // namespace
thread_local LaunchEvents g_launch_ev;
namespace {
struct TimingRec {
  int kind;
  hipEvent_t a, b;
};
std::mutex g_tmu;
uint32_t g_timing = 0;  // bit k: time kernel kind k
int32_t g_timing_depth = -1;  // only this depth index (-1: all)
std::vector<TimingRec> g_recs;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  // timing only: no system-scope fence when the event completes, so no L2
  // writeback and invalidate between the timed kernel and the next one
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// Times one launcher call: its kernels are launched with the event pair
// attached to their dispatch packets (hipExtLaunchKernel), so the start and
// end timestamps are those of the kernels themselves and no marker packet
// sits between kernels (a separate hipEventRecord left the GPU idle about
// 6 us per marker).
struct Launch {
  hipStream_t st;
  bool timing;
  int kind;
  hipEvent_t a = nullptr, b = nullptr;
  Launch(hipStream_t s, bool t, int k) : st(s), timing(t), kind(k) {
    if (timing) {
      std::lock_guard<std::mutex> lk(g_tmu);
      a = take_event();
      b = a ? take_event() : nullptr;
      if (a && !b) {
        g_event_pool.push_back(a);
        a = nullptr;
      }
      g_launch_ev.start = a;
      g_launch_ev.stop = b;
    }
  }
  hipError_t done(hipError_t err) {
    if (a) {
      const bool launched = g_launch_ev.start == nullptr;   // a kernel took the start event
      g_launch_ev = LaunchEvents{};
      std::lock_guard<std::mutex> lk(g_tmu);
      if (launched && err == hipSuccess) {
        g_recs.push_back({kind, a, b});
      } else {
        g_event_pool.push_back(a);
        g_event_pool.push_back(b);
      }
    }
    return err;
  }
};

}  // namespace

// Compute units of the current device (cached per device).
hipError_t cu_count(int *n) {
  static int cached[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (cached[dev] == 0) {
    int v = 0;
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cached[dev] = v;
  }
  *n = cached[dev];
  return hipSuccess;
}

size_t workspace_layout(const Plan &p, char *base, Workspace *ws) {
  const lol_core_config &c = p.cfg;
  const size_t T = (size_t)p.T, d = (size_t)c.d, f = (size_t)c.d_ffn;
  const size_t ns = (size_t)p.n_slots;
  const int max_mtiles = (p.T + kTileM - 1) / kTileM + c.L;
  const int max_mtiles2 = (p.T + kTileM2 - 1) / kTileM2 + c.L;
  size_t off = 0;
  auto carve = [&](size_t bytes) -> char * {
    char *ptr = base ? base + off : nullptr;
    off += align_up(bytes);
    return ptr;
  };
  Workspace w;
  w.flags = (uint32_t *)carve(16);
  w.zpart = (float *)carve(ns * (d / 64) * (size_t)c.L * 4);
  w.zpart0 = (float *)carve((size_t)c.batch * (d / 64) * c.L * 4);
  w.zlog = (float *)carve(ns * (size_t)c.L * 4);
  w.win_exp = (int32_t *)carve(ns * 4);
  w.win_gate = (float *)carve(ns * 4);
  w.win_row0 = (int32_t *)carve(ns * 4);
  w.win_len = (int32_t *)carve(ns * 4);
  w.ecount = (int32_t *)carve((size_t)(c.L + 1) * 4);
  w.toff = (int32_t *)carve((size_t)(c.L + 1) * 4);
  w.mtile = (int32_t *)carve((size_t)max_mtiles * 8);
  w.mtile2 = (int32_t *)carve((size_t)max_mtiles2 * 8);
  w.mcount = (int32_t *)carve(3 * 4);
  w.row_tok = (int32_t *)carve(T * 4);
  w.row_pos = (int32_t *)carve(T * 4);
  w.row_exp = (int32_t *)carve(T * 4);
  w.row_gate = (float *)carve(T * 4);
  w.rope_cs = (float *)carve((size_t)c.W * (p.d_head / 2) * 2 * 4);
  w.u = carve(T * d * p.act_bytes);
  w.qkv = carve(T * 3 * d * p.act_bytes);
  w.o = carve(T * d * p.act_bytes);
  w.h = (float *)carve(T * d * 4);
  w.hid = carve(T * f * p.act_bytes);
  w.wo_p = o_norm_eligible(c) ? (bf16_t *)carve((size_t)c.L * d * d * 2) : nullptr;
  w.max_mtiles = max_mtiles;
  w.max_mtiles2 = max_mtiles2;
  if (ws) *ws = w;
  return off;
}

namespace {
lol_status forward_impl(const lol_core_config *cfg, int64_t n_tokens, const int32_t *doc_start,
                        const int32_t *doc_len, const float *s0, const lol_library *lib,
                        const lol_router *rt, const int32_t *forced_expert,
                        const float *forced_gate, float *s_out, const lol_path *path,
                        void *workspace, size_t workspace_bytes, void *stream, bool allow_timing);
hipError_t scratch_address(void **out);
}  // namespace
}  // namespace lol

using namespace lol;

extern "C" {

int32_t lol_core_k_max(const lol_core_config *cfg) {
  if (validate(cfg) == LOL_EINVAL) return -1;
  return (cfg->n + cfg->W - 1) / cfg->W + 1;
}

lol_status lol_core_validate(const lol_core_config *cfg) { return validate(cfg); }

size_t lol_core_workspace_size(const lol_core_config *cfg) {
  if (validate(cfg) != LOL_OK) return 0;
  return workspace_layout(make_plan(cfg), nullptr, nullptr);
}

lol_status lol_core_forward(const lol_core_config *cfg, const float *s0, const lol_library *lib,
                            const lol_router *rt, const int32_t *forced_expert,
                            const float *forced_gate, float *s_out, const lol_path *path,
                            void *workspace, size_t workspace_bytes, void *stream) {
  const lol_status vs = validate(cfg);
  if (vs != LOL_OK) return vs;
  return lol_core_forward_docs(cfg, (int64_t)cfg->batch * cfg->n, nullptr, nullptr, s0, lib, rt,
                               forced_expert, forced_gate, s_out, path, workspace, workspace_bytes,
                               stream);
}

lol_status lol_core_forward_docs(const lol_core_config *cfg, int64_t n_tokens,
                                 const int32_t *doc_start, const int32_t *doc_len,
                                 const float *s0, const lol_library *lib, const lol_router *rt,
                                 const int32_t *forced_expert, const float *forced_gate,
                                 float *s_out, const lol_path *path, void *workspace,
                                 size_t workspace_bytes, void *stream) {
  return forward_impl(cfg, n_tokens, doc_start, doc_len, s0, lib, rt, forced_expert, forced_gate,
                      s_out, path, workspace, workspace_bytes, stream, true);
}

}  // extern "C"

namespace lol {
namespace {
// Byte offsets of the three matrices inside lol_prepare_weight_panels'
// buffer (wqkv's panels start at 0); returns the buffer's size.
size_t weight_panel_layout(const lol_core_config &c, size_t *off_gu, size_t *off_down) {
  const size_t L = c.L, d = c.d, f = c.d_ffn;
  const size_t n_gu = c.mlp == LOL_MLP_SWIGLU ? 2 * f : f;
  const size_t qkv = L * 3 * d * d * 2, gu = L * n_gu * d * 2, down = L * d * f * 2;
  if (off_gu) *off_gu = qkv;
  if (off_down) *off_down = qkv + gu;
  return qkv + gu + down;
}

// The routed-core forward behind every entry point.  allow_timing = false
// leaves the timing instrumentation off for this call (it creates HIP
// events on first use).
lol_status forward_impl(const lol_core_config *cfg, int64_t n_tokens, const int32_t *doc_start,
                        const int32_t *doc_len, const float *s0, const lol_library *lib,
                        const lol_router *rt, const int32_t *forced_expert,
                        const float *forced_gate, float *s_out, const lol_path *path,
                        void *workspace, size_t workspace_bytes, void *stream, bool allow_timing) {
  const lol_status vs = validate(cfg);
  if (vs != LOL_OK) return vs;
  if (!s0 || !s_out || !lib || !rt) return LOL_EINVAL;
  if ((doc_start == nullptr) != (doc_len == nullptr)) return LOL_EINVAL;
  if (n_tokens < 1 || n_tokens >= (1LL << 30)) return LOL_EINVAL;
  if (!doc_len && n_tokens != (int64_t)cfg->batch * cfg->n) return LOL_EINVAL;
  if (!lib->wqkv || !lib->wo || !lib->w_gu || !lib->w_down || !lib->g_attn || !lib->g_ffn)
    return LOL_EINVAL;
  if ((lib->film_gamma == nullptr) != (lib->film_beta == nullptr)) return LOL_EINVAL;
  if (!rt->w_r || !rt->e_depth) return LOL_EINVAL;
  if ((rt->per_depth != 0 && rt->per_depth != 1) || (lib->film_per_expert != 0 && lib->film_per_expert != 1))
    return LOL_EINVAL;
  if (lib->weight_panels &&
      (cfg->dtype != LOL_BF16 || (reinterpret_cast<uintptr_t>(lib->weight_panels) & 15)))
    return LOL_EINVAL;
  Plan p = make_plan(cfg);
  p.doc_start = doc_start;
  p.doc_len = doc_len;
  p.n_tokens = (int)n_tokens;
  const size_t need = workspace_layout(p, nullptr, nullptr);
  if (!workspace || workspace_bytes < need) return LOL_EWORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return LOL_EINVAL;
  Workspace ws;
  workspace_layout(p, static_cast<char *>(workspace), &ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t timing;
  int32_t timing_depth;
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    timing = allow_timing ? g_timing : 0u;
    timing_depth = g_timing_depth;
  }
  int cur_depth = -1;   // depth index of the launches below (-1: before the first depth)
  const lol_core_config &c = p.cfg;
  const size_t d = c.d, f = c.d_ffn;
  const bool glu = c.mlp == LOL_MLP_SWIGLU;
  hipError_t err;
#define LOL_TRY(kind, call)                           \
  do {                                                \
    Launch _l(st, ((timing >> (kind)) & 1u) && (timing_depth < 0 || timing_depth == cur_depth), kind); \
    err = _l.done(call);                              \
    if (err != hipSuccess) return LOL_EHIP;           \
  } while (0)

  // Depth 1 reads s0 and its blend writes s_out: every token (of every
  // document) lies in exactly one window per depth, so s_out is complete
  // after it (no copy of s0).
  // With the fused output projection (bf16, d a multiple of 256 up to 1024)
  // the blend is split: the O kernel writes s_out = s + gate * Attn and the
  // down projection adds gate * MLP.
  const bool fused_o = o_norm_fused(p);
  // bf16 GEMM inputs written by this library's own kernels go in 32-k
  // panels: a stage of an A tile is then one block of whole lines
  const bool bf16 = c.dtype == LOL_BF16;
  const bool qkv_panels = bf16 && panels_addressable(p, c.d);        // u from the attention norm
  const bool down_panels = bf16 && panels_addressable(p, c.d_ffn);   // hid from the gate/up epilogue
  LOL_TRY(KK_SETUP, launch_setup(p, ws, st));
  // W_o in 16-k panels for the fused output projection, unless the caller
  // prepared them once (lol_prepare_wo_panels)
  if (fused_o && !lib->wo_panels) LOL_TRY(KK_SETUP, launch_pack_wo(c, lib->wo, ws.wo_p, st));
  // the experts' QKV, gate/up and down weights in 32-k panels, when the
  // caller prepared them (lol_prepare_weight_panels)
  const char *wpan = static_cast<const char *>(lib->weight_panels);
  size_t wpan_gu = 0, wpan_down = 0;
  weight_panel_layout(c, &wpan_gu, &wpan_down);
  for (int l = 0; l < c.D; ++l) {
    cur_depth = l;
    const float *s = l == 0 ? s0 : s_out;   // depth input
    DepthGeom g;
    g.depth = l;
    g.delta = (int)(((long long)l * c.S) % c.W);
    g.K = (c.n - 1 + g.delta) / c.W + 1;
    // ragged documents end windows anywhere: no common divisor to exploit
    g.len_gcd = doc_len ? 1 : window_length_gcd(c.n, c.W, g.delta, g.K);
    LOL_TRY(KK_POOL, launch_pool(p, g, s, ws, *rt, st));
    LOL_TRY(KK_ROUTE, launch_route(p, g, s, ws, *rt, forced_expert, forced_gate, path, st));
    LOL_TRY(KK_NORM_ATTN, launch_norm(p, g, 0, s, *lib, ws, qkv_panels ? p.T : 0, st));
    GemmArgs a{};
    a.A = ws.u;
    a.Wt = lib->wqkv;
    a.N = 3 * c.d;
    a.K = c.d;
    a.w_expert_stride = (long long)3 * d * d;
    // bf16 mode rotates q and k in the GEMM epilogue, before their one
    // rounding to bf16; fp32 mode rotates inside its attention kernel
    a.len_gcd = g.len_gcd;
    const bool rope_in_gemm = c.dtype == LOL_BF16 && c.rope_theta != 0.f;
    a.epi = rope_in_gemm ? EPI_QKV_ROPE : EPI_STORE;
    a.rope_cols = rope_in_gemm ? 2 * c.d : 0;
    a.C = ws.qkv;
    a.a_panel_rows = qkv_panels ? p.T : 0;
    if (wpan) {
      a.Wt = wpan;
      a.b_panel_rows = 3 * c.d;
    }
    LOL_TRY(KK_GEMM_QKV, launch_gemm(p, ws, a, st));
    LOL_TRY(KK_ATTN, launch_attention(p, g, ws, fused_o ? p.T : 0, st));
    if (fused_o) {
      LOL_TRY(KK_GEMM_O, launch_o_norm(p, g, ws, s, s_out, *lib, p.T, st));
    } else {
      a = GemmArgs{};
      a.len_gcd = g.len_gcd;
      a.A = ws.o;
      a.Wt = lib->wo;
      a.N = c.d;
      a.K = c.d;
      a.w_expert_stride = (long long)d * d;
      a.epi = EPI_RESID;
      a.C = ws.h;
      a.s_in = s;
      LOL_TRY(KK_GEMM_O, launch_gemm(p, ws, a, st));
      LOL_TRY(KK_NORM_FFN, launch_norm(p, g, 1, s, *lib, ws, 0, st));
    }
    a = GemmArgs{};
    a.len_gcd = g.len_gcd;
    a.A = ws.u;
    a.Wt = lib->w_gu;
    a.N = c.d_ffn;
    a.K = c.d;
    a.w_expert_stride = (long long)(glu ? 2 : 1) * f * d;
    a.glu_offset = c.d_ffn;
    a.epi = glu ? EPI_SWIGLU : EPI_GELU;
    a.C = ws.hid;
    // the fused O kernel leaves u in 32-k panels: whole-line loads per stage
    a.a_panel_rows = fused_o ? p.T : 0;
    a.c_panel_rows = down_panels ? p.T : 0;
    if (wpan) {
      a.Wt = wpan + wpan_gu;
      a.b_panel_rows = (glu ? 2 : 1) * c.d_ffn;
    }
    LOL_TRY(KK_GEMM_GATE_UP, launch_gemm(p, ws, a, st));
    a = GemmArgs{};
    a.len_gcd = g.len_gcd;
    a.A = ws.hid;
    a.Wt = lib->w_down;
    a.N = c.d;
    a.K = c.d_ffn;
    a.w_expert_stride = (long long)d * f;
    a.a_panel_rows = down_panels ? p.T : 0;
    if (fused_o) {
      a.epi = EPI_ACCUM;
      a.s_in = s_out;
      // h is not used on this path: it holds the K-split tail's partial tiles
      a.part = ws.h;
      a.part_slots = (int)((long long)p.T * c.d / (kTileM2 * 256));
    } else {
      a.epi = EPI_BLEND;
      a.s_in = s;
      a.h = ws.h;
    }
    a.s = s_out;
    if (wpan) {
      a.Wt = wpan + wpan_down;
      a.b_panel_rows = c.d;
    }
    LOL_TRY(KK_GEMM_DOWN, launch_gemm(p, ws, a, st));
  }
#undef LOL_TRY
  return LOL_OK;
}

// ---- The forward without a workspace argument ----
// Callers that cannot allocate (inside HIP graph capture, in tight serving
// loops) use a workspace that lives in the library itself: one array per
// device, allocated when the code object is loaded and held until the
// process ends.  Every call on a device shares it.
static __device__ __align__(256) char scratch[LOL_STATIC_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up once per
// device (hipGetSymbolAddress): the host-side name is only a stand-in.
hipError_t scratch_address(void **out) {
  static std::mutex mu;
  static void *addr[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return hipSuccess;
}
}  // namespace
}  // namespace lol

extern "C" {

lol_status lol_core_forward_static(const lol_core_config *cfg, const float *s0,
                                   const lol_library *lib, const lol_router *rt,
                                   const int32_t *forced_expert, const float *forced_gate,
                                   float *s_out, const lol_path *path, void *stream) {
  const lol_status vs = validate(cfg);
  if (vs != LOL_OK) return vs;
  const size_t need = lol_core_workspace_size(cfg);
  if (need > (size_t)LOL_STATIC_SCRATCH_BYTES) return LOL_EWORKSPACE;
  if (!s0 || !s_out || !lib || !rt) return LOL_EINVAL;
  void *ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return LOL_EHIP;
  return forward_impl(cfg, (int64_t)cfg->batch * cfg->n, nullptr, nullptr, s0, lib, rt,
                      forced_expert, forced_gate, s_out, path, ws, LOL_STATIC_SCRATCH_BYTES,
                      stream, false);
}

size_t lol_decode_state_size(const lol_core_config *cfg) {
  if (validate(cfg) != LOL_OK || !decode_supported(*cfg)) return 0;
  return decode_layout(*cfg, nullptr, nullptr);
}

lol_status lol_decode_reset(const lol_core_config *cfg, void *state, size_t state_bytes,
                            void *stream) {
  const lol_status vs = validate(cfg);
  if (vs != LOL_OK) return vs;
  if (!decode_supported(*cfg)) return LOL_EUNSUPPORTED;
  if (!state || state_bytes < decode_layout(*cfg, nullptr, nullptr) ||
      (reinterpret_cast<uintptr_t>(state) & 255))
    return LOL_EWORKSPACE;
  DecodeBufs s;
  decode_layout(*cfg, static_cast<char *>(state), &s);
  if (launch_dec_reset(*cfg, s, -1, static_cast<hipStream_t>(stream)) != hipSuccess) return LOL_EHIP;
  return LOL_OK;
}

lol_status lol_decode_reset_row(const lol_core_config *cfg, void *state, size_t state_bytes,
                                int32_t row, void *stream) {
  const lol_status vs = validate(cfg);
  if (vs != LOL_OK) return vs;
  if (!decode_supported(*cfg)) return LOL_EUNSUPPORTED;
  if (row < 0 || row >= cfg->batch) return LOL_EINVAL;
  if (!state || state_bytes < decode_layout(*cfg, nullptr, nullptr) ||
      (reinterpret_cast<uintptr_t>(state) & 255))
    return LOL_EWORKSPACE;
  DecodeBufs s;
  decode_layout(*cfg, static_cast<char *>(state), &s);
  if (launch_dec_reset(*cfg, s, row, static_cast<hipStream_t>(stream)) != hipSuccess) return LOL_EHIP;
  return LOL_OK;
}

lol_status lol_decode_step(const lol_core_config *cfg, int32_t pos, const float *x,
                           const lol_library *lib, const lol_router *rt,
                           const int32_t *forced_expert, const float *forced_gate, float *y,
                           const lol_path *path, void *state, size_t state_bytes, void *stream) {
  const lol_status vs = validate(cfg);
  if (vs != LOL_OK) return vs;
  if (!decode_supported(*cfg)) return LOL_EUNSUPPORTED;
  if (!x || !y || !lib || !rt) return LOL_EINVAL;
  if (!lib->wqkv || !lib->wo || !lib->w_gu || !lib->w_down || !lib->g_attn || !lib->g_ffn)
    return LOL_EINVAL;
  if ((lib->film_gamma == nullptr) != (lib->film_beta == nullptr)) return LOL_EINVAL;
  if (!rt->w_r || !rt->e_depth) return LOL_EINVAL;
  if ((rt->per_depth != 0 && rt->per_depth != 1) || (lib->film_per_expert != 0 && lib->film_per_expert != 1))
    return LOL_EINVAL;
  if (pos < -1 || pos >= cfg->n) return LOL_EINVAL;
  if (!state || state_bytes < decode_layout(*cfg, nullptr, nullptr) ||
      (reinterpret_cast<uintptr_t>(state) & 255))
    return LOL_EWORKSPACE;
  DecodeBufs s;
  decode_layout(*cfg, static_cast<char *>(state), &s);
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t timing;
  int32_t timing_depth;
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    timing = g_timing;
    timing_depth = g_timing_depth;
  }
  const lol_core_config &c = *cfg;
  int cur_depth = -1;
  hipError_t err;
#define LOL_TRY(kind, call)                           \
  do {                                                \
    Launch _l(st, ((timing >> (kind)) & 1u) && (timing_depth < 0 || timing_depth == cur_depth), kind); \
    err = _l.done(call);                              \
    if (err != hipSuccess) return LOL_EHIP;           \
  } while (0)
  // each document's position lives on the device (the route kernel of depth
  // 0 takes it), so the window geometry of every depth is computed there and
  // a call with pos = -1 has no per-call arguments (it can be captured once
  // in a graph and replayed)
  for (int l = 0; l < c.D; ++l) {
    cur_depth = l;
    const float *xin = l == 0 ? x : y;   // depth input; y holds s^(l) afterwards
    LOL_TRY(KK_ROUTE, launch_dec_route(c, s, l, pos, xin, *lib, *rt, forced_expert, forced_gate,
                                       path, st));
    LOL_TRY(KK_GEMM_QKV, launch_dec_gemv(c, s, l, DEC_QKV, xin, y, *lib, st));
    LOL_TRY(KK_ATTN, launch_dec_attn(c, s, l, st));
    LOL_TRY(KK_GEMM_O, launch_dec_gemv(c, s, l, DEC_O, xin, y, *lib, st));
    LOL_TRY(KK_NORM_FFN, launch_dec_norm(c, s, l, *lib, st));
    LOL_TRY(KK_GEMM_GATE_UP, launch_dec_gemv(c, s, l, DEC_GU, xin, y, *lib, st));
    LOL_TRY(KK_GEMM_DOWN, launch_dec_gemv(c, s, l, DEC_DOWN, xin, y, *lib, st));
  }
#undef LOL_TRY
  return LOL_OK;
}

lol_status lol_decode_read_flags(void *state, uint32_t *flags, void *stream) {
  if (!state || !flags) return LOL_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t *dflags = static_cast<uint32_t *>(state) + 1;  // header word 1
  if (hipMemcpyAsync(flags, dflags, sizeof(uint32_t), hipMemcpyDeviceToHost, st) != hipSuccess)
    return LOL_EHIP;
  if (hipStreamSynchronize(st) != hipSuccess) return LOL_EHIP;
  if (hipMemsetAsync(dflags, 0, sizeof(uint32_t), st) != hipSuccess) return LOL_EHIP;
  if (hipStreamSynchronize(st) != hipSuccess) return LOL_EHIP;
  return LOL_OK;
}

size_t lol_prepare_wo_panels_size(const lol_core_config *cfg) {
  if (validate(cfg) != LOL_OK || !o_norm_eligible(*cfg)) return 0;
  return (size_t)cfg->L * cfg->d * cfg->d * 2;
}

lol_status lol_prepare_wo_panels(const lol_core_config *cfg, const void *wo, void *wo_panels,
                                 void *stream) {
  const lol_status vs = validate(cfg);
  if (vs != LOL_OK) return vs;
  if (!o_norm_eligible(*cfg)) return LOL_EUNSUPPORTED;
  if (!wo || !wo_panels || (reinterpret_cast<uintptr_t>(wo) & 15) ||
      (reinterpret_cast<uintptr_t>(wo_panels) & 15))
    return LOL_EINVAL;
  const size_t bytes = lol_prepare_wo_panels_size(cfg);
  const uintptr_t a = reinterpret_cast<uintptr_t>(wo), b = reinterpret_cast<uintptr_t>(wo_panels);
  if (a < b + bytes && b < a + bytes) return LOL_EINVAL;   // overlapping buffers
  if (launch_pack_wo(*cfg, wo, wo_panels, static_cast<hipStream_t>(stream)) != hipSuccess)
    return LOL_EHIP;
  return LOL_OK;
}

size_t lol_prepare_weight_panels_size(const lol_core_config *cfg) {
  if (validate(cfg) != LOL_OK || cfg->dtype != LOL_BF16) return 0;
  return weight_panel_layout(*cfg, nullptr, nullptr);
}

lol_status lol_prepare_weight_panels(const lol_core_config *cfg, const lol_library *lib,
                                     void *weight_panels, void *stream) {
  const lol_status vs = validate(cfg);
  if (vs != LOL_OK) return vs;
  if (cfg->dtype != LOL_BF16) return LOL_EUNSUPPORTED;
  if (!lib || !weight_panels || (reinterpret_cast<uintptr_t>(weight_panels) & 15)) return LOL_EINVAL;
  const void *src[3] = {lib->wqkv, lib->w_gu, lib->w_down};
  size_t off[3] = {0, 0, 0};
  const size_t bytes = weight_panel_layout(*cfg, &off[1], &off[2]);
  const size_t len[3] = {off[1], off[2] - off[1], bytes - off[2]};
  const uintptr_t b = reinterpret_cast<uintptr_t>(weight_panels);
  for (int i = 0; i < 3; ++i) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(src[i]);
    if (!src[i] || (a & 15)) return LOL_EINVAL;
    if (a < b + bytes && b < a + len[i]) return LOL_EINVAL;   // overlapping buffers
  }
  const int d = cfg->d, f = cfg->d_ffn, L = cfg->L;
  const int n_gu = cfg->mlp == LOL_MLP_SWIGLU ? 2 * f : f;
  char *dst = static_cast<char *>(weight_panels);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (launch_pack_panels(lib->wqkv, dst, L, 3 * d, d, 32, st) != hipSuccess ||
      launch_pack_panels(lib->w_gu, dst + off[1], L, n_gu, d, 32, st) != hipSuccess ||
      launch_pack_panels(lib->w_down, dst + off[2], L, d, f, 32, st) != hipSuccess)
    return LOL_EHIP;
  return LOL_OK;
}

size_t lol_core_buckets_size(const lol_core_config *cfg) {
  if (validate(cfg) != LOL_OK) return 0;
  const Plan p = make_plan(cfg);
  Workspace w;
  workspace_layout(p, nullptr, &w);
  return (size_t)cfg->L + (cfg->L + 1) + (size_t)p.n_slots + 2 + 2 * (size_t)w.max_mtiles +
         2 * (size_t)w.max_mtiles2;
}

lol_status lol_core_read_buckets(const lol_core_config *cfg, const void *workspace,
                                 size_t workspace_bytes, int32_t *out, void *stream) {
  const lol_status vs = validate(cfg);
  if (vs != LOL_OK) return vs;
  if (!out) return LOL_EINVAL;
  const Plan p = make_plan(cfg);
  if (!workspace || workspace_bytes < workspace_layout(p, nullptr, nullptr) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255))
    return LOL_EWORKSPACE;
  Workspace w;
  workspace_layout(p, static_cast<char *>(const_cast<void *>(workspace)), &w);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t L = cfg->L;
  struct Piece { const int32_t *src; size_t count; } pieces[] = {
      {w.ecount, L}, {w.toff, L + 1}, {w.win_row0, (size_t)p.n_slots}, {w.mcount, 2},
      {w.mtile, 2 * (size_t)w.max_mtiles}, {w.mtile2, 2 * (size_t)w.max_mtiles2}};
  int32_t *dst = out;
  for (const Piece &pc : pieces) {
    if (hipMemcpyAsync(dst, pc.src, pc.count * 4, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return LOL_EHIP;
    dst += pc.count;
  }
  return LOL_OK;
}

size_t lol_measure_mfma_bf16_scratch_size(void) {
  int ncu = 0;
  if (cu_count(&ncu) != hipSuccess || ncu < 1) return 0;
  return mfma_ceiling_scratch_bytes(ncu);
}

lol_status lol_measure_mfma_bf16(int32_t shape, int32_t random_operands, int32_t iters,
                                 void *scratch, size_t scratch_bytes, double *tflops, double *ghz,
                                 void *stream) {
  if (!scratch || !tflops || !ghz || iters < 1 || iters > (1 << 24) || (shape != 16 && shape != 32) ||
      (random_operands != 0 && random_operands != 1) ||
      (reinterpret_cast<uintptr_t>(scratch) & 255))
    return LOL_EINVAL;
  int ncu = 0;
  if (cu_count(&ncu) != hipSuccess || ncu < 1) return LOL_EHIP;
  if (scratch_bytes < mfma_ceiling_scratch_bytes(ncu)) return LOL_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // one untimed launch (clocks ramp up, code is loaded), then the measured one
  for (int rep = 0; rep < 2; ++rep)
    if (launch_mfma_ceiling(shape, ncu, rep == 0 ? (iters + 7) / 8 : iters, random_operands, scratch, st) !=
        hipSuccess)
      return LOL_EHIP;
  std::vector<long long> clk((size_t)ncu * 2);
  const char *src = static_cast<const char *>(scratch) + (size_t)ncu * 512 * sizeof(float);
  if (hipMemcpyAsync(clk.data(), src, clk.size() * sizeof(long long), hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return LOL_EHIP;
  long long longest = 0;
  double clock_sum = 0.0;
  for (int b = 0; b < ncu; ++b) {
    const long long cyc = clk[2 * b], ref = clk[2 * b + 1];
    if (ref <= 0) return LOL_EHIP;
    longest = ref > longest ? ref : longest;
    clock_sum += (double)cyc / (double)ref * 0.1;   // s_memrealtime ticks at 100 MHz
  }
  const double seconds = (double)longest * 1e-8;
  *tflops = mfma_ceiling_flops_per_block(iters) * ncu / seconds * 1e-12;
  *ghz = clock_sum / ncu;
  return LOL_OK;
}

lol_status lol_core_read_flags(void *workspace, uint32_t *flags, void *stream) {
  if (!workspace || !flags) return LOL_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t *dflags = static_cast<uint32_t *>(workspace);  // flags are the first workspace word
  if (hipMemcpyAsync(flags, dflags, sizeof(uint32_t), hipMemcpyDeviceToHost, st) != hipSuccess)
    return LOL_EHIP;
  if (hipStreamSynchronize(st) != hipSuccess) return LOL_EHIP;
  if (hipMemsetAsync(dflags, 0, sizeof(uint32_t), st) != hipSuccess) return LOL_EHIP;
  if (hipStreamSynchronize(st) != hipSuccess) return LOL_EHIP;
  return LOL_OK;
}

lol_status lol_core_timing_enable(uint32_t mask) {
  if (mask & ~(uint32_t)LOL_TIMING_ALL) return LOL_EINVAL;
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing = mask;
  return LOL_OK;
}

lol_status lol_core_timing_depth(int32_t depth) {
  if (depth < -1) return LOL_EINVAL;
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing_depth = depth;
  return LOL_OK;
}

lol_status lol_core_timing_collect(double *ms, int32_t *launches) {
  if (!ms || !launches) return LOL_EINVAL;
  std::lock_guard<std::mutex> lk(g_tmu);
  lol_status status = LOL_OK;
  for (TimingRec &r : g_recs) {
    float t = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
      status = LOL_EHIP;
    else {
      ms[r.kind] += t;
      launches[r.kind] += 1;
    }
    g_event_pool.push_back(r.a);
    g_event_pool.push_back(r.b);
  }
  g_recs.clear();
  return status;
}

const char *lol_core_kernel_name(int32_t kind) {
  static const char *names[LOL_KERNEL_KINDS] = {
      "setup",    "pool",     "route",  "bucket", "rowmeta",      "norm_attn",
      "gemm_qkv", "win_attn", "gemm_o", "norm_ffn", "gemm_gate_up", "gemm_down"};
  if (kind < 0 || kind >= LOL_KERNEL_KINDS) return nullptr;
  return names[kind];
}

const char *lol_status_str(lol_status status) {
  switch (status) {
    case LOL_OK: return "ok";
    case LOL_EINVAL: return "invalid argument";
    case LOL_EUNSUPPORTED: return "unsupported configuration";
    case LOL_EWORKSPACE: return "workspace missing or too small";
    case LOL_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

}  // extern "C"
