// Routing kernels of the routed core: window means, prefix router with
// biased top-1 choice, expert bucketing of windows, grouped-row metadata and
// the RoPE angle table.
//
// Method: paper "Library of Layers (LoL)", Sec. 3.2.1 (window partition),
// Sec. 3.2.2 and Algorithm 1 (router input from earlier windows' means,
// first-window rule), App. A (loss-free balancing: the bias enters the
// choice only, the gate is the unbiased probability); review "Library of
// Layers: Routing Whole Transformer Blocks at Runtime", Eqs. 2, 4 and 5.
#include <math.h>

#include "lol_internal.h"

namespace lol {
namespace {

constexpr int kMaxSlots = 8192;  // documents x window slots handled by one bucketing block
constexpr int kZlogLds = 8192;   // window logits (slots x experts) kept in LDS up to this many

__device__ __forceinline__ int win_start(int k, int W, int delta) { return max(0, k * W - delta); }
__device__ __forceinline__ int win_end(int k, int W, int delta, int n) {
  return min(n - 1, (k + 1) * W - delta - 1);
}

// Document b: its first token in the residual stream and its length.
// Without a document table it is row b of the [B][n] layout.  With one, the
// entry is clamped so that the document lies inside the n_tokens rows of the
// stream with 1 <= length <= n; k_route_all flags entries that needed it.
struct DocSpan {
  int start, len;
};
__device__ __forceinline__ DocSpan doc_span(const int32_t *__restrict__ doc_start,
                                            const int32_t *__restrict__ doc_len, int b, int n,
                                            int n_tokens) {
  if (!doc_len) return {b * n, n};
  const int len = min(min(max(doc_len[b], 1), n), n_tokens);
  return {min(max(doc_start[b], 0), n_tokens - len), len};
}
// windows of a document of nb tokens at offset delta
__device__ __forceinline__ int doc_windows(int nb, int W, int delta) { return (nb - 1 + delta) / W + 1; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// butterfly reductions inside aligned groups of G lanes (G a power of two)
__device__ __forceinline__ float group_max(float v, int G) {
  for (int o = G >> 1; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float group_sum(float v, int G) {
  for (int o = G >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int group_min(int v, int G) {
  for (int o = G >> 1; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// a2, and the router's linear layer applied to it.  Block = (window,
// 64-column chunk): mu = mean of s over the window's tokens in the chunk
// (16 row phases x 16 float4 columns, fixed-order reduction), then
// zpart[window][chunk][m] = sum_c W_r[m][c] mu[c] for every expert m.  The
// router input of window k > 0 is the mean of the earlier windows' means, so
// its logits are the mean of their zpart sums (the layer is linear); the
// first window's input (e_l + s_0) / 2 is contracted here as well, by the
// blocks of window 0.
__global__ void __launch_bounds__(256) k_pool(const float *__restrict__ s,
                                              const float *__restrict__ w_r,
                                              const float *__restrict__ e_depth,
                                              float *__restrict__ zpart, float *__restrict__ zpart0,
                                              int n, int d, int L, int W, int delta, int K,
                                              int K_max, int depth,
                                              const int32_t *__restrict__ doc_start,
                                              const int32_t *__restrict__ doc_len, int n_tokens) {
  const int b = blockIdx.x / K, k = blockIdx.x % K, chunk = blockIdx.y, nch = gridDim.y;
  const DocSpan doc = doc_span(doc_start, doc_len, b, n, n_tokens);
  if (k >= doc_windows(doc.len, W, delta)) return;  // past the end of a shorter document
  const int start = win_start(k, W, delta), len = win_end(k, W, delta, doc.len) - start + 1;
  const int c4 = threadIdx.x & 15, ph = threadIdx.x >> 4;
  const int col = chunk * 64 + c4 * 4;
  const float *base = s + ((size_t)doc.start + start) * d + col;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // rows ph, ph + 16, ... in batches of 8 whose loads are all in flight
  // before the first add
  for (int r0 = ph; r0 < len; r0 += 8 * 16) {
    float4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = r0 + 16 * i;
      v[i] = r < len ? *reinterpret_cast<const float4 *>(base + (size_t)r * d)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc.x += v[i].x; acc.y += v[i].y; acc.z += v[i].z; acc.w += v[i].w;
    }
  }
  __shared__ float4 red[16][16];
  __shared__ float mu[64], r0[64];
  red[ph][c4] = acc;
  __syncthreads();
  if (ph == 0) {
    float4 t = red[0][c4];
    for (int i = 1; i < 16; ++i) {
      t.x += red[i][c4].x; t.y += red[i][c4].y; t.z += red[i][c4].z; t.w += red[i][c4].w;
    }
    const float fl = (float)len;
    mu[c4 * 4 + 0] = t.x / fl; mu[c4 * 4 + 1] = t.y / fl;
    mu[c4 * 4 + 2] = t.z / fl; mu[c4 * 4 + 3] = t.w / fl;
  }
  if (k == 0 && threadIdx.x < 64) {
    const int c = chunk * 64 + threadIdx.x;
    r0[threadIdx.x] = 0.5f * (e_depth[(size_t)depth * d + c] + s[(size_t)doc.start * d + c]);
  }
  __syncthreads();
  // one wave per expert (4 waves), lane = column of the chunk
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int m = wave; m < L; m += 4) {
    const float w = w_r[(size_t)m * d + chunk * 64 + lane];
    const float z = wave_sum(w * mu[lane]);
    if (lane == 0) zpart[(((size_t)b * K_max + k) * nch + chunk) * L + m] = z;
    if (k == 0) {
      const float z0 = wave_sum(w * r0[lane]);
      if (lane == 0) zpart0[((size_t)b * nch + chunk) * L + m] = z0;
    }
  }
}

// a3 - a5 in one workgroup of 1024 threads (16 waves), for all documents:
//  1. router logits: Y_j = sum over chunks of zpart_j (= W_r mu_j), then
//     z_k = (Y_0 + .. + Y_{k-1}) / k + b_r for k > 0 and z_0 = the window-0
//     contraction + b_r (one thread per (document, expert), running sum
//     over the windows in order);
//  2. per window (one wave each): a = softmax(z) in fp32, choice = lowest
//     index attaining max(a + bias), gate = a_choice, margin = top1 - top2
//     of a + bias, forcing as documented in the C ABI; slots k >= K get
//     expert -1;
//  3. bucketing: windows grouped by expert, in slot order inside an expert
//     (stable), so every expert's tokens form one contiguous range of grouped
//     rows; per-expert counts and row offsets, the first grouped row of every
//     window, and the M-tile tables (expert, first row) for kTileM- and
//     kTileM2-row tiles;
// The grouped-row metadata (token, window-local position, expert and gate of
// every grouped row) are written by the attention norm, which visits every
// window's rows anyway.
// Integer counts only (LDS atomics on integers), so the result does not
// depend on thread timing.
__global__ void __launch_bounds__(1024) k_route_all(
    const float *__restrict__ zpart, float *__restrict__ zpart0, const float *__restrict__ b_r,
    const float *__restrict__ bias, const int32_t *__restrict__ forced_e,
    const float *__restrict__ forced_g, int32_t *__restrict__ win_exp, float *__restrict__ win_gate,
    int32_t *__restrict__ win_row0, int32_t *__restrict__ path_e, float *__restrict__ path_g,
    float *__restrict__ path_m, uint32_t *__restrict__ flags, int32_t *__restrict__ ecount,
    int32_t *__restrict__ toff_out, int32_t *__restrict__ mtile, int max_mtiles,
    int32_t *__restrict__ mtile2, int max_mtiles2, int32_t *__restrict__ mcount,
    float *__restrict__ zlog_g, int n, int nch, int L, int W, int delta,
    int K, int K_max, int B, int depth, int32_t *__restrict__ win_len,
    const int32_t *__restrict__ doc_start, const int32_t *__restrict__ doc_len, int n_tokens,
    int32_t *__restrict__ path_util) {
  __shared__ int s_exp[kMaxSlots];
  __shared__ int s_len[kMaxSlots];
  __shared__ int cnt_w[kMaxExperts], cnt_t[kMaxExperts];
  __shared__ int toff[kMaxExperts + 1];
  // M-tile tables (128- and 256-row tiles): every expert's full tiles in
  // expert order, then the partial last tiles, so that partial (cheaper)
  // tiles are the last ones a GEMM hands out
  __shared__ int fo[kMaxExperts + 1], po[kMaxExperts + 1], fo2[kMaxExperts + 1], po2[kMaxExperts + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n_slots = B * K_max;
  // the router's own bias and the balancing bias, read once
  __shared__ float s_br[kMaxExperts], s_bias[kMaxExperts];
  if (tid < L) {
    s_br[tid] = b_r ? b_r[tid] : 0.f;
    s_bias[tid] = bias ? bias[tid] : 0.f;
  }
  // window logits live in LDS when they fit, else in the workspace
  __shared__ float s_zlog[kZlogLds];
  float *const zlog = (size_t)n_slots * L <= kZlogLds ? s_zlog : zlog_g;

  // 1. logits of every window, zlog[b][k][m]: first Y_k = sum over chunks
  // (slot k >= 1 holds Y_{k-1}; slot 0 the window-0 contraction), then one
  // wave per (document, expert) turns Y into running means with a scan over k
  for (int i = tid; i < B * K * L; i += blockDim.x) {
    const int m = i % L, k = (i / L) % K, b = i / (L * K);
    // the chunk partials of one window, 16 loads in flight at a time, summed
    // in chunk order
    const float *zp = k == 0 ? zpart0 + (size_t)b * nch * L + m
                             : zpart + ((size_t)b * K_max + k - 1) * nch * L + m;
    float y = 0.f;
    for (int c0 = 0; c0 < nch; c0 += 16) {
      float t[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) t[i] = c0 + i < nch ? zp[(size_t)(c0 + i) * L] : 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) y += t[i];
    }
    zlog[((size_t)b * K_max + k) * L + m] = y;
  }
  __syncthreads();
  // segments of SEG lanes, one (document, expert) each: 4 per wave when a
  // document has at most 16 windows, 2 up to 32, else one per wave with a
  // carry across passes of 64 windows (the per-element sums are the same
  // for every segment width)
  {
    const int SEG = K <= 16 ? 16 : (K <= 32 ? 32 : 64);
    const int pw = 64 / SEG, sl = lane & (SEG - 1), sp = lane / SEG;
    for (int bm0 = wave * pw; bm0 < B * L; bm0 += 16 * pw) {
      const int bm = bm0 + sp;
      const bool okp = bm < B * L;
      const int b = okp ? bm / L : 0, m = okp ? bm % L : 0;
      const float br = s_br[m];
      float carry = 0.f;
      for (int k0 = 0; k0 < K; k0 += SEG) {
        const int k = k0 + sl;
        const bool okk = okp && k < K;
        float *zp = zlog + ((size_t)b * K_max + k) * L + m;
        const float y = okk ? *zp : 0.f;
        // inclusive scan of Y over k >= 1 (slot 0 is not part of the prefix)
        float v = (k >= 1) ? y : 0.f;
        for (int o = 1; o < SEG; o <<= 1) {
          const float t = __shfl_up(v, o, SEG);
          if (sl >= o) v += t;
        }
        v += carry;
        if (okk) *zp = (k == 0 ? y : v / (float)k) + br;
        carry = __shfl(v, SEG - 1, SEG);
      }
    }
  }
  for (int i = tid; i < kMaxExperts; i += blockDim.x) { cnt_w[i] = 0; cnt_t[i] = 0; }
  // a document table must hold, in increasing order, disjoint documents of
  // 1..n tokens inside the stream's n_tokens rows
  if (doc_len && depth == 0) {
    for (int b = tid; b < B; b += blockDim.x) {
      const int st = doc_start[b], ln = doc_len[b];
      bool bad = ln < 1 || ln > n || st < 0 || st > n_tokens - ln;
      if (!bad && b + 1 < B) bad = st + ln > doc_start[b + 1];
      if (bad) atomicOr(flags, (uint32_t)LOL_FLAG_BAD_DOC);
    }
  }
  __syncthreads();

  // 2. score and select: groups of G lanes (G = the power of two >= L), one
  // window per group, lane = expert inside it
  const int G = L <= 1 ? 1 : 1 << (32 - __clz(L - 1));
  const int gl = lane & (G - 1), per_wave = 64 / G;
  for (int slot0 = wave * per_wave; slot0 < n_slots; slot0 += 16 * per_wave) {
    const int slot = slot0 + lane / G;
    const bool in_range = slot < n_slots;
    const int b = slot / K_max, k = slot % K_max;
    const int nb = in_range ? doc_span(doc_start, doc_len, b, n, n_tokens).len : n;
    const bool win_ok = in_range && k < K && k < doc_windows(nb, W, delta);
    const size_t pidx = ((size_t)depth * B + b) * K_max + k;
    const bool live = win_ok && gl < L;
    const float zl = live ? zlog[(size_t)slot * L + gl] : -INFINITY;
    const float zmax = group_max(zl, G);
    const float ez = live ? expf(zl - zmax) : 0.f;
    const float a = ez / group_sum(ez, G);
    const float sc = live ? a + s_bias[gl] : -INFINITY;
    const float top = group_max(sc, G);
    // lowest index attaining the maximum
    const int rho = group_min((live && sc == top) ? gl : 64, G);
    const float second = group_max((live && gl != rho) ? sc : -INFINITY, G);
    const float margin = (L > 1) ? top - second : INFINITY;
    int chosen = rho;
    if (forced_e && win_ok) {
      const int fe = forced_e[pidx];
      if (fe >= L) {
        if (gl == 0) atomicOr(flags, (uint32_t)LOL_FLAG_BAD_FORCED_ID);
      } else if (fe >= 0) {
        chosen = fe;
      }
    }
    // the chosen expert's probability, from lane (group base + chosen)
    float alpha = __shfl(a, (lane & ~(G - 1)) + (chosen & (G - 1)), 64);
    if (forced_g && win_ok) {
      const float fg = forced_g[pidx];
      if (!isnan(fg)) alpha = fg;
    }
    if (in_range && gl == 0) {
      const int e = win_ok ? chosen : -1;
      win_exp[slot] = e;
      win_gate[slot] = win_ok ? alpha : 0.f;
      s_exp[slot] = e;
      s_len[slot] = win_ok ? win_end(k, W, delta, nb) - win_start(k, W, delta) + 1 : 0;
      win_len[slot] = s_len[slot];
      if (path_e) path_e[pidx] = e;
      if (path_g) path_g[pidx] = win_ok ? alpha : 0.f;
      if (path_m) path_m[pidx] = win_ok ? margin : 0.f;
    }
  }
  __syncthreads();

  // 3. bucketing
  for (int slot = tid; slot < n_slots; slot += blockDim.x) {
    const int e = s_exp[slot];
    if (e >= 0) {
      atomicAdd(&cnt_w[e], 1);
      atomicAdd(&cnt_t[e], s_len[slot]);
    }
  }
  __syncthreads();
  if (tid == 0) {
    int t = 0, f = 0, q = 0, f2 = 0, q2 = 0, w = 0;
    for (int e = 0; e < L; ++e) {
      toff[e] = t;
      fo[e] = f;
      po[e] = q;
      fo2[e] = f2;
      po2[e] = q2;
      t += cnt_t[e];
      f += cnt_t[e] / kTileM;
      q += cnt_t[e] % kTileM != 0;
      f2 += cnt_t[e] / kTileM2;
      q2 += cnt_t[e] % kTileM2 != 0;
      w += cnt_w[e];
    }
    toff[L] = t;
    fo[L] = f;
    po[L] = q;
    fo2[L] = f2;
    po2[L] = q2;
    ecount[L] = w;
    mcount[0] = f + q;
    mcount[1] = f2 + q2;
    mcount[2] = f2;   // full 256-row tiles (the table's first entries)
  }
  __syncthreads();
  for (int e = tid; e <= L; e += blockDim.x) toff_out[e] = toff[e];
  for (int e = tid; e < L; e += blockDim.x) {
    ecount[e] = cnt_w[e];
    if (path_util) path_util[(size_t)depth * L + e] = cnt_w[e];
  }
  // first grouped row of every window: one wave per expert walks the slots in
  // order, 64 at a time, with an exclusive scan of the lengths
  for (int e = wave; e < L; e += 16) {
    int base = toff[e];
    for (int s0 = 0; s0 < n_slots; s0 += 64) {
      const int slot = s0 + lane;
      const bool mine = slot < n_slots && s_exp[slot] == e;
      int v = mine ? s_len[slot] : 0;
      int incl = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      if (mine) win_row0[slot] = base + incl - v;
      base += __shfl(incl, 63, 64);
    }
  }
  for (int slot = tid; slot < n_slots; slot += blockDim.x)
    if (s_exp[slot] < 0) win_row0[slot] = -1;
  // tile i: full tile (i - fo[e]) of expert e, or the partial tile of the
  // (i - F)-th expert that has one
  auto tile_entry = [&](int i, const int *fo_, const int *po_, int H, int &e, int &row0) {
    e = -1;
    row0 = 0;
    const int F = fo_[L];
    if (i < F) {
      e = 0;
      while (fo_[e + 1] <= i) ++e;
      row0 = toff[e] + (i - fo_[e]) * H;
    } else if (i - F < po_[L]) {
      const int j = i - F;
      e = 0;
      while (po_[e + 1] <= j) ++e;
      row0 = toff[e] + (fo_[e + 1] - fo_[e]) * H;
    }
  };
  for (int i = tid; i < max_mtiles; i += blockDim.x) {
    int e, row0;
    tile_entry(i, fo, po, kTileM, e, row0);
    mtile[2 * i] = e;
    mtile[2 * i + 1] = row0;
  }
  for (int i = tid; i < max_mtiles2; i += blockDim.x) {
    int e, row0;
    tile_entry(i, fo2, po2, kTileM2, e, row0);
    mtile2[2 * i] = e;
    mtile2[2 * i + 1] = row0;
  }
}

// Per-call set-up: clears the device flag word and fills the RoPE table
// cos / sin of p * theta^(-2j/d_head) for window-local positions p < W,
// evaluated in double and rounded once.
__global__ void k_setup(uint32_t *__restrict__ flags, float *__restrict__ cs, int W, int half,
                        double theta, int use_rope) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx == 0) flags[0] = 0u;
  if (!use_rope || idx >= W * half) return;
  const int p = idx / half, j = idx % half;
  const double ang = (double)p * pow(theta, -2.0 * (double)j / (double)(2 * half));
  cs[2 * idx] = (float)cos(ang);
  cs[2 * idx + 1] = (float)sin(ang);
}

}  // namespace

hipError_t launch_pool(const Plan &p, const DepthGeom &g, const float *s, const Workspace &ws,
                       const lol_router &rt, hipStream_t st) {
  dim3 grid(p.cfg.batch * g.K, p.cfg.d / 64);
  // untied router: this depth's W_r
  const float *w_r = rt.w_r + (rt.per_depth ? (size_t)g.depth * p.cfg.L * p.cfg.d : 0);
  lol_launch(k_pool, grid, dim3(256), 0, st, s, w_r, rt.e_depth, ws.zpart, ws.zpart0,
                     p.cfg.n, p.cfg.d, p.cfg.L, p.cfg.W, g.delta, g.K, p.K_max, g.depth,
                     p.doc_start, p.doc_len, p.n_tokens);
  return hipGetLastError();
}

hipError_t launch_route(const Plan &p, const DepthGeom &g, const float *s, const Workspace &ws,
                        const lol_router &rt, const int32_t *forced_expert,
                        const float *forced_gate, const lol_path *path, hipStream_t st) {
  (void)s;
  // untied router: this depth's b_r
  const float *b_r = rt.b_r && rt.per_depth ? rt.b_r + (size_t)g.depth * p.cfg.L : rt.b_r;
  lol_launch(k_route_all, dim3(1), dim3(1024), 0, st, ws.zpart, ws.zpart0, b_r,
                     rt.expert_bias, forced_expert, forced_gate, ws.win_exp, ws.win_gate,
                     ws.win_row0, path ? path->expert : nullptr, path ? path->gate : nullptr,
                     path ? path->margin : nullptr, ws.flags, ws.ecount, ws.toff, ws.mtile,
                     ws.max_mtiles, ws.mtile2, ws.max_mtiles2, ws.mcount, ws.zlog, p.cfg.n,
                     p.cfg.d / 64, p.cfg.L, p.cfg.W,
                     g.delta, g.K, p.K_max, p.cfg.batch, g.depth, ws.win_len, p.doc_start,
                     p.doc_len, p.n_tokens, path ? path->util : nullptr);
  return hipGetLastError();
}

hipError_t launch_setup(const Plan &p, const Workspace &ws, hipStream_t st) {
  const int half = p.d_head / 2;
  const int total = p.cfg.W * half;
  lol_launch(k_setup, dim3((total + 255) / 256), dim3(256), 0, st, ws.flags, ws.rope_cs,
                     p.cfg.W, half, (double)p.cfg.rope_theta, p.cfg.rope_theta != 0.f ? 1 : 0);
  return hipGetLastError();
}

int max_slots() { return kMaxSlots; }

}  // namespace lol
