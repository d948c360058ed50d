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

__device__ __forceinline__ int win_start(int k, int W, int delta) { return max(0, k * W - delta); }
__device__ __forceinline__ int win_end(int k, int W, int delta, int n) {
  return min(n - 1, (k + 1) * W - delta - 1);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// a2: mu[slot][c] = mean of s over the window's tokens.  Block = (window,
// 64-column chunk); 16 row phases x 16 float4 columns, fixed-order reduction.
__global__ void __launch_bounds__(256) k_pool(const float *__restrict__ s, float *__restrict__ mu,
                                              int n, int d, int W, int delta, int K, int K_max) {
  const int b = blockIdx.x / K, k = blockIdx.x % K;
  const int start = win_start(k, W, delta), len = win_end(k, W, delta, n) - start + 1;
  const int c4 = threadIdx.x & 15, ph = threadIdx.x >> 4;
  const int col = blockIdx.y * 64 + c4 * 4;
  const float *base = s + ((size_t)b * n + start) * d + col;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int r = ph; r < len; r += 16) {
    const float4 v = *reinterpret_cast<const float4 *>(base + (size_t)r * d);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  __shared__ float4 red[16][16];
  red[ph][c4] = acc;
  __syncthreads();
  if (ph == 0) {
    float4 t = red[0][c4];
    for (int i = 1; i < 16; ++i) {
      t.x += red[i][c4].x; t.y += red[i][c4].y; t.z += red[i][c4].z; t.w += red[i][c4].w;
    }
    const float fl = (float)len;
    t.x /= fl; t.y /= fl; t.z /= fl; t.w /= fl;
    *reinterpret_cast<float4 *>(mu + ((size_t)b * K_max + k) * d + col) = t;
  }
}

// a3 + a4: one block per window slot (b, k).  r_0 = (e_l + s_0)/2, r_k =
// mean of mu_0..mu_{k-1}; z = W_r r + b_r (fp32); a = softmax(z); choice =
// first argmax of a + bias; gate = a_choice; forcing as documented in the
// C ABI.  Slots k >= K get expert -1.
__global__ void __launch_bounds__(256) k_route(
    const float *__restrict__ s, const float *__restrict__ mu, const float *__restrict__ w_r,
    const float *__restrict__ b_r, const float *__restrict__ e_depth, const float *__restrict__ bias,
    const int32_t *__restrict__ forced_e, const float *__restrict__ forced_g,
    int32_t *__restrict__ win_exp, float *__restrict__ win_gate, int32_t *__restrict__ path_e,
    float *__restrict__ path_g, float *__restrict__ path_m, uint32_t *__restrict__ flags, int n,
    int d, int L, int K, int K_max, int B, int depth) {
  extern __shared__ float r[];  // [d]
  __shared__ float z[kMaxExperts];
  const int slot = blockIdx.x, b = slot / K_max, k = slot % K_max;
  const size_t pidx = ((size_t)depth * B + b) * K_max + k;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (k >= K) {
    if (tid == 0) {
      win_exp[slot] = -1;
      win_gate[slot] = 0.f;
      if (path_e) path_e[pidx] = -1;
      if (path_g) path_g[pidx] = 0.f;
      if (path_m) path_m[pidx] = 0.f;
    }
    return;
  }
  for (int c = tid; c < d; c += blockDim.x) {
    float v;
    if (k == 0) {
      v = 0.5f * (e_depth[(size_t)depth * d + c] + s[(size_t)b * n * d + c]);
    } else {
      float acc = 0.f;
      for (int j = 0; j < k; ++j) acc += mu[((size_t)b * K_max + j) * d + c];
      v = acc / (float)k;
    }
    r[c] = v;
  }
  __syncthreads();
  for (int m = wave; m < L; m += 4) {
    float acc = 0.f;
    for (int c = lane; c < d; c += 64) acc += w_r[(size_t)m * d + c] * r[c];
    acc = wave_sum(acc);
    if (lane == 0) z[m] = acc + (b_r ? b_r[m] : 0.f);
  }
  __syncthreads();
  if (wave != 0) return;
  const bool live = lane < L;
  const float zl = live ? z[lane] : -INFINITY;
  const float zmax = wave_max(zl);
  const float ez = live ? expf(zl - zmax) : 0.f;
  const float a = ez / wave_sum(ez);
  const float sc = live ? a + (bias ? bias[lane] : 0.f) : -INFINITY;
  const float top = wave_max(sc);
  // lowest index attaining the maximum
  int cand = (live && sc == top) ? lane : 64;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cand = min(cand, __shfl_xor(cand, o, 64));
  const int rho = cand;
  const float second = wave_max((live && lane != rho) ? sc : -INFINITY);
  const float margin = (L > 1) ? top - second : INFINITY;
  int chosen = rho;
  if (forced_e) {
    const int fe = forced_e[pidx];
    if (fe >= L) {
      if (lane == 0) atomicOr(flags, (uint32_t)LOL_FLAG_BAD_FORCED_ID);
    } else if (fe >= 0) {
      chosen = fe;
    }
  }
  float alpha = __shfl(a, chosen, 64);
  if (forced_g) {
    const float fg = forced_g[pidx];
    if (!isnan(fg)) alpha = fg;
  }
  if (lane == 0) {
    win_exp[slot] = chosen;
    win_gate[slot] = alpha;
    if (path_e) path_e[pidx] = chosen;
    if (path_g) path_g[pidx] = alpha;
    if (path_m) path_m[pidx] = margin;
  }
}

// a5: expert bucketing in one block.  Windows are grouped by expert, in slot
// order inside each expert (stable), so every expert's tokens form one
// contiguous range of grouped rows; the M-tile table lists (expert, first
// row) for every kTileM-row tile of every expert.
__global__ void __launch_bounds__(1024) k_bucket(const int32_t *__restrict__ win_exp,
                                                 int32_t *__restrict__ win_row0,
                                                 int32_t *__restrict__ ecount,
                                                 int32_t *__restrict__ toff_out,
                                                 int32_t *__restrict__ mtile, int max_mtiles,
                                                 int32_t *__restrict__ mtile2, int max_mtiles2,
                                                 int32_t *__restrict__ mcount, int n,
                                                 int W, int delta, int K, int K_max, int n_slots,
                                                 int L) {
  __shared__ int s_exp[kMaxSlots];
  __shared__ int s_len[kMaxSlots];
  __shared__ int cnt_w[kMaxExperts], cnt_t[kMaxExperts];
  __shared__ int toff[kMaxExperts + 1], moff[kMaxExperts + 1], moff2[kMaxExperts + 1];
  const int tid = threadIdx.x;
  for (int i = tid; i < kMaxExperts; i += blockDim.x) { cnt_w[i] = 0; cnt_t[i] = 0; }
  for (int slot = tid; slot < n_slots; slot += blockDim.x) {
    const int k = slot % K_max;
    const int e = win_exp[slot];
    s_exp[slot] = e;
    s_len[slot] = (k < K && e >= 0) ? win_end(k, W, delta, n) - win_start(k, W, delta) + 1 : 0;
  }
  __syncthreads();
  for (int slot = tid; slot < n_slots; slot += blockDim.x) {
    const int e = s_exp[slot];
    if (e >= 0) {
      atomicAdd(&cnt_w[e], 1);
      atomicAdd(&cnt_t[e], s_len[slot]);
    }
  }
  __syncthreads();
  if (tid == 0) {
    int t = 0, m = 0, m2 = 0, w = 0;
    for (int e = 0; e < L; ++e) {
      toff[e] = t;
      moff[e] = m;
      moff2[e] = m2;
      t += cnt_t[e];
      m += (cnt_t[e] + kTileM - 1) / kTileM;
      m2 += (cnt_t[e] + kTileM2 - 1) / kTileM2;
      w += cnt_w[e];
    }
    toff[L] = t;
    moff[L] = m;
    moff2[L] = m2;
    ecount[L] = w;
    mcount[0] = m;
    mcount[1] = m2;
  }
  __syncthreads();
  for (int e = tid; e <= L; e += blockDim.x) toff_out[e] = toff[e];
  for (int e = tid; e < L; e += blockDim.x) ecount[e] = cnt_w[e];
  for (int slot = tid; slot < n_slots; slot += blockDim.x) {
    const int e = s_exp[slot];
    if (e < 0) {
      win_row0[slot] = -1;
      continue;
    }
    int before = 0;
    for (int t = 0; t < slot; ++t) before += (s_exp[t] == e) ? s_len[t] : 0;
    win_row0[slot] = toff[e] + before;
  }
  for (int i = tid; i < max_mtiles; i += blockDim.x) {
    int e = -1, row0 = 0;
    if (i < moff[L]) {
      e = 0;
      while (moff[e + 1] <= i) ++e;
      row0 = toff[e] + (i - moff[e]) * kTileM;
    }
    mtile[2 * i] = e;
    mtile[2 * i + 1] = row0;
  }
  for (int i = tid; i < max_mtiles2; i += blockDim.x) {
    int e = -1, row0 = 0;
    if (i < moff2[L]) {
      e = 0;
      while (moff2[e + 1] <= i) ++e;
      row0 = toff[e] + (i - moff2[e]) * kTileM2;
    }
    mtile2[2 * i] = e;
    mtile2[2 * i + 1] = row0;
  }
}

// Grouped-row metadata: token, window-local position, expert and gate of
// every grouped row.
__global__ void __launch_bounds__(256) k_rowmeta(const int32_t *__restrict__ win_exp,
                                                 const float *__restrict__ win_gate,
                                                 const int32_t *__restrict__ win_row0,
                                                 int32_t *__restrict__ row_tok,
                                                 int32_t *__restrict__ row_pos,
                                                 int32_t *__restrict__ row_exp,
                                                 float *__restrict__ row_gate, int n, int W,
                                                 int delta, int K_max) {
  const int slot = blockIdx.x;
  const int e = win_exp[slot];
  if (e < 0) return;
  const int b = slot / K_max, k = slot % K_max;
  const int start = win_start(k, W, delta), len = win_end(k, W, delta, n) - start + 1;
  const int base = win_row0[slot];
  const float g = win_gate[slot];
  for (int p = threadIdx.x; p < len; p += blockDim.x) {
    const int row = base + p;
    row_tok[row] = b * n + start + p;
    row_pos[row] = p;
    row_exp[row] = e;
    row_gate[row] = g;
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

hipError_t launch_pool(const Plan &p, const DepthGeom &g, const float *s, float *mu, hipStream_t st) {
  dim3 grid(p.cfg.batch * g.K, p.cfg.d / 64);
  hipLaunchKernelGGL(k_pool, grid, dim3(256), 0, st, s, mu, p.cfg.n, p.cfg.d, p.cfg.W, g.delta,
                     g.K, p.K_max);
  return hipGetLastError();
}

hipError_t launch_route(const Plan &p, const DepthGeom &g, const float *s, const Workspace &ws,
                        const lol_router &rt, const int32_t *forced_expert,
                        const float *forced_gate, const lol_path *path, hipStream_t st) {
  const size_t smem = (size_t)p.cfg.d * sizeof(float);
  hipLaunchKernelGGL(k_route, dim3(p.n_slots), dim3(256), smem, st, s, ws.mu, rt.w_r, rt.b_r,
                     rt.e_depth, rt.expert_bias, forced_expert, forced_gate, ws.win_exp,
                     ws.win_gate, path ? path->expert : nullptr, path ? path->gate : nullptr,
                     path ? path->margin : nullptr, ws.flags, p.cfg.n, p.cfg.d, p.cfg.L, g.K,
                     p.K_max, p.cfg.batch, g.depth);
  return hipGetLastError();
}

hipError_t launch_bucket(const Plan &p, const DepthGeom &g, const Workspace &ws, hipStream_t st) {
  hipLaunchKernelGGL(k_bucket, dim3(1), dim3(1024), 0, st, ws.win_exp, ws.win_row0, ws.ecount,
                     ws.toff, ws.mtile, ws.max_mtiles, ws.mtile2, ws.max_mtiles2, ws.mcount, p.cfg.n, p.cfg.W, g.delta, g.K, p.K_max,
                     p.n_slots, p.cfg.L);
  return hipGetLastError();
}

hipError_t launch_rowmeta(const Plan &p, const DepthGeom &g, const Workspace &ws, hipStream_t st) {
  hipLaunchKernelGGL(k_rowmeta, dim3(p.n_slots), dim3(256), 0, st, ws.win_exp, ws.win_gate,
                     ws.win_row0, ws.row_tok, ws.row_pos, ws.row_exp, ws.row_gate, p.cfg.n,
                     p.cfg.W, g.delta, p.K_max);
  return hipGetLastError();
}

hipError_t launch_setup(const Plan &p, const Workspace &ws, hipStream_t st) {
  const int half = p.d_head / 2;
  const int total = p.cfg.W * half;
  hipLaunchKernelGGL(k_setup, dim3((total + 255) / 256), dim3(256), 0, st, ws.flags, ws.rope_cs,
                     p.cfg.W, half, (double)p.cfg.rope_theta, p.cfg.rope_theta != 0.f ? 1 : 0);
  return hipGetLastError();
}

int max_slots() { return kMaxSlots; }

}  // namespace lol
