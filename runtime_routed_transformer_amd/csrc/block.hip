// Row-wise and attention kernels of a library block.
//
// Norms: paper "Library of Layers (LoL)", App. A (RMSNorm, and the depth
// FiLM gamma_s * Norm_s(x) + beta_s that replaces each norm); review "Library
// of Layers: Routing Whole Transformer Blocks at Runtime", Eq. 7.
// Attention: paper Sec. 3.2.1 (causal attention restricted to the window),
// review Eq. 1 (scores scaled by 1/sqrt(d_head)), App. A (RoPE, bias-free).
#include <math.h>

#include "lol_internal.h"

namespace lol {
namespace {

__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}
__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <typename T> __device__ __forceinline__ float ld(const T *p);
template <> __device__ __forceinline__ float ld<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float ld<bf16_t>(const bf16_t *p) { return bf2f(*p); }
template <typename T> __device__ __forceinline__ void st(T *p, float v);
template <> __device__ __forceinline__ void st<float>(float *p, float v) { *p = v; }
template <> __device__ __forceinline__ void st<bf16_t>(bf16_t *p, float v) { *p = f2bf(v); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// u[row] = gamma * (g_e * x / sqrt(mean(x^2) + eps)) + beta, one wave per row.
// FROM_S: x = s[row_tok[row]] (attention sublayer); else x = h[row] (MLP).
template <typename act_t, bool FROM_S>
__global__ void __launch_bounds__(256) k_norm(const float *__restrict__ src,
                                              const int32_t *__restrict__ row_tok,
                                              const int32_t *__restrict__ row_exp,
                                              const float *__restrict__ gain,
                                              const float *__restrict__ fg,
                                              const float *__restrict__ fb, act_t *__restrict__ u,
                                              int T, int d, float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= T) return;
  const float *x = src + (FROM_S ? (size_t)row_tok[row] : (size_t)row) * d;
  const float *g = gain + (size_t)row_exp[row] * d;
  act_t *out = u + (size_t)row * d;
  float ss = 0.f;
  if ((d & 255) == 0) {
    for (int c = lane * 4; c < d; c += 256) {
      const float4 v = *reinterpret_cast<const float4 *>(x + c);
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
  } else {
    for (int c = lane; c < d; c += 64) ss += x[c] * x[c];
  }
  const float inv = rsqrtf(wave_sum(ss) / (float)d + eps);
  for (int c = lane; c < d; c += 64) {
    float v = x[c] * inv * g[c];
    if (fg) v = fg[c] * v + fb[c];
    st<act_t>(out + c, v);
  }
}

// Window-causal attention, one wave per (window, head, 64 queries); each
// lane owns one query.  Keys and values of the window are staged through LDS
// 64 rows at a time with RoPE applied on the way in (window-local positions);
// online softmax in fp32.
template <typename act_t, int DH>
__global__ void __launch_bounds__(64) k_attn_simt(const act_t *__restrict__ qkv,
                                                  act_t *__restrict__ o,
                                                  const int32_t *__restrict__ win_exp,
                                                  const int32_t *__restrict__ win_row0,
                                                  const float *__restrict__ rope_cs, int n, int d,
                                                  int W, int delta, int K_max, float scale,
                                                  int use_rope) {
  constexpr int HALF = DH / 2;
  __shared__ float ks[64][DH + 1];
  __shared__ float vs[64][DH + 1];
  const int slot = blockIdx.x, h = blockIdx.y, q0 = blockIdx.z * 64;
  if (win_exp[slot] < 0) return;
  const int k = slot % K_max;
  const int start = max(0, k * W - delta);
  const int len = min(n - 1, (k + 1) * W - delta - 1) - start + 1;
  if (q0 >= len) return;
  const int base = win_row0[slot];
  const int lane = threadIdx.x;
  const int i = q0 + lane;
  const bool valid = i < len;
  const size_t ld3 = (size_t)3 * d;
  float q[DH];
  {
    const act_t *qp = qkv + (size_t)(base + (valid ? i : 0)) * ld3 + h * DH;
#pragma unroll
    for (int c = 0; c < DH; ++c) q[c] = ld<act_t>(qp + c);
    if (use_rope) {
      const float *cs = rope_cs + (size_t)(valid ? i : 0) * HALF * 2;
#pragma unroll
      for (int j = 0; j < HALF; ++j) {
        const float c0 = cs[2 * j], s0 = cs[2 * j + 1];
        const float x1 = q[j], x2 = q[j + HALF];
        q[j] = x1 * c0 - x2 * s0;
        q[j + HALF] = x1 * s0 + x2 * c0;
      }
    }
#pragma unroll
    for (int c = 0; c < DH; ++c) q[c] *= scale;
  }
  float m = -INFINITY, l = 0.f, acc[DH];
#pragma unroll
  for (int c = 0; c < DH; ++c) acc[c] = 0.f;
  const int kend = min(len, q0 + 64);
  for (int j0 = 0; j0 < kend; j0 += 64) {
    __syncthreads();
    const int j = j0 + lane;
    if (j < kend) {
      const act_t *kp = qkv + (size_t)(base + j) * ld3 + d + h * DH;
      const act_t *vp = kp + d;
      float kr[DH];
#pragma unroll
      for (int c = 0; c < DH; ++c) kr[c] = ld<act_t>(kp + c);
      if (use_rope) {
        const float *cs = rope_cs + (size_t)j * HALF * 2;
#pragma unroll
        for (int t = 0; t < HALF; ++t) {
          const float c0 = cs[2 * t], s0 = cs[2 * t + 1];
          const float x1 = kr[t], x2 = kr[t + HALF];
          kr[t] = x1 * c0 - x2 * s0;
          kr[t + HALF] = x1 * s0 + x2 * c0;
        }
      }
#pragma unroll
      for (int c = 0; c < DH; ++c) { ks[lane][c] = kr[c]; vs[lane][c] = ld<act_t>(vp + c); }
    }
    __syncthreads();
    const int jn = min(64, kend - j0);
    for (int jj = 0; jj < jn; ++jj) {
      if (j0 + jj > i) break;
      float sc = 0.f;
#pragma unroll
      for (int c = 0; c < DH; ++c) sc = fmaf(q[c], ks[jj][c], sc);
      const float mn = fmaxf(m, sc);
      const float corr = expf(m - mn), pj = expf(sc - mn);
      l = l * corr + pj;
#pragma unroll
      for (int c = 0; c < DH; ++c) acc[c] = acc[c] * corr + pj * vs[jj][c];
      m = mn;
    }
  }
  if (!valid) return;
  act_t *op = o + (size_t)(base + i) * d + h * DH;
  const float il = 1.0f / l;
#pragma unroll
  for (int c = 0; c < DH; ++c) st<act_t>(op + c, acc[c] * il);
}

template <typename act_t>
hipError_t norm_typed(const Plan &p, int which, const float *s, const lol_library &lib,
                      const Workspace &ws, int depth, hipStream_t st) {
  const int d = p.cfg.d;
  const float *fg = lib.film_gamma ? lib.film_gamma + ((size_t)depth * 2 + which) * d : nullptr;
  const float *fb = lib.film_beta ? lib.film_beta + ((size_t)depth * 2 + which) * d : nullptr;
  dim3 grid((p.T + 3) / 4);
  if (which == 0)
    hipLaunchKernelGGL((k_norm<act_t, true>), grid, dim3(256), 0, st, s, ws.row_tok, ws.row_exp,
                       lib.g_attn, fg, fb, reinterpret_cast<act_t *>(ws.u), p.T, d,
                       p.cfg.rms_eps);
  else
    hipLaunchKernelGGL((k_norm<act_t, false>), grid, dim3(256), 0, st, ws.h, ws.row_tok,
                       ws.row_exp, lib.g_ffn, fg, fb, reinterpret_cast<act_t *>(ws.u), p.T, d,
                       p.cfg.rms_eps);
  return hipGetLastError();
}

template <typename act_t, int DH>
hipError_t attn_typed(const Plan &p, const DepthGeom &g, const Workspace &ws, hipStream_t st) {
  dim3 grid(p.n_slots, p.cfg.n_heads, (p.cfg.W + 63) / 64);
  const float scale = 1.0f / sqrtf((float)DH);
  hipLaunchKernelGGL((k_attn_simt<act_t, DH>), grid, dim3(64), 0, st,
                     reinterpret_cast<const act_t *>(ws.qkv), reinterpret_cast<act_t *>(ws.o),
                     ws.win_exp, ws.win_row0, ws.rope_cs, p.cfg.n, p.cfg.d, p.cfg.W, g.delta,
                     p.K_max, scale, p.cfg.rope_theta != 0.f ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_norm(const Plan &p, const DepthGeom &g, int which, const float *s,
                       const lol_library &lib, const Workspace &ws, hipStream_t st) {
  if (p.cfg.dtype == LOL_BF16) return norm_typed<bf16_t>(p, which, s, lib, ws, g.depth, st);
  return norm_typed<float>(p, which, s, lib, ws, g.depth, st);
}

hipError_t launch_attention(const Plan &p, const DepthGeom &g, const Workspace &ws, hipStream_t st) {
  if (p.cfg.dtype == LOL_BF16)
    return p.d_head == 64 ? attn_typed<bf16_t, 64>(p, g, ws, st) : attn_typed<bf16_t, 32>(p, g, ws, st);
  return p.d_head == 64 ? attn_typed<float, 64>(p, g, ws, st) : attn_typed<float, 32>(p, g, ws, st);
}

}  // namespace lol
