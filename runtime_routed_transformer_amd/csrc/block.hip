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
// NCH > 0: d = 256 NCH; every lane keeps its NCH float4 chunks of the row in
// registers (read once, 16-byte loads) and stores 4 outputs per chunk.
// NCH = 0: any d (multiple of 64), element-wise.
template <typename act_t>
__device__ __forceinline__ void store4(act_t *p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float *p, float a, float b, float c, float d) {
  *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t *p, float a, float b, float c, float d) {
  uint2 pk;
  pk.x = (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
  pk.y = (uint32_t)f2bf(c) | ((uint32_t)f2bf(d) << 16);
  *reinterpret_cast<uint2 *>(p) = pk;
}

template <typename act_t, bool FROM_S, int NCH>
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
  if (NCH > 0) {
    float4 xv[NCH > 0 ? NCH : 1];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      xv[i] = *reinterpret_cast<const float4 *>(x + i * 256 + lane * 4);
      ss += xv[i].x * xv[i].x + xv[i].y * xv[i].y + xv[i].z * xv[i].z + xv[i].w * xv[i].w;
    }
    const float inv = rsqrtf(wave_sum(ss) / (float)d + eps);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = i * 256 + lane * 4;
      const float4 gv = *reinterpret_cast<const float4 *>(g + c);
      float4 v = make_float4(xv[i].x * inv * gv.x, xv[i].y * inv * gv.y, xv[i].z * inv * gv.z,
                             xv[i].w * inv * gv.w);
      if (fg) {
        const float4 a = *reinterpret_cast<const float4 *>(fg + c);
        const float4 b = *reinterpret_cast<const float4 *>(fb + c);
        v = make_float4(a.x * v.x + b.x, a.y * v.y + b.y, a.z * v.z + b.z, a.w * v.w + b.w);
      }
      store4<act_t>(out + c, v.x, v.y, v.z, v.w);
    }
  } else {
    float ss = 0.f;
    for (int c = lane; c < d; c += 64) ss += x[c] * x[c];
    const float inv = rsqrtf(wave_sum(ss) / (float)d + eps);
    for (int c = lane; c < d; c += 64) {
      float v = x[c] * inv * g[c];
      if (fg) v = fg[c] * v + fb[c];
      st<act_t>(out + c, v);
    }
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

// bf16 window-causal attention on MFMA (v_mfma_f32_32x32x16_bf16).
// Block = (window, head, chunk of 256 queries), 4 waves.  Keys and values
// stream through LDS in chunks of 256 keys (K row-major with RoPE applied,
// V transposed).  Each wave owns query blocks of 32 (wave w takes blocks w
// and 7-w of the chunk, which balances the causal triangle) and computes
// S^T = K Q^T, so every lane holds one query's scores for 16 of 32 keys:
// the online softmax needs one exchange with the lane 32 apart.  Then
// O^T += V^T P^T, with the key order inside each 16-key MFMA step permuted
// to match where the scores already sit in the lane.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

template <int DH>
__global__ void __launch_bounds__(256) k_attn_mfma(const bf16_t *__restrict__ qkv,
                                                   bf16_t *__restrict__ o,
                                                   const int32_t *__restrict__ win_exp,
                                                   const int32_t *__restrict__ win_row0,
                                                   const float *__restrict__ rope_cs, int n, int d,
                                                   int W, int delta, int K_max, float qscale,
                                                   int use_rope) {
  constexpr int CH = 256;           // keys / queries per chunk
  constexpr int LDKR = DH + 8;      // K row stride (elements)
  constexpr int LDV = CH + 4;       // V^T row stride: 2-bank reads hit 32 distinct bank pairs
  constexpr int HALF = DH / 2;
  constexpr int KS = DH / 16;       // MFMA k-steps over the head dimension
  constexpr int DB = DH / 32;       // 32-wide output blocks over the head dimension
  __shared__ __attribute__((aligned(16))) bf16_t Ks[CH * LDKR];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[DH * LDV];
  const int slot = blockIdx.x, h = blockIdx.y, qc = blockIdx.z;
  if (win_exp[slot] < 0) return;
  const int k = slot % K_max;
  const int start = max(0, k * W - delta);
  const int len = min(n - 1, (k + 1) * W - delta - 1) - start + 1;
  const int q_begin = qc * CH;
  if (q_begin >= len) return;
  const int base = win_row0[slot];
  const size_t ld3 = (size_t)3 * d;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hl = lane >> 5, col = lane & 31;

  // ---- this wave's two query blocks: Q fragments (RoPE, scale) in registers
  int qblk[2] = {wave, 7 - wave};
  bf16x8_t qf[2][KS];
  float m_run[2], l_run[2];
  f32x16_t acc[2][DB];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int qpos = q_begin + qblk[b] * 32 + col;         // window-local query position
    const int qrow = min(qpos, len - 1);
    const bf16_t *qp = qkv + (size_t)(base + qrow) * ld3 + h * DH;
    float x[KS][8];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 raw = *reinterpret_cast<const uint4 *>(qp + ks * 16 + hl * 8);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[ks][2 * j] = __uint_as_float(w[j] << 16);
        x[ks][2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    }
    if (use_rope) {
      const float *cs = rope_cs + (size_t)qrow * HALF * 2;
#pragma unroll
      for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int dd = ks * 16 + hl * 8 + j;                // < HALF; partner dd + HALF
          const float c0 = cs[2 * dd], s0 = cs[2 * dd + 1];
          const float x1 = x[ks][j], x2 = x[ks + KS / 2][j];
          x[ks][j] = x1 * c0 - x2 * s0;
          x[ks + KS / 2][j] = x1 * s0 + x2 * c0;
        }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[b][ks][j] = (__bf16)(x[ks][j] * qscale);
    m_run[b] = -INFINITY;
    l_run[b] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][db][i] = 0.f;
  }

  for (int kc = 0; kc <= qc; ++kc) {
    const int k_begin = kc * CH;
    __syncthreads();
    // ---- stage K (RoPE) row-major and V transposed; zero rows past the window
    {
      const int kpos = k_begin + tid;
      float x[DH];
      if (kpos < len) {
        const bf16_t *kp = qkv + (size_t)(base + kpos) * ld3 + d + h * DH;
#pragma unroll
        for (int c = 0; c < DH; c += 8) {
          const uint4 raw = *reinterpret_cast<const uint4 *>(kp + c);
          const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x[c + 2 * j] = __uint_as_float(w[j] << 16);
            x[c + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
          }
        }
        if (use_rope) {
          const float *cs = rope_cs + (size_t)kpos * HALF * 2;
#pragma unroll
          for (int j = 0; j < HALF; ++j) {
            const float c0 = cs[2 * j], s0 = cs[2 * j + 1];
            const float x1 = x[j], x2 = x[j + HALF];
            x[j] = x1 * c0 - x2 * s0;
            x[j + HALF] = x1 * s0 + x2 * c0;
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < DH; ++c) x[c] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < DH; c += 8) {
        uint4 pk;
        pk.x = (uint32_t)f2bf(x[c]) | ((uint32_t)f2bf(x[c + 1]) << 16);
        pk.y = (uint32_t)f2bf(x[c + 2]) | ((uint32_t)f2bf(x[c + 3]) << 16);
        pk.z = (uint32_t)f2bf(x[c + 4]) | ((uint32_t)f2bf(x[c + 5]) << 16);
        pk.w = (uint32_t)f2bf(x[c + 6]) | ((uint32_t)f2bf(x[c + 7]) << 16);
        *reinterpret_cast<uint4 *>(&Ks[tid * LDKR + c]) = pk;
      }
      // V^T: thread = (key pair, half of the head dims); packed 32-bit writes
      const int pr = tid & 127, dh0 = (tid >> 7) * HALF;
      const int k0 = k_begin + 2 * pr;
      const bf16_t *v0 = qkv + (size_t)(base + min(k0, len - 1)) * ld3 + 2 * d + h * DH + dh0;
      const bf16_t *v1 = qkv + (size_t)(base + min(k0 + 1, len - 1)) * ld3 + 2 * d + h * DH + dh0;
      const bool ok0 = k0 < len, ok1 = k0 + 1 < len;
#pragma unroll
      for (int c = 0; c < HALF; c += 8) {
        const uint4 a = *reinterpret_cast<const uint4 *>(v0 + c);
        const uint4 b = *reinterpret_cast<const uint4 *>(v1 + c);
        const uint32_t wa[4] = {ok0 ? a.x : 0u, ok0 ? a.y : 0u, ok0 ? a.z : 0u, ok0 ? a.w : 0u};
        const uint32_t wb[4] = {ok1 ? b.x : 0u, ok1 ? b.y : 0u, ok1 ? b.z : 0u, ok1 ? b.w : 0u};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo = (wa[j] & 0xFFFFu) | (wb[j] << 16);          // dim c+2j
          const uint32_t hi = (wa[j] >> 16) | (wb[j] & 0xFFFF0000u);      // dim c+2j+1
          *reinterpret_cast<uint32_t *>(&Vt[(dh0 + c + 2 * j) * LDV + 2 * pr]) = lo;
          *reinterpret_cast<uint32_t *>(&Vt[(dh0 + c + 2 * j + 1) * LDV + 2 * pr]) = hi;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int q_lo = q_begin + qblk[b] * 32;            // first query of the block
      if (q_lo >= len) continue;
      const int q = q_lo + col;
      // key blocks of this chunk that the query block can see
      const int kb_end = (kc < qc) ? CH / 32 : qblk[b] + 1;
      for (int kb = 0; kb < kb_end; ++kb) {
        f32x16_t sc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8_t kf =
              *reinterpret_cast<const bf16x8_t *>(&Ks[(kb * 32 + col) * LDKR + ks * 16 + hl * 8]);
          sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[b][ks], sc, 0, 0, 0);
        }
        // sc[i] = score(key = k_begin + kb*32 + (i/4)*8 + 4*hl + i%4, query q), log2 units
        if (kc == qc && kb == qblk[b]) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k_begin + kb * 32 + (i >> 2) * 8 + 4 * hl + (i & 3);
            if (key > q) sc[i] = -INFINITY;
          }
        }
        float mx = sc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run[b], mx);
        const float corr = exp2f(m_run[b] - m_new);
        float p[16], rs = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p[i] = exp2f(sc[i] - m_new);
          rs += p[i];
        }
        rs += __shfl_xor(rs, 32, 64);
        l_run[b] = l_run[b] * corr + rs;
        m_run[b] = m_new;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[b][db][i] *= corr;
#pragma unroll
        for (int step = 0; step < 2; ++step) {
          bf16x8_t pb;
#pragma unroll
          for (int j = 0; j < 8; ++j) pb[j] = (__bf16)p[8 * step + j];
          const int key0 = kb * 32 + 16 * step + 4 * hl;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16_t *vr = &Vt[(db * 32 + col) * LDV + key0];
            const uint2 lo = *reinterpret_cast<const uint2 *>(vr);
            const uint2 hi = *reinterpret_cast<const uint2 *>(vr + 8);
            bf16x8_t va;
            const uint32_t w[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              va[2 * j] = __builtin_bit_cast(__bf16, (bf16_t)(w[j] & 0xFFFFu));
              va[2 * j + 1] = __builtin_bit_cast(__bf16, (bf16_t)(w[j] >> 16));
            }
            acc[b][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, acc[b][db], 0, 0, 0);
          }
        }
      }
    }
  }
  // ---- O[q][d] = acc / l ; lane holds d = db*32 + (i/4)*8 + 4*hl + i%4 of query col
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int q = q_begin + qblk[b] * 32 + col;
    if (q >= len) continue;
    const float il = 1.0f / l_run[b];
    bf16_t *op = o + (size_t)(base + q) * d + h * DH;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 pk;
        pk.x = (uint32_t)f2bf(acc[b][db][4 * g] * il) | ((uint32_t)f2bf(acc[b][db][4 * g + 1] * il) << 16);
        pk.y = (uint32_t)f2bf(acc[b][db][4 * g + 2] * il) | ((uint32_t)f2bf(acc[b][db][4 * g + 3] * il) << 16);
        *reinterpret_cast<uint2 *>(op + db * 32 + g * 8 + 4 * hl) = pk;
      }
  }
}

template <typename act_t, int NCH>
void norm_launch(const Plan &p, int which, const float *s, const lol_library &lib,
                 const Workspace &ws, const float *fg, const float *fb, hipStream_t st) {
  dim3 grid((p.T + 3) / 4);
  if (which == 0)
    hipLaunchKernelGGL((k_norm<act_t, true, NCH>), grid, dim3(256), 0, st, s, ws.row_tok,
                       ws.row_exp, lib.g_attn, fg, fb, reinterpret_cast<act_t *>(ws.u), p.T,
                       p.cfg.d, p.cfg.rms_eps);
  else
    hipLaunchKernelGGL((k_norm<act_t, false, NCH>), grid, dim3(256), 0, st, ws.h, ws.row_tok,
                       ws.row_exp, lib.g_ffn, fg, fb, reinterpret_cast<act_t *>(ws.u), p.T,
                       p.cfg.d, p.cfg.rms_eps);
}

template <typename act_t>
hipError_t norm_typed(const Plan &p, int which, const float *s, const lol_library &lib,
                      const Workspace &ws, int depth, hipStream_t st) {
  const int d = p.cfg.d;
  const float *fg = lib.film_gamma ? lib.film_gamma + ((size_t)depth * 2 + which) * d : nullptr;
  const float *fb = lib.film_beta ? lib.film_beta + ((size_t)depth * 2 + which) * d : nullptr;
  switch ((d % 256 == 0) ? d / 256 : 0) {
    case 1: norm_launch<act_t, 1>(p, which, s, lib, ws, fg, fb, st); break;
    case 2: norm_launch<act_t, 2>(p, which, s, lib, ws, fg, fb, st); break;
    case 3: norm_launch<act_t, 3>(p, which, s, lib, ws, fg, fb, st); break;
    case 4: norm_launch<act_t, 4>(p, which, s, lib, ws, fg, fb, st); break;
    case 5: norm_launch<act_t, 5>(p, which, s, lib, ws, fg, fb, st); break;
    case 6: norm_launch<act_t, 6>(p, which, s, lib, ws, fg, fb, st); break;
    case 7: norm_launch<act_t, 7>(p, which, s, lib, ws, fg, fb, st); break;
    case 8: norm_launch<act_t, 8>(p, which, s, lib, ws, fg, fb, st); break;
    default: norm_launch<act_t, 0>(p, which, s, lib, ws, fg, fb, st); break;
  }
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

template <int DH>
hipError_t attn_mfma(const Plan &p, const DepthGeom &g, const Workspace &ws, hipStream_t st) {
  dim3 grid(p.n_slots, p.cfg.n_heads, (p.cfg.W + 255) / 256);
  // scores come out in log2 units: softmax uses exp2
  const float qscale = 1.4426950408889634f / sqrtf((float)DH);
  hipLaunchKernelGGL((k_attn_mfma<DH>), grid, dim3(256), 0, st,
                     reinterpret_cast<const bf16_t *>(ws.qkv), reinterpret_cast<bf16_t *>(ws.o),
                     ws.win_exp, ws.win_row0, ws.rope_cs, p.cfg.n, p.cfg.d, p.cfg.W, g.delta,
                     p.K_max, qscale, p.cfg.rope_theta != 0.f ? 1 : 0);
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
    return p.d_head == 64 ? attn_mfma<64>(p, g, ws, st) : attn_mfma<32>(p, g, ws, st);
  return p.d_head == 64 ? attn_typed<float, 64>(p, g, ws, st) : attn_typed<float, 32>(p, g, ws, st);
}

}  // namespace lol
