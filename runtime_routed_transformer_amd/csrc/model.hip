// Around the routed core: the token embedding and the vocabulary readout
// (paper "Library of Layers (LoL)", Appendix A, Algorithm 1: the prelude
// reads the token sequence; the coda ends in the vocabulary readout).  The
// prelude and coda themselves are fixed-order stacks of ordinary blocks
// (paper Sec. 3.1) and run through lol_core_forward with one window per
// document and a forced path (see lol_core.h).
#include <math.h>

#include "lol_internal.h"

namespace lol {
namespace {

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// s[t][c .. c+3] = table[tokens[t]][c .. c+3]; one thread per 4 columns
template <typename W>
__global__ void __launch_bounds__(256) k_embed(const int32_t *__restrict__ tokens, const W *__restrict__ table,
                                               int V, int d, float *__restrict__ s, long long quads) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= quads) return;
  const int q4 = d / 4;
  const long long t = i / q4;
  const int c = (int)(i % q4) * 4;
  const int tok = tokens[t];
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (tok >= 0 && tok < V) {
    const W *row = table + (size_t)tok * d + c;
    if (sizeof(W) == 2) {
      const uint2 raw = *reinterpret_cast<const uint2 *>(row);
      v = make_float4(bf16_to_f32((bf16_t)(raw.x & 0xFFFFu)), bf16_to_f32((bf16_t)(raw.x >> 16)),
                      bf16_to_f32((bf16_t)(raw.y & 0xFFFFu)), bf16_to_f32((bf16_t)(raw.y >> 16)));
    } else {
      v = *reinterpret_cast<const float4 *>(row);
    }
  }
  *reinterpret_cast<float4 *>(s + (size_t)t * d + c) = v;
}

// u[t] = g * s[t] / sqrt(mean(s[t]^2) + eps), one wave per row.  bf16: u in
// 32-column panels [d/32][T][32] (the A layout the GEMM loads whole lines
// from); fp32: u row-major.
template <typename act_t>
__global__ void __launch_bounds__(256) k_head_norm(const float *__restrict__ s, const float *__restrict__ g,
                                                   act_t *__restrict__ u, int T, int d, float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= T) return;
  const float *x = s + (size_t)row * d;
  float ss = 0.f;
  for (int c = lane * 4; c < d; c += 256) {
    const float4 v = *reinterpret_cast<const float4 *>(x + c);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  const float inv = rsqrtf(ss / (float)d + eps);
  for (int c = lane * 4; c < d; c += 256) {
    const float4 v = *reinterpret_cast<const float4 *>(x + c);
    const float4 gv = *reinterpret_cast<const float4 *>(g + c);
    const float a = v.x * inv * gv.x, b = v.y * inv * gv.y, e = v.z * inv * gv.z, f = v.w * inv * gv.w;
    if (sizeof(act_t) == 2) {
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
      pk.y = (uint32_t)f32_to_bf16(e) | ((uint32_t)f32_to_bf16(f) << 16);
      *reinterpret_cast<uint2 *>(reinterpret_cast<bf16_t *>(u) + ((size_t)(c >> 5) * T + row) * 32 + (c & 31)) = pk;
    } else {
      *reinterpret_cast<float4 *>(reinterpret_cast<float *>(u) + (size_t)row * d + c) = make_float4(a, b, e, f);
    }
  }
}

// Tile tables of one "expert" holding all T rows: 128- and 256-row tiles.
__global__ void k_dense_tiles(int32_t *__restrict__ mtile, int max1, int32_t *__restrict__ mtile2, int max2,
                              int32_t *__restrict__ mcount, int32_t *__restrict__ toff, int T) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < max1) {
    mtile[2 * i] = i * kTileM < T ? 0 : -1;
    mtile[2 * i + 1] = i * kTileM;
  }
  if (i < max2) {
    mtile2[2 * i] = i * kTileM2 < T ? 0 : -1;
    mtile2[2 * i + 1] = i * kTileM2;
  }
  if (i == 0) {
    mcount[0] = (T + kTileM - 1) / kTileM;
    mcount[1] = (T + kTileM2 - 1) / kTileM2;
    mcount[2] = T / kTileM2;   // full 256-row tiles
    toff[0] = 0;
    toff[1] = T;
  }
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// workspace of the readout: u, then the two tile tables, counts and offsets
size_t head_layout(int T, int d, int dtype, char *base, Workspace *ws) {
  const size_t ab = dtype == LOL_BF16 ? 2 : 4;
  const int max1 = (T + kTileM - 1) / kTileM + 1, max2 = (T + kTileM2 - 1) / kTileM2 + 1;
  size_t off = 0;
  auto carve = [&](size_t bytes) -> char * {
    char *p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  Workspace w{};
  w.u = carve((size_t)T * d * ab);
  w.mtile = (int32_t *)carve((size_t)max1 * 8);
  w.mtile2 = (int32_t *)carve((size_t)max2 * 8);
  w.mcount = (int32_t *)carve(12);
  w.toff = (int32_t *)carve(8);
  w.max_mtiles = max1;
  w.max_mtiles2 = max2;
  if (ws) *ws = w;
  return off;
}

bool head_sizes_ok(int T, int d, int V, int dtype) {
  if (T < 1 || d < 1 || V < 1) return false;
  if (dtype == LOL_BF16) return d % 128 == 0 && V % 128 == 0;
  if (dtype == LOL_FP32) return d % 64 == 0 && V % 64 == 0;
  return false;
}

}  // namespace
}  // namespace lol

using namespace lol;

extern "C" {

lol_status lol_embed(const int32_t *tokens, int32_t T, const void *table, int32_t V, int32_t d,
                     int32_t dtype, float *s, void *stream) {
  if (!tokens || !table || !s || T < 1 || V < 1 || d < 4 || d % 4 != 0) return LOL_EINVAL;
  if (dtype != LOL_BF16 && dtype != LOL_FP32) return LOL_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const long long quads = (long long)T * (d / 4);
  const dim3 grid((unsigned)((quads + 255) / 256));
  if (dtype == LOL_BF16)
    lol_launch(k_embed<bf16_t>, grid, dim3(256), 0, st, tokens, static_cast<const bf16_t *>(table), V, d, s, quads);
  else
    lol_launch(k_embed<float>, grid, dim3(256), 0, st, tokens, static_cast<const float *>(table), V, d, s, quads);
  return hipGetLastError() == hipSuccess ? LOL_OK : LOL_EHIP;
}

size_t lol_lm_head_workspace_size(int32_t T, int32_t d, int32_t V, int32_t dtype) {
  if (!head_sizes_ok(T, d, V, dtype)) return 0;
  return head_layout(T, d, dtype, nullptr, nullptr);
}

lol_status lol_lm_head(const float *s, int32_t T, int32_t d, const float *g_final, float eps,
                       const void *w_vocab, int32_t V, int32_t dtype, float *logits,
                       void *workspace, size_t workspace_bytes, void *stream) {
  if (!s || !g_final || !w_vocab || !logits || !(eps > 0.f)) return LOL_EINVAL;
  if (!head_sizes_ok(T, d, V, dtype)) return LOL_EINVAL;
  const size_t need = head_layout(T, d, dtype, nullptr, nullptr);
  if (!workspace || workspace_bytes < need) return LOL_EWORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return LOL_EINVAL;
  Workspace ws;
  head_layout(T, d, dtype, static_cast<char *>(workspace), &ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == LOL_BF16;
  const int mx = ws.max_mtiles > ws.max_mtiles2 ? ws.max_mtiles : ws.max_mtiles2;
  lol_launch(k_dense_tiles, dim3((mx + 255) / 256), dim3(256), 0, st, ws.mtile, ws.max_mtiles, ws.mtile2,
             ws.max_mtiles2, ws.mcount, ws.toff, T);
  if (bf16)
    lol_launch(k_head_norm<bf16_t>, dim3((T + 3) / 4), dim3(256), 0, st, s, g_final,
               reinterpret_cast<bf16_t *>(ws.u), T, d, eps);
  else
    lol_launch(k_head_norm<float>, dim3((T + 3) / 4), dim3(256), 0, st, s, g_final,
               reinterpret_cast<float *>(ws.u), T, d, eps);
  if (hipGetLastError() != hipSuccess) return LOL_EHIP;
  // the logits GEMM: one expert of T rows, W_vocab [V][d]
  Plan p{};
  p.cfg.dtype = dtype;
  p.cfg.L = 1;
  p.cfg.d = d;
  p.T = T;
  p.d_head = 64;
  p.act_bytes = bf16 ? 2 : 4;
  GemmArgs a{};
  a.A = ws.u;
  a.Wt = w_vocab;
  a.N = V;
  a.K = d;
  a.w_expert_stride = (long long)V * d;
  a.epi = bf16 ? EPI_STORE_F32 : EPI_STORE;
  a.C = logits;
  a.len_gcd = T;
  a.a_panel_rows = bf16 ? T : 0;
  return launch_gemm(p, ws, a, st) == hipSuccess ? LOL_OK : LOL_EHIP;
}

}  // extern "C"
