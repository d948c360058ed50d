// Incremental decode of the routed core: one new token per document per
// call, carried through every routed depth.
//
// Review "Library of Layers: Routing Whole Transformer Blocks at Runtime",
// "Deriving prefix-only routing": a window's router input depends only on
// earlier, completed windows (window 0: the document's first token and the
// depth vector), so its route and gate are fixed when its first token
// arrives, and serving keeps per-depth window boundaries and summaries.
// Blog "Library of Layers: a transformer that picks its own layer order",
// "What it costs": attention stays inside a window, so a depth only needs
// the open window's keys and values.
//
// The state holds each document's next position and, per depth and
// document, the sum of the completed windows' means, the running sum and
// length of the open window, its expert and gate, and its keys and values.
// One call runs, per depth:
//   k_dec_route   positions (depth 0), close/open windows, route a window
//                 that opens, attention RMSNorm + FiLM (one block per document)
//   k_dec_gemv    QKV projection (grouped by expert)
//   k_dec_attn    RoPE, cache append, attention over the open window
//   k_dec_gemv    output projection + residual
//   k_dec_norm    MLP RMSNorm + FiLM
//   k_dec_gemv    gate/up + SwiGLU (or GELU)
//   k_dec_gemv    down projection + gated blend
// A token's rows are few (one per document), so the projections are
// matrix-vector products bound by reading the weights once: every wave
// streams one weight row (one gate/up pair) of one expert with 16-byte
// loads, and all rows (documents) routed to that expert share the read.
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

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t v) { return bf2f(v); }
template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { return f2bf(v); }

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
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum over the 256 threads of a block (red: 4 floats of LDS).
__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d) {
  *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store4(bf16_t *p, float a, float b, float c, float d) {
  uint2 pk;
  pk.x = (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
  pk.y = (uint32_t)f2bf(c) | ((uint32_t)f2bf(d) << 16);
  *reinterpret_cast<uint2 *>(p) = pk;
}

// out = FiLM(g * x / sqrt(mean(x^2) + eps)) over one row of d <= 4096, by a
// block of 256 threads (paper App. A RMSNorm with the depth FiLM of the
// review's Eq. 7).  Every load of the row, the gain and FiLM is issued
// before the reduction, so the row costs one memory round trip.
template <typename act_t>
__device__ __forceinline__ void norm_row(const float *__restrict__ x, int d,
                                         const float *__restrict__ g,
                                         const float *__restrict__ fg,
                                         const float *__restrict__ fb, float eps,
                                         act_t *__restrict__ out, float *red) {
  float4 xv[4], gv[4], av[4], bv[4];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = (i * 256 + (int)threadIdx.x) * 4;
    if (c < d) {
      xv[i] = *reinterpret_cast<const float4 *>(x + c);
      gv[i] = *reinterpret_cast<const float4 *>(g + c);
      if (fg) {
        av[i] = *reinterpret_cast<const float4 *>(fg + c);
        bv[i] = *reinterpret_cast<const float4 *>(fb + c);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if ((i * 256 + (int)threadIdx.x) * 4 < d)
      ss += xv[i].x * xv[i].x + xv[i].y * xv[i].y + xv[i].z * xv[i].z + xv[i].w * xv[i].w;
  const float inv = rsqrtf(block_sum(ss, red) / (float)d + eps);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = (i * 256 + (int)threadIdx.x) * 4;
    if (c >= d) continue;
    float4 v = make_float4(xv[i].x * inv * gv[i].x, xv[i].y * inv * gv[i].y,
                           xv[i].z * inv * gv[i].z, xv[i].w * inv * gv[i].w);
    if (fg)
      v = make_float4(av[i].x * v.x + bv[i].x, av[i].y * v.y + bv[i].y, av[i].z * v.z + bv[i].z,
                      av[i].w * v.w + bv[i].w);
    store4(out + c, v.x, v.y, v.z, v.w);
  }
}

// Resets rows [row0, row1) of the state: next position 0, window routes to
// expert 0 (and, with flags, the flag word and the RoPE table).
__global__ void k_dec_reset(int32_t *__restrict__ hdr, int32_t *__restrict__ row_next,
                            int32_t *__restrict__ cur_len, int32_t *__restrict__ expert,
                            float *__restrict__ gate, int B, int D, int row0, int row1, int all,
                            float *__restrict__ cs, int W, int half, double theta, int use_rope) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (all && idx == 0) hdr[1] = 0;
  const int nr = row1 - row0;
  if (idx < nr) row_next[row0 + idx] = 0;
  if (idx < D * nr) {
    const int l = idx / nr, b = row0 + idx % nr;
    cur_len[l * B + b] = 0;
    expert[l * B + b] = 0;
    gate[l * B + b] = 0.f;
  }
  if (all && use_rope && idx < W * half) {
    // cos / sin of p * theta^(-2j/d_head) at window-local position p
    const int p = idx / half, j = idx % half;
    const double ang = (double)p * pow(theta, -2.0 * (double)j / (double)(2 * half));
    cs[2 * idx] = (float)cos(ang);
    cs[2 * idx + 1] = (float)sin(ang);
  }
}

// One block per document.  At depth 0 the block takes the document's
// position for this call (`pos` >= 0: every document's, checked against the
// state; -1: the document's own next position) and advances it; every depth
// then reads it back.  At position pos of depth index `depth` (window
// offset delta) the token lies in window k = (pos + delta) / W:
//  - if the token opens window k, window k-1 is closed (its mean joins the
//    prefix sum), the router input is built (the depth vector and the token
//    for k = 0, else the mean of the k completed windows' means), the fp32
//    router scores it (softmax, lowest index attaining max(a + bias), gate =
//    a of the applied expert, margin top1 - top2, forcing), and the open
//    window's running sum restarts at the token;
//  - else the token joins the open window's running sum.
// Then u = FiLM_attn(RMSNorm_e(token)) for the window's expert e.
template <typename act_t>
__global__ void __launch_bounds__(256) k_dec_route(
    const float *__restrict__ x, int d, int L, int B, int depth, int pos_arg, int n, int W,
    int delta, int K_max, int32_t *__restrict__ hdr, int32_t *__restrict__ row_next,
    int32_t *__restrict__ row_cur, float *__restrict__ prefix, float *__restrict__ cur_sum,
    int32_t *__restrict__ cur_len, int32_t *__restrict__ expert, float *__restrict__ gate,
    const float *__restrict__ w_r, const float *__restrict__ b_r, const float *__restrict__ e_vec,
    const float *__restrict__ bias, const int32_t *__restrict__ forced_e,
    const float *__restrict__ forced_g, int32_t *__restrict__ path_e, float *__restrict__ path_g,
    float *__restrict__ path_m, const float *__restrict__ g_attn, const float *__restrict__ fg,
    const float *__restrict__ fb, int film_stride, float eps, act_t *__restrict__ u) {
  extern __shared__ float s_r[];   // [d] router input
  __shared__ float s_z[kMaxExperts];
  __shared__ float red[4];
  __shared__ int s_e, s_pos;
  const int b = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float *xr = x + (size_t)b * d;
  const size_t sidx = (size_t)depth * B + b;
  float *pre = prefix + sidx * d;
  float *cs = cur_sum + sidx * d;
  if (tid == 0) {
    int ps;
    if (depth == 0) {
      const int nxt = row_next[b];
      ps = pos_arg >= 0 ? pos_arg : nxt;
      bool bad = pos_arg >= 0 && nxt != pos_arg;
      if (ps < 0 || ps >= n) {   // past the document's last slot: stay in bounds
        bad = true;
        ps = min(max(ps, 0), n - 1);
      }
      if (bad) atomicOr(reinterpret_cast<unsigned int *>(hdr + 1), (unsigned)LOL_FLAG_BAD_POS);
      row_cur[b] = ps;
      row_next[b] = ps + 1;
    } else {
      ps = row_cur[b];
    }
    s_pos = ps;
  }
  __syncthreads();
  const int pos = s_pos;
  const int k = (pos + delta) / W;
  const bool opens = pos == max(0, k * W - delta);
  if (!opens) {
    for (int c = tid; c < d; c += 256) cs[c] += xr[c];
    const int e = min(max(expert[sidx], 0), L - 1);
    if (tid == 0) cur_len[sidx] += 1;
    norm_row<act_t>(xr, d, g_attn + (size_t)e * d, fg ? fg + (size_t)e * film_stride : nullptr,
                    fb ? fb + (size_t)e * film_stride : nullptr, eps, u + (size_t)b * d, red);
    return;
  }
  const float inv_prev = 1.f / (float)max(cur_len[sidx], 1);
  for (int c = tid; c < d; c += 256) {
    const float xc = xr[c];
    const float p = k > 0 ? pre[c] + cs[c] * inv_prev : 0.f;
    pre[c] = p;
    s_r[c] = k > 0 ? p / (float)k : 0.5f * (e_vec[c] + xc);
    cs[c] = xc;
  }
  __syncthreads();
  for (int m = wave; m < L; m += 4) {
    const float *wm = w_r + (size_t)m * d;
    float acc = 0.f;
    for (int c = lane; c < d; c += 64) acc += wm[c] * s_r[c];
    acc = wave_sum(acc);
    if (lane == 0) s_z[m] = acc + (b_r ? b_r[m] : 0.f);
  }
  __syncthreads();
  if (wave == 0) {
  const bool live = lane < L;
  const float zl = live ? s_z[lane] : -INFINITY;
  const float zmax = wave_max(zl);
  const float ez = live ? expf(zl - zmax) : 0.f;
  const float a = ez / wave_sum(ez);
  const float sc = live ? a + (bias ? bias[lane] : 0.f) : -INFINITY;
  const float top = wave_max(sc);
  const int rho = wave_min_i((live && sc == top) ? lane : 64);
  const float second = wave_max((live && lane != rho) ? sc : -INFINITY);
  const float margin = L > 1 ? top - second : INFINITY;
  const size_t pidx = sidx * K_max + k;
  int chosen = rho;
  if (forced_e) {
    const int fe = forced_e[pidx];
    if (fe >= L) {
      if (lane == 0) atomicOr(reinterpret_cast<unsigned int *>(hdr + 1), (unsigned)LOL_FLAG_BAD_FORCED_ID);
    } else if (fe >= 0) {
      chosen = fe;
    }
  }
  float alpha = __shfl(a, chosen, 64);
  if (forced_g) {
    const float fgv = forced_g[pidx];
    if (!isnan(fgv)) alpha = fgv;
  }
  if (lane == 0) {
    expert[sidx] = chosen;
    gate[sidx] = alpha;
    cur_len[sidx] = 1;
    if (path_e) path_e[pidx] = chosen;
    if (path_g) path_g[pidx] = alpha;
    if (path_m) path_m[pidx] = margin;
    s_e = chosen;
  }
  }
  __syncthreads();
  const int e = s_e;
  norm_row<act_t>(xr, d, g_attn + (size_t)e * d, fg ? fg + (size_t)e * film_stride : nullptr,
                  fb ? fb + (size_t)e * film_stride : nullptr, eps, u + (size_t)b * d, red);
}

// u = FiLM_ffn(RMSNorm_e(h)) of every document's token, one block each.
template <typename act_t>
__global__ void __launch_bounds__(256) k_dec_norm(const float *__restrict__ h, int d, int L,
                                                  const int32_t *__restrict__ expert,
                                                  const float *__restrict__ g_ffn,
                                                  const float *__restrict__ fg,
                                                  const float *__restrict__ fb, int film_stride,
                                                  float eps, act_t *__restrict__ u) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  const int e = min(max(expert[b], 0), L - 1);
  norm_row<act_t>(h + (size_t)b * d, d, g_ffn + (size_t)e * d,
                  fg ? fg + (size_t)e * film_stride : nullptr,
                  fb ? fb + (size_t)e * film_stride : nullptr, eps, u + (size_t)b * d, red);
}

// Sum of the N values of each lane over the 64 lanes of a wave: every
// exchange step halves the values a lane carries (the partner keeps the
// other half), then plain butterflies finish.  Afterwards a lane holds the
// total of value index lane >> (6 - log2 N), N a power of two <= 64.
template <int N>
__device__ __forceinline__ float wave_reduce_many(float (&v)[N], int lane) {
#pragma unroll
  for (int s = 0; s < 6; ++s) {
    const int o = 32 >> s;
    if ((N >> s) > 1) {
      const int n2 = (N >> s) / 2;
      const bool hi = (lane & o) != 0;
#pragma unroll
      for (int i = 0; i < n2; ++i) {
        float lo_v = v[i], hi_v = v[i + n2];
        // opaque register values: keeps the compiler from turning the two
        // selects below into one dynamically indexed (scratch) array access
        asm volatile("" : "+v"(lo_v), "+v"(hi_v));
        const float send = hi ? lo_v : hi_v;
        const float keep = hi ? hi_v : lo_v;
        v[i] = keep + __shfl_xor(send, o, 64);
      }
    } else {
      v[0] += __shfl_xor(v[0], o, 64);
    }
  }
  return v[0];
}

template <int N> struct Log2 { static constexpr int v = 1 + Log2<N / 2>::v; };
template <> struct Log2<1> { static constexpr int v = 0; };

// 16 bytes of weights or activations
template <typename wt> struct Vec16;
template <> struct Vec16<bf16_t> {
  uint4 v;
  __device__ __forceinline__ float dot(const Vec16 &a, float acc) const {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.x),
                                          __builtin_bit_cast(bf16x2_t, a.v.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.y),
                                          __builtin_bit_cast(bf16x2_t, a.v.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.z),
                                          __builtin_bit_cast(bf16x2_t, a.v.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.w),
                                          __builtin_bit_cast(bf16x2_t, a.v.w), acc, false);
    return acc;
  }
};
template <> struct Vec16<float> {
  float4 v;
  __device__ __forceinline__ float dot(const Vec16 &a, float acc) const {
    acc = fmaf(v.x, a.v.x, acc);
    acc = fmaf(v.y, a.v.y, acc);
    acc = fmaf(v.z, a.v.z, acc);
    return fmaf(v.w, a.v.w, acc);
  }
};
template <typename wt> __device__ __forceinline__ Vec16<wt> ld16(const wt *p) {
  Vec16<wt> r;
  r.v = *reinterpret_cast<const decltype(r.v) *>(p);
  return r;
}
template <typename wt> __device__ __forceinline__ Vec16<wt> zero16() {
  Vec16<wt> r;
  r.v = {};
  return r;
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }
__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

struct DecGemv {
  const void *A;            // [B][K] act: the documents' inputs
  const void *W;            // [L][rows][K] weights (act type)
  long long w_estride;      // elements between experts
  int K;
  int n_cols;               // output columns (SwiGLU: f; the up rows start at glu_off)
  int glu_off;
  int B, L;
  const int32_t *expert;    // [B] this depth's expert of each document
  const float *gate;        // [B]
  const float *x;           // [B][n_cols] depth input (RESID, BLEND)
  const float *h;           // [B][n_cols] (BLEND)
  float *out;               // [B][n_cols] fp32 (STORE, RESID, BLEND; may equal x)
  void *out_act;            // [B][n_cols] act (SWIGLU, GELU)
};

enum DecEpi { DEC_STORE = 0, DEC_RESID = 1, DEC_SWIGLU = 2, DEC_GELU = 3, DEC_BLEND = 4 };

// Grouped matrix-vector products of one depth.  blockIdx.y = g picks the
// g-th distinct expert among the documents (in order of first appearance);
// blocks of a g past the distinct count exit.  Each wave owns CPW output
// columns (2 CPW weight rows with SwiGLU: gate row c and up row glu_off + c)
// and works alone (no block barrier): per chunk of KC inputs it issues every
// 16-byte weight load of its rows together with the inputs of up to MR
// documents of the group (from L2, straight into registers), then the
// products, so a chunk costs one memory round trip.  A lane's sums over its
// inputs are reduced across the wave once per pass.
template <typename wt, int CPW, int EPI, int MR, int NT>
__global__ void __launch_bounds__(256) k_dec_gemv(DecGemv a) {
  constexpr int VEC = 16 / (int)sizeof(wt);
  constexpr int STEP = 64 * VEC;           // inputs one wave load covers
  constexpr int KC = NT * STEP;            // inputs per chunk (NT loads per weight row per lane)
  constexpr bool GLU = EPI == DEC_SWIGLU;
  constexpr int NV = GLU ? 2 * CPW : CPW;  // weight rows per wave
  constexpr int NR = NV * MR;              // sums per lane
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col0 = (blockIdx.x * (blockDim.x >> 6) + wave) * CPW;
  if (col0 >= a.n_cols) return;

  // the group: g-th distinct expert, and its documents (bit mask)
  const int el = lane < a.B ? min(max(a.expert[lane], 0), a.L - 1) : -1;
  bool dup = false;
  for (int j = 0; j < a.B; ++j) {
    const int ej = __shfl(el, j, 64);
    if (j < lane && ej == el) dup = true;
  }
  const unsigned long long first = __ballot(lane < a.B && !dup);
  const int g = blockIdx.y;
  if (__popcll(first) <= g) return;
  unsigned long long mm = first;
  for (int i = 0; i < g; ++i) mm &= mm - 1;
  const int e = __shfl(el, __ffsll((long long)mm) - 1, 64);
  unsigned long long rows = __ballot(lane < a.B && el == e);

  const int K = a.K;
  const wt *We = static_cast<const wt *>(a.W) + (size_t)e * a.w_estride;
  const wt *wrow[NV];
  bool wok[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int j = GLU ? v / 2 : v;
    const int c = col0 + j;
    wok[v] = c < a.n_cols;
    const int r = (GLU && (v & 1)) ? a.glu_off + c : c;
    wrow[v] = We + (size_t)(wok[v] ? r : 0) * K;
  }

  while (rows) {
    // the next pass: up to MR documents of the group (padding repeats the first)
    int rowid[MR];
    int mr = 0;
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      if (rows) {
        rowid[r] = __ffsll((long long)rows) - 1;
        rows &= rows - 1;
        mr = r + 1;
      } else {
        rowid[r] = rowid[0];
      }
    }
    float acc[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) acc[i] = 0.f;
    for (int k0 = 0; k0 < K; k0 += KC) {
      Vec16<wt> w[NT][NV];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int kk = k0 + t * STEP + lane * VEC;
#pragma unroll
        for (int v = 0; v < NV; ++v)
          w[t][v] = (wok[v] && kk < K) ? ld16<wt>(wrow[v] + kk) : zero16<wt>();
      }
      Vec16<wt> av[NT][MR];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int kk = k0 + t * STEP + lane * VEC;
        if (kk < K) {
#pragma unroll
          for (int r = 0; r < MR; ++r)
            av[t][r] = ld16<wt>(static_cast<const wt *>(a.A) + (size_t)rowid[r] * K + kk);
        } else {
#pragma unroll
          for (int r = 0; r < MR; ++r) av[t][r] = zero16<wt>();
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < MR; ++r)
#pragma unroll
          for (int v = 0; v < NV; ++v) acc[v * MR + r] = w[t][v].dot(av[t][r], acc[v * MR + r]);
    }
    const float tot = wave_reduce_many<NR>(acc, lane);
    constexpr int SH = 6 - Log2<NR>::v;
    // SwiGLU: the up row's sum sits MR values (MR << SH lanes) after the gate's
    const float up = GLU ? __shfl(tot, (lane + (MR << SH)) & 63, 64) : 0.f;
    const int idx = lane >> SH;
    const int v = idx / MR, r = idx % MR;
    if ((lane & ((1 << SH) - 1)) != 0 || r >= mr || (GLU && (v & 1))) continue;
    const int c = col0 + (GLU ? v / 2 : v);
    if (c >= a.n_cols) continue;
    int row = rowid[0];
#pragma unroll
    for (int q = 1; q < MR; ++q)
      if (q == r) row = rowid[q];
    const size_t o = (size_t)row * a.n_cols + c;
    if (EPI == DEC_STORE) {
      a.out[o] = tot;
    } else if (EPI == DEC_RESID) {
      a.out[o] = a.x[o] + tot;
    } else if (EPI == DEC_SWIGLU) {
      static_cast<wt *>(a.out_act)[o] = from_f<wt>(silu(tot) * up);
    } else if (EPI == DEC_GELU) {
      static_cast<wt *>(a.out_act)[o] = from_f<wt>(gelu_erf(tot));
    } else {
      const float xv = a.x[o];
      const float y = a.h[o] + tot;
      a.out[o] = xv + a.gate[row] * (y - xv);
    }
  }
}

// Attention of every document's token (block x = document, y = head, 4
// waves) over the open window of one depth: q and k of the token are rotated
// at its window-local position p (RoPE, rotate-half pairs), rounded to the
// operand type, k and v are appended to the cache at slot p, and the token
// attends to slots 0..p (paper Sec. 3.2.1: causal inside the window; review
// Eq. 1: scores scaled by 1/sqrt(d_head)).  Keys go one per thread, 256 at
// a time: the first 256 keys' K and V rows are requested together at the
// start (16-byte loads), before the token's own projections are read; the
// values are staged in LDS for the weighted sum (lanes over dimensions, keys
// split over the 4 waves), then the 4 waves' sums are added.
template <typename act_t, int DH>
__global__ void __launch_bounds__(256) k_dec_attn(const float *__restrict__ qkv,
                                                  act_t *__restrict__ kc, act_t *__restrict__ vc,
                                                  act_t *__restrict__ o,
                                                  const float *__restrict__ rope_cs, int d, int H,
                                                  int W, int delta,
                                                  const int32_t *__restrict__ row_cur, float scale,
                                                  int use_rope) {
  extern __shared__ float s_p[];   // [W] scores, then weights
  __shared__ float s_q[DH], s_k[DH], s_v[DH];
  __shared__ float s_red[4];
  __shared__ float s_o[4][DH];
  __shared__ __attribute__((aligned(16))) act_t s_vrow[256][DH];   // values of keys 0..255
  constexpr int HALF = DH / 2;
  constexpr int V = 16 / (int)sizeof(act_t);   // elements per 16-byte load
  constexpr int NV = DH / V;                   // loads per row
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // the token's window-local position at this depth
  const int pos = row_cur[b];
  const int p = pos - max(0, (pos + delta) / W * W - delta);
  const float *qr = qkv + (size_t)b * 3 * d + h * DH;
  const size_t cbase = ((size_t)b * H + h) * W * DH;
  act_t *kcache = kc + cbase, *vcache = vc + cbase;
  // keys 0..255 (those before the token): rows requested first
  Vec16<act_t> k0[NV], v0[NV];
  if (tid < p) {
#pragma unroll
    for (int t = 0; t < NV; ++t) {
      k0[t] = ld16<act_t>(kcache + (size_t)tid * DH + t * V);
      v0[t] = ld16<act_t>(vcache + (size_t)tid * DH + t * V);
    }
  }
  if (tid < DH) {
    float q = qr[tid], k = qr[d + tid];
    const float v = qr[2 * d + tid];
    if (use_rope) {
      const int j = tid % HALF;
      const float c = rope_cs[((size_t)p * HALF + j) * 2], s = rope_cs[((size_t)p * HALF + j) * 2 + 1];
      const int partner = tid < HALF ? tid + HALF : tid - HALF;
      const float qp = qr[partner], kp = qr[d + partner];
      q = tid < HALF ? q * c - qp * s : q * c + qp * s;
      k = tid < HALF ? k * c - kp * s : k * c + kp * s;
    }
    const act_t qa = from_f<act_t>(q), ka = from_f<act_t>(k), va = from_f<act_t>(v);
    s_q[tid] = to_f<act_t>(qa);
    s_k[tid] = to_f<act_t>(ka);
    s_v[tid] = to_f<act_t>(va);
    kcache[(size_t)p * DH + tid] = ka;
    vcache[(size_t)p * DH + tid] = va;
  }
  __syncthreads();
  // scores of keys j = tid, tid + 256, ...
  auto key_dot = [&](const Vec16<act_t> (&kv)[NV]) {
    float sc = 0.f;
#pragma unroll
    for (int t = 0; t < NV; ++t) {
      const act_t *kp = reinterpret_cast<const act_t *>(&kv[t].v);
#pragma unroll
      for (int i = 0; i < V; ++i) sc += s_q[t * V + i] * to_f<act_t>(kp[i]);
    }
    return sc;
  };
  float mloc = -INFINITY;
  if (tid <= p) {
    float sc = 0.f;
    if (tid == p) {
#pragma unroll
      for (int t = 0; t < DH; ++t) sc += s_q[t] * s_k[t];
    } else {
      sc = key_dot(k0);
    }
    s_p[tid] = sc * scale;
    mloc = sc * scale;
  }
  for (int j = tid + 256; j <= p; j += 256) {
    float sc = 0.f;
    if (j == p) {
#pragma unroll
      for (int t = 0; t < DH; ++t) sc += s_q[t] * s_k[t];
    } else {
      Vec16<act_t> kv[NV];
#pragma unroll
      for (int t = 0; t < NV; ++t) kv[t] = ld16<act_t>(kcache + (size_t)j * DH + t * V);
      sc = key_dot(kv);
    }
    s_p[j] = sc * scale;
    mloc = fmaxf(mloc, sc * scale);
  }
  mloc = wave_max(mloc);
  if (lane == 0) s_red[wave] = mloc;
  __syncthreads();
  const float mx = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  float lsum = 0.f;
  for (int j = tid; j <= p; j += 256) {
    const float w = expf(s_p[j] - mx);
    s_p[j] = w;
    lsum += w;
  }
  lsum = wave_sum(lsum);
  __syncthreads();   // every thread has read s_red
  if (lane == 0) s_red[wave] = lsum;
  // sum over keys of w_j v_j: lanes over dimensions, keys split over the 4
  // waves; the first 256 keys' values come from LDS (staged from the rows
  // requested at the start), later ones from the cache
  if (tid < p) {
#pragma unroll
    for (int t = 0; t < NV; ++t) *reinterpret_cast<decltype(v0[t].v) *>(&s_vrow[tid][t * V]) = v0[t].v;
  }
  __syncthreads();
  if (lane < DH) {
    float acc = 0.f;
    const int j1 = min(p, 256);
    int j = wave;
    for (; j + 12 < j1; j += 16)
      acc += s_p[j] * to_f<act_t>(s_vrow[j][lane]) + s_p[j + 4] * to_f<act_t>(s_vrow[j + 4][lane]) +
             s_p[j + 8] * to_f<act_t>(s_vrow[j + 8][lane]) + s_p[j + 12] * to_f<act_t>(s_vrow[j + 12][lane]);
    for (; j < j1; j += 4) acc += s_p[j] * to_f<act_t>(s_vrow[j][lane]);
    for (; j < p; j += 4) acc += s_p[j] * to_f<act_t>(vcache[(size_t)j * DH + lane]);
    if (j == p) acc += s_p[p] * s_v[lane];
    s_o[wave][lane] = acc;
  }
  __syncthreads();
  if (tid < DH) {
    const float inv = 1.f / (s_red[0] + s_red[1] + s_red[2] + s_red[3]);
    o[(size_t)b * d + h * DH + tid] =
        from_f<act_t>((s_o[0][tid] + s_o[1][tid] + s_o[2][tid] + s_o[3][tid]) * inv);
  }
}

template <typename wt, int CPW, int EPI, int MR, int NT>
hipError_t gemv_launch_mr(const DecGemv &a, hipStream_t st) {
  constexpr int WPB = 4;   // waves per block (they share nothing)
  dim3 grid((a.n_cols + WPB * CPW - 1) / (WPB * CPW), min(a.B, a.L));
  lol_launch(k_dec_gemv<wt, CPW, EPI, MR, NT>, grid, dim3(64 * WPB), 0, st, a);
  return hipGetLastError();
}

template <typename wt, int CPW, int EPI, int NT>
hipError_t gemv_launch(const DecGemv &a, hipStream_t st) {
  // documents per pass: the batch rounded up to a power of two, at most 8
  // (8 documents per pass with half the columns per wave: the sums and
  // inputs of a pass stay in registers)
  constexpr int CPW8 = CPW > 1 ? CPW / 2 : 1;
  if (a.B <= 1) return gemv_launch_mr<wt, CPW, EPI, 1, NT>(a, st);
  if (a.B <= 2) return gemv_launch_mr<wt, CPW, EPI, 2, NT>(a, st);
  if (a.B <= 4) return gemv_launch_mr<wt, CPW, EPI, 4, NT>(a, st);
  return gemv_launch_mr<wt, CPW8, EPI, 8, NT>(a, st);
}

// One output column (SwiGLU: one gate/up pair) per wave: with few documents
// the fixed part of a wave (group lookup, one round trip, the reduction)
// outweighs its bytes, so more waves in flight hide more of it (measured:
// 4 columns per wave for QKV and 2 pairs for gate/up were 10-15% slower).
// The down projection reads 4 loads per row per chunk (two chunks at K =
// 4096).
template <typename wt>
hipError_t gemv_typed(const DecGemv &a, int which, bool glu, hipStream_t st) {
  switch (which) {
    case DEC_QKV: return gemv_launch<wt, 1, DEC_STORE, 2>(a, st);
    case DEC_O: return gemv_launch<wt, 1, DEC_RESID, 2>(a, st);
    case DEC_GU:
      return glu ? gemv_launch<wt, 1, DEC_SWIGLU, 2>(a, st)
                 : gemv_launch<wt, 4, DEC_GELU, 2>(a, st);
    default: return gemv_launch<wt, 1, DEC_BLEND, 4>(a, st);
  }
}

template <typename act_t>
hipError_t attn_launch(const lol_core_config &c, const DecodeBufs &s, int depth, int delta,
                       hipStream_t st) {
  const int dh = c.d / c.n_heads;
  const size_t per_depth = (size_t)c.batch * c.n_heads * c.W * dh;
  act_t *kc = static_cast<act_t *>(s.kc) + (size_t)depth * per_depth;
  act_t *vc = static_cast<act_t *>(s.vc) + (size_t)depth * per_depth;
  const float scale = 1.0f / sqrtf((float)dh);
  const int use_rope = c.rope_theta != 0.f ? 1 : 0;
  dim3 grid(c.batch, c.n_heads);
  const uint32_t shm = (uint32_t)c.W * sizeof(float);   // scores of up to W keys
  if (dh == 64)
    lol_launch(k_dec_attn<act_t, 64>, grid, dim3(256), shm, st, s.qkv, kc, vc,
               static_cast<act_t *>(s.o), s.rope_cs, c.d, c.n_heads, c.W, delta, s.row_cur, scale,
               use_rope);
  else
    lol_launch(k_dec_attn<act_t, 32>, grid, dim3(256), shm, st, s.qkv, kc, vc,
               static_cast<act_t *>(s.o), s.rope_cs, c.d, c.n_heads, c.W, delta, s.row_cur, scale,
               use_rope);
  return hipGetLastError();
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

bool decode_supported(const lol_core_config &c) {
  return c.batch <= 64 && c.d <= 4096 && c.W <= 8192;
}

size_t decode_layout(const lol_core_config &c, char *base, DecodeBufs *out) {
  const size_t B = c.batch, d = c.d, f = c.d_ffn, D = c.D;
  const size_t act = c.dtype == LOL_BF16 ? 2 : 4;
  const size_t dh = d / c.n_heads;
  size_t off = 0;
  auto carve = [&](size_t bytes) -> char * {
    char *ptr = base ? base + off : nullptr;
    off += align_up(bytes);
    return ptr;
  };
  DecodeBufs s;
  s.hdr = (int32_t *)carve(2 * 4);
  s.row_next = (int32_t *)carve(B * 4);
  s.row_cur = (int32_t *)carve(B * 4);
  s.prefix = (float *)carve(D * B * d * 4);
  s.cur_sum = (float *)carve(D * B * d * 4);
  s.cur_len = (int32_t *)carve(D * B * 4);
  s.expert = (int32_t *)carve(D * B * 4);
  s.gate = (float *)carve(D * B * 4);
  s.kc = carve(D * B * c.n_heads * (size_t)c.W * dh * act);
  s.vc = carve(D * B * c.n_heads * (size_t)c.W * dh * act);
  s.rope_cs = (float *)carve((size_t)c.W * (dh / 2) * 2 * 4);
  s.u = carve(B * d * act);
  s.qkv = (float *)carve(B * 3 * d * 4);
  s.o = carve(B * d * act);
  s.h = (float *)carve(B * d * 4);
  s.hid = carve(B * f * act);
  if (out) *out = s;
  return off;
}

hipError_t launch_dec_reset(const lol_core_config &c, const DecodeBufs &s, int row, hipStream_t st) {
  const int half = c.d / c.n_heads / 2;
  const bool all = row < 0;
  const int row0 = all ? 0 : row, row1 = all ? c.batch : row + 1;
  const int total = max(max(c.D * (row1 - row0), all ? c.W * half : 0), 1);
  lol_launch(k_dec_reset, dim3((total + 255) / 256), dim3(256), 0, st, s.hdr, s.row_next,
             s.cur_len, s.expert, s.gate, c.batch, c.D, row0, row1, all ? 1 : 0, s.rope_cs, c.W,
             half, (double)c.rope_theta, c.rope_theta != 0.f ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_dec_route(const lol_core_config &c, const DecodeBufs &s, int depth, int pos,
                            const float *x, const lol_library &lib,
                            const lol_router &rt, const int32_t *forced_e, const float *forced_g,
                            const lol_path *path, hipStream_t st) {
  const int d = c.d, L = c.L;
  const int K_max = (c.n + c.W - 1) / c.W + 1;
  const float *w_r = rt.w_r + (rt.per_depth ? (size_t)depth * L * d : 0);
  const float *b_r = rt.b_r ? rt.b_r + (rt.per_depth ? (size_t)depth * L : 0) : nullptr;
  // FiLM rows of (depth, attention sublayer): [D][2][d], or [D][L][2][d] per expert
  const size_t film_off = ((size_t)depth * (lib.film_per_expert ? L : 1) * 2 + 0) * d;
  const float *fg = lib.film_gamma ? lib.film_gamma + film_off : nullptr;
  const float *fb = lib.film_beta ? lib.film_beta + film_off : nullptr;
  const int film_stride = lib.film_per_expert ? 2 * d : 0;
  const uint32_t shm = (uint32_t)d * sizeof(float);
  int32_t *pe = path ? path->expert : nullptr;
  float *pg = path ? path->gate : nullptr, *pm = path ? path->margin : nullptr;
  const int delta = (int)(((long long)depth * c.S) % c.W);
  if (c.dtype == LOL_BF16)
    lol_launch(k_dec_route<bf16_t>, dim3(c.batch), dim3(256), shm, st, x, d, L, c.batch, depth,
               pos, c.n, c.W, delta, K_max, s.hdr, s.row_next, s.row_cur, s.prefix, s.cur_sum,
               s.cur_len, s.expert, s.gate, w_r,
               b_r, rt.e_depth + (size_t)depth * d, rt.expert_bias, forced_e, forced_g, pe, pg, pm,
               lib.g_attn, fg, fb, film_stride, c.rms_eps, static_cast<bf16_t *>(s.u));
  else
    lol_launch(k_dec_route<float>, dim3(c.batch), dim3(256), shm, st, x, d, L, c.batch, depth,
               pos, c.n, c.W, delta, K_max, s.hdr, s.row_next, s.row_cur, s.prefix, s.cur_sum,
               s.cur_len, s.expert, s.gate, w_r,
               b_r, rt.e_depth + (size_t)depth * d, rt.expert_bias, forced_e, forced_g, pe, pg, pm,
               lib.g_attn, fg, fb, film_stride, c.rms_eps, static_cast<float *>(s.u));
  return hipGetLastError();
}

hipError_t launch_dec_norm(const lol_core_config &c, const DecodeBufs &s, int depth,
                           const lol_library &lib, hipStream_t st) {
  const int d = c.d, L = c.L;
  const size_t film_off = ((size_t)depth * (lib.film_per_expert ? L : 1) * 2 + 1) * d;
  const float *fg = lib.film_gamma ? lib.film_gamma + film_off : nullptr;
  const float *fb = lib.film_beta ? lib.film_beta + film_off : nullptr;
  const int film_stride = lib.film_per_expert ? 2 * d : 0;
  const int32_t *ex = s.expert + (size_t)depth * c.batch;
  if (c.dtype == LOL_BF16)
    lol_launch(k_dec_norm<bf16_t>, dim3(c.batch), dim3(256), 0, st, s.h, d, L, ex, lib.g_ffn, fg,
               fb, film_stride, c.rms_eps, static_cast<bf16_t *>(s.u));
  else
    lol_launch(k_dec_norm<float>, dim3(c.batch), dim3(256), 0, st, s.h, d, L, ex, lib.g_ffn, fg,
               fb, film_stride, c.rms_eps, static_cast<float *>(s.u));
  return hipGetLastError();
}

hipError_t launch_dec_attn(const lol_core_config &c, const DecodeBufs &s, int depth,
                           hipStream_t st) {
  const int delta = (int)(((long long)depth * c.S) % c.W);
  if (c.dtype == LOL_BF16) return attn_launch<bf16_t>(c, s, depth, delta, st);
  return attn_launch<float>(c, s, depth, delta, st);
}

hipError_t launch_dec_gemv(const lol_core_config &c, const DecodeBufs &s, int depth, int which,
                           const float *x, float *y, const lol_library &lib, hipStream_t st) {
  const size_t d = c.d, f = c.d_ffn;
  const bool glu = c.mlp == LOL_MLP_SWIGLU;
  DecGemv a{};
  a.B = c.batch;
  a.L = c.L;
  a.expert = s.expert + (size_t)depth * c.batch;
  a.gate = s.gate + (size_t)depth * c.batch;
  switch (which) {
    case DEC_QKV:
      a.A = s.u; a.W = lib.wqkv; a.w_estride = (long long)(3 * d * d); a.K = (int)d;
      a.n_cols = (int)(3 * d); a.out = s.qkv;
      break;
    case DEC_O:
      a.A = s.o; a.W = lib.wo; a.w_estride = (long long)(d * d); a.K = (int)d;
      a.n_cols = (int)d; a.x = x; a.out = s.h;
      break;
    case DEC_GU:
      a.A = s.u; a.W = lib.w_gu; a.w_estride = (long long)((glu ? 2 : 1) * f * d); a.K = (int)d;
      a.n_cols = (int)f; a.glu_off = (int)f; a.out_act = s.hid;
      break;
    case DEC_DOWN:
      a.A = s.hid; a.W = lib.w_down; a.w_estride = (long long)(d * f); a.K = (int)f;
      a.n_cols = (int)d; a.x = x; a.h = s.h; a.out = y;
      break;
    default:
      return hipErrorInvalidValue;
  }
  if (c.dtype == LOL_BF16) return gemv_typed<bf16_t>(a, which, glu, st);
  return gemv_typed<float>(a, which, glu, st);
}

}  // namespace lol
