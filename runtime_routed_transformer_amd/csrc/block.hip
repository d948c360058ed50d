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
// FROM_S (attention sublayer): blocks walk the windows (block (c, slot) takes
// positions 4c .. 4c + 3 of window slot `slot`), x = s[token], and the wave
// also writes the grouped row's metadata (token, window-local position,
// expert, gate) for the kernels after it.  Else (MLP) x = h[row], rows in
// grouped order.
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

// Window geometry and grouped-row metadata for the attention norm.
struct NormWin {
  const int32_t *win_exp, *win_len, *win_row0;
  const float *win_gate;
  const int32_t *doc_start, *doc_len;   // packed documents, or NULL
  int W, delta, K_max, n, n_tokens;
  int32_t *row_tok, *row_pos, *row_exp;
  float *row_gate;
};

template <typename act_t, bool FROM_S, int NCH>
__global__ void __launch_bounds__(256) k_norm(const float *__restrict__ src,
                                              const int32_t *__restrict__ row_exp_in,
                                              const float *__restrict__ gain,
                                              const float *__restrict__ fg,
                                              const float *__restrict__ fb, act_t *__restrict__ u,
                                              const int32_t *__restrict__ n_rows, int d, float eps,
                                              int panel_rows, int film_stride, NormWin nw) {
  // the row is wave-uniform: its metadata arrive through scalar loads
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  int row, e;
  const float *x;
  if constexpr (FROM_S) {
    const int slot = blockIdx.y, p = blockIdx.x * 4 + wave;
    e = nw.win_exp[slot];
    if (e < 0 || p >= nw.win_len[slot]) return;
    row = nw.win_row0[slot] + p;
    const int b = slot / nw.K_max, k = slot - b * nw.K_max;
    // document b's first token (clamped into the stream like the router's)
    int d0 = b * nw.n;
    if (nw.doc_len) {
      const int len = min(min(max(nw.doc_len[b], 1), nw.n), nw.n_tokens);
      d0 = min(max(nw.doc_start[b], 0), nw.n_tokens - len);
    }
    const int tok = d0 + max(0, k * nw.W - nw.delta) + p;
    if (lane == 0) {
      nw.row_tok[row] = tok;
      nw.row_pos[row] = p;
      nw.row_exp[row] = e;
      nw.row_gate[row] = nw.win_gate[slot];
    }
    x = src + (size_t)tok * d;
  } else {
    row = blockIdx.x * 4 + wave;
    // grouped rows in use this depth (the grid covers the most there can be;
    // packed documents fill fewer, and the rows past them hold no metadata)
    if (row >= *n_rows) return;
    x = src + (size_t)row * d;
    e = row_exp_in[row];
  }
  const float *g = gain + (size_t)e * d;
  // FiLM of this depth and sublayer; per expert when film_stride > 0
  if (fg) {
    fg += (size_t)e * film_stride;
    fb += (size_t)e * film_stride;
  }
  act_t *out = u + (size_t)row * d;
  if (NCH > 0) {
    // every load of the row (x, the expert gain, FiLM) is issued before the
    // reduction, so the row waits for one round trip instead of one per chunk
    constexpr int N1 = NCH > 0 ? NCH : 1;
    float4 xv[N1], gv[N1], av[N1], bv[N1];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = i * 256 + lane * 4;
      xv[i] = *reinterpret_cast<const float4 *>(x + c);
      gv[i] = *reinterpret_cast<const float4 *>(g + c);
      if (fg) {
        av[i] = *reinterpret_cast<const float4 *>(fg + c);
        bv[i] = *reinterpret_cast<const float4 *>(fb + c);
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      ss += xv[i].x * xv[i].x + xv[i].y * xv[i].y + xv[i].z * xv[i].z + xv[i].w * xv[i].w;
    const float inv = rsqrtf(wave_sum(ss) / (float)d + eps);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = i * 256 + lane * 4;
      float4 v = make_float4(xv[i].x * inv * gv[i].x, xv[i].y * inv * gv[i].y,
                             xv[i].z * inv * gv[i].z, xv[i].w * inv * gv[i].w);
      if (fg)
        v = make_float4(av[i].x * v.x + bv[i].x, av[i].y * v.y + bv[i].y, av[i].z * v.z + bv[i].z,
                        av[i].w * v.w + bv[i].w);
      // panel_rows > 0 (NCH > 0 only): u in 32-column panels [d/32][panel_rows][32]
      act_t *dst = panel_rows ? u + ((size_t)(c >> 5) * panel_rows + row) * 32 + (c & 31) : out + c;
      store4<act_t>(dst, v.x, v.y, v.z, v.w);
    }
  } else {
    float ss = 0.f;
    for (int c = lane; c < d; c += 64) ss += x[c] * x[c];
    const float inv = rsqrtf(wave_sum(ss) / (float)d + eps);
    for (int c = lane; c < d; c += 64) {
      float v = x[c] * inv * g[c];
      if (fg) v = fg[c] * v + fb[c];
      st<act_t>(panel_rows ? u + ((size_t)(c >> 5) * panel_rows + row) * 32 + (c & 31) : out + c, v);
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
                                                  const int32_t *__restrict__ win_len,
                                                  const float *__restrict__ rope_cs, int d,
                                                  float scale, int use_rope) {
  constexpr int HALF = DH / 2;
  __shared__ float ks[64][DH + 1];
  __shared__ float vs[64][DH + 1];
  const int slot = blockIdx.x, h = blockIdx.y, q0 = blockIdx.z * 64;
  if (win_exp[slot] < 0) return;
  const int len = win_len[slot];  // tokens of the window (its document's end clips the last one)
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
// q and k arrive rotated (RoPE is applied in the QKV projection's epilogue).
// Block = (window, head, chunk of 256 queries), 4 waves, three blocks per
// CU.  Keys and values of a chunk of 128 keys at a time are copied row-major
// into LDS by direct global-to-LDS loads (no register staging), 16-byte chunks of each row XOR-swizzled so
// that the fragment reads below are free of bank conflicts.  Each wave owns
// query blocks of 32 (wave w takes blocks w and 7-w of the chunk, which
// balances the causal triangle) and computes S^T = K Q^T, so every lane holds
// one query's scores for 16 of 32 keys: the online softmax needs one exchange
// with the lane 32 apart.  Then O^T += V^T P^T, where the V^T operand comes
// from row-major V through the LDS transpose read (ds_read_b64_tr_b16: in
// each group of 16 lanes, lane i receives element i % 4 of the 8-byte pieces
// that lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4 address), and the key order
// inside each 16-key MFMA step is the one in which the scores already sit.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

template <int DH> struct AttnLds {
  static constexpr int RB = 2 * DH;        // bytes per K or V row
  static constexpr int NCK = DH / 8;       // 16-byte chunks per row
  static constexpr int RPI = 1024 / RB;    // rows per 1 KiB direct load
  // K: physical chunk = logical ^ kswz(row).  16 lanes read one logical
  // chunk of 16 consecutive rows; with this swizzle they cover all 64 banks.
  static __device__ __forceinline__ int kswz(int r) { return (r / (256 / RB)) & (NCK - 1); }
  // V: the transpose reads of one half-wave touch 4 consecutive rows and
  // 64 bytes of each; for 128-byte rows, rows 2 and 3 of each group of 4
  // move to the other half of the row.
  static __device__ __forceinline__ int vswz(int r) { return DH == 64 ? ((r >> 1) & 1) << 2 : 0; }
};

template <int DH>
__global__ void __launch_bounds__(256, 3) k_attn_mfma(const bf16_t *__restrict__ qkv,
                                                      bf16_t *__restrict__ o,
                                                      const int32_t *__restrict__ win_exp,
                                                      const int32_t *__restrict__ win_row0,
                                                      const int32_t *__restrict__ win_len, int d,
                                                      float qscale, int o_panel_rows) {
  using LY = AttnLds<DH>;
  constexpr int CH = 256;            // keys / queries per chunk
  constexpr int RB = LY::RB, NCK = LY::NCK, RPI = LY::RPI;
  constexpr int KS = DH / 16;        // MFMA k-steps over the head dimension
  constexpr int DB = DH / 32;        // 32-wide output blocks over the head dimension
  // keys per LDS chunk: 32 KiB of K and V, so three blocks share a CU (four
  // would leave under 128 registers per lane and spill; 256-key chunks
  // allowed only two and measured 38.6 vs 34.9 us at mid_bf16)
  constexpr int KC = CH / 2;
  constexpr int NI = KC * RB / 1024 / 4;  // 1 KiB loads per wave per operand
  __shared__ __attribute__((aligned(1024))) char lds[2 * KC * RB];
  char *const Kl = lds;
  char *const Vl = lds + KC * RB;
  // query chunks in reverse dispatch order: in a window longer than one
  // chunk the last chunks see the most keys, so they start first and the
  // light ones fill in behind them
  const int slot = blockIdx.x, h = blockIdx.y, qc = gridDim.z - 1 - blockIdx.z;
  if (win_exp[slot] < 0) return;
  const int len = win_len[slot];  // tokens of the window (its document's end clips the last one)
  const int q_begin = qc * CH;
  if (q_begin >= len) return;
  const int base = win_row0[slot];
  const size_t ld3 = (size_t)3 * d;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar LDS addresses
  const int hl = lane >> 5, col = lane & 31;

  // ---- this wave's two query blocks: Q fragments straight from HBM
  const int qblk[2] = {wave, 7 - wave};
  bf16x8_t qf[2][KS];
  float m_run[2], l_run[2];
  f32x16_t acc[2][DB];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int qrow = min(q_begin + qblk[b] * 32 + col, len - 1);
    const bf16_t *qp = qkv + (size_t)(base + qrow) * ld3 + h * DH + hl * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[b][ks] = *reinterpret_cast<const bf16x8_t *>(qp + ks * 16);
    m_run[b] = -INFINITY;
    l_run[b] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][db][i] = 0.f;
  }

  // ---- per-lane pieces of the direct loads: row lr of each 1 KiB, physical chunk pc
  const int lr = lane / NCK, pc = lane % NCK;
  // transpose-read addressing: lane (group g = lane/16, p = lane%16) reads
  // row 4 (g/2) + p/4 (+8 for the second read) and the 4 columns from
  // (g%2) 16 + 4 (p%4) of each 32-column block
  const int g16 = lane >> 4, p16 = lane & 15;
  const int tr_row = 4 * (g16 >> 1) + (p16 >> 2);
  const int tr_col = (g16 & 1) * 16 + 4 * (p16 & 3);
  // Both swizzles depend only on row bits below 32 (K: bits 1-3 or 2-3; V:
  // bit 1), so every fragment address is a per-lane constant plus
  // kb * 32 rows: no address arithmetic inside the key loop.
  int k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = col * RB + (((2 * ks + hl) ^ LY::kswz(col)) << 4);
  int v_off[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int c = db * 32 + tr_col;                     // first of the 4 columns
    v_off[db] = tr_row * RB + ((((c >> 3) ^ LY::vswz(tr_row)) << 4) + ((c & 4) << 1));
  }

  // key chunks of KC keys up to the block's last query
  const int nkc = (min(q_begin + CH, len) + KC - 1) / KC;
  for (int kc = 0; kc < nkc; ++kc) {
    const int k_begin = kc * KC;
    if (kc > 0) __syncthreads();   // every wave is done with the previous chunk
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int piece = wave + 4 * i;
      const int r = piece * RPI + lr;                       // row inside the chunk
      const int key = min(k_begin + r, len - 1);            // rows past the window repeat the last key
      const bf16_t *rowp = qkv + (size_t)(base + key) * ld3 + h * DH;
      __builtin_amdgcn_global_load_lds((gbl_void_t *)(rowp + d + ((pc ^ LY::kswz(r)) << 3)),
                                       (lds_void_t *)(Kl + piece * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gbl_void_t *)(rowp + 2 * d + ((pc ^ LY::vswz(r)) << 3)),
                                       (lds_void_t *)(Vl + piece * 1024), 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's direct loads have landed
    __syncthreads();
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int q_lo = q_begin + qblk[b] * 32;            // first query of the block
      if (q_lo >= len) continue;
      const int q = q_lo + col;
      // key blocks of this chunk that the query block can see (32-key block
      // indices over the window: the chunk starts at kb0, the query block is qg)
      const int kb0 = kc * (KC / 32), qg = qc * (CH / 32) + qblk[b];
      if (qg < kb0) continue;
      const int kb_end = min(KC / 32, qg - kb0 + 1);
      for (int kb = 0; kb < kb_end; ++kb) {
        f32x16_t sc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[i] = 0.f;
        const char *kbase = Kl + kb * 32 * RB;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8_t kf = *reinterpret_cast<const bf16x8_t *>(kbase + k_off[ks]);
          sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[b][ks], sc, 0, 0, 0);
        }
        // sc[i] = q.k for key = k_begin + kb*32 + (i/4)*8 + 4*hl + i%4, query q
        if (kb0 + kb == qg) {
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
        // Softmax weights 2^((s - m) * log2(e) / sqrt(d_head)) against a
        // reference maximum m that only moves (rescaling the running sum and
        // output) when some lane's scores exceed it by more than 2^8; below
        // that the weights stay <= 256, exact enough in fp32 and in the bf16
        // operand.  The raw exp2 is exact to about 1 ulp and flushes tiny
        // weights to zero.
        if (__builtin_amdgcn_ballot_w64((mx - m_run[b]) * qscale > 8.f)) {
          const float m_new = fmaxf(m_run[b], mx);
          const float corr = __builtin_amdgcn_exp2f((m_run[b] - m_new) * qscale);
          l_run[b] *= corr;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[b][db][i] *= corr;
          m_run[b] = m_new;
        }
        const float mc = m_run[b] * qscale;
        float p[16], rs = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], qscale, -mc));
          rs += p[i];
        }
        rs += __shfl_xor(rs, 32, 64);
        l_run[b] += rs;
#pragma unroll
        for (int step = 0; step < 2; ++step) {
          bf16x8_t pb;
#pragma unroll
          for (int j = 0; j < 8; ++j) pb[j] = (__bf16)p[8 * step + j];
          // rows kb*32 + 16 step + tr_row (keys +0..3) and 8 rows on
          const char *vbase = Vl + (kb * 32 + 16 * step) * RB;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            // (element-wise copies out of the v4i16 form of this read are
            // miscompiled by this compiler: only its low dword survives)
            const bf16x4_t lo =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(vbase + v_off[db]));
            const bf16x4_t hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(vbase + v_off[db] + 8 * RB));
            const bf16x8_t va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
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
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 pk;
        pk.x = (uint32_t)f2bf(acc[b][db][4 * g] * il) | ((uint32_t)f2bf(acc[b][db][4 * g + 1] * il) << 16);
        pk.y = (uint32_t)f2bf(acc[b][db][4 * g + 2] * il) | ((uint32_t)f2bf(acc[b][db][4 * g + 3] * il) << 16);
        // 4 consecutive columns, inside one 16-column panel when o is in panels
        const int col = h * DH + db * 32 + g * 8 + 4 * hl;
        bf16_t *op = o_panel_rows ? o + ((size_t)(col >> 4) * o_panel_rows + base + q) * 16 + (col & 15)
                                  : o + (size_t)(base + q) * d + col;
        *reinterpret_cast<uint2 *>(op) = pk;
      }
  }
}

template <typename act_t, int NCH>
void norm_launch(const Plan &p, int which, const float *s, const lol_library &lib,
                 const Workspace &ws, const float *fg, const float *fb, int panel_rows, int delta,
                 hipStream_t st) {
  const int film_stride = lib.film_per_expert ? 2 * p.cfg.d : 0;
  const int32_t *n_rows = ws.toff + p.cfg.L;   // total grouped rows, written by the router
  NormWin nw{ws.win_exp, ws.win_len, ws.win_row0, ws.win_gate, p.doc_start, p.doc_len,
             p.cfg.W, delta, p.K_max, p.cfg.n, p.n_tokens, ws.row_tok, ws.row_pos, ws.row_exp,
             ws.row_gate};
  if (which == 0)
    lol_launch((k_norm<act_t, true, NCH>), dim3((p.cfg.W + 3) / 4, p.n_slots), dim3(256), 0, st, s,
                       ws.row_exp, lib.g_attn, fg, fb, reinterpret_cast<act_t *>(ws.u), n_rows,
                       p.cfg.d, p.cfg.rms_eps, panel_rows, film_stride, nw);
  else
    lol_launch((k_norm<act_t, false, NCH>), dim3((p.T + 3) / 4), dim3(256), 0, st, ws.h,
                       ws.row_exp, lib.g_ffn, fg, fb, reinterpret_cast<act_t *>(ws.u), n_rows,
                       p.cfg.d, p.cfg.rms_eps, panel_rows, film_stride, nw);
}

template <typename act_t>
hipError_t norm_typed(const Plan &p, int which, const float *s, const lol_library &lib,
                      const Workspace &ws, int depth, int delta, int panel_rows, hipStream_t st) {
  const int d = p.cfg.d;
  // FiLM rows of (depth, sublayer): [D][2][d], or [D][L][2][d] per expert
  // (then the kernel adds expert * 2d)
  const size_t film_off = ((size_t)depth * (lib.film_per_expert ? p.cfg.L : 1) * 2 + which) * d;
  const float *fg = lib.film_gamma ? lib.film_gamma + film_off : nullptr;
  const float *fb = lib.film_beta ? lib.film_beta + film_off : nullptr;
  switch ((d % 256 == 0) ? d / 256 : 0) {
    case 1: norm_launch<act_t, 1>(p, which, s, lib, ws, fg, fb, panel_rows, delta, st); break;
    case 2: norm_launch<act_t, 2>(p, which, s, lib, ws, fg, fb, panel_rows, delta, st); break;
    case 3: norm_launch<act_t, 3>(p, which, s, lib, ws, fg, fb, panel_rows, delta, st); break;
    case 4: norm_launch<act_t, 4>(p, which, s, lib, ws, fg, fb, panel_rows, delta, st); break;
    case 5: norm_launch<act_t, 5>(p, which, s, lib, ws, fg, fb, panel_rows, delta, st); break;
    case 6: norm_launch<act_t, 6>(p, which, s, lib, ws, fg, fb, panel_rows, delta, st); break;
    case 7: norm_launch<act_t, 7>(p, which, s, lib, ws, fg, fb, panel_rows, delta, st); break;
    case 8: norm_launch<act_t, 8>(p, which, s, lib, ws, fg, fb, panel_rows, delta, st); break;
    default: norm_launch<act_t, 0>(p, which, s, lib, ws, fg, fb, panel_rows, delta, st); break;
  }
  return hipGetLastError();
}

template <typename act_t, int DH>
hipError_t attn_typed(const Plan &p, const DepthGeom &g, const Workspace &ws, hipStream_t st) {
  dim3 grid(p.n_slots, p.cfg.n_heads, (p.cfg.W + 63) / 64);
  const float scale = 1.0f / sqrtf((float)DH);
  lol_launch((k_attn_simt<act_t, DH>), grid, dim3(64), 0, st,
                     reinterpret_cast<const act_t *>(ws.qkv), reinterpret_cast<act_t *>(ws.o),
                     ws.win_exp, ws.win_row0, ws.win_len, ws.rope_cs, p.cfg.d, scale,
                     p.cfg.rope_theta != 0.f ? 1 : 0);
  return hipGetLastError();
}

template <int DH>
hipError_t attn_mfma(const Plan &p, const DepthGeom &g, const Workspace &ws, int o_panel_rows,
                     hipStream_t st) {
  dim3 grid(p.n_slots, p.cfg.n_heads, (p.cfg.W + 255) / 256);
  // scores come out in log2 units: softmax uses exp2
  const float qscale = 1.4426950408889634f / sqrtf((float)DH);
  lol_launch((k_attn_mfma<DH>), grid, dim3(256), 0, st,
                     reinterpret_cast<const bf16_t *>(ws.qkv), reinterpret_cast<bf16_t *>(ws.o),
                     ws.win_exp, ws.win_row0, ws.win_len, p.cfg.d, qscale, o_panel_rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_norm(const Plan &p, const DepthGeom &g, int which, const float *s,
                       const lol_library &lib, const Workspace &ws, int panel_rows, hipStream_t st) {
  if (panel_rows && (p.cfg.dtype != LOL_BF16 || p.cfg.d % 32 != 0)) return hipErrorInvalidValue;
  if (p.cfg.dtype == LOL_BF16)
    return norm_typed<bf16_t>(p, which, s, lib, ws, g.depth, g.delta, panel_rows, st);
  return norm_typed<float>(p, which, s, lib, ws, g.depth, g.delta, 0, st);
}

hipError_t launch_attention(const Plan &p, const DepthGeom &g, const Workspace &ws, int o_panel_rows,
                            hipStream_t st) {
  if (p.cfg.dtype == LOL_BF16)
    return p.d_head == 64 ? attn_mfma<64>(p, g, ws, o_panel_rows, st)
                          : attn_mfma<32>(p, g, ws, o_panel_rows, st);
  if (o_panel_rows) return hipErrorInvalidValue;   // fp32 mode keeps o row-major
  return p.d_head == 64 ? attn_typed<float, 64>(p, g, ws, st) : attn_typed<float, 32>(p, g, ws, st);
}

}  // namespace lol
