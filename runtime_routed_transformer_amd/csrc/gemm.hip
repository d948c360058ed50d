// Grouped expert GEMMs of the routed core, with fused epilogues.
//
// Every library block's projections (paper "Library of Layers (LoL)",
// App. A: bias-free attention, SwiGLU MLP; the GELU variant is the tiny
// workload's two-matrix MLP) run as one grouped GEMM per projection over all
// windows of a depth: windows routed to the same expert form one contiguous
// range of grouped rows (bucketing), and each M tile of kTileM rows belongs
// to one expert.  C[m][n] = sum_k A[m][k] * W_e[n][k]; both operands are
// contiguous along k.
//
// bf16 mode: v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  The weight
// tile is the MFMA's A operand and the activation tile its B operand, so each
// lane ends with 4 consecutive output columns of one row (vector stores), and
// a SwiGLU tile interleaves gate and up rows so that each lane holds both
// halves of its hidden columns.
// fp32 mode: an LDS-tiled FMA kernel with the same tiles and epilogues.
#include <math.h>

#include "lol_internal.h"

namespace lol {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }
__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

struct GemmParams {
  const void *A;
  const void *Wt;
  long long w_stride;
  int N;          // logical output columns
  int K;
  int ldc;        // row stride of the output
  int glu_offset;
  int n_tiles_n;
  const int32_t *mtile;
  const int32_t *toff;
  const int32_t *row_tok;
  const float *row_gate;
  void *C;
  float *s;
  const float *h;
};

// Writes 4 consecutive logical columns [col, col+4) of grouped row `row`.
template <int EPI, typename act_t>
__device__ __forceinline__ void epilogue4(const GemmParams &P, int row, int col, float v0, float v1,
                                          float v2, float v3) {
  if (EPI == EPI_STORE || EPI == EPI_GELU) {
    if (EPI == EPI_GELU) { v0 = gelu_erf(v0); v1 = gelu_erf(v1); v2 = gelu_erf(v2); v3 = gelu_erf(v3); }
    act_t *C = reinterpret_cast<act_t *>(P.C) + (size_t)row * P.ldc + col;
    if (sizeof(act_t) == 2) {
      uint2 pk;
      pk.x = (uint32_t)f2bf(v0) | ((uint32_t)f2bf(v1) << 16);
      pk.y = (uint32_t)f2bf(v2) | ((uint32_t)f2bf(v3) << 16);
      *reinterpret_cast<uint2 *>(C) = pk;
    } else {
      *reinterpret_cast<float4 *>(C) = make_float4(v0, v1, v2, v3);
    }
  } else if (EPI == EPI_RESID) {
    const size_t tok = (size_t)P.row_tok[row];
    const float4 x = *reinterpret_cast<const float4 *>(P.s + tok * P.ldc + col);
    *reinterpret_cast<float4 *>(reinterpret_cast<float *>(P.C) + (size_t)row * P.ldc + col) =
        make_float4(x.x + v0, x.y + v1, x.z + v2, x.w + v3);
  } else if (EPI == EPI_BLEND) {
    const size_t tok = (size_t)P.row_tok[row];
    const float g = P.row_gate[row];
    float4 *sp = reinterpret_cast<float4 *>(P.s + tok * P.ldc + col);
    const float4 x = *sp;
    const float4 hv = *reinterpret_cast<const float4 *>(P.h + (size_t)row * P.ldc + col);
    *sp = make_float4(x.x + g * (hv.x + v0 - x.x), x.y + g * (hv.y + v1 - x.y),
                      x.z + g * (hv.z + v2 - x.z), x.w + g * (hv.w + v3 - x.w));
  }
}

template <typename act_t>
__device__ __forceinline__ void store_glu4(const GemmParams &P, int row, int col, const float *g,
                                           const float *u) {
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = silu(g[j]) * u[j];
  epilogue4<EPI_STORE, act_t>(P, row, col, v[0], v[1], v[2], v[3]);
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel.  4 waves in a 2 x 2 grid; each wave owns TM x TN blocks of
// 32 x 32 outputs, so the block tile is (64 TM) x (64 TN) and k advances by
// BK = 64 per stage.  Stage k+1 is fetched from global memory into registers
// while stage k is multiplied out of one of two LDS buffers; one barrier per
// stage.
// ---------------------------------------------------------------------------
constexpr int BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row (144 B): conflict-free 16-B fragment reads

template <int EPI, int TM, int TN>
__global__ void __launch_bounds__(256) k_gemm_bf16(GemmParams P) {
  constexpr int BMt = 64 * TM, BNt = 64 * TN;
  constexpr int AV = BMt / 32, BV = BNt / 32;  // 16-byte vectors per thread per stage
  constexpr int STAGE = (BMt + BNt) * LDK;     // elements per LDS buffer
  extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
  const int mt = blockIdx.x / P.n_tiles_n, nt = blockIdx.x % P.n_tiles_n;
  const int e = P.mtile[2 * mt];
  if (e < 0) return;
  const int row0 = P.mtile[2 * mt + 1];
  const int row_end = P.toff[e + 1];
  const int K = P.K;
  const bf16_t *A = reinterpret_cast<const bf16_t *>(P.A);
  const bf16_t *Wt = reinterpret_cast<const bf16_t *>(P.Wt) + (size_t)e * P.w_stride;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int kv = tid & 7, r_base = tid >> 3;  // each thread: one 16-byte chunk of rows r_base + 32 i

  const bf16_t *a_src[AV];
  const bf16_t *b_src[BV];
#pragma unroll
  for (int i = 0; i < AV; ++i) {
    const int arow = min(row0 + r_base + 32 * i, row_end - 1);
    a_src[i] = A + (size_t)arow * K + kv * 8;
  }
#pragma unroll
  for (int i = 0; i < BV; ++i) {
    const int r = r_base + 32 * i;
    int wrow;
    if (EPI == EPI_SWIGLU) {
      constexpr int WR = TN * 32, HALF = TN * 16;  // weight rows per wave column, gate half
      const int wc = r / WR, within = r % WR;
      const int hidden = nt * (BNt / 2) + wc * HALF + (within % HALF);
      wrow = (within < HALF ? 0 : P.glu_offset) + hidden;
    } else {
      wrow = nt * BNt + r;
    }
    b_src[i] = Wt + (size_t)wrow * K + kv * 8;
  }
  uint4 ra[AV], rb[BV];
#pragma unroll
  for (int i = 0; i < AV; ++i) ra[i] = *reinterpret_cast<const uint4 *>(a_src[i]);
#pragma unroll
  for (int i = 0; i < BV; ++i) rb[i] = *reinterpret_cast<const uint4 *>(b_src[i]);
  {
    bf16_t *As = smem, *Bs = smem + BMt * LDK;
#pragma unroll
    for (int i = 0; i < AV; ++i) *reinterpret_cast<uint4 *>(&As[(r_base + 32 * i) * LDK + kv * 8]) = ra[i];
#pragma unroll
    for (int i = 0; i < BV; ++i) *reinterpret_cast<uint4 *>(&Bs[(r_base + 32 * i) * LDK + kv * 8]) = rb[i];
  }
  __syncthreads();

  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  const int frow = lane & 31, fk = (lane >> 5) * 8;
  const int nk = K / BK;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    // prefetch stage kt+1 (the last iteration re-reads the final stage, unused)
    const int knext = min(kt + 1, nk - 1) * BK;
#pragma unroll
    for (int i = 0; i < AV; ++i) ra[i] = *reinterpret_cast<const uint4 *>(a_src[i] + knext);
#pragma unroll
    for (int i = 0; i < BV; ++i) rb[i] = *reinterpret_cast<const uint4 *>(b_src[i] + knext);
    const bf16_t *As = smem + cur * STAGE, *Bs = As + BMt * LDK;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 fw[TN], fx[TM];
#pragma unroll
      for (int i = 0; i < TN; ++i)
        fw[i] = *reinterpret_cast<const bf16x8 *>(&Bs[(wn * TN * 32 + i * 32 + frow) * LDK + kk + fk]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fx[i] = *reinterpret_cast<const bf16x8 *>(&As[(wm * TM * 32 + i * 32 + frow) * LDK + kk + fk]);
#pragma unroll
      for (int in = 0; in < TN; ++in)
#pragma unroll
        for (int im = 0; im < TM; ++im)
          acc[in][im] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[in], fx[im], acc[in][im], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      bf16_t *An = smem + (cur ^ 1) * STAGE, *Bn = An + BMt * LDK;
#pragma unroll
      for (int i = 0; i < AV; ++i) *reinterpret_cast<uint4 *>(&An[(r_base + 32 * i) * LDK + kv * 8]) = ra[i];
#pragma unroll
      for (int i = 0; i < BV; ++i) *reinterpret_cast<uint4 *>(&Bn[(r_base + 32 * i) * LDK + kv * 8]) = rb[i];
    }
    __syncthreads();
  }

  // lane holds C[m = im*32 + lane%32][n = in*32 + g*8 + 4*(lane/32) + j], g, j < 4
  const int cq = (lane >> 5) * 4;
#pragma unroll
  for (int im = 0; im < TM; ++im) {
    const int row = row0 + wm * TM * 32 + im * 32 + (lane & 31);
    if (row >= row_end) continue;
    if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int in = 0; in < TN / 2; ++in)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int hcol = nt * (BNt / 2) + wn * TN * 16 + in * 32 + g * 8 + cq;
          float gv[4], uv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            gv[j] = acc[in][im][g * 4 + j];
            uv[j] = acc[in + TN / 2][im][g * 4 + j];
          }
          store_glu4<bf16_t>(P, row, hcol, gv, uv);
        }
    } else {
#pragma unroll
      for (int in = 0; in < TN; ++in)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = nt * BNt + wn * TN * 32 + in * 32 + g * 8 + cq;
          epilogue4<EPI, bf16_t>(P, row, col, acc[in][im][g * 4], acc[in][im][g * 4 + 1],
                                 acc[in][im][g * 4 + 2], acc[in][im][g * 4 + 3]);
        }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel: tile 128 rows x 64 logical columns x 16 k; each thread
// computes 8 rows x 4 columns (x2 for SwiGLU: gate and up).
// ---------------------------------------------------------------------------
constexpr int BM = kTileM;  // 128 rows per fp32 tile
constexpr int FBN = 64;
constexpr int FBK = 16;

template <int EPI>
__global__ void __launch_bounds__(256) k_gemm_f32(GemmParams P) {
  constexpr int NB = (EPI == EPI_SWIGLU) ? 2 * FBN : FBN;  // weight rows per tile
  __shared__ float As[FBK][BM + 4];
  __shared__ float Bs[FBK][NB + 4];
  const int mt = blockIdx.x / P.n_tiles_n, nt = blockIdx.x % P.n_tiles_n;
  const int e = P.mtile[2 * mt];
  if (e < 0) return;
  const int row0 = P.mtile[2 * mt + 1];
  const int row_end = P.toff[e + 1];
  const int K = P.K;
  const float *A = reinterpret_cast<const float *>(P.A);
  const float *Wt = reinterpret_cast<const float *>(P.Wt) + (size_t)e * P.w_stride;
  const int tid = threadIdx.x;
  const int tm = tid >> 4, tn = tid & 15;  // 16 row groups of 8, 16 column groups of 4
  float acc[8][4], accu[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) { acc[i][j] = 0.f; accu[i][j] = 0.f; }

  for (int k0 = 0; k0 < K; k0 += FBK) {
    // A: 128 rows x 16 k = 512 float4, two per thread
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = tid + i * 256, r = v >> 2, kq = (v & 3) * 4;
      const int arow = min(row0 + r, row_end - 1);
      const float4 x = *reinterpret_cast<const float4 *>(A + (size_t)arow * K + k0 + kq);
      As[kq][r] = x.x; As[kq + 1][r] = x.y; As[kq + 2][r] = x.z; As[kq + 3][r] = x.w;
    }
    for (int v = tid; v < NB * 4; v += 256) {
      const int r = v >> 2, kq = (v & 3) * 4;
      int wrow;
      if (EPI == EPI_SWIGLU)
        wrow = (r < FBN ? nt * FBN + r : P.glu_offset + nt * FBN + (r - FBN));
      else
        wrow = nt * FBN + r;
      const float4 x = *reinterpret_cast<const float4 *>(Wt + (size_t)wrow * K + k0 + kq);
      Bs[kq][r] = x.x; Bs[kq + 1][r] = x.y; Bs[kq + 2][r] = x.z; Bs[kq + 3][r] = x.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      float a[8], b[4], bu[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] = As[kk][tm * 8 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tn * 4 + j];
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int j = 0; j < 4; ++j) bu[j] = Bs[kk][FBN + tn * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
          if (EPI == EPI_SWIGLU) accu[i][j] = fmaf(a[i], bu[j], accu[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = row0 + tm * 8 + i;
    if (row >= row_end) continue;
    const int col = nt * FBN + tn * 4;
    if (EPI == EPI_SWIGLU)
      store_glu4<float>(P, row, col, acc[i], accu[i]);
    else
      epilogue4<EPI, float>(P, row, col, acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
  }
}

template <int EPI>
hipError_t launch_typed(const Plan &p, const Workspace &ws, const GemmArgs &a, hipStream_t st) {
  GemmParams P;
  P.A = a.A;
  P.Wt = a.Wt;
  P.w_stride = a.w_expert_stride;
  P.N = a.N;
  P.K = a.K;
  P.ldc = a.N;
  P.glu_offset = a.glu_offset;
  P.mtile = ws.mtile;
  P.toff = ws.toff;
  P.row_tok = ws.row_tok;
  P.row_gate = ws.row_gate;
  P.C = a.C;
  P.s = a.s;
  P.h = a.h;
  if (p.cfg.dtype == LOL_BF16) {
    // 256 x 256 tiles for the wide projections (QKV, gate/up); 256 x 128 for
    // the d-wide ones (O, down), which otherwise leave CUs idle in the tail
    const bool wide = (EPI == EPI_SWIGLU ? 2 * a.N : a.N) >= 2048;
    if (wide && a.N % (EPI == EPI_SWIGLU ? 128 : 256) == 0) {
      constexpr int TM = 4, TN = 4;
      P.mtile = ws.mtile2;
      P.n_tiles_n = (EPI == EPI_SWIGLU) ? a.N / (32 * TN) : a.N / (64 * TN);
      const size_t smem = 2 * (size_t)(64 * TM + 64 * TN) * LDK * sizeof(bf16_t);
      hipFuncSetAttribute((const void *)k_gemm_bf16<EPI, TM, TN>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
      hipLaunchKernelGGL((k_gemm_bf16<EPI, TM, TN>), dim3(ws.max_mtiles2 * P.n_tiles_n), dim3(256),
                         smem, st, P);
    } else {
      constexpr int TM = 4, TN = 2;
      P.mtile = ws.mtile2;
      P.n_tiles_n = (EPI == EPI_SWIGLU) ? a.N / (32 * TN) : a.N / (64 * TN);
      const size_t smem = 2 * (size_t)(64 * TM + 64 * TN) * LDK * sizeof(bf16_t);
      hipFuncSetAttribute((const void *)k_gemm_bf16<EPI, TM, TN>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
      hipLaunchKernelGGL((k_gemm_bf16<EPI, TM, TN>), dim3(ws.max_mtiles2 * P.n_tiles_n), dim3(256),
                         smem, st, P);
    }
  } else {
    P.n_tiles_n = a.N / FBN;
    hipLaunchKernelGGL(k_gemm_f32<EPI>, dim3(ws.max_mtiles * P.n_tiles_n), dim3(256), 0, st, P);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const Plan &p, const Workspace &ws, const GemmArgs &a, hipStream_t st) {
  switch (a.epi) {
    case EPI_STORE: return launch_typed<EPI_STORE>(p, ws, a, st);
    case EPI_RESID: return launch_typed<EPI_RESID>(p, ws, a, st);
    case EPI_SWIGLU: return launch_typed<EPI_SWIGLU>(p, ws, a, st);
    case EPI_GELU: return launch_typed<EPI_GELU>(p, ws, a, st);
    case EPI_BLEND: return launch_typed<EPI_BLEND>(p, ws, a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace lol
