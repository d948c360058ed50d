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
// bf16 MFMA kernel: tile 128 (rows) x 128 (weight rows) x 64 (k), 4 waves in
// a 2 x 2 grid, each wave 64 x 64 outputs as 2 x 2 blocks of 32 x 32.
// ---------------------------------------------------------------------------
constexpr int BM = kTileM;  // 128
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row (144 B): conflict-free 16-B fragment reads

template <int EPI>
__global__ void __launch_bounds__(256) k_gemm_bf16(GemmParams P) {
  __shared__ __attribute__((aligned(16))) bf16_t As[BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[BN * LDK];
  const int mt = blockIdx.x / P.n_tiles_n, nt = blockIdx.x % P.n_tiles_n;
  const int e = P.mtile[2 * mt];
  if (e < 0) return;
  const int row0 = P.mtile[2 * mt + 1];
  const int row_end = P.toff[e + 1];
  const int K = P.K;
  const bf16_t *A = reinterpret_cast<const bf16_t *>(P.A);
  const bf16_t *Wt = reinterpret_cast<const bf16_t *>(P.Wt) + (size_t)e * P.w_stride;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  // global -> register staging: 4 x 16 B of A and of B per thread per k-step
  const bf16_t *a_src[4];
  const bf16_t *b_src[4];
  int lds_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int v = tid + i * 256, r = v >> 3, kv = v & 7;
    const int arow = min(row0 + r, row_end - 1);
    a_src[i] = A + (size_t)arow * K + kv * 8;
    int wrow;
    if (EPI == EPI_SWIGLU) {
      const int wc = r >> 6, within = r & 63;
      const int hidden = nt * 64 + wc * 32 + (within & 31);
      wrow = (within < 32 ? 0 : P.glu_offset) + hidden;
    } else {
      wrow = nt * BN + r;
    }
    b_src[i] = Wt + (size_t)wrow * K + kv * 8;
    lds_off[i] = r * LDK + kv * 8;
  }
  uint4 ra[4], rb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = *reinterpret_cast<const uint4 *>(a_src[i]);
    rb[i] = *reinterpret_cast<const uint4 *>(b_src[i]);
  }
  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  const int frow = lane & 31, fk = (lane >> 5) * 8;
  for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint4 *>(&As[lds_off[i]]) = ra[i];
      *reinterpret_cast<uint4 *>(&Bs[lds_off[i]]) = rb[i];
    }
    __syncthreads();
    if (k0 + BK < K) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = *reinterpret_cast<const uint4 *>(a_src[i] + k0 + BK);
        rb[i] = *reinterpret_cast<const uint4 *>(b_src[i] + k0 + BK);
      }
    }
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 fw[2], fx[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fw[i] = *reinterpret_cast<const bf16x8 *>(&Bs[(wn * 64 + i * 32 + frow) * LDK + kk + fk]);
        fx[i] = *reinterpret_cast<const bf16x8 *>(&As[(wm * 64 + i * 32 + frow) * LDK + kk + fk]);
      }
#pragma unroll
      for (int in = 0; in < 2; ++in)
#pragma unroll
        for (int im = 0; im < 2; ++im)
          acc[in][im] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[in], fx[im], acc[in][im], 0, 0, 0);
    }
    __syncthreads();
  }

  // lane holds C[m = im*32 + lane%32][n = in*32 + g*8 + 4*(lane/32) + j], g, j < 4
  const int cq = (lane >> 5) * 4;
#pragma unroll
  for (int im = 0; im < 2; ++im) {
    const int row = row0 + wm * 64 + im * 32 + (lane & 31);
    if (row >= row_end) continue;
    if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int hcol = nt * 64 + wn * 32 + g * 8 + cq;
        float gv[4], uv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) { gv[j] = acc[0][im][g * 4 + j]; uv[j] = acc[1][im][g * 4 + j]; }
        store_glu4<bf16_t>(P, row, hcol, gv, uv);
      }
    } else {
#pragma unroll
      for (int in = 0; in < 2; ++in)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = nt * BN + wn * 64 + in * 32 + g * 8 + cq;
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
    const int cols_per_tile = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
    P.n_tiles_n = a.N / cols_per_tile;
    hipLaunchKernelGGL(k_gemm_bf16<EPI>, dim3(ws.max_mtiles * P.n_tiles_n), dim3(256), 0, st, P);
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
