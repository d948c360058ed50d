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

#include <type_traits>

#include "lol_internal.h"

namespace lol {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

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
  const int32_t *mcount;   // [0]: M tiles in use in mtile
  const int32_t *toff;
  const int32_t *row_tok;
  const float *row_gate;
  void *C;
  const float *s_in;       // residual stream read (RESID, BLEND)
  float *s;                // residual stream written (BLEND)
  const float *h;
  const int32_t *row_pos;  // QKV_ROPE: window-local position of each grouped row
  const float *rope_cs;    // QKV_ROPE: [W][half][2] cos, sin of p * theta^(-2j/d_head)
  int rope_cols;           // QKV_ROPE: columns [0, rope_cols) hold q and k
  int half;                // QKV_ROPE: d_head / 2
  float rope_log2_theta;   // QKV_ROPE: log2 of the RoPE base
  int a_panel_rows;        // 0: A is [rows][K]; else A is in 32-k panels [K/32][a_panel_rows][32]
  int b_panel_rows;        // 0: an expert's weights are [N_w][K]; else 32-k panels [K/32][N_w][32]
  int c_panel_rows;        // bf16 store epilogues: 0 = C is [rows][ldc]; else 32-column panels
  int gm;                  // m-tiles per group of the tile order (see "Tile order")
  float *part;             // K-split tail (EPI_ACCUM, 256 x 256): fp32 partial tiles [part_slots][256][256]
  int part_slots;          // 0: tail tiles are not split
};

// Writes 4 consecutive logical columns [col, col+4) of grouped row `row`.
template <int EPI, typename act_t>
__device__ __forceinline__ void epilogue4(const GemmParams &P, int row, int col, float v0, float v1,
                                          float v2, float v3) {
  if (EPI == EPI_STORE || EPI == EPI_GELU || EPI == EPI_QKV_ROPE) {
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
    const float4 x = *reinterpret_cast<const float4 *>(P.s_in + tok * P.ldc + col);
    *reinterpret_cast<float4 *>(reinterpret_cast<float *>(P.C) + (size_t)row * P.ldc + col) =
        make_float4(x.x + v0, x.y + v1, x.z + v2, x.w + v3);
  } else if (EPI == EPI_BLEND) {
    const size_t tok = (size_t)P.row_tok[row];
    const float g = P.row_gate[row];
    float4 *sp = reinterpret_cast<float4 *>(P.s + tok * P.ldc + col);
    const float4 x = *reinterpret_cast<const float4 *>(P.s_in + tok * P.ldc + col);
    const float4 hv = *reinterpret_cast<const float4 *>(P.h + (size_t)row * P.ldc + col);
    *sp = make_float4(x.x + g * (hv.x + v0 - x.x), x.y + g * (hv.y + v1 - x.y),
                      x.z + g * (hv.z + v2 - x.z), x.w + g * (hv.w + v3 - x.w));
  } else if (EPI == EPI_ACCUM) {
    const size_t tok = (size_t)P.row_tok[row];
    const float g = P.row_gate[row];
    const float4 x = *reinterpret_cast<const float4 *>(P.s_in + tok * P.ldc + col);
    *reinterpret_cast<float4 *>(P.s + tok * P.ldc + col) =
        make_float4(x.x + g * v0, x.y + g * v1, x.z + g * v2, x.w + g * v3);
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
// bf16 MFMA kernel.  A workgroup of WM x WN waves computes one tile (rows x
// output columns of W); each wave owns 128 x 64 outputs as 16 x 16 blocks of
// v_mfma_f32_16x16x32_bf16, or 64 x 64 as 32 x 32 blocks of
// v_mfma_f32_32x32x16_bf16 in the small-problem shapes (the shape table
// below).
//
// Main loop: k advances by BK = 32 per stage through a ring of NSTAGE LDS
// stages filled by direct global-to-LDS loads (16 bytes per lane, no
// register staging).  Fragment reads of the next stage start right after
// the stage barrier, under the MFMAs of the current one.
//
// LDS layout of one operand in one stage: rows of 32 k = 64 bytes, four
// 16-byte chunks per row; logical chunk c of row r sits at chunk
// c ^ swz(r), swz(r) = (r >> 2) & 3.  One load instruction fills 16
// consecutive rows (1 KiB); the swizzle is applied on the global side (each
// lane picks which chunk of its row to fetch).  A fragment read has every
// quarter-wave read one logical chunk of 16 consecutive rows; with the
// swizzle these 16 lanes cover all 64 four-byte banks.  The read runs at
// the full rate (4 clocks per 128-bit instruction, measured) only when, in
// addition, lanes l and l + 16 read 16-byte slots whose index XOR has even
// parity; an odd XOR costs 2 more clocks per half-wave.  The 32 x 32
// fragments (lanes l and l + 16 read the same chunk of rows 16 apart)
// satisfy this as they are; the 16 x 16 fragments order their k-chunks
// for it.
//
// Epilogue: each wave stages 32 rows of its results at a time in LDS (fp32,
// XOR-swizzled 16-byte slots) and reads them back row-wise, so that every
// global access of the epilogue (bf16 stores, residual reads and writes) is
// a run of 8 consecutive columns per lane and whole rows per group of lanes.
//
// Persistent tiles (256 x 256 shape, one workgroup per CU): the workgroup
// walks its XCD's range of tiles.  After a tile's main loop it requests the
// next tile's first two stages into two ring slots, then runs the epilogue
// through the other two, so the next tile's first loads travel under the
// epilogue (measured about 1% faster than one tile per workgroup).
//
// Tile order: tiles are numbered (m-tile, n-tile) in groups of GM m-tiles
// (n-tile major inside a group) and dealt to the 8 XCDs in contiguous
// ranges (workgroup i runs on XCD i mod 8), so that tiles sharing an A or B
// slice run close together in time on one XCD's L2.
//
// Mixed tiles (2 x 4 shape, gate/up): where every expert's row count is a
// multiple of 128 but not of 256, an expert's last 256-row m-tile holds 128
// rows, and a 256 x 256 tile of it leaves one wave row idle: such tiles
// formed a partial extra round.  The mixed variant runs the full m-tiles as
// 256 x 256 tiles and each half-filled one as "wide" 128 x 512 tiles, both
// wave rows on its 128 activation rows and each on its own 256 weight rows
// (n-tiles 2 nt and 2 nt + 1): the same MACs per tile, so the number of
// rounds is that of the aligned depths.  A stage slot holds 128 + 512 rows
// (40 KiB): pieces 0-7 are A rows 0-127, 8-15 A rows 128-255 or B rows
// 0-127, 16-31 B rows 0-255 or 128-383, 32-39 (wide only) B rows 384-511;
// every loading wave issues ten pieces per stage either way, a 256 x 256
// tile's last two through a buffer resource with no records (nothing is
// read), so the stage wait counts are the same for both kinds.
// ---------------------------------------------------------------------------
constexpr int TN = 2;                   // 32-wide units per wave along N (64 output columns)
constexpr int BK = 32;
// m-tiles per group: 2 for every projection.  With row-major weights 4 was
// as fast for the wide ones (8,192 weight rows and more) and moved less
// L2-miss traffic; with the weights in 32-k panels 2 is faster there too
// (same-box A/B at mid_bf16, two runs each: 3.493 / 3.493 M tokens/s
// against 3.482 / 3.485 with 4 for gate/up and 3.485 / 3.491 with 8;
// gate/up at the unshifted depths 205-210 against 209-218 us with 4; 4 for
// every projection 3.473, and 1 for the narrow ones 3.482)
constexpr int GM = 2;
// Four shapes of workgroup, WM x WN waves:
//   2 x 2: 256 x 128 tile, 4 waves, 3-stage ring of 72 KiB, two per CU;
//   2 x 4: 256 x 256 tile, 8 waves, 4-stage ring of 128 KiB, one per CU
//          (persistent); its mixed variant also runs 128 x 512 tiles, with
//          a 4-stage ring of 160 KiB (see "Mixed tiles");
//   1 x 4: 128 x 256 tile, 4 waves, 3-stage ring of 72 KiB, two per CU;
//   1 x 8: 128 x 512 tile, 8 waves, 4-stage ring of 160 KiB (all of the
//          LDS), one per CU (persistent);
//   2 x 2 with 64 x 64 per wave (TM = 2): 128 x 128 tile, 4 waves, 3-stage
//          ring of 48 KiB, three per CU, for problems too small to fill the
//          CUs with larger tiles: all four SIMDs of a CU work even when
//          there is one tile per CU (small_bf16's down projection, 256
//          tiles, ran on two-wave 128 x 128 tiles with two SIMDs idle).
// Every other shape gives each wave 128 x 64 outputs (TM = 4): 2 x 2 and
// 1 x 4 move the same bytes per MAC; 1 x 4 and 1 x 8 use the 128-row tile
// tables, which fit expert row counts that are multiples of 128 without a
// partial tile, and 1 x 8 loads 1.25x the stage bytes of 2 x 4 per MAC
// where two 1 x 4 workgroups load 1.5x.
// NSV > 0 overrides the ring depth (and gives the workgroup the CU alone):
// the 128 x 128 shape with an 8-stage ring for problems with at most one
// tile per CU, where a stage's matrix work (256 clocks per wave) is far
// shorter than a load's latency and only a deep ring keeps it fed.
// MXV != 0: the 2 x 4 shape that also runs "wide" tiles, 128 x 512: both
// wave rows on the same 128 activation rows, each on its own 256 weight rows
// (see "Mixed tiles"); its stage slots hold 128 + 512 rows (40 KiB).
template <int WM, int WN, int TMV = 4, int NSV = 0, int MXV = 0> struct Shape {
  static constexpr int TM = TMV;                         // 32-row units per wave along M
  static constexpr int NW = WM * WN;                     // waves
  static constexpr int BMT = 32 * TM * WM;               // rows of A per tile
  static constexpr int BNT = 32 * TN * WN;               // weight rows per tile
  static constexpr int NSTAGE = NSV ? NSV : (NW == 8 ? 4 : 3);
  static constexpr bool MIX = MXV != 0;
  static_assert(!MIX || (WM == 2 && WN == 4 && TMV == 4 && NSV == 0), "mixed tiles: the 2 x 4 shape");
  static constexpr int STAGE_BYTES = MIX ? (kTileM + 2 * BNT) * BK * 2 : (BMT + BNT) * BK * 2;
  static constexpr int LDS = NSTAGE * STAGE_BYTES;
  static constexpr int PER_CU = NSV ? 1 : NW == 8 ? 1 : (TM == 2 ? 3 : 2);
  // one workgroup per CU walks a range of tiles (see "Persistent tiles")
  static constexpr bool PERSIST = NW == 8;
  static_assert(BMT == kTileM || BMT == kTileM2, "M tiles come from the 128- or 256-row tables");
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }

// Direct global-to-LDS load of 16 bytes per lane through a buffer resource:
// per-lane byte offset voff plus a wave-uniform byte offset soff, so that a
// stage needs no per-lane 64-bit address arithmetic
constexpr int kBufferFlags = 0x00020000;   // raw buffer, 32-bit data format, no swizzle
__device__ __forceinline__ void lds_dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, void *lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds, 16, (int)voff, soff, 0, 0);
}

// Stage barrier: wait until at most VM vector-memory operations (the
// direct-to-LDS stage loads) and LG LDS operations of this wave are in flight,
// then s_barrier.  Built from the compiler's own intrinsics so that its
// wait-count tracking knows about them; the empty asm statements keep memory
// accesses from being moved across, and the scheduling barriers keep the
// MFMA blocks on their side.
template <int VM, int LG>
__device__ __forceinline__ void stage_barrier() {
  static_assert(VM >= 0 && VM < 64 && LG >= 0 && LG < 16, "counter range");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LG << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Scheduling hint for "NR fragment reads (for the next step), then NM MFMAs
// (on fragments already in registers)": every read first, so that each has
// the whole MFMA block to arrive.
template <int NR, int NM>
__device__ __forceinline__ void reads_then_mfmas() {
  __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);  // the LDS reads
  __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);  // the MFMAs
}

// Scheduling hint for an MFMA block that also carries N stage loads: N
// groups of "a share of the M MFMAs, then one load".  Issued as one burst
// right after the stage barrier, the loads of all waves queue in the CU's
// memory pipeline together and hold up the MFMAs behind them; spread over
// the block they enter it one at a time (gate/up main loop 57.9 -> 49.7
// kilo-clocks per 256 x 256 tile, down 232 -> 202, same-box probe).
template <int N, int M, int Q = 0>
__device__ __forceinline__ void mfma_load_groups() {
  if constexpr (Q < N) {
    __builtin_amdgcn_sched_group_barrier(0x008, (M * (Q + 1)) / N - (M * Q) / N, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    mfma_load_groups<N, M, Q + 1>();
  }
}

// silu(x) = x / (1 + e^-x) with the hardware exp2 and reciprocal (about one
// ulp each, far below the bf16 rounding of the result).
__device__ __forceinline__ float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;  // round to nearest even (v_cvt_pk_bf16_f32)
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// ---- K-split tail (persistent 256 x 256 tiles, the down projection's
// EPI_ACCUM).  A persistent launch runs each XCD's tiles in rounds of one
// tile per workgroup.  Ragged expert row counts (packed documents, windows
// whose lengths are not multiples of 256) add a few partial m-tiles and so
// a short last round that costs nearly a whole tile's time on a handful of
// CUs.  When that round holds at most half the XCD's workgroups, its tiles
// are cut along K into `split` pieces that run side by side: each piece
// stores its fp32 partial tile into a slot of P.part, and k_split_accum then
// sums a tile's pieces in piece order (a fixed order: the result does not
// depend on timing) and applies the epilogue.
constexpr int kSplitMax = 8, kSplitMin = 2;
struct TailSplit {
  int per, nf;      // tiles per XCD range; tiles of this XCD
  int full, tail;   // tiles run whole; tail tiles (the short last round)
  int split, spx;   // pieces per tail tile (1: none); partial slots per XCD
};
__host__ __device__ inline TailSplit tail_split(int R, int xcd, int ustep, int nk, int part_slots) {
  TailSplit t;
  t.per = (R + 7) >> 3;
  const int rest = R - xcd * t.per;
  t.nf = rest < 0 ? 0 : (rest < t.per ? rest : t.per);
  t.tail = t.nf % ustep;
  t.full = t.nf - t.tail;
  t.spx = part_slots >> 3;
  t.split = 1;
  if (t.tail > 0) {
    int sp = ustep / t.tail;
    if (t.spx / t.tail < sp) sp = t.spx / t.tail;
    if (kSplitMax < sp) sp = kSplitMax;
    // whole groups of 4 stages per piece
    while (sp > 1 && (nk % sp != 0 || (nk / sp) % 4 != 0)) --sp;
    t.split = sp < kSplitMin ? 1 : sp;
  }
  if (t.split == 1) t.full = t.nf;
  return t;
}
// m-tile and n-tile of tile t of the tile order (see "Tile order")
__device__ __forceinline__ void tile_mn(int t, int n_mt, int n_nt, int GM_, int &mt, int &nt) {
  const int grp = t / (GM_ * n_nt), within = t - grp * (GM_ * n_nt);
  const int gm = min(GM_, n_mt - grp * GM_);
  mt = grp * GM_ + within % gm;
  nt = within / gm;
}

template <int EPI, int WM, int WN, int TMV, int NSV, int MXV>
__global__ void __launch_bounds__(64 * WM * WN, (Shape<WM, WN, TMV, NSV, MXV>::PER_CU)) k_gemm_bf16(GemmParams P) {
  using S = Shape<WM, WN, TMV, NSV, MXV>;
  constexpr bool MIX = S::MIX;
  constexpr int TM = S::TM;
  constexpr int NW = S::NW, BMT = S::BMT, BNT = S::BNT, NSTAGE = S::NSTAGE;
  constexpr int STAGE_BYTES = S::STAGE_BYTES;
  constexpr int A_BYTES = BMT * BK * 2;
  constexpr int AQ = BMT / 16 / NW, BQ = BNT / 16 / NW;  // 1-KiB load instructions per wave per stage
  constexpr int NQ = AQ + BQ;

  constexpr bool PERSIST = S::PERSIST;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  // ---- tiles of this workgroup (see "Tile order"): unit u of its XCD's
  // range; a persistent workgroup then steps by the workgroups per XCD.
  // Mixed tiles: units [0, nf) are 256 x 256 tiles of the full m-tiles,
  // [nf, nf + nw) wide tiles (n-tiles 2 nt and 2 nt + 1 of a half-filled
  // m-tile), spread evenly over the XCDs.
  const int n_mt = MIX ? P.mcount[1] : P.mcount[0];   // m-tiles run as 256 x 256
  const int n_nt = P.n_tiles_n;
  const int R = n_mt * n_nt;
  const int RW = MIX ? (P.mcount[0] - n_mt) * (n_nt >> 1) : 0;
  const int per = (R + 7) >> 3, perw = (RW + 7) >> 3;
  const int xcd = blockIdx.x & 7;
  const int nf = max(0, min(per, R - xcd * per));
  const int nw = max(0, min(perw, RW - xcd * perw));
  const int ustep = gridDim.x >> 3;
  int u = blockIdx.x >> 3;
  // K-split tail: units [ts.full, ts.full + ts.tail * ts.split) are pieces,
  // piece q = kc * tail + j of tail tile j, in partial slot xcd * spx + q
  constexpr bool SPLIT = EPI == EPI_ACCUM && PERSIST && !MIX && BMT == kTileM2 && BNT == 256;
  const int nk_all = P.K / BK;
  TailSplit ts{};
  ts.full = nf;
  ts.split = 1;
  if constexpr (SPLIT) ts = tail_split(R, xcd, ustep, nk_all, P.part_slots);
  auto locate = [&](int uu, int &mt_, int &nt_, int &e_, int &row0_, int &row_end_, bool &wide_, int &kc_,
                    int &slot_) -> bool {
    wide_ = false;
    kc_ = -1;
    slot_ = 0;
    if (uu < ts.full) {
      tile_mn(xcd * per + uu, n_mt, n_nt, P.gm, mt_, nt_);
    } else if (SPLIT && ts.split > 1 && uu - ts.full < ts.tail * ts.split) {
      const int q = uu - ts.full;
      tile_mn(xcd * per + ts.full + q % ts.tail, n_mt, n_nt, P.gm, mt_, nt_);
      kc_ = q / ts.tail;
      slot_ = xcd * ts.spx + q;
    } else if (MIX && uu - nf < nw) {
      const int h = xcd * perw + uu - nf;
      mt_ = n_mt + h / (n_nt >> 1);
      nt_ = h % (n_nt >> 1);
      wide_ = true;
    } else {
      return false;
    }
    // uniform across the wave (the compiler loses track of it through the
    // tail arithmetic and would take the tile's buffer resources as divergent)
    mt_ = __builtin_amdgcn_readfirstlane(mt_);
    nt_ = __builtin_amdgcn_readfirstlane(nt_);
    e_ = P.mtile[2 * mt_];
    if (e_ < 0) return false;
    row0_ = P.mtile[2 * mt_ + 1];
    row_end_ = P.toff[e_ + 1];
    return true;
  };
  int mt, nt, e, row0, row_end, kc, pslot;
  bool wide;
  if (!locate(u, mt, nt, e, row0, row_end, wide, kc, pslot)) return;
  // stages of the tile (a piece: its share of K, from stage kc * nk)
  auto tile_nk = [&](int kc_) { return kc_ >= 0 ? nk_all / ts.split : nk_all; };
  const int K = P.K;
  const bf16_t *A = reinterpret_cast<const bf16_t *>(P.A);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar LDS addresses

  // ---- per-lane global sources of this wave's load instructions
  const int lrow = lane >> 2, lchunk = lane & 3;
  // sources: a per-tile base (wave-uniform) plus a 32-bit element offset per
  // lane and load instruction
  // buffer resources (base = this tile's first A row / its expert's weights;
  // 2^32 - 1 bytes of range, the offsets stay inside the operands) and
  // per-lane byte offsets; a stage adds a scalar offset
  __amdgpu_buffer_rsrc_t a_rsrc, b_rsrc;
  // Persistent 8-wave shapes: only the first wave of each SIMD (waves
  // 0 .. NW/2-1) issues the stage loads, twice as many each.  The issue
  // arbiter favours the older of a SIMD's two waves, which reaches every
  // stage barrier about a third of a stage before the younger (clock
  // stamps); with the loads moved to it the two arrive closer together
  // (measured 1-2% faster).
  constexpr bool LB = PERSIST && TM == 4;
  constexpr int LW = LB ? NW / 2 : NW;
  constexpr int LAQ = LB ? 2 * AQ : AQ, LBQ = LB ? 2 * BQ : BQ;
  // mixed tiles: ten 1 KiB pieces per loading wave and stage, piece
  // p = wave + 4 i of the 40 KiB slot (see "Mixed tiles")
  constexpr int LNQ = MIX ? 10 : LAQ + LBQ;
  const bool loader = !LB || wave < LW;
  uint32_t soff[LNQ];
  bool ld_wide = false;   // the tile whose stages are being loaded is wide
  __amdgpu_buffer_rsrc_t z_rsrc;   // no records: every access out of range, nothing read
  if (MIX) z_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(P.Wt), 0, 0, kBufferFlags);
  // A row stride and per-stage step: row-major, or 32-k panels (a stage of
  // the tile is then one contiguous block of whole lines)
  const int a_rs = P.a_panel_rows ? BK : K;
  const size_t a_ks = P.a_panel_rows ? (size_t)P.a_panel_rows * BK : BK;
  const int b_rs = P.b_panel_rows ? BK : K;
  const int b_ks = P.b_panel_rows ? P.b_panel_rows * BK : BK;
  // weight row of row r (< BNT) of n-tile nt_'s B tile
  auto wrow_of = [&](int nt_, int r) -> int {
    if (EPI == EPI_SWIGLU) {
      // each wave column's 64 B rows: 32 gate rows, then the 32 up rows of
      // the same hidden columns
      const int wc = r >> 6, in_wc = r & 63;
      const int hidden = nt_ * (BNT / 2) + wc * 32 + (in_wc & 31);
      return (in_wc < 32 ? 0 : P.glu_offset) + hidden;
    }
    return nt_ * BNT + r;
  };
  auto set_src = [&](int e_, int row0_, int row_end_, int nt_, bool wide_, int kc_) {
    const size_t kst0 = kc_ >= 0 ? (size_t)kc_ * tile_nk(kc_) : 0;   // first stage of a piece
    a_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(A + (size_t)row0_ * a_rs + kst0 * a_ks), 0,
                                               -1, kBufferFlags);
    b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(reinterpret_cast<const bf16_t *>(P.Wt) + (size_t)e_ * P.w_stride + kst0 * b_ks), 0,
        -1, kBufferFlags);
    const int last = row_end_ - 1 - row0_;                   // last valid row of the A tile
    if constexpr (MIX) {
      // pieces 0-7: A rows 0-127; 8-15: A rows 128-255 (256 x 256) or B
      // rows 0-127 (wide); 16-31: B rows 0-255 (256 x 256) or 128-383
      // (wide); 32-39: B rows 384-511 (wide; nothing otherwise)
      ld_wide = wide_;
#pragma unroll
      for (int i = 0; i < LNQ; ++i) {
        const int pc = wave % LW + LW * i;
        if (i < 2 || (i < 4 && !wide_)) {
          const int r = pc * 16 + lrow;
          soff[i] = ((uint32_t)min(r, last) * a_rs + ((lchunk ^ swz(r)) << 3)) * 2;
        } else {
          const int r = (pc - (wide_ ? 8 : 16)) * 16 + lrow;   // row of the 512 (or 256) B rows
          const int wrow = wrow_of(wide_ ? 2 * nt_ + (r >> 8) : nt_, r & (BNT - 1));
          soff[i] = ((uint32_t)wrow * b_rs + ((lchunk ^ swz(r)) << 3)) * 2;
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < LAQ; ++i) {
      const int r = (wave % LW + LW * i) * 16 + lrow;        // row inside the A tile
      soff[i] = ((uint32_t)min(r, last) * a_rs + ((lchunk ^ swz(r)) << 3)) * 2;   // bytes
    }
#pragma unroll
    for (int i = 0; i < LBQ; ++i) {
      const int r = (wave % LW + LW * i) * 16 + lrow;        // row inside the B tile
      soff[LAQ + i] = ((uint32_t)wrow_of(nt_, r) * b_rs + ((lchunk ^ swz(r)) << 3)) * 2;   // bytes
    }
  };
  set_src(e, row0, row_end, nt, wide, kc);
  auto issue_l = [&](int stage, int slot) {
    char *base = smem + slot * STAGE_BYTES;
    const int a_so = (int)(stage * a_ks * 2), b_so = stage * b_ks * 2;   // bytes
    if constexpr (MIX) {
      const __amdgpu_buffer_rsrc_t r23 = ld_wide ? b_rsrc : a_rsrc, r89 = ld_wide ? b_rsrc : z_rsrc;
      const int so23 = ld_wide ? b_so : a_so;
#pragma unroll
      for (int i = 0; i < LNQ; ++i) {
        char *dst = base + (wave % LW + LW * i) * 1024;
        if (i < 2)
          lds_dma16_buf(a_rsrc, soff[i], a_so, dst);
        else if (i < 4)
          lds_dma16_buf(r23, soff[i], so23, dst);
        else if (i < 8)
          lds_dma16_buf(b_rsrc, soff[i], b_so, dst);
        else
          lds_dma16_buf(r89, soff[i], b_so, dst);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < LAQ; ++i) lds_dma16_buf(a_rsrc, soff[i], a_so, base + (wave % LW + LW * i) * 1024);
#pragma unroll
    for (int i = 0; i < LBQ; ++i)
      lds_dma16_buf(b_rsrc, soff[LAQ + i], b_so, base + A_BYTES + (wave % LW + LW * i) * 1024);
  };
  auto issue = [&](int stage, int slot) {
    if (loader) issue_l(stage, slot);
  };

  // ---- fragments.  v_mfma_f32_16x16x32_bf16 with the weights as operand A:
  // lane l holds row l % 16 of a 16-row block at logical 16-byte chunk l / 16
  // (k 8 (l / 16) .. + 7) of both operands, and ends with
  // C[m = l % 16][n = 4 (l / 16) + j], j < 4, of its 16 x 16 block: four
  // consecutive output columns per lane.  (The 32 x 32 x 16 instruction
  // moves twice the accumulator bytes per MAC and, on random operands,
  // draws enough more power to run these GEMMs 6-12% slower.)  A wave's
  // 64 x 128 (columns x rows) block is NWB x NXB such blocks; a stage's
  // MFMAs run in four quarters: weight blocks 0-1 or 2-3 times activation
  // blocks 0 .. HX-1 or HX .. NXB-1.
  constexpr int NWB = 2 * TN;   // 16-row weight blocks per wave
  constexpr int NXB = 2 * TM;   // 16-row activation blocks per wave
  constexpr int HX = TM;        // activation blocks per half-stage
  const int wm = wave / WN, wn = wave % WN;
  const int frow = lane & 15;
  // quarter q of the wave (lanes 16 q .. 16 q + 15) takes logical k-chunk
  // pi(q) = 0, 3, 1, 2 of both operands (the MFMA's k order is free as long
  // as both operands share it): a 128-bit read runs at full rate only when
  // lanes l and l + 16 sit at 16-byte slots whose XOR has even parity
  const int kq = (lane >> 5) ^ (((lane >> 4) & 1) * 3);
  const int coff = (kq ^ swz(frow)) << 4;                    // swz of every row of the block
  // byte offsets in a stage slot: this wave's activation rows, then its
  // weight rows (a wide tile: A rows 0-127 for both wave rows, and wave row
  // wm's 256 weight rows from 8 KiB + 256 wm rows on)
  int a_frag, b_frag;
  auto set_frags = [&](bool wide_) {
    const bool wd = MIX && wide_;
    a_frag = ((wd ? 0 : wm * NXB * 16) + frow) * 64 + coff;
    b_frag = (wd ? kTileM * BK * 2 : A_BYTES) + ((wd ? wm * BNT : 0) + wn * NWB * 16 + frow) * 64 + coff;
  };
  set_frags(wide);

  f32x4 acc[NWB][NXB];

  bf16x8 fw[NWB], fx0[HX], fx1[HX];   // the stage's weights and its two activation halves
  // TM == 2 (64 x 64 waves: the small-problem shapes, up to one wave per
  // SIMD, where the loop waits on LDS latency): v_mfma_f32_32x32x16_bf16
  // with two 16-k steps per stage, each with 4 MFMAs of 32 cycles covering
  // the next step's fragment reads, measured faster there than the 16 x 16
  // schedule.  Lane l reads row l % 32 of a 32-row block at logical chunk
  // 2 kk + l / 32 and ends with C[m = l % 32][n = 8 g + 4 (l / 32) + j],
  // g, j < 4, of its 32 x 32 block.
  constexpr bool M32 = TM == 2;
  const int frow32 = lane & 31;
  const int coff32_0 = ((lane >> 5) ^ swz(frow32)) << 4, coff32_1 = ((2 + (lane >> 5)) ^ swz(frow32)) << 4;
  const int a_frag32 = (wm * TM * 32 + frow32) * 64;
  const int b_frag32 = A_BYTES + (wn * TN * 32 + frow32) * 64;
  f32x16 acc32[M32 ? TN : 1][M32 ? TM : 1];
  bf16x8 gw0[M32 ? TN : 1], gx0[M32 ? TM : 1], gw1[M32 ? TN : 1], gx1[M32 ? TM : 1];
  auto read_frags32 = [&](bf16x8 *w, bf16x8 *x, int slot, int co) {
    const char *base = smem + slot * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < TN; ++i) w[i] = *reinterpret_cast<const bf16x8 *>(base + b_frag32 + i * 32 * 64 + co);
#pragma unroll
    for (int i = 0; i < TM; ++i) x[i] = *reinterpret_cast<const bf16x8 *>(base + a_frag32 + i * 32 * 64 + co);
  };
  auto mfmas32 = [&](const bf16x8 *w, const bf16x8 *x) {
#pragma unroll
    for (int in = 0; in < (M32 ? TN : 1); ++in)
#pragma unroll
      for (int im = 0; im < (M32 ? TM : 1); ++im)
        acc32[in][im] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[in], x[im], acc32[in][im], 0, 0, 0);
  };
  // weight blocks 2 wh, 2 wh + 1
  auto read_w = [&](int slot, int wh) {
    const char *base = smem + slot * STAGE_BYTES + wh * 2 * 16 * 64;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      fw[2 * wh + i] = *reinterpret_cast<const bf16x8 *>(base + b_frag + i * 16 * 64);
  };
  auto read_x = [&](bf16x8 *x, int slot, int half) {
    const char *base = smem + slot * STAGE_BYTES + half * HX * 16 * 64;
#pragma unroll
    for (int i = 0; i < HX; ++i) x[i] = *reinterpret_cast<const bf16x8 *>(base + a_frag + i * 16 * 64);
  };
  // quarter (WH, XH): weight blocks 2 WH, 2 WH + 1 times activation half XH
  auto mfmas = [&](const bf16x8 *x, auto wh_tag, auto xh_tag) {
    constexpr int WH = decltype(wh_tag)::value, XH = decltype(xh_tag)::value;
#pragma unroll
    for (int jn = 2 * WH; jn < 2 * WH + 2; ++jn)
#pragma unroll
      for (int i = 0; i < HX; ++i)
        acc[jn][XH * HX + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[jn], x[i], acc[jn][XH * HX + i], 0, 0, 0);
  };

  // Order inside iteration kt (stage kt in slot kt % NSTAGE):
  //   wait for activation half 0 and weight blocks 0-1 of stage kt; read
  //   activation half 1; quarter (0, 0); wait for weight blocks 2-3;
  //   quarter (1, 0);
  //   barrier: stage kt+1 has landed and every fragment read of this wave
  //   is done, so after it the slot of stage kt-1 is free on every wave;
  //   read activation half 0 of stage kt+1; load stage kt+NSTAGE-1 into
  //   the free slot; quarter (0, 1); read weight blocks 0-1 of stage kt+1;
  //   quarter (1, 1); read its weight blocks 2-3.
  // Every read has at least 8 MFMAs (a quarter) to arrive before its first
  // use, and the fragments take 48 registers.
  // (Requesting stages one iteration earlier, into the slot of stage kt,
  // measured no faster.)  The explicit LDS waits sit where the reads have
  // had an MFMA block to arrive, so the compiler needs none of its own in
  // front of the MFMAs.
  int nk = tile_nk(kc);
  int gb = 0;   // ring slot of the tile's stage 0 (rotates from tile to tile)
  auto slot = [&](int st) { return (int)((unsigned)(gb + st) % NSTAGE); };
#pragma unroll
  for (int st = 0; st < NSTAGE - 1; ++st)
    if (st < nk) issue(st, slot(st));
  const int out_cols = (EPI == EPI_SWIGLU) ? BNT / 2 : BNT;
  constexpr bool ROPE = EPI == EPI_QKV_ROPE;
  int rpos[ROPE ? NXB : 1];
  // (cos, sin) of frequencies f .. f + 3 at position pos, f = 16 q + 4 (lane / 16)
  // (q = 0, and q = 1 for d_head = 64), for each 16-row half of a 32-row block
  float4 tq[ROPE ? 2 : 1][2][2];
  // computed, not loaded: frequency f turns theta^(-f / half) / (2 pi)
  // revolutions per position; the hardware sine and cosine take revolutions
  float frev[ROPE ? 2 : 1][4];
  if (ROPE) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = 16 * q + 4 * (lane >> 4) + i;
        frev[q][i] = __builtin_amdgcn_exp2f(-(float)f / (float)P.half * P.rope_log2_theta) * 0.15915494309189535f;
      }
  }
  auto rope_table = [&](int pos, float4 (&t)[2][2]) {
    // (the fraction of the position's revolutions, exact to about 2^-24 W)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (q == 0 || P.half == 32) {
        float c[4], sn[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float r = __builtin_amdgcn_fractf((float)pos * frev[q][i]);
          c[i] = __builtin_amdgcn_cosf(r);
          sn[i] = __builtin_amdgcn_sinf(r);
        }
        t[q][0] = make_float4(c[0], sn[0], c[1], sn[1]);
        t[q][1] = make_float4(c[2], sn[2], c[3], sn[3]);
      }
    }
  };
  for (;;) {
#pragma unroll
    for (int a = 0; a < NWB; ++a)
#pragma unroll
      for (int b = 0; b < NXB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[a][b][i] = 0.f;
    if constexpr (M32) {
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc32[a][b][i] = 0.f;
    }
    // A wave whose 128 rows all lie past the expert's last row (the second
    // wave row of a partial tile with at most 128 rows) skips its fragment
    // reads and MFMAs and only keeps the barriers and its share of the loads.
    const bool active = (MIX && wide) || wm * 32 * TM < row_end - row0;
    auto main_loop = [&](auto act_tag, auto ldr_tag) {
      constexpr bool ACT = decltype(act_tag)::value;
      constexpr bool LDR = decltype(ldr_tag)::value;
      constexpr int WNQ = LDR ? LNQ : 0;   // this wave's loads per stage
      // stage 0 landed (stages 1 .. NSTAGE-2 may be in flight; for a tile after
      // the first, also the previous epilogue's stores, which are younger than
      // stages 0 and 1 and older than stage NSTAGE-2)
      if (nk >= NSTAGE - 1)
        stage_barrier<WNQ * (NSTAGE - 2), 0>();
      else
        stage_barrier<0, 0>();
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      if constexpr (M32) {
        if (ACT) read_frags32(gw0, gx0, slot(0), coff32_0);
        auto step32 = [&](int kt, int s_kt, int s_next, int s_load, auto load_tag) {
          constexpr bool LOAD = decltype(load_tag)::value;
          __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
          if (ACT) {
            read_frags32(gw1, gx1, s_kt, coff32_1);
            mfmas32(gw0, gx0);
            reads_then_mfmas<TM + TN, TM * TN>();
          }
          if (LOAD)
            stage_barrier<WNQ * (NSTAGE - 3), 0>();
          else
            stage_barrier<0, 0>();
          if (ACT) read_frags32(gw0, gx0, s_next, coff32_0);   // (last stage: a stale slot, unused)
          if (LOAD && LDR) issue_l(kt + NSTAGE - 1, s_load);
          if (ACT) {
            mfmas32(gw1, gx1);
            __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);
            if (LOAD && LDR)
              mfma_load_groups<LNQ, TM * TN>();
            else
              __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);
          }
        };
        int kt = 0;
        for (; kt + NSTAGE - 1 < nk; ++kt)
          step32(kt, slot(kt), slot(kt + 1), slot(kt + NSTAGE - 1), std::true_type{});
        for (; kt < nk; ++kt) step32(kt, slot(kt), slot(kt + 1), 0, std::false_type{});
        return;
      }
      if (ACT) {
        // in the order the steady state leaves its reads in flight
        read_x(fx0, slot(0), 0);
        read_w(slot(0), 0);
        read_w(slot(0), 1);
      }
      auto stage_step = [&](int kt, int s_kt, int s_next, int s_load, auto load_tag) {
        constexpr bool LOAD = decltype(load_tag)::value;
        // activation half 0 and weight blocks 0-1 landed (blocks 2-3 may not)
        __builtin_amdgcn_s_waitcnt(0xc07f | (2 << 8));
        if (ACT) {
          read_x(fx1, s_kt, 1);
          mfmas(fx0, I0{}, I0{});
          reads_then_mfmas<HX, 2 * HX>();
        }
        // weight blocks 2-3 landed (activation half 1 may not)
        __builtin_amdgcn_s_waitcnt(0xc07f | (HX << 8));
        if (ACT) {
          mfmas(fx0, I1{}, I0{});
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * HX, 0);
        }
        if (LOAD)
          // at the barrier stages kt+2 .. kt+NSTAGE-2 may still be in flight;
          // stage kt+NSTAGE-1 goes into the slot of stage kt-1
          stage_barrier<WNQ * (NSTAGE - 3), 0>();
        else
          stage_barrier<0, 0>();   // drain: nothing left to load
        if (ACT) read_x(fx0, s_next, 0);   // (on the last stage a stale slot, unused)
        if (LOAD && LDR) issue_l(kt + NSTAGE - 1, s_load);
        if (ACT) {
          mfmas(fx1, I0{}, I1{});
          __builtin_amdgcn_sched_group_barrier(0x100, HX, 0);        // the LDS reads
          if (LOAD && LDR)
            mfma_load_groups<LNQ, 2 * HX>();                          // MFMAs, stage loads among them
          else
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * HX, 0);
          read_w(s_next, 0);
          mfmas(fx1, I1{}, I1{});
          reads_then_mfmas<2, 2 * HX>();
          read_w(s_next, 1);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      };
      int kt = 0;
      for (; kt + NSTAGE - 1 < nk; ++kt)
        stage_step(kt, slot(kt), slot(kt + 1), slot(kt + NSTAGE - 1), std::true_type{});
      for (; kt < nk; ++kt) stage_step(kt, slot(kt), slot(kt + 1), 0, std::false_type{});
    };
    if (loader) {
      if (active)
        main_loop(std::true_type{}, std::true_type{});
      else
        main_loop(std::false_type{}, std::true_type{});
    } else {
      if (active)
        main_loop(std::true_type{}, std::false_type{});
      else
        main_loop(std::false_type{}, std::false_type{});
    }
    stage_barrier<0, 0>();  // every wave is done with the ring: reuse it below

    // next tile (persistent): its stages 0 .. NSTAGE-3 go into the ring now,
    // under this tile's epilogue, which stages through the other two slots
    int mt2 = 0, nt2 = 0, e2 = 0, r02 = 0, re2 = 0, kc2 = -1, pslot2 = 0;
    bool wide2 = false;
    const bool more = PERSIST && locate(u + ustep, mt2, nt2, e2, r02, re2, wide2, kc2, pslot2);
    const int gb2 = (int)((unsigned)(gb + nk) % NSTAGE);
    const int nk2 = tile_nk(kc2);
    if (PERSIST && more) {
      set_src(e2, r02, re2, nt2, wide2, kc2);
#pragma unroll
      for (int st = 0; st < NSTAGE - 2; ++st)
        if (st < nk2) issue(st, (gb2 + st) % NSTAGE);
    }

    // ---- epilogue.  acc[jn][xb] holds C[m = xb*16 + lane%16][n = jn*16 +
    // 4*(lane/16) + j] (j < 4) of this wave's 128 x 64 block.  SwiGLU:
    // acc[0], acc[1] are the gate and acc[2], acc[3] the up projection of the
    // same 32 hidden columns.
    // the lane index, opaque to the compiler: keeps the epilogue's address
    // arithmetic from being hoisted out of the tile loop (registers are
    // short across the main loop)
    int lane_e = lane;
    asm volatile("" : "+v"(lane_e));
    constexpr int NC = (EPI == EPI_SWIGLU) ? 32 : 64;   // output columns per wave
    constexpr int SLOTS = NC / 4;                       // 16-byte slots per staged row
    constexpr int LPR = NC / 8;                         // lanes per row on read-back
    constexpr int RPP = 64 / LPR;                       // rows per read-back pass
    float *stage_f =
        PERSIST ? reinterpret_cast<float *>(smem + ((gb2 + NSTAGE - 2 + wave / (NW / 2)) % NSTAGE) * STAGE_BYTES) +
                      (wave % (NW / 2)) * 32 * NC
                : reinterpret_cast<float *>(smem) + wave * 32 * NC;
    static_assert(!PERSIST || (NW / 2) * 32 * NC * 4 <= STAGE_BYTES, "epilogue staging: half the waves per slot");
    auto sslot = [&](int r, int c) {                    // physical slot of logical slot c
      return r * SLOTS + (c ^ (SLOTS == 16 ? (r & 15) : ((r >> 1) & 7)));
    };
    const int rr = lane_e / LPR, cc = (lane_e % LPR) * 2;   // read-back row in pass, first slot
    // this wave's first row in the tile and its n-tile (a wide tile: rows
    // 0-127 for both wave rows, n-tile 2 nt + wm)
    const int wrow0 = (MIX && wide) ? 0 : wm * TM * 32;
    const int col_base = ((MIX && wide) ? 2 * nt + wm : nt) * out_cols + wn * NC;
    // RoPE: window positions of this lane's rows and the (cos, sin) values
    // of its first 32-row block
    const bool rope = ROPE && col_base < P.rope_cols;
    if (ROPE && rope && !M32) {
#pragma unroll
      for (int xb = 0; xb < NXB; ++xb)
        rpos[xb] = P.row_pos[min(row0 + wrow0 + xb * 16 + (lane_e & 15), row_end - 1)];
      rope_table(rpos[0], tq[0]);
      rope_table(rpos[1], tq[1]);
    }
    // RoPE (QKV, q and k columns): before staging, every lane_e holds one row of
    // each 16-row block and, for each of its columns in the low half of a
    // head, also the partner column d_head/2 to the right, in the same
    // register of another block: acc[q] / acc[q + 2] for d_head = 64 (the
    // wave's 64 columns are one head), acc[2 h] / acc[2 h + 1] for d_head = 32
    // (two heads).  The rotation is done there, on the fp32 accumulators.
#pragma unroll
    for (int im = 0; im < TM; ++im) {
      if (ROPE && rope && !M32) {
        // pair (x, y) at frequency f: x' = x cos - y sin, y' = x sin + y cos
        auto rot = [](f32x4 &a, f32x4 &b, int j, float c, float sn) {
          const float x = a[j], y = b[j];
          a[j] = x * c - y * sn;
          b[j] = x * sn + y * c;
        };
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int xb = 2 * im + h2;
          const float4(&t)[2][2] = tq[h2];
          if (P.half == 32) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              rot(acc[q][xb], acc[q + 2][xb], 0, t[q][0].x, t[q][0].y);
              rot(acc[q][xb], acc[q + 2][xb], 1, t[q][0].z, t[q][0].w);
              rot(acc[q][xb], acc[q + 2][xb], 2, t[q][1].x, t[q][1].y);
              rot(acc[q][xb], acc[q + 2][xb], 3, t[q][1].z, t[q][1].w);
            }
          } else {  // d_head = 32
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              rot(acc[2 * hh][xb], acc[2 * hh + 1][xb], 0, t[0][0].x, t[0][0].y);
              rot(acc[2 * hh][xb], acc[2 * hh + 1][xb], 1, t[0][0].z, t[0][0].w);
              rot(acc[2 * hh][xb], acc[2 * hh + 1][xb], 2, t[0][1].x, t[0][1].y);
              rot(acc[2 * hh][xb], acc[2 * hh + 1][xb], 3, t[0][1].z, t[0][1].w);
            }
          }
        }
        // the next block's (cos, sin) values
        if (im + 1 < TM) {
          rope_table(rpos[2 * im + 2], tq[0]);
          rope_table(rpos[2 * im + 3], tq[1]);
        }
      }
      if constexpr (M32) {
        // RoPE (d_head 64: acc32[0] / acc32[1]; 32: blocks g and g + 2 of one
        // acc32), with the (cos, sin) entries of this lane's row
        if (ROPE && rope) {
          const int pos = P.row_pos[min(row0 + wm * TM * 32 + im * 32 + (lane_e & 31), row_end - 1)];
          const float *cs = P.rope_cs + (size_t)pos * P.half * 2 + 8 * (lane_e >> 5);
          auto rot = [](f32x16 &a, int i, f32x16 &b, int k, float c, float sn) {
            const float x = a[i], y = b[k];
            a[i] = x * c - y * sn;
            b[k] = x * sn + y * c;
          };
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            if (g >= 2 && P.half != 32) break;
            const float4 t0 = *reinterpret_cast<const float4 *>(cs + 16 * g);
            const float4 t1 = *reinterpret_cast<const float4 *>(cs + 16 * g + 4);
            if (P.half == 32) {
              rot(acc32[0][im], 4 * g + 0, acc32[1][im], 4 * g + 0, t0.x, t0.y);
              rot(acc32[0][im], 4 * g + 1, acc32[1][im], 4 * g + 1, t0.z, t0.w);
              rot(acc32[0][im], 4 * g + 2, acc32[1][im], 4 * g + 2, t1.x, t1.y);
              rot(acc32[0][im], 4 * g + 3, acc32[1][im], 4 * g + 3, t1.z, t1.w);
            } else {
#pragma unroll
              for (int in = 0; in < TN; ++in) {
                rot(acc32[in][im], 4 * g + 0, acc32[in][im], 4 * g + 8, t0.x, t0.y);
                rot(acc32[in][im], 4 * g + 1, acc32[in][im], 4 * g + 9, t0.z, t0.w);
                rot(acc32[in][im], 4 * g + 2, acc32[in][im], 4 * g + 10, t1.x, t1.y);
                rot(acc32[in][im], 4 * g + 3, acc32[in][im], 4 * g + 11, t1.z, t1.w);
              }
            }
          }
        }
#pragma unroll
        for (int in = 0; in < (EPI == EPI_SWIGLU ? 1 : TN); ++in)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float4 v;
            if (EPI == EPI_SWIGLU) {
              v.x = silu_fast(acc32[0][im][4 * g + 0]) * acc32[1][im][4 * g + 0];
              v.y = silu_fast(acc32[0][im][4 * g + 1]) * acc32[1][im][4 * g + 1];
              v.z = silu_fast(acc32[0][im][4 * g + 2]) * acc32[1][im][4 * g + 2];
              v.w = silu_fast(acc32[0][im][4 * g + 3]) * acc32[1][im][4 * g + 3];
            } else {
              v = make_float4(acc32[in][im][4 * g], acc32[in][im][4 * g + 1], acc32[in][im][4 * g + 2],
                              acc32[in][im][4 * g + 3]);
              if (EPI == EPI_GELU) {
                v.x = gelu_erf(v.x); v.y = gelu_erf(v.y); v.z = gelu_erf(v.z); v.w = gelu_erf(v.w);
              }
            }
            const int c = in * 8 + 2 * g + (lane_e >> 5);
            *reinterpret_cast<float4 *>(stage_f + sslot(lane_e & 31, c) * 4) = v;
          }
      }
      // stage this 32-row block: its two 16-row blocks, four columns per lane
      // and block
#pragma unroll
      for (int h2 = 0; h2 < (M32 ? 0 : 2); ++h2) {
        const int xb = 2 * im + h2;
        const int r = 16 * h2 + (lane_e & 15);
#pragma unroll
        for (int jn = 0; jn < (EPI == EPI_SWIGLU ? NWB / 2 : NWB); ++jn) {
          float4 v;
          if (EPI == EPI_SWIGLU) {
            const f32x4 g = acc[jn][xb], up = acc[jn + NWB / 2][xb];
            v.x = silu_fast(g[0]) * up[0];
            v.y = silu_fast(g[1]) * up[1];
            v.z = silu_fast(g[2]) * up[2];
            v.w = silu_fast(g[3]) * up[3];
          } else {
            v = make_float4(acc[jn][xb][0], acc[jn][xb][1], acc[jn][xb][2], acc[jn][xb][3]);
            if (EPI == EPI_GELU) {
              v.x = gelu_erf(v.x); v.y = gelu_erf(v.y); v.z = gelu_erf(v.z); v.w = gelu_erf(v.w);
            }
          }
          const int c = jn * 4 + (lane_e >> 4);   // logical 16-byte slot of the row
          *reinterpret_cast<float4 *>(stage_f + sslot(r, c) * 4) = v;
        }
      }
      // read back whole rows: lane_e -> row rr (+ RPP * pass), 8 columns from 4 * cc
      constexpr int NP = 32 / RPP;
      const int col = col_base + cc * 4;
      int row[NP];
      bool ok[NP];
      float4 v0[NP], v1[NP];
#pragma unroll
      for (int pass = 0; pass < NP; ++pass) {
        const int r = rr + pass * RPP;
        v0[pass] = *reinterpret_cast<const float4 *>(stage_f + sslot(r, cc) * 4);
        v1[pass] = *reinterpret_cast<const float4 *>(stage_f + sslot(r, cc + 1) * 4);
        const int rw = row0 + wrow0 + im * 32 + r;
        ok[pass] = rw < row_end;
        row[pass] = ok[pass] ? rw : row_end - 1;   // rows past the expert: read a valid row, store nothing
      }
      if (SPLIT && kc >= 0) {
        // a piece of a K-split tail tile: its fp32 partial, row-major 256 x 256
        float *pp = P.part + (size_t)pslot * (kTileM2 * 256);
#pragma unroll
        for (int pass = 0; pass < NP; ++pass) {
          if (!ok[pass]) continue;
          float4 *q = reinterpret_cast<float4 *>(pp + (size_t)(wrow0 + im * 32 + rr + pass * RPP) * 256 +
                                                 (col - nt * BNT));
          q[0] = v0[pass];
          q[1] = v1[pass];
        }
      } else if (EPI == EPI_RESID || EPI == EPI_BLEND || EPI == EPI_ACCUM) {
        // every load of the block first (token ids, then the residual rows),
        // then the arithmetic and the stores: the loads overlap each other
        const float *__restrict__ sres = P.s_in;
        const float *__restrict__ hres = P.h;
        size_t tok[NP];
        float gt[NP];
#pragma unroll
        for (int pass = 0; pass < NP; ++pass) {
          tok[pass] = (size_t)P.row_tok[row[pass]];
          gt[pass] = EPI == EPI_BLEND || EPI == EPI_ACCUM ? P.row_gate[row[pass]] : 0.f;
        }
        float4 x0[NP], x1[NP], h0[NP], h1[NP];
#pragma unroll
        for (int pass = 0; pass < NP; ++pass) {
          const float4 *sp = reinterpret_cast<const float4 *>(sres + tok[pass] * P.ldc + col);
          x0[pass] = sp[0];
          x1[pass] = sp[1];
          if (EPI == EPI_BLEND) {
            const float4 *hp = reinterpret_cast<const float4 *>(hres + (size_t)row[pass] * P.ldc + col);
            h0[pass] = hp[0];
            h1[pass] = hp[1];
          }
        }
#pragma unroll
        for (int pass = 0; pass < NP; ++pass) {
          if (!ok[pass]) continue;
          const float4 a0 = v0[pass], a1 = v1[pass], s0 = x0[pass], s1 = x1[pass];
          if (EPI == EPI_RESID) {
            float4 *hp = reinterpret_cast<float4 *>(reinterpret_cast<float *>(P.C) + (size_t)row[pass] * P.ldc + col);
            hp[0] = make_float4(s0.x + a0.x, s0.y + a0.y, s0.z + a0.z, s0.w + a0.w);
            hp[1] = make_float4(s1.x + a1.x, s1.y + a1.y, s1.z + a1.z, s1.w + a1.w);
          } else if (EPI == EPI_ACCUM) {
            const float g = gt[pass];
            float4 *sp = reinterpret_cast<float4 *>(P.s + tok[pass] * P.ldc + col);
            sp[0] = make_float4(s0.x + g * a0.x, s0.y + g * a0.y, s0.z + g * a0.z, s0.w + g * a0.w);
            sp[1] = make_float4(s1.x + g * a1.x, s1.y + g * a1.y, s1.z + g * a1.z, s1.w + g * a1.w);
          } else {
            const float g = gt[pass];
            const float4 q0 = h0[pass], q1 = h1[pass];
            float4 *sp = reinterpret_cast<float4 *>(P.s + tok[pass] * P.ldc + col);
            sp[0] = make_float4(s0.x + g * (q0.x + a0.x - s0.x), s0.y + g * (q0.y + a0.y - s0.y),
                                s0.z + g * (q0.z + a0.z - s0.z), s0.w + g * (q0.w + a0.w - s0.w));
            sp[1] = make_float4(s1.x + g * (q1.x + a1.x - s1.x), s1.y + g * (q1.y + a1.y - s1.y),
                                s1.z + g * (q1.z + a1.z - s1.z), s1.w + g * (q1.w + a1.w - s1.w));
          }
        }
      } else if (EPI == EPI_STORE_F32) {
#pragma unroll
        for (int pass = 0; pass < NP; ++pass) {
          if (!ok[pass]) continue;
          float4 *cp = reinterpret_cast<float4 *>(reinterpret_cast<float *>(P.C) + (size_t)row[pass] * P.ldc + col);
          cp[0] = v0[pass];
          cp[1] = v1[pass];
        }
      } else {
#pragma unroll
        for (int pass = 0; pass < NP; ++pass) {
          if (!ok[pass]) continue;
          uint4 pk;
          pk.x = pack_bf16x2(v0[pass].x, v0[pass].y);
          pk.y = pack_bf16x2(v0[pass].z, v0[pass].w);
          pk.z = pack_bf16x2(v1[pass].x, v1[pass].y);
          pk.w = pack_bf16x2(v1[pass].z, v1[pass].w);
          bf16_t *cp = P.c_panel_rows
                           ? reinterpret_cast<bf16_t *>(P.C) + ((size_t)(col >> 5) * P.c_panel_rows + row[pass]) * 32 + (col & 31)
                           : reinterpret_cast<bf16_t *>(P.C) + (size_t)row[pass] * P.ldc + col;
          *reinterpret_cast<uint4 *>(cp) = pk;
        }
      }
    }
    if (!PERSIST || !more) break;
    // every wave is done with the staging slots: stage NSTAGE-2 of the next
    // tile goes into one of them (no wait on the loads and stores in flight)
    stage_barrier<63, 0>();
    u += ustep;
    mt = mt2; nt = nt2; e = e2; row0 = r02; row_end = re2; gb = gb2;
    kc = kc2; pslot = pslot2; nk = nk2;
    if (MIX) {
      wide = wide2;
      set_frags(wide);
    }
    if (NSTAGE - 2 < nk) issue(NSTAGE - 2, slot(NSTAGE - 2));
  }  // tiles
}

// ---------------------------------------------------------------------------
// Output projection fused with the feed-forward sublayer's RMSNorm + FiLM
// (paper "Library of Layers (LoL)", App. A block: h = x + Attn(.), then the
// MLP reads Norm_ffn(h); review Eq. 7 FiLM).  bf16, d = 256 TN.
//
// A workgroup owns 64 grouped rows and all d output columns, so the whole of
// h for its rows exists in its registers and the norm needs no second pass
// over HBM: h is never stored.  8 waves side by side, each 64 rows x 32 TN
// columns = TN x 2 blocks of v_mfma_f32_32x32x16_bf16.  Every wave reads
// the same 64 activation rows and its own slice of W_o.
//
// Main loop: one 16-k step per stage (2 KiB of activations + 32 d bytes of
// weights), 4 stages in a ring, all four in flight: stage kt + 4 goes into
// the slot of stage kt once every wave has read its fragments.  Rows of 16 k
// = 32 bytes, two 16-byte chunks; logical chunk c of row r sits at c ^ ((r
// >> 3) & 1), which spreads the 16 rows of a fragment read over all 64 banks.
//
// Epilogue, per 32-row half: every wave stages its accumulators in LDS as
// fp32 rows (16-byte chunk c of row r at c ^ (r & 15)), then each wave takes
// 4 whole rows: h = s_in[t] + y, one wave reduction of h^2, u = FiLM(g_e h /
// rms) in bf16 and s[t] = s_in[t] + gate y, all as contiguous row accesses.
// ---------------------------------------------------------------------------
// W [L][rows][K] (row n, contiguous k) -> Wp [L][K/PW][rows][PW]: the
// PW-k panel p of expert e holds W[e][n][PW p .. PW p + PW) for every n, in
// n order, so that one PW-column step of an expert's weights is one
// contiguous block of whole lines.  One thread per 16-byte piece, numbered
// in Wp order, so the stores are contiguous.  PW = 16 for the fused output
// projection's W_o, 32 for the grouped GEMMs' stages.
template <int PW>
__global__ void __launch_bounds__(256) k_pack_panels(const bf16_t *__restrict__ W, bf16_t *__restrict__ Wp,
                                                     int rows, int K, long long pieces) {
  constexpr int PPR = PW / 8;                  // 16-byte pieces per panel row
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= pieces) return;
  const int q = (int)(i % PPR);
  const long long nn = i / PPR;                // (e, panel, n) in Wp order
  const int n = (int)(nn % rows);
  const long long ep = nn / rows;              // e * (K / PW) + panel
  const int panel = (int)(ep % (K / PW));
  const long long e = ep / (K / PW);
  const uint4 v = *reinterpret_cast<const uint4 *>(W + ((size_t)e * rows + n) * K + panel * PW + q * 8);
  *reinterpret_cast<uint4 *>(Wp + (size_t)i * 8) = v;
}

struct ONormParams {
  const bf16_t *A;         // o in 16-k panels, [d/16][a_panel_rows][16]
  int a_panel_rows;        // rows of each panel of o (T)
  const bf16_t *Wp;        // W_o in 16-k panels, [L][d/16][d][16]
  const int32_t *mtile;    // 128-row tile table: (expert, first row)
  const int32_t *mcount;
  const int32_t *toff;
  const int32_t *row_tok;
  const float *row_gate;
  const float *s_in;
  float *s;
  const float *gain;       // Norm_ffn gains, [L][d]
  const float *fg, *fb;    // FiLM of this depth's MLP sublayer, [d] (null: off)
  int film_stride;         // > 0: per-expert FiLM, expert e's rows at fg + e * film_stride
  bf16_t *u;
  int u_panel_rows;        // 0: u is [T][d]; else u is in 32-k panels [d/32][u_panel_rows][32]
  float eps;
  int cpx;                 // CUs per XCD (0: no tail sub-units)
};

constexpr int kONormRows = 64;
constexpr int kONormStages = 4;
constexpr int kONormBK = 16;

template <int TN> struct ONormShape {
  static constexpr int D = 256 * TN;
  static constexpr int A_STAGE = kONormRows * kONormBK * 2;   // 2 KiB
  static constexpr int STAGE = A_STAGE + D * kONormBK * 2;
  static constexpr int LDS = kONormStages * STAGE;
  static_assert(32 * D * 4 <= LDS, "epilogue staging of 32 fp32 rows fits in the ring");
};

__device__ __forceinline__ void lds_dma4_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, void *lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds, 4, (int)voff, soff, 0, 0);
}

__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int TN>
__global__ void __launch_bounds__(512, 1) k_gemm_o_norm(ONormParams P) {
  using S = ONormShape<TN>;
  constexpr int D = S::D, A_STAGE = S::A_STAGE, STAGE = S::STAGE, NS = kONormStages;
  constexpr int NQ = 1 + TN;              // load instructions per wave per stage
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  // ---- tile: the 64-row half (t & 1) of 128-row table entry t >> 1; the
  // 8 XCDs take contiguous ranges of tiles (workgroup i runs on XCD i mod 8),
  // so that the tiles of one expert share W_o in one L2
  const int n_t = 2 * P.mcount[0];
  const int per = (n_t + 7) >> 3;
  const int u_ = blockIdx.x >> 3;
  // Tail sub-units: ragged expert rows (packed documents) add a few units,
  // which would run as a second round of whole units on a few CUs of each
  // XCD.  When the overrun is at most half the XCD's CUs (and the grid has
  // the room), each overrun unit runs instead as two 32-row sub-units,
  // whose workgroups skip the MFMAs of the missing half.
  const int tail = per - P.cpx;
  const bool subs = P.cpx > 0 && tail > 0 && P.cpx + 2 * tail <= (int)(gridDim.x >> 3);
  int t, sub = -1;
  if (!subs || u_ < P.cpx) {
    t = (blockIdx.x & 7) * per + u_;
    if (u_ >= per || t >= n_t) return;
  } else {
    const int q = u_ - P.cpx;
    if (q >= 2 * tail) return;
    t = (blockIdx.x & 7) * per + P.cpx + (q >> 1);
    if (t >= n_t) return;
    sub = q & 1;
  }
  const int e = P.mtile[2 * (t >> 1)];
  if (e < 0) return;
  const int row0 = P.mtile[2 * (t >> 1) + 1] + (t & 1) * kONormRows + (sub > 0 ? kONormRows / 2 : 0);
  const int row_end = sub >= 0 ? min(P.toff[e + 1], row0 + kONormRows / 2) : P.toff[e + 1];
  if (row0 >= row_end) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar LDS addresses

  // ---- load sources.  Activations: wave w fetches rows 8 w .. 8 w + 7, 4
  // bytes per lane (lane -> row 8 w + lane / 8, dword lane % 8 of the row's
  // 32 bytes); o is in 16-k panels, so a stage of the tile's 64 rows is one
  // contiguous 2 KiB block.  Weights: instruction q of wave w fetches rows
  // (w + 8 q) 32 + lane / 2, 16 bytes per lane (physical chunk lane % 2).
  const int last = row_end - 1 - row0;
  const int ar = wave * 8 + (lane >> 3);
  const int a_chunk = ((lane >> 2) & 1) ^ ((ar >> 3) & 1);
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(P.A + (size_t)row0 * kONormBK), 0, -1, kBufferFlags);
  const uint32_t a_off = ((uint32_t)min(ar, last) * kONormBK + a_chunk * 8 + (lane & 3) * 2) * 2;   // bytes
  const int a_step = P.a_panel_rows * kONormBK * 2;   // bytes from one 16-k panel to the next
  // weights in 16-k panels: stage k0 / 16 of expert e is the contiguous
  // block Wp[e][k0 / 16][0 .. d)[0 .. 16), so every request is a whole line
  const __amdgpu_buffer_rsrc_t b_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(P.Wp + (size_t)e * D * D), 0, -1, kBufferFlags);
  uint32_t boff[TN];
#pragma unroll
  for (int q = 0; q < TN; ++q) {
    const int br = (wave + 8 * q) * 32 + (lane >> 1);
    boff[q] = ((uint32_t)br * kONormBK + (((lane & 1) ^ ((br >> 3) & 1)) << 3)) * 2;   // bytes
  }
  auto issue = [&](int stage, int slot) {
    char *base = smem + slot * STAGE;
    lds_dma4_buf(a_rsrc, a_off, stage * a_step, base + wave * 256);
    const int b_so = stage * (D * kONormBK) * 2;
#pragma unroll
    for (int q = 0; q < TN; ++q) lds_dma16_buf(b_rsrc, boff[q], b_so, base + A_STAGE + (wave + 8 * q) * 1024);
  };

  // ---- fragments: lane reads row (lane & 31) of each 32-row block at logical
  // chunk lane >> 5
  const int frow = lane & 31;
  const int coff = (((lane >> 5) ^ ((frow >> 3) & 1)) << 4) + frow * 32;
  const int b_frag = A_STAGE + wave * 32 * TN * 32 + coff;
  f32x16 acc[TN][2];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
  bf16x8 fw[2][TN], fx[2][2];
  auto read_frags = [&](int buf, int slot) {
    const char *base = smem + slot * STAGE;
#pragma unroll
    for (int i = 0; i < TN; ++i) fw[buf][i] = *reinterpret_cast<const bf16x8 *>(base + b_frag + i * 32 * 32);
#pragma unroll
    for (int i = 0; i < 2; ++i) fx[buf][i] = *reinterpret_cast<const bf16x8 *>(base + coff + i * 32 * 32);
  };

  constexpr int nk = D / kONormBK;   // >= 16
#pragma unroll
  for (int st = 0; st < NS; ++st) issue(st, st);
  stage_barrier<NQ * (NS - 1), 0>();   // stage 0 landed on every wave
  read_frags(0, 0);
  // step kt: the fragments of stage kt were read during step kt - 1.  After
  // the barrier stage kt + 1 has landed everywhere and no wave reads slot kt
  // any more, so stage kt + 4 goes there.  Past the last stage the loads
  // repeat it into slots nobody reads again (and the last step reads a stale
  // slot), which keeps every step free of branches and its wait counts fixed.
  // (The barrier's own lgkmcnt(0) covers this wave's reads of stage kt; an
  // extra explicit wait in front of it made the compiler add another one
  // between the MFMAs.)
  // (a sub-unit: IM = 1, the MFMAs of the first 32-row block only)
  auto main_loop = [&](auto im_tag) {
    constexpr int IM = decltype(im_tag)::value;
    auto step = [&](int kt, auto cur_tag) {
      constexpr int cur = decltype(cur_tag)::value;
      stage_barrier<NQ * 2, 0>();
      issue(min(kt + NS, nk - 1), (int)((unsigned)kt % NS));
      read_frags(cur ^ 1, (int)((unsigned)(kt + 1) % NS));
#pragma unroll
      for (int in = 0; in < TN; ++in)
#pragma unroll
        for (int im = 0; im < IM; ++im)
          acc[in][im] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[cur][in], fx[cur][im], acc[in][im], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, TN + 2, 0);   // the fragment reads
      mfma_load_groups<NQ, IM * TN>();                          // MFMAs, stage loads among them
    };
    for (int kt = 0; kt < nk; kt += 2) {
      step(kt, std::integral_constant<int, 0>{});
      step(kt + 1, std::integral_constant<int, 1>{});
    }
  };
  if (sub >= 0)
    main_loop(std::integral_constant<int, 1>{});
  else
    main_loop(std::integral_constant<int, 2>{});
  stage_barrier<0, 0>();   // every wave is done with the ring: the epilogue reuses it

  // ---- epilogue.  acc[in][im] holds y[m = im*32 + lane%32][n = wave*32*TN +
  // in*32 + g*8 + 4*(lane/32) + j] (g, j < 4).
  int lane_e = lane;
  asm volatile("" : "+v"(lane_e));
  float *stg = reinterpret_cast<float *>(smem);
  constexpr int CH = D / 4;   // 16-byte chunks per staged row
  const float *gain = P.gain + (size_t)e * D;
  float4 gv[TN], av[TN], bv[TN];
#pragma unroll
  for (int i = 0; i < TN; ++i) {
    const int c = (i * 64 + lane_e) * 4;
    gv[i] = *reinterpret_cast<const float4 *>(gain + c);
    if (P.fg) {
      av[i] = *reinterpret_cast<const float4 *>(P.fg + (size_t)e * P.film_stride + c);
      bv[i] = *reinterpret_cast<const float4 *>(P.fb + (size_t)e * P.film_stride + c);
    } else {
      av[i] = make_float4(1.f, 1.f, 1.f, 1.f);
      bv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int im = 0; im < 2; ++im) {
    if (im && sub >= 0) break;        // a sub-unit's rows are all in the first block
    if (im) stage_barrier<63, 0>();   // every wave is done reading the first half
    {
      const int r = lane_e & 31;
#pragma unroll
      for (int in = 0; in < TN; ++in)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = wave * 8 * TN + in * 8 + 2 * g + (lane_e >> 5);
          *reinterpret_cast<float4 *>(stg + (r * CH + (c ^ (r & 15))) * 4) =
              make_float4(acc[in][im][4 * g], acc[in][im][4 * g + 1], acc[in][im][4 * g + 2],
                          acc[in][im][4 * g + 3]);
        }
    }
    stage_barrier<63, 0>();
    // rows 4 wave .. 4 wave + 3 of this half, two at a time: every load of the
    // pair first
#pragma unroll
    for (int j0 = 0; j0 < 4; j0 += 2) {
      int grow[2];
      size_t tok[2];
      float gate[2];
      float4 x[2][TN], y[2][TN];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wave * 4 + j0 + j;
        grow[j] = row0 + im * 32 + r;
        const int rr = min(grow[j], row_end - 1);   // past the expert: read a valid row, store nothing
        tok[j] = (size_t)P.row_tok[rr];
        gate[j] = P.row_gate[rr];
#pragma unroll
        for (int i = 0; i < TN; ++i) {
          const int c = i * 64 + lane_e;
          x[j][i] = *reinterpret_cast<const float4 *>(P.s_in + tok[j] * D + c * 4);
          y[j][i] = *reinterpret_cast<const float4 *>(stg + (r * CH + (c ^ (r & 15))) * 4);
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (grow[j] >= row_end) continue;
        float4 h[TN];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < TN; ++i) {
          h[i] = make_float4(x[j][i].x + y[j][i].x, x[j][i].y + y[j][i].y, x[j][i].z + y[j][i].z,
                             x[j][i].w + y[j][i].w);
          ss += h[i].x * h[i].x + h[i].y * h[i].y + h[i].z * h[i].z + h[i].w * h[i].w;
        }
        const float rinv = rsqrtf(wave_sum64(ss) / (float)D + P.eps);
        const float gt = gate[j];
#pragma unroll
        for (int i = 0; i < TN; ++i) {
          const int c = (i * 64 + lane_e) * 4;
          *reinterpret_cast<float4 *>(P.s + tok[j] * D + c) =
              make_float4(x[j][i].x + gt * y[j][i].x, x[j][i].y + gt * y[j][i].y,
                          x[j][i].z + gt * y[j][i].z, x[j][i].w + gt * y[j][i].w);
          const float v0 = av[i].x * (h[i].x * rinv * gv[i].x) + bv[i].x;
          const float v1 = av[i].y * (h[i].y * rinv * gv[i].y) + bv[i].y;
          const float v2 = av[i].z * (h[i].z * rinv * gv[i].z) + bv[i].z;
          const float v3 = av[i].w * (h[i].w * rinv * gv[i].w) + bv[i].w;
          uint2 pk;
          pk.x = pack_bf16x2(v0, v1);
          pk.y = pack_bf16x2(v2, v3);
          bf16_t *up = P.u_panel_rows
                           ? P.u + ((size_t)(c >> 5) * P.u_panel_rows + grow[j]) * 32 + (c & 31)
                           : P.u + (size_t)grow[j] * D + c;
          *reinterpret_cast<uint2 *>(up) = pk;
        }
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


// Finishes the K-split tail tiles of a persistent EPI_ACCUM launch of
// gemm_grid workgroups: each tail tile's pieces summed in piece order, then
// s[t] = s_in[t] + g y for its rows, the epilogue the whole tile would have
// applied.  Block (8 j + xcd, rg): tail tile j of XCD xcd, rows 16 rg ..
// 16 rg + 15 of the tile (small blocks: the sums spread over many CUs;
// 64-row blocks measured 4% slower on packed documents); blocks past the tail (or past the expert's rows)
// do nothing (the host cannot tell how many there are: the tile counts are
// the router's).
__global__ void __launch_bounds__(256) k_split_accum(GemmParams P, int gemm_grid) {
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int n_mt = P.mcount[0], n_nt = P.n_tiles_n;
  const TailSplit ts = tail_split(n_mt * n_nt, xcd, gemm_grid >> 3, P.K / BK, P.part_slots);
  if (ts.split < 2 || j >= ts.tail) return;
  int mt, nt;
  tile_mn(xcd * ts.per + ts.full + j, n_mt, n_nt, P.gm, mt, nt);
  const int e = P.mtile[2 * mt];
  if (e < 0) return;
  const int r0 = P.mtile[2 * mt + 1] + blockIdx.y * 16, row_end = P.toff[e + 1];
  if (r0 >= row_end) return;
  constexpr size_t SLOT = (size_t)kTileM2 * 256;
  // piece kc of tail tile j sits in slot xcd * spx + kc * tail + j
  const float *part = P.part + (size_t)(xcd * ts.spx + j) * SLOT + (size_t)blockIdx.y * 16 * 256;
  const size_t pstep = (size_t)ts.tail * SLOT;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = threadIdx.x + 256 * i;   // 16 rows x 64 float4
    const int r = idx >> 6, c = (idx & 63) * 4;
    const int row = r0 + r;
    if (row >= row_end) continue;
    float4 y = *reinterpret_cast<const float4 *>(part + (size_t)r * 256 + c);
    for (int kc = 1; kc < ts.split; ++kc) {
      const float4 q = *reinterpret_cast<const float4 *>(part + kc * pstep + (size_t)r * 256 + c);
      y.x += q.x;
      y.y += q.y;
      y.z += q.z;
      y.w += q.w;
    }
    const size_t tok = (size_t)P.row_tok[row];
    const float g = P.row_gate[row];
    const int col = nt * 256 + c;
    const float4 x = *reinterpret_cast<const float4 *>(P.s_in + tok * P.ldc + col);
    *reinterpret_cast<float4 *>(P.s + tok * P.ldc + col) =
        make_float4(x.x + g * y.x, x.y + g * y.y, x.z + g * y.z, x.w + g * y.w);
  }
}

// exact_mt: the number of 256-row m-tiles when the host knows it (every
// expert's row count a multiple of 256), else -1
template <int EPI, int WM, int WN, int TMV = 4, int NSV = 0, int MXV = 0>
hipError_t launch_shape(GemmParams P, const Workspace &ws, int n_w, hipStream_t st, int exact_mt = -1) {
  using S = Shape<WM, WN, TMV, NSV, MXV>;
  const bool tall = S::BMT == kTileM2;
  P.mtile = tall ? ws.mtile2 : ws.mtile;
  P.mcount = tall ? ws.mcount + 1 : ws.mcount;
  P.n_tiles_n = n_w / S::BNT;
  const hipError_t e = hipFuncSetAttribute((const void *)k_gemm_bf16<EPI, WM, WN, TMV, NSV, MXV>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, S::LDS);
  if (e != hipSuccess) return e;
  int grid = (((tall ? ws.max_mtiles2 : ws.max_mtiles) * P.n_tiles_n + 7) / 8) * 8;
  if (S::PERSIST) {
    // one workgroup per CU, a multiple of the 8 XCDs, never more than the tiles
    int ncu = 0;
    const hipError_t ec = cu_count(&ncu);
    if (ec != hipSuccess) return ec;
    grid = min(grid, max(8, ncu / 8 * 8));
  }
  // K-split tail: on when the partial slots allow two pieces per XCD and
  // the tiles may leave a short last round (always possible when the host
  // does not know the tile count; when it does, only if some XCD splits)
  bool split = false;
  if constexpr (EPI == EPI_ACCUM && S::PERSIST && !S::MIX && S::BMT == kTileM2 && S::BNT == 256) {
    split = P.part && P.part_slots >= 16;
    if (split && exact_mt >= 0) {
      split = false;
      for (int x = 0; x < 8; ++x)
        if (tail_split(exact_mt * P.n_tiles_n, x, grid >> 3, P.K / BK, P.part_slots).split > 1) split = true;
    }
  }
  if (!split) P.part_slots = 0;
  lol_launch((k_gemm_bf16<EPI, WM, WN, TMV, NSV, MXV>), dim3(grid), dim3(64 * S::NW), S::LDS, st, P);
  if (split) {
    const hipError_t e1 = hipGetLastError();
    if (e1 != hipSuccess) return e1;
    const int max_tail = (grid >> 3) / kSplitMin;   // a longer tail is not split
    lol_launch(k_split_accum, dim3(8 * (max_tail > 0 ? max_tail : 1), kTileM2 / 16), dim3(256), 0, st, P, grid);
  }
  return hipGetLastError();
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
  P.mcount = ws.mcount;
  P.toff = ws.toff;
  P.row_tok = ws.row_tok;
  P.row_gate = ws.row_gate;
  P.C = a.C;
  P.s_in = a.s_in;
  P.s = a.s;
  P.h = a.h;
  P.row_pos = ws.row_pos;
  P.rope_cs = ws.rope_cs;
  P.rope_cols = a.rope_cols;
  P.half = p.d_head / 2;
  P.rope_log2_theta = p.cfg.rope_theta > 0.f ? log2f(p.cfg.rope_theta) : 0.f;
  P.a_panel_rows = a.a_panel_rows;
  P.c_panel_rows = a.c_panel_rows;
  P.b_panel_rows = a.b_panel_rows;
  P.gm = GM;
  P.part = a.part;
  P.part_slots = EPI == EPI_ACCUM && a.part ? a.part_slots : 0;
  if ((a.a_panel_rows || a.b_panel_rows || a.c_panel_rows) && p.cfg.dtype != LOL_BF16)
    return hipErrorInvalidValue;
  if (a.c_panel_rows && (EPI == EPI_RESID || EPI == EPI_BLEND || EPI == EPI_ACCUM)) return hipErrorInvalidValue;
  if (EPI == EPI_QKV_ROPE && (p.cfg.dtype != LOL_BF16 || (p.d_head != 32 && p.d_head != 64)))
    return hipErrorInvalidValue;  // fp32 mode rotates inside its attention kernel
  // the bf16 kernel takes K in groups of 4 32-k stages (d and d_ffn are
  // multiples of 128 in bf16 mode)
  if (p.cfg.dtype == LOL_BF16 && a.K % (4 * BK) != 0) return hipErrorInvalidValue;
  if (p.cfg.dtype == LOL_BF16) {
    // 256 x 256 tiles (persistent) when every expert's row count is a
    // multiple of 256 and such tiles fill the CUs; otherwise tiles from the
    // 128-row table, which leave no partial tile when rows come in multiples
    // of 128: 128 x 512 (persistent) when N allows and they fill the CUs,
    // for long K (the down projection) or with the weights in 32-k panels,
    // else 128 x 256 (measured: with row-major weights 128 x 512 is faster
    // at K = 4096 and slower at K = 1024, where its 512 weight rows per
    // stage are 1,024 half-line requests; in panels it is faster at K =
    // 1,024 too, QKV at the shifted depths of mid_bf16 112 -> 101 us;
    // gate/up measured faster with 256 x 256 either way);
    // 256 x 128 when N is not a multiple of 256
    const int n_w = EPI == EPI_SWIGLU ? 2 * a.N : a.N;   // weight rows
    if (n_w % 256 == 0) {
      int ncu = 0;
      const hipError_t ec = cu_count(&ncu);
      if (ec != hipSuccess) return ec;
      const bool rows256 = a.len_gcd % kTileM2 == 0 || EPI == EPI_SWIGLU || EPI == EPI_GELU;
      const bool rows128 = a.len_gcd % kTileM == 0;
      const long long tiles256 = (long long)(p.T / kTileM2) * (n_w / 256);
      // short K (16 stages or fewer): two 256 x 128 workgroups per CU, whose
      // prologues, epilogues and barriers overlap each other's matrix work,
      // beat the persistent 256 x 256 tile (small_bf16, K = 512: gate/up
      // 49.2 -> 45.4 us, QKV 27.8 -> 26.6 us, same box)
      if (a.K <= 16 * BK && rows256 && tiles256 >= ncu) return launch_shape<EPI, 2, 2>(P, ws, n_w, st);
      // mixed tiles (gate/up): expert rows in multiples of 128 but not of
      // 256 (the depths shifted by half a window) and the weights in panels
      // (a wide tile reads 512 weight rows per stage): 256 x 256 tiles for
      // the full m-tiles and 128 x 512 for the half-filled ones, which then
      // add no partial round of tiles (mid_bf16, same box: gate/up at the
      // shifted depths 241-252 -> 228-235 us, forward 3.335 -> 3.352 M
      // tokens/s; QKV measured slower so than with 128 x 512 tiles at those
      // depths: 117 against 98-108 us)
      if constexpr (EPI == EPI_SWIGLU) {
        if (rows128 && a.len_gcd % kTileM2 != 0 && a.b_panel_rows && (n_w / 256) % 2 == 0 &&
            tiles256 >= ncu)
          return launch_shape<EPI, 2, 4, 4, 0, 1>(P, ws, n_w, st);
      }
      if (rows256 && tiles256 >= ncu)
        return launch_shape<EPI, 2, 4>(P, ws, n_w, st, a.len_gcd % kTileM2 == 0 ? p.T / kTileM2 : -1);
      // expert rows that leave partial tiles in either table (windows whose
      // lengths are not multiples of 128, packed documents): the persistent
      // 256 x 256 shape, whose waves skip the MFMAs of rows past the expert
      // (same-box A/B: forced_bf16 down 226 -> 201 us, QKV 151 -> 147 us;
      // mid_bf16_packed down 284 -> 240 us)
      if (!rows128 && tiles256 >= ncu) return launch_shape<EPI, 2, 4>(P, ws, n_w, st);
      const long long tiles512 = (long long)(p.T / kTileM) * (n_w / 512);
      if ((a.K >= 2048 || a.b_panel_rows) && n_w % 512 == 0 && tiles512 >= ncu)
        return launch_shape<EPI, 1, 8>(P, ws, n_w, st);
      // a small problem whose 128 x 256 tiles would not fill the workgroup
      // slots (two per CU) in one round: 128 x 128 tiles of four 64 x 64
      // waves, three per CU, double the tile count and keep every SIMD busy
      const long long tiles128x256 = (long long)(p.T / kTileM) * (n_w / 256);
      const long long tiles128x128 = 2 * tiles128x256;
      if (tiles128x128 <= ncu) return launch_shape<EPI, 2, 2, 2, 8>(P, ws, n_w, st);
      if (tiles128x256 < 2LL * ncu) return launch_shape<EPI, 2, 2, 2>(P, ws, n_w, st);
      return launch_shape<EPI, 1, 4>(P, ws, n_w, st);
    }
    return launch_shape<EPI, 2, 2>(P, ws, n_w, st);
  } else {
    P.n_tiles_n = a.N / FBN;
    lol_launch(k_gemm_f32<EPI>, dim3(ws.max_mtiles * P.n_tiles_n), dim3(256), 0, st, P);
  }
  return hipGetLastError();
}

template <int TN>
hipError_t launch_o_norm_tn(const ONormParams &P, const Workspace &ws, hipStream_t st) {
  constexpr int LDS = ONormShape<TN>::LDS;
  const hipError_t e = hipFuncSetAttribute((const void *)k_gemm_o_norm<TN>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
  if (e != hipSuccess) return e;
  // 64-row halves of the 128-row table, per XCD; room for the tail's
  // sub-units when the halves can overrun the XCD's CUs by at most half
  int ncu = 0;
  const hipError_t ec = cu_count(&ncu);
  if (ec != hipSuccess) return ec;
  ONormParams Q = P;
  Q.cpx = ncu / 8;
  const int per_max = (2 * ws.max_mtiles + 7) / 8;
  const int tail_max = per_max - Q.cpx;
  const int slots = tail_max > 0 && 2 * tail_max <= Q.cpx ? Q.cpx + 2 * tail_max : per_max;
  lol_launch((k_gemm_o_norm<TN>), dim3(8 * slots), dim3(512), LDS, st, Q);
  return hipGetLastError();
}

}  // namespace

bool o_norm_eligible(const lol_core_config &c) {
  return c.dtype == LOL_BF16 && c.d % 256 == 0 && c.d <= 1024;
}

bool o_norm_fused(const Plan &p) {
  const int d = p.cfg.d;
  if (!o_norm_eligible(p.cfg)) return false;
  // o and u are read and written in panels whose per-stage steps are 32-bit
  // byte offsets
  if (!panels_addressable(p, d)) return false;
  int dev = 0, lds = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return false;
  return lds >= kONormStages * (kONormRows * kONormBK * 2 + d * kONormBK * 2);
}

hipError_t launch_o_norm(const Plan &p, const DepthGeom &g, const Workspace &ws, const float *s_in,
                         float *s, const lol_library &lib, int u_panel_rows, hipStream_t st) {
  if (!o_norm_fused(p)) return hipErrorInvalidValue;
  const int d = p.cfg.d;
  ONormParams P;
  P.A = reinterpret_cast<const bf16_t *>(ws.o);
  P.a_panel_rows = p.T;   // the attention kernel wrote o in 16-k panels
  // W_o in panels: the caller's (prepared once) or the forward's own copy
  P.Wp = lib.wo_panels ? reinterpret_cast<const bf16_t *>(lib.wo_panels) : ws.wo_p;
  P.mtile = ws.mtile;
  P.mcount = ws.mcount;
  P.toff = ws.toff;
  P.row_tok = ws.row_tok;
  P.row_gate = ws.row_gate;
  P.s_in = s_in;
  P.s = s;
  P.gain = lib.g_ffn;
  // FiLM of the MLP sublayer (index 1) of this depth: [D][2][d], or
  // [D][L][2][d] per expert (the kernel adds expert * 2d)
  const size_t film_off = ((size_t)g.depth * (lib.film_per_expert ? p.cfg.L : 1) * 2 + 1) * d;
  P.fg = lib.film_gamma ? lib.film_gamma + film_off : nullptr;
  P.fb = lib.film_beta ? lib.film_beta + film_off : nullptr;
  P.film_stride = lib.film_per_expert ? 2 * d : 0;
  P.u = reinterpret_cast<bf16_t *>(ws.u);
  P.u_panel_rows = u_panel_rows;
  P.eps = p.cfg.rms_eps;
  switch (d / 256) {
    case 1: return launch_o_norm_tn<1>(P, ws, st);
    case 2: return launch_o_norm_tn<2>(P, ws, st);
    case 3: return launch_o_norm_tn<3>(P, ws, st);
    case 4: return launch_o_norm_tn<4>(P, ws, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_pack_panels(const void *w, void *wp, int L, int rows, int K, int pw, hipStream_t st) {
  if (!w || !wp || (pw != 16 && pw != 32) || K % pw != 0) return hipErrorInvalidValue;
  const long long pieces = (long long)L * rows * K / 8;   // 16-byte pieces
  const dim3 grid((unsigned)((pieces + 255) / 256));
  const bf16_t *src = reinterpret_cast<const bf16_t *>(w);
  bf16_t *dst = reinterpret_cast<bf16_t *>(wp);
  if (pw == 16)
    lol_launch(k_pack_panels<16>, grid, dim3(256), 0, st, src, dst, rows, K, pieces);
  else
    lol_launch(k_pack_panels<32>, grid, dim3(256), 0, st, src, dst, rows, K, pieces);
  return hipGetLastError();
}

hipError_t launch_pack_wo(const lol_core_config &c, const void *wo, void *wo_p, hipStream_t st) {
  return launch_pack_panels(wo, wo_p, c.L, c.d, c.d, 16, st);
}

hipError_t launch_gemm(const Plan &p, const Workspace &ws, const GemmArgs &a, hipStream_t st) {
  switch (a.epi) {
    case EPI_STORE: return launch_typed<EPI_STORE>(p, ws, a, st);
    case EPI_RESID: return launch_typed<EPI_RESID>(p, ws, a, st);
    case EPI_SWIGLU: return launch_typed<EPI_SWIGLU>(p, ws, a, st);
    case EPI_GELU: return launch_typed<EPI_GELU>(p, ws, a, st);
    case EPI_BLEND: return launch_typed<EPI_BLEND>(p, ws, a, st);
    case EPI_QKV_ROPE: return launch_typed<EPI_QKV_ROPE>(p, ws, a, st);
    case EPI_ACCUM: return launch_typed<EPI_ACCUM>(p, ws, a, st);
    case EPI_STORE_F32:
      if (p.cfg.dtype != LOL_BF16) return hipErrorInvalidValue;
      return launch_typed<EPI_STORE_F32>(p, ws, a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace lol
