// Internal declarations shared by the HIP translation units of liblol_core.
// Not part of the C ABI (that is include/lol_core.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lol_core.h"

namespace lol {

typedef uint16_t bf16_t;  // raw bfloat16 bits

// Kernel kinds for the timing instrumentation (order = lol_core_kernel_name).
enum KernelKind {
  KK_SETUP = 0,
  KK_POOL,
  KK_ROUTE,
  KK_BUCKET,
  KK_ROWMETA,
  KK_NORM_ATTN,
  KK_GEMM_QKV,
  KK_ATTN,
  KK_GEMM_O,
  KK_NORM_FFN,
  KK_GEMM_GATE_UP,
  KK_GEMM_DOWN,
};

// Rows of one M tile of the grouped GEMMs.  Bucketing builds one tile table
// per height: kTileM rows and kTileM2 rows.
constexpr int kTileM = 128;
constexpr int kTileM2 = 256;
constexpr int kMaxExperts = 64;

// Window geometry of one depth, computed on the host.
struct DepthGeom {
  int depth;      // 0-based depth index l-1
  int delta;      // ((l-1) S) mod W
  int K;          // windows per document at this depth
  int len_gcd;    // greatest common divisor of the window lengths at this depth
};

// Device buffers carved from the caller's workspace.
struct Workspace {
  uint32_t *flags;     // [4]
  float *zpart;        // [B*K_max][d/64][L] router logits of each window mean, per 64-column chunk
  float *zpart0;       // [B][d/64][L]       the same for the first-window input (e_l + s_0)/2
  float *zlog;         // [B*K_max][L]       router logits of every window
  int32_t *win_exp;    // [B*K_max]          expert of each window slot (-1 = none)
  float *win_gate;     // [B*K_max]
  int32_t *win_row0;   // [B*K_max]          first grouped row of each window slot
  int32_t *win_len;    // [B*K_max]          tokens of each window slot (0 = none)
  int32_t *ecount;     // [L+1]              windows per expert (+ total)
  int32_t *toff;       // [L+1]              grouped-row offset of each expert
  int32_t *mtile;      // [max_mtiles][2]    (expert, first row) per kTileM-row tile, -1 = idle
  int32_t *mtile2;     // [max_mtiles2][2]   the same for kTileM2-row tiles
  int32_t *mcount;     // [3]                tiles in use in mtile, mtile2; full tiles in mtile2
  int32_t *row_tok;    // [T]                token (b*n + i) of each grouped row
  int32_t *row_pos;    // [T]                window-local position
  int32_t *row_exp;    // [T]
  float *row_gate;     // [T]
  float *rope_cs;      // [W][d_head/2][2]   cos, sin of p * theta^(-2j/d_head)
  void *u;             // [T][d]   act       normed input of a GEMM
  void *qkv;           // [T][3d]  act
  void *o;             // [T][d]   act       attention output
  float *h;            // [T][d]   fp32      after the attention sublayer
  void *hid;           // [T][f]   act       MLP hidden
  bf16_t *wo_p;        // [L][d/16][d][16] bf16  W_o in 16-k panels (fused output projection only)
  int max_mtiles, max_mtiles2;
};

struct Plan {
  lol_core_config cfg;
  int K_max, d_head, T, n_slots;
  size_t act_bytes;    // 2 (bf16) or 4 (fp32)
  // packed documents (DEVICE [batch] each, NULL for the [batch][n] layout):
  // document b is tokens doc_start[b] .. + doc_len[b] - 1 of a stream of
  // n_tokens rows (n_tokens = batch n without a table)
  const int32_t *doc_start = nullptr, *doc_len = nullptr;
  int n_tokens = 0;
};

// Timing events of the launcher call in progress (set by the forward's
// timing wrapper for the kinds being timed, empty otherwise).  The first
// kernel a launcher starts takes the start event and every kernel the stop
// event, so the pair spans all of the call's kernels.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchEvents g_launch_ev;

// Every kernel of the library is launched through this, with the timing
// events (if any) attached to its dispatch packet; without events it is a
// plain launch.
template <typename F, typename... Args>
inline void lol_launch(F kernel, const dim3 &grid, const dim3 &block, uint32_t shmem, hipStream_t st,
                       Args... args) {
  hipEvent_t a = g_launch_ev.start;
  g_launch_ev.start = nullptr;
  if (!a && !g_launch_ev.stop)
    hipLaunchKernelGGL(kernel, grid, block, shmem, st, args...);
  else
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, a, g_launch_ev.stop, 0u, args...);
}

size_t workspace_layout(const Plan &p, char *base, Workspace *ws);
// compute units of the current device (cached per device)
hipError_t cu_count(int *n);

// ---- launchers (all asynchronous on `st`) ----
// window means, contracted with the router weights per 64-column chunk
hipError_t launch_pool(const Plan &p, const DepthGeom &g, const float *s, const Workspace &ws,
                       const lol_router &rt, hipStream_t st);
// router (logits of the prefix inputs, softmax, choice, forcing) and expert
// bucketing (the grouped-row metadata come from the attention norm)
hipError_t launch_route(const Plan &p, const DepthGeom &g, const float *s, const Workspace &ws,
                        const lol_router &rt, const int32_t *forced_expert, const float *forced_gate,
                        const lol_path *path, hipStream_t st);
// clears the flag word and builds the RoPE table
hipError_t launch_setup(const Plan &p, const Workspace &ws, hipStream_t st);
// which = 0: walks every window's tokens: u = FiLM(Norm_attn(s[token])) at the
// token's grouped row, and the grouped-row metadata (row_tok, row_pos,
// row_exp, row_gate) the later kernels read; which = 1: u = FiLM(Norm_ffn(h)).
// panel_rows > 0 (bf16) writes u in 32-column panels [d/32][panel_rows][32].
hipError_t launch_norm(const Plan &p, const DepthGeom &g, int which, const float *s,
                       const lol_library &lib, const Workspace &ws, int panel_rows, hipStream_t st);
// o_panel_rows > 0 (bf16): o is written in 16-k panels [d/16][o_panel_rows][16]
// (the fused output projection reads it so); 0: o is [T][d]
hipError_t launch_attention(const Plan &p, const DepthGeom &g, const Workspace &ws, int o_panel_rows,
                            hipStream_t st);

enum GemmEpilogue {
  EPI_STORE = 0,    // C (act) = acc
  EPI_RESID = 1,    // h (fp32) = s_in[row_tok] + acc
  EPI_SWIGLU = 2,   // hid (act) = silu(acc_gate) * acc_up
  EPI_GELU = 3,     // hid (act) = gelu(acc)
  EPI_BLEND = 4,    // s[row_tok] = s_in[row_tok] + gate * (h + acc - s_in[row_tok])
  EPI_QKV_ROPE = 5, // C (act) = acc, with RoPE at the row's window position on
                    // the q and k columns (bf16 mode only)
  EPI_ACCUM = 6,    // s[row_tok] = s_in[row_tok] + gate * acc (s_in may equal s)
  EPI_STORE_F32 = 7, // C (fp32) = acc (bf16 mode: the vocabulary logits)
};

struct GemmArgs {
  const void *A;        // [T][K] act, grouped rows
  const void *Wt;       // [L][N_w][K] weights (act type)
  int N;                // output columns of C (for SwiGLU: f)
  int K;
  long long w_expert_stride;  // elements between experts
  int glu_offset;       // SwiGLU: row offset of W_up inside an expert (= f)
  GemmEpilogue epi;
  void *C;              // output (act or fp32 depending on epilogue)
  const float *s_in;    // residual stream read (RESID, BLEND)
  float *s;             // residual stream written (BLEND; may equal s_in)
  const float *h;       // BLEND
  int rope_cols;        // QKV_ROPE: columns [0, rope_cols) are rotated (2 d; 0 = no RoPE)
  int len_gcd;          // gcd of the depth's window lengths: every expert's row count is a multiple
  int a_panel_rows;     // 0: A is [T][K]; else 32-k panels [K/32][a_panel_rows][32] (bf16 only)
  int b_panel_rows;     // 0: each expert's weights are [N_w][K]; else 32-k panels
                        // [K/32][b_panel_rows][32] per expert, b_panel_rows = N_w (bf16 only)
  int c_panel_rows;     // SwiGLU / GELU / STORE (bf16): 0 = C is [T][N]; else 32-column panels
  float *part;          // ACCUM (bf16): room for the K-split tail's fp32 partial tiles, part_slots
  int part_slots;       // of 256 x 256 floats each (none: nullptr, 0)
};
hipError_t launch_gemm(const Plan &p, const Workspace &ws, const GemmArgs &a, hipStream_t st);

// Output projection fused with the feed-forward sublayer's input norm (bf16,
// d a multiple of 256 up to 1024).  Per grouped row r of token t, expert e
// and gate g, with y = o[r] W_o[e]^T and h = s_in[t] + y:
//   u[r] = FiLM_ffn(RMSNorm_e(h))  (bf16)   and   s[t] = s_in[t] + g y,
// so that the down projection finishes the gated blend with EPI_ACCUM.
// h is never stored.  s may equal s_in.
bool o_norm_eligible(const lol_core_config &c);   // bf16, d a multiple of 256 up to 1024
// An activation buffer of T rows and `cols` bf16 columns can be kept in k
// panels: the GEMMs step from one panel to the next with a 32-bit byte
// offset, so the whole buffer must stay under 2 GiB.
inline bool panels_addressable(const Plan &p, int cols) {
  return (long long)p.T * cols * 2 <= 0x7FFFFFFFLL;
}
bool o_norm_fused(const Plan &p);                  // eligible and the device's LDS holds the ring
// W_o [L][d][d] -> 16-k panels [L][d/16][d][16]: one 16-k stage of all d
// rows of an expert becomes one contiguous block
hipError_t launch_pack_wo(const lol_core_config &c, const void *wo, void *wo_p, hipStream_t st);
// w [L][rows][K] bf16 -> wp [L][K/pw][rows][pw] (pw = 16 or 32)
hipError_t launch_pack_panels(const void *w, void *wp, int L, int rows, int K, int pw, hipStream_t st);
// u_panel_rows > 0 writes u in 32-k panels [d/32][u_panel_rows][32] (the
// A layout the next GEMM reads with GemmArgs::a_panel_rows)
hipError_t launch_o_norm(const Plan &p, const DepthGeom &g, const Workspace &ws, const float *s_in,
                         float *s, const lol_library &lib, int u_panel_rows, hipStream_t st);

// ---- measurement: the matrix cores' sustained bf16 rate (ceiling.hip) ----
size_t mfma_ceiling_scratch_bytes(int blocks);
// shape 32: v_mfma_f32_32x32x16_bf16; 16: v_mfma_f32_16x16x32_bf16
hipError_t launch_mfma_ceiling(int shape, int blocks, int iters, int random, void *scratch,
                               hipStream_t st);
double mfma_ceiling_flops_per_block(int iters);

// ---- incremental decode (one token per document per call) ----
// Device buffers carved from the caller's decode state.
struct DecodeBufs {
  int32_t *hdr;        // [1] flags
  int32_t *row_next;   // [B]        position of each document's next token
  int32_t *row_cur;    // [B]        position of the token of the call in progress
  float *prefix;       // [D][B][d]  sum of the completed windows' means
  float *cur_sum;      // [D][B][d]  sum of the open window's depth inputs
  int32_t *cur_len;    // [D][B]     tokens in the open window
  int32_t *expert;     // [D][B]     route of the open window
  float *gate;         // [D][B]
  void *kc, *vc;       // [D][B][H][W][d_head] act: keys (rotated) and values of the open window
  float *rope_cs;      // [W][d_head/2][2]
  void *u;             // [B][d]   act   normed input of QKV, then of gate/up
  float *qkv;          // [B][3d]  fp32  projections before RoPE
  void *o;             // [B][d]   act   attention output
  float *h;            // [B][d]   fp32  after the attention sublayer
  void *hid;           // [B][f]   act   MLP hidden
};
enum DecodeProj { DEC_QKV = 0, DEC_O = 1, DEC_GU = 2, DEC_DOWN = 3 };
// sizes the decode kernels handle (on top of a valid config): batch <= 64,
// d <= 4096, W <= 8192
bool decode_supported(const lol_core_config &c);
size_t decode_layout(const lol_core_config &c, char *base, DecodeBufs *s);
// row < 0: every document (positions, routes, flags, RoPE table); else one
// document: its next position 0 and its window routes
hipError_t launch_dec_reset(const lol_core_config &c, const DecodeBufs &s, int row, hipStream_t st);
// window bookkeeping and routing of depth index `depth` for each document's
// token (pos >= 0: every document at pos; -1: each at its own next
// position), then the attention norm into s.u
hipError_t launch_dec_route(const lol_core_config &c, const DecodeBufs &s, int depth, int pos,
                            const float *x, const lol_library &lib,
                            const lol_router &rt, const int32_t *forced_e, const float *forced_g,
                            const lol_path *path, hipStream_t st);
// MLP norm of s.h into s.u
hipError_t launch_dec_norm(const lol_core_config &c, const DecodeBufs &s, int depth,
                           const lol_library &lib, hipStream_t st);
// attention of each document's token over its open window
hipError_t launch_dec_attn(const lol_core_config &c, const DecodeBufs &s, int depth,
                           hipStream_t st);
// one projection (DecodeProj) grouped by expert; x = depth input, y = depth output
hipError_t launch_dec_gemv(const lol_core_config &c, const DecodeBufs &s, int depth, int which,
                           const float *x, float *y, const lol_library &lib, hipStream_t st);

}  // namespace lol
