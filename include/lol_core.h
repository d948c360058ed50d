/*
 * lol_core.h -- C ABI of the Library-of-Layers routed-core forward pass on
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes: the routed core of Algorithm 1 in the paper "Library of
 * Layers (LoL): Adaptively Ordering Transformer Layers at Runtime"
 * (Appendix A), i.e. for every routed depth l = 1..D:
 *   - windows of W tokens whose boundaries shift by ((l-1) S) mod W
 *     (paper Sec. 3.2.1; review "Library of Layers: Routing Whole
 *     Transformer Blocks at Runtime", Eq. 2);
 *   - per window a router input built from earlier windows' means, or from
 *     the first token and a depth vector for window 0 (paper Sec. 3.2.2;
 *     review Eq. 4);
 *   - a linear router in fp32, softmax, and a top-1 choice of one library
 *     block by probability plus balancing bias, gated by the unbiased
 *     probability (paper App. A, loss-free balancing; review Eq. 5; blog
 *     "Library of Layers: a transformer that picks its own layer order",
 *     "How the order is chosen");
 *   - the chosen pre-norm block (RMSNorm with depth FiLM, bias-free QKV,
 *     RoPE, attention causal inside the window, output projection, SwiGLU
 *     or GELU MLP; paper App. A; review Eqs. 1 and 7);
 *   - the gated residual blend s + alpha (E(s) - s) (Algorithm 1, blend
 *     step; blog "The forward pass, term by term", step 5).
 *
 * Conventions for every entry point:
 *   - Pointers marked DEVICE point to device memory of the current HIP
 *     device; pointers marked HOST to host memory.  The caller owns every
 *     buffer; the library allocates nothing inside lol_core_forward.
 *   - lol_core_forward is asynchronous on `stream` (a hipStream_t passed as
 *     void*; NULL = the default stream).  Host-checkable errors are returned
 *     before anything is launched.  No C++ exception crosses the ABI.
 *   - Layouts are row-major.  Each batch row is one document.
 *   - K_max = ceil(n / W) + 1 bounds the windows of any depth.
 */
#ifndef LOL_CORE_H
#define LOL_CORE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LOL_OK = 0,
  LOL_EINVAL = 1,        /* a NULL required pointer or an invalid size/argument */
  LOL_EUNSUPPORTED = 2,  /* valid for the method, outside what these kernels handle */
  LOL_EWORKSPACE = 3,    /* workspace NULL or smaller than lol_core_workspace_size */
  LOL_EHIP = 4           /* a HIP runtime call failed (launch, event, copy) */
} lol_status;

typedef enum { LOL_FP32 = 0, LOL_BF16 = 1 } lol_dtype;
typedef enum { LOL_MLP_SWIGLU = 0, LOL_MLP_GELU = 1 } lol_mlp;

/* Sizes and numeric settings of one routed core.
 *   batch, n      documents and tokens per document (T = batch * n rows)
 *   d, n_heads    model width and heads; d_head = d / n_heads must be 32 or 64
 *   d_ffn         MLP hidden width f
 *   L, D          library size (1..64) and routed depth (>= 1)
 *   W, S          window size (>= 1) and per-depth boundary shift (>= 0)
 *   mlp           lol_mlp: SwiGLU (three matrices) or exact-erf GELU (two)
 *   dtype         lol_dtype of the block matrices and of the GEMM/attention
 *                 operands; the residual stream, norms, softmax and router
 *                 are fp32 in both modes
 *   rms_eps       RMSNorm epsilon (> 0)
 *   rope_theta    RoPE base (window-local positions, rotate-half pairs
 *                 (j, j + d_head/2)); 0 disables RoPE
 * Supported sizes: d % 64 == 0 and d_ffn % 64 == 0; in bf16 mode also
 * d % 128 == 0 and d_ffn % 128 == 0. */
typedef struct {
  int32_t batch, n, d, n_heads, d_ffn, L, D, W, S;
  int32_t mlp;
  int32_t dtype;
  float rms_eps;
  float rope_theta;
} lol_core_config;

/* The shared library {E_1..E_L} (DEVICE).  Matrices are [out][in]:
 *   wqkv   [L][3d][d]  rows W_q, then W_k, then W_v
 *   wo     [L][d][d]
 *   w_gu   SwiGLU [L][2f][d] (W_gate rows, then W_up rows); GELU [L][f][d]
 *   w_down [L][d][f]
 * element type = cfg.dtype (bf16 stored as raw 16-bit patterns).
 *   g_attn, g_ffn          [L][d] fp32 RMSNorm gains of each expert
 *   film_gamma, film_beta  fp32 FiLM after each norm (index s = 0 for the
 *                          attention norm, 1 for the MLP norm); both NULL =
 *                          no FiLM (gamma 1, beta 0).  Layout by
 *                          film_per_expert:
 *                            0: [D][2][d], per depth, shared by all experts
 *                               (the paper's gamma_{l,s}, beta_{l,s});
 *                            1: [D][L][2][d], per depth and expert (the
 *                               released configs' depth_expert_film): a
 *                               window uses the FiLM of its chosen expert.
 *   wo_panels              NULL, or W_o already rearranged by
 *                          lol_prepare_wo_panels (see there).  When the
 *                          forward's fused output projection is used (bf16,
 *                          d a multiple of 256 up to 1024) and this is NULL,
 *                          every forward rearranges W_o into its workspace
 *                          first; given, the forward reads it and does not.
 *                          Must hold the panels of the same wo.
 *   weight_panels          NULL, or wqkv, w_gu and w_down already
 *                          rearranged by lol_prepare_weight_panels (see
 *                          there; bf16 only).  Given, the forward's grouped
 *                          QKV, gate/up and down GEMMs read their weights
 *                          from it and not from wqkv, w_gu, w_down (which
 *                          must still be set: the decode kernels read
 *                          them).  Must hold the panels of the same
 *                          matrices.
 * Callers that build this struct must set every member (NULL / 0 where not
 * used). */
typedef struct {
  const void *wqkv, *wo, *w_gu, *w_down;
  const float *g_attn, *g_ffn;
  const float *film_gamma, *film_beta;
  int32_t film_per_expert;
  const void *wo_panels;
  const void *weight_panels;
} lol_library;

/* The router (DEVICE, fp32):
 *   w_r, b_r (b_r NULL = 0): logits z = W_r r + b_r, with
 *     per_depth = 0: w_r [L][d], b_r [L], tied across depths (the default
 *                    of the released code);
 *     per_depth = 1: w_r [D][L][d], b_r [D][L], one router per routed depth
 *                    (the paper's untied-router ablation, Fig. 9)
 *   e_depth [D][d]: the learned vector of each depth used by window 0
 *   expert_bias [L] (NULL = 0): balancing bias, used for the choice only */
typedef struct {
  const float *w_r, *b_r, *e_depth, *expert_bias;
  int32_t per_depth;
} lol_router;

/* Per-window routing path (DEVICE), [D][batch][K_max], indexed by depth,
 * document and window ordinal; slots k >= K_l hold expert -1, gate 0,
 * margin 0.  expert: chosen library index; gate: alpha applied to the
 * update; margin: (a+b)_top1 - (a+b)_top2 of the free router (+inf when
 * L = 1).
 * util (DEVICE [D][L] int32): the number of windows routed to each expert
 * at each depth, the per-depth expert utilisation the paper plots as a
 * heat map (Sec. 4.2, Fig. 4); written by the forwards, not by decode.
 * Any member may be NULL (not written); callers that build this struct
 * must set every member. */
typedef struct {
  int32_t *expert;
  float *gate;
  float *margin;
  int32_t *util;
} lol_path;

/* ceil(n / W) + 1, or -1 for an invalid config.  HOST, pure. */
int32_t lol_core_k_max(const lol_core_config *cfg);

/* LOL_OK if the config is valid and supported, else the status that
 * lol_core_forward would return for it.  HOST, pure. */
lol_status lol_core_validate(const lol_core_config *cfg);

/* Bytes of device workspace lol_core_forward needs for cfg (0 if invalid).
 * HOST, pure. */
size_t lol_core_workspace_size(const lol_core_config *cfg);

/* The routed-core forward pass (Algorithm 1 of the paper, routed depths).
 *   s0            DEVICE [batch][n][d] fp32, the prelude output s^(0)
 *   lib, rt       library and router, as above
 *   forced_expert DEVICE [D][batch][K_max] int32 or NULL; entry >= 0
 *                 replaces the router's choice for that window (the router
 *                 still runs), -1 leaves it free.  Ids >= L are treated as
 *                 free and raise LOL_FLAG_BAD_FORCED_ID (lol_core_read_flags).
 *   forced_gate   DEVICE [D][batch][K_max] fp32 or NULL; a non-NaN entry
 *                 replaces alpha, NaN keeps the router's probability of the
 *                 applied expert (the review's note on forcing a path:
 *                 forcing supplies an expert id and a gate)
 *   s_out         DEVICE [batch][n][d] fp32, receives s^(D); may equal s0
 *   path          HOST struct of DEVICE pointers, or NULL
 *   workspace     DEVICE scratch of workspace_bytes >= lol_core_workspace_size
 *   stream        hipStream_t (as void*) the work is queued on
 * Returns LOL_OK once the work is queued.  Inputs must stay unchanged and
 * the workspace unused by others until the stream reaches the end of it. */
lol_status lol_core_forward(const lol_core_config *cfg, const float *s0,
                            const lol_library *lib, const lol_router *rt,
                            const int32_t *forced_expert, const float *forced_gate,
                            float *s_out, const lol_path *path,
                            void *workspace, size_t workspace_bytes, void *stream);

/* The same forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): no workspace argument; the forward uses a buffer inside the
 * library instead, LOL_STATIC_SCRATCH_BYTES of device memory that each GPU
 * the library runs on holds from the library's load until the process
 * ends.  Arguments, results and errors as lol_core_forward, plus:
 *   LOL_EWORKSPACE  when lol_core_workspace_size(cfg) exceeds
 *                   LOL_STATIC_SCRATCH_BYTES (checked before any launch);
 *   LOL_EHIP        when the buffer's device address cannot be obtained.
 * Every call on one GPU shares the one buffer, which keeps the last call's
 * contents: calls that overlap on a GPU (other streams, other host
 * threads) race and give unspecified results; calls queued in order on one
 * stream are safe.  The device flags of these calls are cleared at the
 * start of each call and cannot be read (a bad forced id is still treated
 * as free).  Kernel timing (lol_core_timing_enable) does not apply.  It
 * calls no allocating routine: hipMalloc, hipFree and event creation are
 * never reached. */
#define LOL_STATIC_SCRATCH_BYTES (64u << 20)
lol_status lol_core_forward_static(const lol_core_config *cfg, const float *s0,
                                   const lol_library *lib, const lol_router *rt,
                                   const int32_t *forced_expert, const float *forced_gate,
                                   float *s_out, const lol_path *path, void *stream);

/* Packed documents: the same forward over a batch of documents of
 * different lengths laid out back to back in one token stream.  Each
 * document is partitioned into windows, routed and attended exactly as if
 * it were a row of its own: the router's running mean of window means
 * restarts at every document's first window, window 0 uses the document's
 * own first token, and no attention crosses a document (paper App. A uses
 * document-blocked attention; the explainer "Library of Layers: a
 * transformer that picks its own layer order", The forward pass, term by
 * term, has the router's prefix sum restart at each document boundary; the
 * review "Library of Layers: Routing Whole Transformer Blocks at Runtime",
 * Deriving prefix-only routing, asks for routing isolated per document in
 * packed execution).
 *   cfg           as for lol_core_forward, with batch = number of
 *                 documents and n = the longest a document may be (window
 *                 slots and workspace are sized by n)
 *   n_tokens      rows of s0 and s_out, 1 <= n_tokens < 2^30
 *   doc_start     DEVICE [batch] int32, first row of each document
 *   doc_len       DEVICE [batch] int32, its length
 *   s0, s_out     DEVICE [n_tokens][d] fp32; rows outside every document
 *                 are not written (s_out may equal s0)
 *   forced_expert, forced_gate, path
 *                 [D][batch][K_max] as for lol_core_forward, indexed by
 *                 document; slots past a document's last window hold
 *                 expert -1, gate 0, margin 0 in `path`
 * The documents must be disjoint, in increasing order of doc_start, each of
 * 1..n tokens inside [0, n_tokens).  A table that breaks this raises
 * LOL_FLAG_BAD_DOC; the kernels then clamp every entry into range (so no
 * access leaves the buffers) but the result is unspecified.  Both tables
 * NULL is lol_core_forward on the [batch][n] layout (n_tokens = batch n);
 * one NULL is LOL_EINVAL. */
lol_status lol_core_forward_docs(const lol_core_config *cfg, int64_t n_tokens,
                                 const int32_t *doc_start, const int32_t *doc_len,
                                 const float *s0, const lol_library *lib, const lol_router *rt,
                                 const int32_t *forced_expert, const float *forced_gate,
                                 float *s_out, const lol_path *path,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* ---- Static weight preparation ------------------------------------------
 * The fused output projection reads W_o in 16-k panels, [L][d/16][d][16]:
 * panel p of expert e holds W_o[e][j][16 p .. 16 p + 15] for every output
 * row j in order, so that one 16-column step of an expert's W_o is one
 * contiguous block.  The weights do not change between forwards, so a
 * caller can rearrange them once and pass the result as
 * lol_library.wo_panels.
 * lol_prepare_wo_panels_size: bytes of that buffer for cfg, or 0 when cfg
 * does not use the fused output projection (fp32, or d not a multiple of
 * 256, or d > 1024) or is invalid.  HOST, pure.
 * lol_prepare_wo_panels: wo (DEVICE [L][d][d] bf16) -> wo_panels (DEVICE,
 * the size above, 16-byte aligned; must not overlap wo).  Asynchronous on
 * stream.  LOL_EUNSUPPORTED when the size above is 0, LOL_EINVAL for NULL
 * or misaligned pointers. */
size_t lol_prepare_wo_panels_size(const lol_core_config *cfg);
lol_status lol_prepare_wo_panels(const lol_core_config *cfg, const void *wo, void *wo_panels,
                                 void *stream);

/* The experts' block matrices (paper "Library of Layers (LoL)", App. A:
 * the library of transformer blocks) do not change between forwards either.
 * The grouped QKV, gate/up and down GEMMs read an expert's weights 32
 * columns of k at a time.  Row-major, such a step takes 64 bytes from each
 * weight row: half of a 128-byte line, the other half a step later.  In
 * 32-k panels, [L][K/32][N_w][32] for a matrix [L][N_w][K] (panel p of
 * expert e holds W[e][j][32 p .. 32 p + 31] for every row j in order), a
 * step of a tile is one contiguous block of whole lines.  The buffer holds
 * the panels of wqkv (N_w = 3d, K = d), then of w_gu (N_w = 2 d_ffn for
 * SwiGLU, d_ffn for GELU; K = d), then of w_down (N_w = d, K = d_ffn), back
 * to back; pass it as lol_library.weight_panels.
 * lol_prepare_weight_panels_size: bytes of that buffer for cfg (the sum of
 * the three matrices' sizes), or 0 for fp32 or an invalid cfg.  HOST, pure.
 * lol_prepare_weight_panels: lib->wqkv, lib->w_gu, lib->w_down (DEVICE,
 * bf16) -> weight_panels (DEVICE, the size above, 16-byte aligned; must not
 * overlap them).  Asynchronous on stream.  LOL_EUNSUPPORTED when the size
 * above is 0, LOL_EINVAL for NULL or misaligned pointers. */
size_t lol_prepare_weight_panels_size(const lol_core_config *cfg);
lol_status lol_prepare_weight_panels(const lol_core_config *cfg, const lol_library *lib,
                                     void *weight_panels, void *stream);

/* ---- Expert bucketing of the last routed depth --------------------------
 * A forward groups every depth's windows by chosen expert (the grouped
 * dispatch of the explainer "Library of Layers: a transformer that picks
 * its own layer order", What it costs): windows routed to expert e, in
 * (document, window) order, form one contiguous range of "grouped rows",
 * one row per token, and the expert GEMMs walk that range in tiles of 128
 * or 256 rows.  lol_core_read_buckets copies those tables, as the workspace
 * holds them after the last routed depth of the most recent forward on it,
 * into `out` (DEVICE int32, lol_core_buckets_size(cfg) entries), laid out
 * back to back as
 *   counts   [L]            windows routed to each expert
 *   row_off  [L + 1]        first grouped row of each expert; row_off[L] =
 *                           tokens routed
 *   win_row0 [batch K_max]  first grouped row of window slot b K_max + k,
 *                           -1 for a slot without a window
 *   n_tiles  [2]            tiles in use in the 128- and 256-row tables
 *   tiles128 [M128][2]      (expert, first grouped row) per 128-row tile:
 *                           every expert's full tiles in expert order, then
 *                           each expert's partial last tile in expert
 *                           order; unused entries (-1, 0)
 *   tiles256 [M256][2]      the same for 256-row tiles
 * with M128 = ceil(batch n / 128) + L and M256 = ceil(batch n / 256) + L.
 * Asynchronous on stream (device-to-device copies).  For inspection and
 * tests; the forward does not need it. */
size_t lol_core_buckets_size(const lol_core_config *cfg);
lol_status lol_core_read_buckets(const lol_core_config *cfg, const void *workspace,
                                 size_t workspace_bytes, int32_t *out, void *stream);

/* Device-side error flags of the last forward that used `workspace` (and,
 * LOL_FLAG_BAD_POS, of decode calls on a decode state). */
#define LOL_FLAG_BAD_FORCED_ID 1u
#define LOL_FLAG_BAD_DOC 2u
#define LOL_FLAG_BAD_POS 4u
/* Copies the flag word to *flags (HOST) and clears it; synchronises
 * `stream`. */
lol_status lol_core_read_flags(void *workspace, uint32_t *flags, void *stream);

/* Kernel-duration instrumentation, for measurement only.
 * lol_core_timing_enable(mask): while bit k of `mask` is set,
 * lol_core_forward records a HIP event pair on its stream around every
 * launch of kernel kind k (0 <= k < LOL_KERNEL_KINDS; mask 0 disables,
 * LOL_TIMING_ALL enables every kind).  lol_core_timing_collect waits for
 * those events and adds, per kind, the summed milliseconds and the launch
 * count to ms[k] and launches[k] (HOST arrays of LOL_KERNEL_KINDS), then
 * forgets them. */
#define LOL_KERNEL_KINDS 12
#define LOL_TIMING_ALL 0xFFFu
lol_status lol_core_timing_enable(uint32_t mask);
/* Restricts the timing above to the launches of depth index `depth`
 * (0 <= depth < D of the forwards that follow); -1 (the default) times
 * every depth.  Each timed launch costs the stream a few microseconds (the
 * events are attached to the kernel's dispatch, created without a
 * system-scope fence), so a caller that needs one kernel's average
 * duration inside a timed region can sample one depth per forward.
 * LOL_EINVAL for depth < -1. */
lol_status lol_core_timing_depth(int32_t depth);
lol_status lol_core_timing_collect(double *ms, int32_t *launches);
/* Name of kernel kind k (0 <= k < LOL_KERNEL_KINDS), or NULL. */
const char *lol_core_kernel_name(int32_t kind);

/* Measurement only: the bf16 matrix-core rate this GPU sustains, for the
 * roofline's ceiling beside the datasheet peak.  One workgroup of 8 waves
 * per compute unit issues nothing but one bf16 MFMA shape on operands held
 * in registers (no memory traffic): shape 32 = v_mfma_f32_32x32x16_bf16,
 * `iters` x 8 instructions per wave; shape 16 = v_mfma_f32_16x16x32_bf16
 * (the grouped GEMMs' instruction), twice as many for the same MACs; in
 * either case on operands that are identical in every instruction
 * (random_operands = 0) or random bf16 values of GEMM-like size (1).  The chip's clock follows
 * its power draw, which depends on how many multiplier bits the operands
 * toggle, so the two settings bracket what a GEMM can reach.
 *   scratch   DEVICE, >= lol_measure_mfma_bf16_scratch_size() bytes,
 *             256-byte aligned
 *   tflops    HOST, receives the measured dense bf16 TFLOP/s
 *   ghz       HOST, receives the mean shader clock during the run (s_memtime
 *             cycles over the 100 MHz s_memrealtime ticks)
 * Launches twice (a short untimed run, then the measured one) and
 * synchronises stream.  LOL_EINVAL for bad arguments (shape other than 16
 * or 32 included), LOL_EWORKSPACE for a small scratch. */
size_t lol_measure_mfma_bf16_scratch_size(void);
lol_status lol_measure_mfma_bf16(int32_t shape, int32_t random_operands, int32_t iters,
                                 void *scratch, size_t scratch_bytes, double *tflops, double *ghz,
                                 void *stream);

/* ---- Incremental decode -------------------------------------------------
 * The routed core one token at a time, for `batch` documents (every call
 * brings one token of each document, at the position the state holds for
 * it).  The review "Library of Layers: Routing Whole Transformer Blocks at
 * Runtime", Deriving prefix-only
 * routing, notes that a window's router reads only earlier, completed
 * windows (window 0: the document's first token and the depth vector), so a
 * window's route and gate are fixed when its first token arrives and a
 * server keeps each depth's window boundaries and summaries; the explainer
 * "Library of Layers: a transformer that picks its own layer order", What
 * it costs, notes that attention never leaves a window.  A decode state
 * holds, per depth and document, the sum of the completed windows' means,
 * the open window's running sum, length, expert and gate, and the open
 * window's keys and values ([W] slots per head).  Feeding tokens 0 .. n-1
 * gives, token by token, the s^(D) rows and path of lol_core_forward on the
 * whole documents, up to rounding (the projections' operands are rounded
 * to bf16 at the same points, the attention weights stay fp32 here, and
 * the sums run in another order).
 * Supported: every config lol_core_validate accepts with batch <= 64,
 * d <= 4096 and W <= 8192 (else LOL_EUNSUPPORTED). */

/* Bytes of the device decode state for cfg (0 if invalid or unsupported).
 * HOST, pure. */
size_t lol_decode_state_size(const lol_core_config *cfg);

/* Starts new documents in every row of `state` (DEVICE, state_bytes >= the
 * size above, 256-byte aligned): each row's next position is 0; clears the
 * flags.  Asynchronous on stream. */
lol_status lol_decode_reset(const lol_core_config *cfg, void *state, size_t state_bytes,
                            void *stream);

/* Starts a new document in row `row` only (0 <= row < batch, else
 * LOL_EINVAL): its next position is 0; the other rows continue.  For
 * serving, where documents join and leave the batch at any step.  Launches
 * one kernel and no memset, so it may be captured in a graph.  Asynchronous
 * on stream. */
lol_status lol_decode_reset_row(const lol_core_config *cfg, void *state, size_t state_bytes,
                                int32_t row, void *stream);

/* One token per document through every routed depth.
 *   pos           -1: each row's token is at the row's own next position
 *                 (0 after its reset, then 1, 2, ...; rows may differ); the
 *                 call then has no per-call arguments besides the buffers,
 *                 so it may be captured once in a graph and replayed.
 *                 0 <= pos < n: every row's token is at pos, which must be
 *                 each row's next position (lockstep use).  A row whose
 *                 position differs from pos, or reaches n, raises
 *                 LOL_FLAG_BAD_POS and its result is unspecified (the
 *                 kernels stay in bounds)
 *   x             DEVICE [batch][d] fp32, s^(0) of the tokens
 *   lib, rt       as for lol_core_forward
 *   forced_expert, forced_gate
 *                 DEVICE [D][batch][K_max] or NULL, as for lol_core_forward;
 *                 read for the windows that open at this position
 *   y             DEVICE [batch][d] fp32, receives s^(D) of the tokens; may
 *                 equal x
 *   path          HOST struct of DEVICE [D][batch][K_max] pointers, or NULL:
 *                 the entries of the windows that open at this position are
 *                 written (expert, gate, margin); others are left untouched
 *   state         the decode state (DEVICE); its per-call scratch is inside
 * Returns LOL_OK once queued; LOL_EINVAL for NULL inputs or pos outside
 * [-1, n); LOL_EWORKSPACE for a state that is missing, too small or not
 * 256-byte aligned.  Calls on one state must run in order on one stream. */
lol_status lol_decode_step(const lol_core_config *cfg, int32_t pos, const float *x,
                           const lol_library *lib, const lol_router *rt,
                           const int32_t *forced_expert, const float *forced_gate, float *y,
                           const lol_path *path, void *state, size_t state_bytes, void *stream);

/* Copies the decode state's flag word (LOL_FLAG_BAD_FORCED_ID,
 * LOL_FLAG_BAD_POS) to *flags (HOST) and clears it; synchronises stream. */
lol_status lol_decode_read_flags(void *state, uint32_t *flags, void *stream);

/* ---- Around the core: token embedding and vocabulary readout ----------
 * The paper's Algorithm 1 (Appendix A) runs a causal prelude on the token
 * sequence, the routed core, then the causal coda and the vocabulary
 * readout; its Sec. 3.1 describes prelude and coda as fixed-order stacks of
 * decoder layers with full causal attention.  Such a stack of P layers is
 * lol_core_forward with W >= n, S = 0, L = D = P, every window forced to
 * expert l at depth l with gate 1, and no FiLM: one window per document,
 * s + 1 (E(s) - s) = E(s).  The two entry points below are the parts that
 * are not blocks. */

/* Embedding lookup: s[t][:] = table[tokens[t]][:], converted to fp32.
 *   tokens  DEVICE [T] int32 token ids; an id outside [0, V) yields a zero row
 *   table   DEVICE [V][d], element type dtype (bf16 as raw 16-bit patterns)
 *   s       DEVICE [T][d] fp32 output
 * T >= 1, V >= 1, d % 4 == 0.  Asynchronous on stream. */
lol_status lol_embed(const int32_t *tokens, int32_t T, const void *table, int32_t V, int32_t d,
                     int32_t dtype, float *s, void *stream);

/* Bytes of device workspace lol_lm_head needs (0 for invalid sizes). */
size_t lol_lm_head_workspace_size(int32_t T, int32_t d, int32_t V, int32_t dtype);

/* Vocabulary readout: logits[t][v] = sum_k u[t][k] * w_vocab[v][k] with
 * u[t] = g_final * s[t] / sqrt(mean(s[t]^2) + eps), a final RMSNorm with a
 * gain; the softmax over v is left to the consumer (the loss or a sampler
 * takes it from the logits).  bf16 mode rounds u to bf16 and accumulates
 * in fp32, like every GEMM of the core.
 *   s        DEVICE [T][d] fp32 (the coda's output)
 *   g_final  DEVICE [d] fp32
 *   w_vocab  DEVICE [V][d], element type dtype
 *   logits   DEVICE [T][V] fp32 output
 * Supported: bf16: d % 128 == 0, V % 128 == 0; fp32: d % 64 == 0,
 * V % 64 == 0.  LOL_EWORKSPACE if the workspace is too small. */
lol_status lol_lm_head(const float *s, int32_t T, int32_t d, const float *g_final, float eps,
                       const void *w_vocab, int32_t V, int32_t dtype, float *logits,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Static description of a status code. */
const char *lol_status_str(lol_status status);

#ifdef __cplusplus
}
#endif

#endif /* LOL_CORE_H */
