"""Seeded synthetic workloads for the Library-of-Layers routed core.

This module is the only code that both the CPU oracle (``oracle/``) and the
HIP path see.  It draws inputs and nothing else: it holds none of the
method's arithmetic (no partition, pooling, routing, norm, attention or MLP).

Shapes follow the paper "Library of Layers (LoL): Adaptively Ordering
Transformer Layers at Runtime" (arXiv HTML, Appendix A, architecture
paragraph): bias-free attention, RMSNorm gains, SwiGLU MLP with three
matrices; one exception is the tiny fp32 workload, which uses a two-matrix
GELU MLP.  No dataset is used anywhere: the pages' corpora (FineWeb, math,
sudoku and maze traces) are replaced by i.i.d. Gaussian hidden states of the
same shapes.

Weight layouts (all row-major, "[out][in]", so every GEMM operand is
contiguous along the reduction dimension):

  wqkv    [L][3d][d]   rows 0..d-1 = W_q, d..2d-1 = W_k, 2d..3d-1 = W_v
  wo      [L][d][d]
  w_gu    [L][2f][d]   SwiGLU: rows 0..f-1 = W_gate, f..2f-1 = W_up
                       GELU:   [L][f][d] = W_1
  w_down  [L][d][f]    (GELU: W_2)
  g_attn, g_ffn [L][d] RMSNorm gains, fp32
  film_gamma, film_beta [D][2][d] depth FiLM (index 0 = attention norm,
                       1 = MLP norm), fp32, or None for "no FiLM";
                       [D][L][2][d] with film_mode "depth_expert"
  w_r [L][d], b_r [L], e_depth [D][d], expert_bias [L]  router, fp32;
                       w_r [D][L][d], b_r [D][L] with router "per_depth"
                       (untied)

bf16 workloads round every block matrix to bf16 once (round to nearest even);
``*_f32`` holds those rounded values exactly as fp32 for the oracle and
``*_bf16`` the raw 16-bit patterns for the device.
"""
from __future__ import annotations

import dataclasses
import json
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

WEIGHT_STD = 0.02


@dataclass(frozen=True)
class CoreConfig:
    name: str
    batch: int
    n: int
    d: int
    n_heads: int
    d_ffn: int
    L: int
    D: int
    W: int
    S: int
    mlp: str          # "swiglu" | "gelu"
    dtype: str        # "fp32" | "bf16"
    seed: int
    film: bool = True
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    bias_mode: str = "zero"      # "zero" | "skewed" (large-library load skew)
    path_mode: str = "free"      # "free" | "forced_seq" (one id sequence for all windows)
    router: str = "tied"         # "tied" | "per_depth" (one router per routed depth)
    film_mode: str = "depth"     # "depth" (shared by experts) | "depth_expert"
    router_std: float = WEIGHT_STD   # std of W_r; larger values give peaked routes with clear margins

    @property
    def d_head(self) -> int:
        return self.d // self.n_heads

    @property
    def tokens(self) -> int:
        return self.batch * self.n

    @property
    def k_max(self) -> int:
        # enough window slots for any depth: ceil(n / W) + 1
        return -(-self.n // self.W) + 1

    def scaled(self, batch: int, n: int, name: Optional[str] = None) -> "CoreConfig":
        return dataclasses.replace(self, batch=batch, n=n,
                                   name=name or f"{self.name}@{batch}x{n}")

    def with_(self, **kw) -> "CoreConfig":
        return dataclasses.replace(self, **kw)


# The five workloads.  Index 0 is the tiny fp32 case, 1 the small bf16 core,
# 2 the mid bf16 core (the throughput workload), 3 the sparse large library
# with skewed load, 4 the forced-path reuse extreme.
CONFIGS = [
    CoreConfig("tiny_fp32", batch=1, n=64, d=64, n_heads=2, d_ffn=256, L=3, D=3,
               W=16, S=8, mlp="gelu", dtype="fp32", seed=0),
    CoreConfig("small_bf16", batch=8, n=1024, d=512, n_heads=8, d_ffn=2048, L=4,
               D=4, W=128, S=64, mlp="swiglu", dtype="bf16", seed=1),
    CoreConfig("mid_bf16", batch=4, n=4096, d=1024, n_heads=16, d_ffn=4096, L=8,
               D=8, W=256, S=128, mlp="swiglu", dtype="bf16", seed=2),
    CoreConfig("sparse_bf16", batch=4, n=4096, d=1024, n_heads=16, d_ffn=4096,
               L=32, D=6, W=256, S=128, mlp="swiglu", dtype="bf16", seed=3,
               bias_mode="skewed"),
    CoreConfig("forced_bf16", batch=16, n=2048, d=768, n_heads=12, d_ffn=3072,
               L=2, D=12, W=64, S=32, mlp="swiglu", dtype="bf16", seed=4,
               path_mode="forced_seq"),
]
CONFIG_BY_NAME = {c.name: c for c in CONFIGS}
# Variants of the mid workload (not among the five above): one router per
# routed depth and FiLM per depth and expert (paper App. B Fig. 9; the
# released configs' depth_expert_film), for bench.py --workload.
VARIANT_CONFIGS = [
    CONFIG_BY_NAME["mid_bf16"].with_(name="mid_bf16_untied_expertfilm", router="per_depth",
                                     film_mode="depth_expert"),
]
CONFIG_BY_NAME.update({c.name: c for c in VARIANT_CONFIGS})


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns fp32 values."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32)


def bf16_bits(x_rounded: np.ndarray) -> np.ndarray:
    """The upper 16 bits of already bf16-rounded fp32 values."""
    u = np.ascontiguousarray(x_rounded, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


@dataclass
class CoreInputs:
    cfg: CoreConfig
    s0: np.ndarray                 # [B][n][d] fp32
    wqkv: np.ndarray               # fp32 values (bf16-exact in bf16 workloads)
    wo: np.ndarray
    w_gu: np.ndarray
    w_down: np.ndarray
    g_attn: np.ndarray             # [L][d]
    g_ffn: np.ndarray
    film_gamma: Optional[np.ndarray]   # [D][2][d], [D][L][2][d] (depth_expert) or None
    film_beta: Optional[np.ndarray]
    w_r: np.ndarray                # [L][d], or [D][L][d] (per_depth)
    b_r: np.ndarray                # [L], or [D][L] (per_depth)
    e_depth: np.ndarray            # [D][d]
    expert_bias: np.ndarray        # [L]
    forced_expert: Optional[np.ndarray]  # [D][B][K_max] int32, -1 = free, or None

    def block_weights(self):
        return self.wqkv, self.wo, self.w_gu, self.w_down

    def device_weight(self, name: str) -> np.ndarray:
        """The array the device receives for a block matrix (bf16 bits or fp32)."""
        w = getattr(self, name)
        return bf16_bits(w) if self.cfg.dtype == "bf16" else w


def _normal(rng, shape, std):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def generate(cfg: CoreConfig) -> CoreInputs:
    """Draw every input of ``cfg`` from ``numpy.random.default_rng(cfg.seed)``.

    Order of draws: s0; then per expert wqkv, wo, w_gu (or w_1), w_down
    (or w_2), g_attn, g_ffn; then FiLM gamma, beta; then W_r and e_depth;
    then, for the forced-sequence workload, the per-depth expert ids.
    Projections, W_r and e_depth are N(0, 0.02^2) (W_r: N(0, router_std^2),
    0.02 unless a test asks for peaked routes); gains and FiLM gamma are
    1 + N(0, 0.02^2); FiLM beta is N(0, 0.02^2); b_r = 0; expert_bias = 0
    (the skewed workload's bias is calibrated afterwards by the test harness).
    """
    rng = np.random.default_rng(cfg.seed)
    B, n, d, f, L, D = cfg.batch, cfg.n, cfg.d, cfg.d_ffn, cfg.L, cfg.D
    if d % cfg.n_heads:
        raise ValueError("d must be a multiple of n_heads")
    s0 = rng.standard_normal((B, n, d), dtype=np.float32)
    n_up = 2 * f if cfg.mlp == "swiglu" else f
    wqkv = np.empty((L, 3 * d, d), np.float32)
    wo = np.empty((L, d, d), np.float32)
    w_gu = np.empty((L, n_up, d), np.float32)
    w_down = np.empty((L, d, f), np.float32)
    g_attn = np.empty((L, d), np.float32)
    g_ffn = np.empty((L, d), np.float32)
    for m in range(L):
        wqkv[m] = _normal(rng, (3 * d, d), WEIGHT_STD)
        wo[m] = _normal(rng, (d, d), WEIGHT_STD)
        w_gu[m] = _normal(rng, (n_up, d), WEIGHT_STD)
        w_down[m] = _normal(rng, (d, f), WEIGHT_STD)
        g_attn[m] = 1.0 + _normal(rng, (d,), WEIGHT_STD)
        g_ffn[m] = 1.0 + _normal(rng, (d,), WEIGHT_STD)
    if cfg.film:
        fshape = (D, L, 2, d) if cfg.film_mode == "depth_expert" else (D, 2, d)
        film_gamma = (1.0 + _normal(rng, fshape, WEIGHT_STD)).astype(np.float32)
        film_beta = _normal(rng, fshape, WEIGHT_STD)
    else:
        film_gamma = film_beta = None
    per_depth = cfg.router == "per_depth"
    w_r = _normal(rng, (D, L, d) if per_depth else (L, d), cfg.router_std)
    e_depth = _normal(rng, (D, d), WEIGHT_STD)
    b_r = np.zeros((D, L) if per_depth else L, np.float32)
    expert_bias = np.zeros(L, np.float32)
    forced = None
    if cfg.path_mode == "forced_seq":
        seq = rng.integers(0, L, size=D).astype(np.int32)
        forced = np.broadcast_to(seq[:, None, None], (D, B, cfg.k_max)).astype(np.int32).copy()
    if cfg.dtype == "bf16":
        wqkv, wo, w_gu, w_down = (bf16_round(w) for w in (wqkv, wo, w_gu, w_down))
    return CoreInputs(cfg, s0, wqkv, wo, w_gu, w_down, g_attn, g_ffn,
                      film_gamma, film_beta, w_r, b_r, e_depth, expert_bias, forced)


# The skewed workloads' balancing bias, calibrated once against target loads
# (a frozen input of those workloads) and stored by ``oracle/write_bias_fixture.py``.
SKEWED_BIAS_FIXTURE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "data",
                                   "skewed_bias.json")


def load_skewed_bias(inp: "CoreInputs") -> None:
    """Set ``inp.expert_bias`` from the stored fixture for a skewed workload
    (raises if the fixture has no entry for exactly this config)."""
    cfg = inp.cfg
    if cfg.bias_mode != "skewed":
        return
    with open(SKEWED_BIAS_FIXTURE) as fh:
        table = json.load(fh)
    entry = table.get(cfg.name)
    if entry is None or entry["config"] != dataclasses.asdict(cfg):
        raise KeyError(f"no stored skewed bias for config {cfg.name} (run "
                       "`python -m oracle.write_bias_fixture`)")
    bits = np.array([int(h, 16) for h in entry["bias_f32_bits"]], np.uint32)
    inp.expert_bias = bits.view(np.float32).copy()


# --------------------------------------------------------------------------
# Full model around the routed core (paper Appendix A, Algorithm 1: causal
# prelude on the token sequence, routed core, causal coda, vocabulary
# readout; Sec. 3.1: prelude and coda are fixed-order stacks of decoder
# layers with full causal attention).
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class FullConfig:
    name: str
    core: CoreConfig
    vocab: int
    prelude: int      # layers before the routed core
    coda: int         # layers after it
    seed: int


@dataclass
class FullInputs:
    cfg: FullConfig
    tokens: np.ndarray          # [B][n] int32 in [0, vocab)
    embedding: np.ndarray       # [V][d] fp32 values (bf16-exact in bf16 mode)
    prelude: CoreInputs         # a stack: L = D = prelude, one window per document, forced path
    core: CoreInputs
    coda: CoreInputs
    g_final: np.ndarray         # [d] fp32 final RMSNorm gain
    w_vocab: np.ndarray         # [V][d] fp32 values (bf16-exact in bf16 mode)


def stack_config(core: CoreConfig, layers: int, seed: int, name: str) -> CoreConfig:
    """A fixed-order stack of ``layers`` blocks as a routed-core config: one
    window per document (W = n, S = 0), library = the stack's layers, no FiLM."""
    return core.with_(name=name, L=layers, D=layers, W=core.n, S=0, film=False, seed=seed,
                      bias_mode="zero", path_mode="free", router="tied", film_mode="depth")


def stack_path(cfg: CoreConfig) -> np.ndarray:
    """Forced ids of a stack: layer l at depth l, every window."""
    return np.broadcast_to(np.arange(cfg.D, dtype=np.int32)[:, None, None],
                           (cfg.D, cfg.batch, cfg.k_max)).copy()


def generate_full(cfg: FullConfig) -> FullInputs:
    """Core inputs as ``generate(cfg.core)``; the stacks from seeds + 1 and
    + 2; then tokens, embedding, final gain and readout from seed + 3.
    Embedding and readout rows are N(0, 0.02^2) like every weight, the final
    gain 1 + N(0, 0.02^2), tokens uniform over the vocabulary."""
    core = generate(cfg.core)
    pre = generate(stack_config(cfg.core, cfg.prelude, cfg.seed + 1, cfg.name + "/prelude"))
    coda = generate(stack_config(cfg.core, cfg.coda, cfg.seed + 2, cfg.name + "/coda"))
    pre.forced_expert = stack_path(pre.cfg)
    coda.forced_expert = stack_path(coda.cfg)
    rng = np.random.default_rng(cfg.seed + 3)
    B, n, d, V = cfg.core.batch, cfg.core.n, cfg.core.d, cfg.vocab
    tokens = rng.integers(0, V, size=(B, n)).astype(np.int32)
    emb = _normal(rng, (V, d), WEIGHT_STD)
    g_final = (1.0 + _normal(rng, (d,), WEIGHT_STD)).astype(np.float32)
    w_vocab = _normal(rng, (V, d), WEIGHT_STD)
    if cfg.core.dtype == "bf16":
        emb, w_vocab = bf16_round(emb), bf16_round(w_vocab)
    return FullInputs(cfg, tokens, emb, pre, core, coda, g_final, w_vocab)


# The pages fix no vocabulary size; 32,768 (a multiple of the readout's
# 128-wide tiles) stands in for it.  The 1B setup of the pages uses 4 prelude
# and 4 coda layers around 8 routed depths (paper Sec. 4.2).
FULL_CONFIGS = [
    FullConfig("full_mid_bf16", CONFIG_BY_NAME["mid_bf16"], vocab=32768, prelude=4, coda=4,
               seed=40),
]
FULL_BY_NAME = {c.name: c for c in FULL_CONFIGS}


# --------------------------------------------------------------------------
# Packed documents: documents of different lengths laid out back to back in
# one token stream, each partitioned, routed and attended as its own row
# (paper App. A: document-blocked attention; the explainer's router prefix
# sum restarts at every document boundary).
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class PackedConfig:
    name: str
    core: CoreConfig   # widths, library, windows; n = the longest a document may be
    total: int         # document tokens in the stream
    min_len: int       # shortest document drawn
    gap: int           # unused rows before every document (0 = back to back)
    seed: int


@dataclass
class PackedInputs:
    cfg: PackedConfig
    core: CoreInputs        # batch = number of documents; document b is core.s0[b, :length[b]]
    start: np.ndarray       # int32 [B] first row of each document in the stream
    length: np.ndarray      # int32 [B]
    n_tokens: int           # rows of the stream

    def stream(self) -> np.ndarray:
        """The packed residual stream [n_tokens][d]; rows outside every
        document hold a constant 1000 (never read by the core)."""
        d = self.core.cfg.d
        out = np.full((self.n_tokens, d), 1000.0, np.float32)
        for b, (a, ln) in enumerate(zip(self.start, self.length)):
            out[a:a + ln] = self.core.s0[b, :ln]
        return out


def doc_lengths(total: int, n_max: int, min_len: int, rng) -> list:
    """Lengths log-uniform in [min_len, n_max] (rounded), drawn until they
    cover ``total`` tokens; the last one is cut to fit."""
    out, left = [], total
    while left > 0:
        x = int(round(float(np.exp(rng.uniform(np.log(min_len), np.log(n_max))))))
        x = min(max(x, min_len), n_max, left)
        out.append(x)
        left -= x
    return out


def generate_packed(cfg: PackedConfig, lengths: Optional[list] = None) -> PackedInputs:
    """Document lengths from ``default_rng(cfg.seed)`` (or as given), then
    every core input as ``generate(cfg.core)`` with batch = the number of
    documents; document b is placed ``cfg.gap`` rows after the end of b - 1."""
    rng = np.random.default_rng(cfg.seed)
    lens = list(lengths) if lengths is not None else doc_lengths(cfg.total, cfg.core.n,
                                                                  cfg.min_len, rng)
    if not lens or min(lens) < 1 or max(lens) > cfg.core.n:
        raise ValueError("document lengths must lie in [1, n]")
    core = generate(cfg.core.with_(name=cfg.name, batch=len(lens)))
    starts, pos = [], 0
    for ln in lens:
        pos += cfg.gap
        starts.append(pos)
        pos += ln
    return PackedInputs(cfg, core, np.asarray(starts, np.int32), np.asarray(lens, np.int32),
                        pos + cfg.gap)


# The mid core on 16,384 packed tokens (as many as its 4 x 4,096 layout) in
# documents of 64 .. 4,096 tokens.
PACKED_CONFIGS = [
    PackedConfig("mid_bf16_packed", CONFIG_BY_NAME["mid_bf16"], total=16384, min_len=64, gap=0,
                 seed=50),
]
PACKED_BY_NAME = {c.name: c for c in PACKED_CONFIGS}
