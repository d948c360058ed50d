"""Plain, slow CPU oracle of the Library-of-Layers routed-core forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (``runtime_routed_transformer_amd/csrc``); the two meet only in the
seeded input generator, which holds none of the method's arithmetic.

Sources (the four pages on the method):
  [paper]  "Library of Layers (LoL): Adaptively Ordering Transformer Layers
           at Runtime", arXiv HTML: Sec. 3.2.1 (strided window attention),
           Sec. 3.2.2 (router), Appendix A (Algorithm 1, architecture and
           loss-free balancing paragraphs, FiLM).
  [blog]   "Library of Layers: a transformer that picks its own layer order"
           (ai.satyajit.si): "The forward pass, term by term" and "How the
           order is chosen" (the router in fp32, biased top-1).
  [review] "Library of Layers: Routing Whole Transformer Blocks at Runtime"
           (zhongzhuzhou.org): Eqs. (1)-(5), (7) and the reader's Algorithm 1.

Arithmetic: everything in float64 (inputs are fp32 or bf16-exact fp32 values,
upcast exactly), except the router's score-and-select step: the blog ("How
the order is chosen") states that the router casts its input to fp32 before
its linear layer, so this oracle also evaluates that step in fp32 and both
sides decide the argmax in the same precision.  Activations are never
rounded to bf16.

Readings of points the pages leave open:
  * RMSNorm eps = 1e-6; Norm_s(x) = g_s * x / sqrt(mean(x^2) + eps) with a
    per-expert gain g_s, followed by the depth FiLM gamma_{l,s}, beta_{l,s}
    that is shared by all experts (review Eq. 7; paper App. A).  Variant
    "depth_expert" (the released configs' depth_expert_film flag, blog
    "Where the configs and the text disagree"): one FiLM pair per depth and
    expert, taken from the window's chosen expert.
  * Router tied across depths (blog "How the order is chosen": tied by
    default).  Variant "per_depth" (paper App. B, Fig. 9, untied router):
    W_r and b_r of routed depth l route that depth; e^(l) is per depth in
    both.
  * RoPE: theta = 10000, rotate-half pairing (j, j + d_h/2), angle
    pos * theta^(-2j/d_h), positions = token index in the document.
  * Bias-free attention with scale 1/sqrt(d_h) and a causal mask confined
    to the window; pre-norm block h = x + Attn(Norm(x)), y = h + MLP(Norm(h)).
  * SwiGLU MLP silu(u W_g^T) * (u W_u^T) then W_d; GELU variant uses the
    exact erf form with two matrices.
  * Argmax ties go to the lowest expert index; margin = top-1 minus top-2 of
    (a + b) in probability units (+inf when L = 1).
  * Forcing: forced id >= 0 replaces the router's choice; the gate is the
    forced gate if given and not NaN, else the router's unbiased a_rho.
  * Packed documents: each document is partitioned, routed and attended as
    a row of its own (window offsets from its first token, window 0 from
    its own first token, prefix means over its own windows only).

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
(worked values printed on the pages, closed forms, library routines on
special cases, brute force and invariants).  The end-to-end values of a
random forward are pinned only through those invariants; the pages print no
numeric forward output.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import List, Optional, Tuple

import numpy as np
from scipy.special import erf


# --------------------------------------------------------------------------
# a1. Strided window partition
#   [paper] Sec. 3.2.1 and Algorithm 1 (window preparation): the offset is
#   delta_l = ((l-1) S) mod W and position i belongs to window
#   floor((i + delta_l) / W).  [review] Eq. (2): no cyclic wrap, the modulo
#   applies to the offset only.
# --------------------------------------------------------------------------
def window_offset(depth: int, W: int, S: int) -> int:
    return ((depth - 1) * S) % W


def window_ids(n: int, W: int, S: int, depth: int) -> np.ndarray:
    """w_l(i) for i = 0..n-1 (depth is 1-based)."""
    delta = window_offset(depth, W, S)
    return (np.arange(n) + delta) // W


def partition(n: int, W: int, S: int, depth: int) -> List[Tuple[int, int]]:
    """Windows of depth ``depth`` as (first, last) inclusive, in ordinal order.

    Built from the set definition I_k = {i : w_l(i) = k}: the ordinals are
    consecutive from 0, so each I_k is a run of consecutive positions.
    """
    w = window_ids(n, W, S, depth)
    out = []
    for k in range(int(w[-1]) + 1):
        members = np.nonzero(w == k)[0]
        out.append((int(members[0]), int(members[-1])))
    return out


# --------------------------------------------------------------------------
# a2, a3. Window means and the prefix router input
#   [paper] Algorithm 1: mu_k = Mean(s_{I_k}); r_0 = (e^(l) + s_0) / 2 with a
#   learned depth vector; r_k = (1/k) sum_{j<k} mu_j (mean of prior windows
#   only).  [review] Eq. (4): equal weight per window, not per token.
# --------------------------------------------------------------------------
def window_means(s_row: np.ndarray, windows) -> np.ndarray:
    return np.stack([s_row[a:b + 1].mean(axis=0) for a, b in windows])


def router_inputs(s_row: np.ndarray, windows, e_depth: np.ndarray) -> np.ndarray:
    mu = window_means(s_row, windows)
    r = np.empty_like(mu)
    r[0] = 0.5 * (e_depth + s_row[0])
    for k in range(1, len(windows)):
        r[k] = mu[:k].sum(axis=0) / k
    return r


# --------------------------------------------------------------------------
# a4. Score and select
#   [blog] "The forward pass, term by term", steps 3 and 4, and "How the
#   order is chosen": the router's linear layer runs in fp32, then a
#   softmax and a biased top-1 whose weight is the unbiased score.  [paper] App. A (loss-free
#   balancing): rho = argmax_m (a_m + b_m), alpha = a_rho.  [review] Eq. (5).
#   Training noise is off at inference ([review] reader's Algorithm 1 note).
# --------------------------------------------------------------------------
@dataclass
class Route:
    expert: int
    gate: float      # alpha = a_rho (unbiased), or the forced gate
    margin: float    # (a+b)_top1 - (a+b)_top2, +inf for a one-expert library
    probs: np.ndarray  # a (fp32)


def route(r: np.ndarray, w_r: np.ndarray, b_r: np.ndarray,
          expert_bias: np.ndarray) -> Route:
    r32 = np.asarray(r, np.float64).astype(np.float32)
    # fp32 linear layer; the dot products are formed exactly in float64 and
    # rounded once to fp32 (the correctly rounded fp32 result)
    z = (w_r.astype(np.float64) @ r32.astype(np.float64)).astype(np.float32)
    z = (z + b_r.astype(np.float32)).astype(np.float32)
    ez = np.exp(z - z.max())                      # fp32 exp
    a = (ez / ez.sum(dtype=np.float32)).astype(np.float32)
    scores = (a + expert_bias.astype(np.float32)).astype(np.float32)
    rho = int(np.argmax(scores))                  # first maximum = lowest index
    if len(scores) > 1:
        margin = float(scores[rho]) - float(np.max(np.delete(scores, rho)))
    else:
        margin = math.inf
    return Route(rho, float(a[rho]), margin, a)


# --------------------------------------------------------------------------
# a6-a12. One library block on one window
#   [paper] App. A: RoPE, RMSNorm, SwiGLU, bias-free attention; depth FiLM
#   gamma_s * Norm_s(x) + beta_s in place of each norm.  [paper] Sec. 3.2.1:
#   causal attention restricted to the window.  [review] Eq. (1) (scale
#   1/sqrt(d_h)) and Eq. (7) (FiLM).  [blog] step 5: a full pre-norm
#   residual block.
# --------------------------------------------------------------------------
@dataclass
class BlockParams:
    wq: np.ndarray    # [d][d]  (out, in)
    wk: np.ndarray
    wv: np.ndarray
    wo: np.ndarray    # [d][d]
    w_up: np.ndarray  # SwiGLU: W_u [f][d]; GELU: W_1 [f][d]
    w_gate: Optional[np.ndarray]  # SwiGLU: W_g [f][d]; GELU: None
    w_down: np.ndarray  # [d][f]
    g_attn: np.ndarray
    g_ffn: np.ndarray


def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    return gain * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE on x [len][H][d_h] at the given positions."""
    if theta == 0.0:
        return x
    dh = x.shape[-1]
    half = dh // 2
    inv_freq = theta ** (-2.0 * np.arange(half) / dh)          # omega_j
    ang = positions[:, None].astype(np.float64) * inv_freq[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def window_causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """softmax(q k^T / sqrt(d_h)) v over keys j <= i, all inside one window.

    q, k, v: [len][H][d_h] -> [len][H][d_h]
    """
    ln, H, dh = q.shape
    out = np.empty_like(q)
    allowed = np.tril(np.ones((ln, ln), dtype=bool))
    for h in range(H):
        sc = (q[:, h, :] @ k[:, h, :].T) / math.sqrt(dh)
        sc = np.where(allowed, sc, -np.inf)
        sc = sc - sc.max(axis=1, keepdims=True)
        p = np.exp(sc)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, h, :]
    return out


def silu(x):
    return x / (1.0 + np.exp(-x))


def gelu_erf(x):
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def expert_block(x: np.ndarray, p: BlockParams, n_heads: int, positions: np.ndarray,
                 film: Optional[Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]],
                 eps: float, rope_theta: float) -> np.ndarray:
    """E_m(x) for one window x [len][d] (float64); returns y [len][d]."""
    ln, d = x.shape
    dh = d // n_heads
    u = rms_norm(x, p.g_attn, eps)
    if film is not None:
        u = film[0] * u + film[1]
    q = (u @ p.wq.T).reshape(ln, n_heads, dh)
    k = (u @ p.wk.T).reshape(ln, n_heads, dh)
    v = (u @ p.wv.T).reshape(ln, n_heads, dh)
    q = rope(q, positions, rope_theta)
    k = rope(k, positions, rope_theta)
    o = window_causal_attention(q, k, v).reshape(ln, d)
    h = x + o @ p.wo.T
    u2 = rms_norm(h, p.g_ffn, eps)
    if film is not None:
        u2 = film[2] * u2 + film[3]
    if p.w_gate is not None:
        mid = silu(u2 @ p.w_gate.T) * (u2 @ p.w_up.T)
    else:
        mid = gelu_erf(u2 @ p.w_up.T)
    return h + mid @ p.w_down.T


# --------------------------------------------------------------------------
# The routed core: Algorithm 1 of [paper] App. A, routed-depth loop only
# (the prelude output s^(0) is the input, the coda is not part of it).
# Every window at depth l reads s^(l-1); the new states replace the old ones
# only after all windows ([review] reader's Algorithm 1 and the note after
# it: window means are taken from the unchanged depth input).
# --------------------------------------------------------------------------
@dataclass
class OracleResult:
    s: np.ndarray              # s^(D) [B][n][d] float32
    s64: np.ndarray            # s^(D) float64 (before the final rounding)
    expert: np.ndarray         # [D][B][K_max] int32, -1 beyond K_l
    gate: np.ndarray           # [D][B][K_max] float32, 0 beyond K_l
    margin: np.ndarray         # [D][B][K_max] float32


def expert_params(inp, m: int) -> BlockParams:
    cfg = inp.cfg
    d, f = cfg.d, cfg.d_ffn
    f64 = lambda a: np.asarray(a, np.float64)
    wqkv = f64(inp.wqkv[m])
    if cfg.mlp == "swiglu":
        w_gate, w_up = f64(inp.w_gu[m][:f]), f64(inp.w_gu[m][f:])
    else:
        w_gate, w_up = None, f64(inp.w_gu[m])
    return BlockParams(wqkv[:d], wqkv[d:2 * d], wqkv[2 * d:], f64(inp.wo[m]),
                       w_up, w_gate, f64(inp.w_down[m]),
                       f64(inp.g_attn[m]), f64(inp.g_ffn[m]))


def forward(inp, forced_expert: Optional[np.ndarray] = None,
            forced_gate: Optional[np.ndarray] = None,
            rows: Optional[List[int]] = None, n_tokens: Optional[int] = None) -> OracleResult:
    """Run the routed core on ``inp`` (a ``CoreInputs``).

    forced_expert / forced_gate: [D][B][K_max]; id -1 (or gate NaN) = free.
    rows / n_tokens: optionally restrict to some batch rows and to the first
    ``n_tokens`` positions of each (a document prefix; by the causality of the
    core, outputs and routes inside the prefix equal those of the full run).
    """
    cfg = inp.cfg
    rows = list(range(cfg.batch)) if rows is None else list(rows)
    n = cfg.n if n_tokens is None else int(n_tokens)
    D, L, K_max = cfg.D, cfg.L, cfg.k_max
    params = [expert_params(inp, m) for m in range(L)]
    per_depth = getattr(cfg, "router", "tied") == "per_depth"
    per_expert_film = getattr(cfg, "film_mode", "depth") == "depth_expert"
    w_r_all = np.asarray(inp.w_r, np.float32)
    b_r_all = np.asarray(inp.b_r, np.float32)
    bias = np.asarray(inp.expert_bias, np.float32)
    s = np.asarray(inp.s0[rows, :n], np.float64).copy()
    expert = np.full((D, len(rows), K_max), -1, np.int32)
    gate = np.zeros((D, len(rows), K_max), np.float32)
    margin = np.zeros((D, len(rows), K_max), np.float32)
    for depth in range(1, D + 1):
        windows = partition(n, cfg.W, cfg.S, depth)
        # the router of this depth (untied) or the shared one
        w_r = w_r_all[depth - 1] if per_depth else w_r_all
        b_r = b_r_all[depth - 1] if per_depth else b_r_all

        def film_of(rho):
            # (gamma_attn, beta_attn, gamma_ffn, beta_ffn) of this depth, and
            # of expert rho in the per-(depth, expert) variant
            if inp.film_gamma is None:
                return None
            fg = np.asarray(inp.film_gamma[depth - 1], np.float64)
            fb = np.asarray(inp.film_beta[depth - 1], np.float64)
            if per_expert_film:
                fg, fb = fg[rho], fb[rho]
            return (fg[0], fb[0], fg[1], fb[1])
        s_next = s.copy()
        for bi, b in enumerate(rows):
            r = router_inputs(s[bi], windows, np.asarray(inp.e_depth[depth - 1], np.float64))
            for k, (a0, a1) in enumerate(windows):
                rt = route(r[k], w_r, b_r, bias)
                rho, alpha = rt.expert, rt.gate
                if forced_expert is not None and forced_expert[depth - 1, b, k] >= 0:
                    rho = int(forced_expert[depth - 1, b, k])
                    alpha = float(rt.probs[rho])
                if forced_gate is not None and not np.isnan(forced_gate[depth - 1, b, k]):
                    alpha = float(forced_gate[depth - 1, b, k])
                x = s[bi, a0:a1 + 1]
                y = expert_block(x, params[rho], cfg.n_heads, np.arange(a0, a1 + 1), film_of(rho),
                                 cfg.rms_eps, cfg.rope_theta)
                s_next[bi, a0:a1 + 1] = x + np.float64(np.float32(alpha)) * (y - x)
                expert[depth - 1, bi, k] = rho
                gate[depth - 1, bi, k] = alpha
                margin[depth - 1, bi, k] = rt.margin
        s = s_next
    return OracleResult(s.astype(np.float32), s, expert, gate, margin)


# --------------------------------------------------------------------------
# Packed documents
#   [paper] Appendix A: attention is blocked by document (no token attends
#   to another document).  [blog] "The forward pass, term by term": the
#   router's cumulative sum over window means restarts at each document
#   boundary.  [review] "Deriving prefix-only routing": packed execution
#   needs the routing summaries reset and isolated per document.
# Reading: a document of a packed stream is partitioned from its own first
# token (window offsets count from it), routed with its own window-0 rule
# and its own prefix means, and attended inside itself, so its result is the
# core's result on that document run alone as a row of its own length.
# --------------------------------------------------------------------------
def forward_docs(inp, lengths, forced_expert: Optional[np.ndarray] = None,
                 forced_gate: Optional[np.ndarray] = None) -> List[OracleResult]:
    """Document b = the first ``lengths[b]`` tokens of row b of ``inp.s0``;
    returns one result per document (batch axis of length 1), each computed
    with only that document's tokens present."""
    out = []
    for b, ln in enumerate(lengths):
        fe = None if forced_expert is None else forced_expert[:, b:b + 1]
        fg = None if forced_gate is None else forced_gate[:, b:b + 1]
        one = dataclasses.replace(inp, s0=np.asarray(inp.s0[b:b + 1, :int(ln)]))
        one_cfg = dataclasses.replace(inp.cfg, batch=1, n=int(ln))
        one = dataclasses.replace(one, cfg=one_cfg)
        r = forward(one, forced_expert=None if fe is None else _fit_slots(fe, one_cfg.k_max),
                    forced_gate=None if fg is None else _fit_slots(fg, one_cfg.k_max))
        out.append(r)
    return out


def _fit_slots(a: np.ndarray, k: int) -> np.ndarray:
    """The first k window slots of a [D][1][K_max] forcing array."""
    return np.ascontiguousarray(a[:, :, :k])


# --------------------------------------------------------------------------
# Incremental decode
#   [review] "Deriving prefix-only routing": a window's route and gate are
#   fixed when the window opens, since the router reads only earlier,
#   completed windows (and, for window 0, the document's first token);
#   serving keeps per-depth window boundaries and summaries.  [blog] "What it
#   costs": attention never leaves the window, so a depth only needs the open
#   window's keys and values, computed by the block that window runs.
# One token of a document enters at a time.  At every routed depth the
# state is: the sum of the completed windows' means, the running sum and
# length of the open window, its route, and its keys and values.  When a
# token opens a window, the window before it (if any) is closed and its mean
# joins the prefix sum, the new window is routed from the prefix (or by the
# window-0 rule) and its cache starts empty.  The token then runs the
# window's block against the cached keys and values plus its own.
# --------------------------------------------------------------------------
@dataclass
class DecodeState:
    prefix: np.ndarray       # [D][d] sum of completed window means
    cur_sum: np.ndarray      # [D][d] sum of the open window's depth inputs
    cur_len: np.ndarray      # [D]
    expert: np.ndarray       # [D] route of the open window
    gate: np.ndarray         # [D]
    keys: list               # [D] list of [H][d_h] arrays (rotated)
    values: list             # [D] list of [H][d_h] arrays


def decode_state(D: int, d: int) -> DecodeState:
    return DecodeState(np.zeros((D, d)), np.zeros((D, d)), np.zeros(D, np.int64),
                       np.full(D, -1, np.int64), np.zeros(D), [[] for _ in range(D)],
                       [[] for _ in range(D)])


def block_step(x: np.ndarray, p: BlockParams, n_heads: int, pos: int, film, eps: float,
               rope_theta: float, keys: list, values: list) -> np.ndarray:
    """E_m on one token x [d] at document position ``pos``: its key and value
    join ``keys`` / ``values`` (the open window's), and its query attends to
    all of them."""
    d = x.shape[0]
    dh = d // n_heads
    u = rms_norm(x[None], p.g_attn, eps)
    if film is not None:
        u = film[0] * u + film[1]
    at = np.array([pos])
    q = rope((u @ p.wq.T).reshape(1, n_heads, dh), at, rope_theta)[0]
    k = rope((u @ p.wk.T).reshape(1, n_heads, dh), at, rope_theta)[0]
    v = (u @ p.wv.T).reshape(n_heads, dh)
    keys.append(k)
    values.append(v)
    K = np.stack(keys)          # [j][H][d_h]
    V = np.stack(values)
    o = np.empty((n_heads, dh))
    for h in range(n_heads):
        sc = K[:, h, :] @ q[h] / math.sqrt(dh)
        w = np.exp(sc - sc.max())
        o[h] = (w / w.sum()) @ V[:, h, :]
    hh = x + o.reshape(d) @ p.wo.T
    u2 = rms_norm(hh[None], p.g_ffn, eps)[0]
    if film is not None:
        u2 = film[2] * u2 + film[3]
    if p.w_gate is not None:
        mid = silu(u2 @ p.w_gate.T) * (u2 @ p.w_up.T)
    else:
        mid = gelu_erf(u2 @ p.w_up.T)
    return hh + mid @ p.w_down.T


def decode(inp, n_tokens: int, forced_expert: Optional[np.ndarray] = None,
           forced_gate: Optional[np.ndarray] = None,
           rows: Optional[List[int]] = None) -> OracleResult:
    """Feed tokens 0 .. n_tokens-1 of each document (row of ``inp.s0``) one
    at a time; returns s^(D) of every token and the path, laid out as
    ``forward``'s result."""
    cfg = inp.cfg
    rows = list(range(cfg.batch)) if rows is None else list(rows)
    D, L, W, K_max = cfg.D, cfg.L, cfg.W, cfg.k_max
    params = [expert_params(inp, m) for m in range(L)]
    per_depth = getattr(cfg, "router", "tied") == "per_depth"
    per_expert_film = getattr(cfg, "film_mode", "depth") == "depth_expert"
    bias = np.asarray(inp.expert_bias, np.float32)
    out = np.zeros((len(rows), n_tokens, cfg.d))
    expert = np.full((D, len(rows), K_max), -1, np.int32)
    gate = np.zeros((D, len(rows), K_max), np.float32)
    margin = np.zeros((D, len(rows), K_max), np.float32)
    for bi, b in enumerate(rows):
        st = decode_state(D, cfg.d)
        for i in range(n_tokens):
            x = np.asarray(inp.s0[b, i], np.float64)
            for l in range(D):
                delta = window_offset(l + 1, W, cfg.S)
                k = (i + delta) // W
                if i == max(0, k * W - delta):
                    # the token opens window k: close k - 1, route k
                    if k > 0:
                        st.prefix[l] += st.cur_sum[l] / st.cur_len[l]
                    r = (0.5 * (np.asarray(inp.e_depth[l], np.float64) + x) if k == 0
                         else st.prefix[l] / k)
                    w_r = np.asarray(inp.w_r[l] if per_depth else inp.w_r, np.float32)
                    b_r = np.asarray(inp.b_r[l] if per_depth else inp.b_r, np.float32)
                    rt = route(r, w_r, b_r, bias)
                    rho, alpha = rt.expert, rt.gate
                    if forced_expert is not None and forced_expert[l, b, k] >= 0:
                        rho = int(forced_expert[l, b, k])
                        alpha = float(rt.probs[rho])
                    if forced_gate is not None and not np.isnan(forced_gate[l, b, k]):
                        alpha = float(forced_gate[l, b, k])
                    st.expert[l], st.gate[l] = rho, alpha
                    st.cur_sum[l] = 0.0
                    st.cur_len[l] = 0
                    st.keys[l], st.values[l] = [], []
                    expert[l, bi, k], gate[l, bi, k], margin[l, bi, k] = rho, alpha, rt.margin
                st.cur_sum[l] += x
                st.cur_len[l] += 1
                rho = int(st.expert[l])
                film = None
                if inp.film_gamma is not None:
                    fg = np.asarray(inp.film_gamma[l], np.float64)
                    fb = np.asarray(inp.film_beta[l], np.float64)
                    if per_expert_film:
                        fg, fb = fg[rho], fb[rho]
                    film = (fg[0], fb[0], fg[1], fb[1])
                y = block_step(x, params[rho], cfg.n_heads, i, film, cfg.rms_eps,
                               cfg.rope_theta, st.keys[l], st.values[l])
                x = x + np.float64(np.float32(st.gate[l])) * (y - x)
            out[bi, i] = x
    return OracleResult(out.astype(np.float32), out, expert, gate, margin)


# --------------------------------------------------------------------------
# Around the core: embedding, fixed-order stacks, vocabulary readout
#   [paper] Appendix A, Algorithm 1: the prelude is applied to the token
#   sequence, the routed core follows, then the causal coda and the
#   vocabulary readout.  Sec. 3.1: prelude and coda are fixed-order stacks
#   of decoder layers with full causal attention.
# Readings: the token sequence enters through an embedding table (one row
# per token id); the readout is a final RMSNorm with a gain followed by a
# linear map onto the vocabulary, giving logits (the pages' softmax over
# them is left to the consumer); the vocabulary size is a free parameter.
# --------------------------------------------------------------------------
def embed(tokens: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Rows of the embedding table, float64 [B][n][d]."""
    return np.asarray(table, np.float64)[np.asarray(tokens)]


def causal_stack(x: np.ndarray, params: List[BlockParams], n_heads: int, eps: float,
                 theta: float) -> np.ndarray:
    """Apply the blocks in order to one document x [n][d], attention causal
    over the whole document (the window is the document)."""
    positions = np.arange(x.shape[0])
    for p in params:
        x = expert_block(x, p, n_heads, positions, None, eps, theta)
    return x


def lm_head(s: np.ndarray, g_final: np.ndarray, w_vocab: np.ndarray, eps: float) -> np.ndarray:
    """logits = RMSNorm_g(s) W_vocab^T, float64."""
    return rms_norm(np.asarray(s, np.float64), np.asarray(g_final, np.float64), eps) @ \
        np.asarray(w_vocab, np.float64).T


@dataclass
class FullResult:
    logits: np.ndarray         # [B][n][V] float64
    prelude_out: np.ndarray    # [B][n][d] float64 (s^(0) of the core)
    core: OracleResult         # the routed core on it
    coda_out: np.ndarray       # [B][n][d] float64


def full_forward(full, core_forced_expert: Optional[np.ndarray] = None,
                 core_forced_gate: Optional[np.ndarray] = None) -> FullResult:
    """Algorithm 1 end to end: embedding, prelude stack, routed core, coda
    stack, readout.  ``full`` is a ``FullInputs``; the forcing arrays go to
    the routed core as in ``forward``."""
    core_cfg = full.core.cfg
    pre = [expert_params(full.prelude, m) for m in range(full.prelude.cfg.L)]
    coda = [expert_params(full.coda, m) for m in range(full.coda.cfg.L)]
    x = embed(full.tokens, full.embedding)
    h0 = np.stack([causal_stack(x[b], pre, core_cfg.n_heads, core_cfg.rms_eps, core_cfg.rope_theta)
                   for b in range(core_cfg.batch)])
    # the core's input s^(0) is fp32, as on the device
    core_in = dataclasses.replace(full.core, s0=h0.astype(np.float32))
    res = forward(core_in, forced_expert=core_forced_expert, forced_gate=core_forced_gate)
    hD = np.stack([causal_stack(res.s64[b], coda, core_cfg.n_heads, core_cfg.rms_eps,
                                core_cfg.rope_theta) for b in range(core_cfg.batch)])
    logits = np.stack([lm_head(hD[b], full.g_final, full.w_vocab, core_cfg.rms_eps)
                       for b in range(core_cfg.batch)])
    return FullResult(logits, h0, res, hD)
