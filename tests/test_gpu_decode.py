"""GPU parity of incremental decode (lol_decode_step): documents fed one
token at a time through the routed depths, against the oracle.

The oracle side is ``oracle.decode`` for the small cases and
``oracle.forward`` on the same document prefix for the larger ones (the
CPU pins show the two agree to 1e-11: a window's route is fixed when it
opens, review "Deriving prefix-only routing").  As in the forward's parity,
windows whose top-1 margin is at most 1e-3 are forced to the oracle's
choice; ids must match on every other window, and s^(D) of every token must
agree to the mode's tolerance.
"""
import sys

import numpy as np
import pytest

import oracle
from runtime_routed_transformer_amd.workloads import CONFIG_BY_NAME, CoreConfig
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _decode_gpu(inp, forced_expert, forced_gate, n_tokens, in_place=False):
    import torch
    from runtime_routed_transformer_amd.core import DeviceCore, DeviceDecoder

    core = DeviceCore(inp)
    core.set_forcing(forced_expert=forced_expert, forced_gate=forced_gate)
    core.path_expert.fill_(-7)
    dec = DeviceDecoder(core)
    out = torch.empty((inp.cfg.batch, n_tokens, inp.cfg.d), dtype=torch.float32, device=core.device)
    for pos in range(n_tokens):
        x = core.s0[:, pos].contiguous()
        y = dec.step(pos, x, y=x if in_place else None)
        out[:, pos] = y
    torch.cuda.synchronize(core.device)
    flags = dec.flags()
    return out.cpu().numpy(), core.path_numpy(), flags


def _check(inp, n_tokens, use_decode_oracle, forced_gate=None, in_place=False):
    cfg = inp.cfg
    rows = list(range(cfg.batch))
    if use_decode_oracle:
        ref = oracle.decode(inp, n_tokens, forced_expert=inp.forced_expert, forced_gate=forced_gate)
    else:
        ref = oracle.forward(inp, forced_expert=inp.forced_expert, forced_gate=forced_gate,
                             n_tokens=n_tokens)
    forced, compared = parity.forced_for_gpu(inp, ref, rows, n_tokens)
    s_gpu, (pe, pg, pm), flags = _decode_gpu(inp, forced, forced_gate, n_tokens, in_place)
    s_ref = ref.s64
    s0 = inp.s0[:, :n_tokens].astype(np.float64)
    rel = float(np.abs(s_gpu - s_ref).max() / np.abs(s_ref).max())
    upd = float(np.abs((s_gpu - s0) - (s_ref - s0)).max() / np.abs(s_ref - s0).max())
    free_cmp = compared & (ref.margin > parity.MARGIN)
    if inp.forced_expert is not None:
        free_cmp &= inp.forced_expert < 0
    mism = int(np.count_nonzero(free_cmp & (pe != ref.expert)))
    gate_err = float(np.abs(pg - ref.gate)[compared].max())
    margin_err = parity.margin_error(pm[compared], ref.margin[compared])
    # every window slot that opened was written; the others kept the fill
    opened = compared
    assert np.all(pe[opened] >= 0) and np.all(pe[~opened] == -7)
    print(f"{cfg.name}: rel_err={rel:.3e} update_err={upd:.3e} ids "
          f"{int(free_cmp.sum()) - mism}/{int(free_cmp.sum())} gate_err={gate_err:.2e} "
          f"margin_err={margin_err:.2e} flags={flags}", flush=True)
    tol = parity.TOL[cfg.dtype]
    assert flags == 0
    assert mism == 0
    assert rel <= tol and upd <= parity.UPDATE_TOL[cfg.dtype]
    # gates come from fp32 routers on depth inputs that, in bf16 mode, carry
    # the bf16 GEMM operands' rounding of every earlier depth
    assert gate_err <= parity.GATE_TOL[cfg.dtype]
    assert margin_err <= parity.MARGIN_TOL[cfg.dtype]
    return s_gpu


SMALL = CONFIG_BY_NAME["small_bf16"]
CASES = [
    # (config, tokens, oracle.decode?)
    (CONFIG_BY_NAME["tiny_fp32"], 64, True),
    (SMALL.scaled(2, 200), 200, False),
    (CONFIG_BY_NAME["mid_bf16"].scaled(2, 300), 300, False),
    # the benchmark's decode configuration: the 4 documents of the mid
    # workload (4 per pass), the first 300 positions (two windows at depth 1)
    (CONFIG_BY_NAME["mid_bf16"].scaled(4, 300).with_(name="mid_bf16_decode@4x300"), 300, False),
    # 32 experts with skewed bias: up to 4 distinct experts per depth
    (CONFIG_BY_NAME["sparse_bf16"].scaled(4, 270), 270, False),
    # every document on one expert per depth: 20 rows share each weight read
    # (passes of 8, 8 and 4 documents)
    (CONFIG_BY_NAME["forced_bf16"].scaled(20, 72), 72, False),
    # untied router, FiLM per depth and expert
    (SMALL.with_(name="small_untied_expertfilm", router="per_depth",
                 film_mode="depth_expert").scaled(2, 160), 160, False),
    # bf16 GELU, d_head 32, S = 0 (fixed windows), ragged last window
    (CoreConfig("dec_gelu_bf16", batch=3, n=75, d=128, n_heads=4, d_ffn=256, L=3, D=3, W=32,
                S=0, mlp="gelu", dtype="bf16", seed=61), 75, True),
    # one expert (margin +inf, gate 1), no FiLM, no RoPE, S > W
    (CoreConfig("dec_l1_fp32", batch=2, n=40, d=64, n_heads=1, d_ffn=128, L=1, D=2, W=12, S=17,
                mlp="swiglu", dtype="fp32", seed=62, film=False, rope_theta=0.0), 40, True),
    # the largest batch (64 documents: passes of 8 per expert group), 6 experts
    (CoreConfig("dec_b64_bf16", batch=64, n=20, d=128, n_heads=2, d_ffn=256, L=6, D=2, W=8, S=3,
                mlp="swiglu", dtype="bf16", seed=65), 20, True),
    # W = 1: every token opens a window at every depth (the router runs on
    # every token; the cache holds one slot)
    (CoreConfig("dec_w1_bf16", batch=3, n=12, d=128, n_heads=2, d_ffn=128, L=3, D=3, W=1, S=0,
                mlp="swiglu", dtype="bf16", seed=66), 12, True),
    # windows longer than 256 tokens: keys past the first 256 are read from
    # the cache inside the score and value loops (d_head 64 and 32)
    (CoreConfig("dec_w320_bf16", batch=2, n=700, d=128, n_heads=2, d_ffn=256, L=3, D=2, W=320,
                S=100, mlp="swiglu", dtype="bf16", seed=68), 700, False),
    (CoreConfig("dec_w300_fp32", batch=1, n=620, d=64, n_heads=2, d_ffn=128, L=2, D=2, W=300,
                S=77, mlp="gelu", dtype="fp32", seed=69), 620, False),
    # at the decode limits: d = 4,096 (64 heads) and W = 8,192 (a window
    # longer than the document at both depths)
    (CoreConfig("dec_limits_d4096_w8192", batch=2, n=40, d=4096, n_heads=64, d_ffn=256, L=3, D=2,
                W=8192, S=4000, mlp="swiglu", dtype="bf16", seed=70), 40, True),
    # one-token documents; 5 documents (3 per pass group size rounds up to 8)
    (CoreConfig("dec_one_token", batch=5, n=1, d=128, n_heads=4, d_ffn=256, L=2, D=3, W=4, S=1,
                mlp="gelu", dtype="bf16", seed=67), 1, True),
]


@pytest.mark.parametrize("cfg,n_tokens,use_dec", CASES, ids=[c[0].name for c in CASES])
def test_decode_parity(cfg, n_tokens, use_dec):
    print(f"case {cfg.name} tokens {n_tokens}", flush=True)
    inp = parity.prepare(cfg)
    _check(inp, n_tokens, use_dec)


def test_decode_forced_gates_and_in_place():
    """Forced ids and gates, y written over x, on an fp32 and a bf16 case."""
    for cfg in (CONFIG_BY_NAME["tiny_fp32"].with_(name="tiny_forced"),
                CoreConfig("dec_forced_bf16", batch=2, n=90, d=256, n_heads=4, d_ffn=512, L=4,
                           D=3, W=24, S=10, mlp="swiglu", dtype="bf16", seed=63)):
        print(f"case {cfg.name}", flush=True)
        inp = parity.prepare(cfg)
        rng = np.random.default_rng(7)
        shape = (cfg.D, cfg.batch, cfg.k_max)
        fe = rng.integers(-1, cfg.L, size=shape).astype(np.int32)
        fg = np.where(rng.random(shape) < 0.5, np.nan, rng.uniform(0, 1, shape)).astype(np.float32)
        inp.forced_expert = fe
        _check(inp, cfg.n, True, forced_gate=fg, in_place=True)


def test_decode_is_deterministic_and_flags_bad_positions():
    import torch
    from runtime_routed_transformer_amd import binding as B
    from runtime_routed_transformer_amd.core import DeviceCore, DeviceDecoder

    cfg = CoreConfig("dec_flags", batch=2, n=48, d=128, n_heads=2, d_ffn=256, L=3, D=2, W=16,
                     S=5, mlp="swiglu", dtype="bf16", seed=64)
    inp = parity.prepare(cfg)
    core = DeviceCore(inp)
    dec = DeviceDecoder(core)
    runs = []
    for _ in range(2):
        dec.reset()
        outs = [dec.step(p, core.s0[:, p].contiguous()).clone() for p in range(cfg.n)]
        runs.append(torch.stack(outs, 1).cpu().numpy())
    np.testing.assert_array_equal(runs[0], runs[1])
    assert dec.flags() == 0
    # a skipped position is flagged (the kernels stay in bounds)
    dec.reset()
    dec.step(0, core.s0[:, 0].contiguous())
    dec.step(2, core.s0[:, 2].contiguous())
    assert dec.flags() == B.LOL_FLAG_BAD_POS
    # a forced id outside the library is flagged and the window routed freely
    dec.reset()
    core.set_forcing(forced_expert=np.full((cfg.D, cfg.batch, cfg.k_max), cfg.L, np.int32))
    free = runs[0][:, 0]
    got = dec.step(0, core.s0[:, 0].contiguous()).cpu().numpy()
    assert dec.flags() == B.LOL_FLAG_BAD_FORCED_ID
    np.testing.assert_array_equal(got, free)


def test_decode_rows_at_their_own_positions():
    """Serving: every row at its own position (pos = -1).  Rows restart
    their documents at different steps (lol_decode_reset_row); each row's
    output at every step equals the oracle's decode of its document at the
    row's position."""
    import torch
    from runtime_routed_transformer_amd.core import DeviceCore, DeviceDecoder

    cfg = CoreConfig("dec_rows", batch=3, n=40, d=128, n_heads=2, d_ffn=256, L=3, D=3, W=8, S=3,
                     mlp="swiglu", dtype="bf16", seed=70)
    inp = parity.prepare(cfg)
    steps, restart = 30, {1: 5, 2: 11}
    ref = oracle.forward(inp, n_tokens=steps)
    forced, _ = parity.forced_for_gpu(inp, ref, list(range(cfg.batch)), steps)
    core = DeviceCore(inp)
    core.set_forcing(forced_expert=forced)
    dec = DeviceDecoder(core)
    start = [0] * cfg.batch
    got = np.zeros((steps, cfg.batch, cfg.d))
    want = np.zeros_like(got)
    for t in range(steps):
        for b, t0 in restart.items():
            if t == t0:
                dec.reset_row(b)
                start[b] = t
        pos = [t - start[b] for b in range(cfg.batch)]
        x = torch.stack([core.s0[b, pos[b]] for b in range(cfg.batch)]).contiguous()
        got[t] = dec.step(None, x).cpu().numpy()
        want[t] = np.stack([ref.s64[b, pos[b]] for b in range(cfg.batch)])
    assert dec.flags() == 0
    rel = float(np.abs(got - want).max() / np.abs(want).max())
    print(f"rows at own positions: rel_err={rel:.3e}", flush=True)
    assert rel <= parity.TOL["bf16"]


def test_decode_step_replays_from_a_graph():
    """With pos = -1 a decode step has no per-call arguments: captured once
    in a HIP graph (torch.cuda.graph) and replayed per token, it gives the
    eager steps' outputs bit for bit."""
    import torch
    from runtime_routed_transformer_amd.core import DeviceCore, DeviceDecoder

    cfg = CoreConfig("dec_graph", batch=2, n=24, d=128, n_heads=2, d_ffn=256, L=3, D=2, W=8, S=3,
                     mlp="swiglu", dtype="bf16", seed=71)
    inp = parity.prepare(cfg)
    core = DeviceCore(inp)
    dec = DeviceDecoder(core)
    eager = [dec.step(None, core.s0[:, p].contiguous()).clone() for p in range(cfg.n)]
    assert dec.flags() == 0
    x_in = torch.empty((cfg.batch, cfg.d), dtype=torch.float32, device=core.device)
    y_out = torch.empty_like(x_in)
    dec.reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dec.step(None, x_in, y=y_out)
    dec.reset()     # capture ran nothing; start the documents again
    torch.cuda.synchronize()
    for p in range(cfg.n):
        x_in.copy_(core.s0[:, p])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_out, eager[p]), f"position {p}"
    assert dec.flags() == 0
