"""GPU parity: the HIP routed core (through the C ABI) against the CPU oracle.

Sizes the oracle finishes in seconds but that still span several GEMM tiles,
several windows per document and ragged tails (half windows, partial M
tiles); then every workload at its full size in the launch configuration
the benchmark times, compared on sampled documents and a document prefix
(by the core's causality those outputs equal the full run's), and edge cases.
"""
import math
import sys

import numpy as np
import pytest

from runtime_routed_transformer_amd.workloads import CONFIG_BY_NAME, CoreConfig
from tests import parity

pytestmark = pytest.mark.gpu


def _report(rep):
    print(rep, flush=True)
    sys.stdout.flush()
    assert rep.ok, str(rep)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from runtime_routed_transformer_amd import binding
    binding.load()


SCALED = [
    CONFIG_BY_NAME["tiny_fp32"],
    CONFIG_BY_NAME["small_bf16"].scaled(2, 384),
    CONFIG_BY_NAME["mid_bf16"].scaled(2, 640),
    # 2,048 tokens: enough 256 x 256 gate/up tiles to fill the CUs, so the
    # shifted depths (half windows at the document edges) run mixed tiles
    CONFIG_BY_NAME["mid_bf16"].scaled(2, 1024),
    CONFIG_BY_NAME["sparse_bf16"].scaled(2, 640),
    CONFIG_BY_NAME["forced_bf16"].scaled(3, 224),
]


@pytest.mark.parametrize("cfg", SCALED, ids=lambda c: c.name)
def test_parity_scaled(cfg):
    print(f"[parity] {cfg.name}", flush=True)
    _report(parity.run(parity.prepare(cfg)))


@pytest.mark.parametrize("name", ["small_bf16", "mid_bf16", "sparse_bf16", "forced_bf16"])
def test_parity_full_size_sampled(name):
    cfg = CONFIG_BY_NAME[name]
    print(f"[parity-full] {cfg.name}", flush=True)
    inp = parity.prepare(cfg)
    _report(parity.run(inp, rows=[0, cfg.batch - 1], n_tokens=min(cfg.n, 3 * cfg.W + cfg.W // 2)))


def test_parity_bench_workload_complete():
    """The benchmark's workload (mid_bf16: 4 documents of 4,096 tokens, 8
    experts, 8 depths) compared with the oracle on every token of every
    document, not on a sample."""
    cfg = CONFIG_BY_NAME["mid_bf16"]
    print(f"[parity-complete] {cfg.name}", flush=True)
    _report(parity.run(parity.prepare(cfg)))


EDGE = [
    CoreConfig("edge_fp32_ragged", batch=2, n=37, d=64, n_heads=2, d_ffn=128, L=3, D=4, W=5, S=3,
               mlp="swiglu", dtype="fp32", seed=21),
    CoreConfig("edge_bf16_ragged", batch=2, n=150, d=128, n_heads=2, d_ffn=256, L=3, D=3, W=40,
               S=13, mlp="swiglu", dtype="bf16", seed=22),
    CoreConfig("edge_bf16_gelu_nofilm", batch=1, n=200, d=256, n_heads=4, d_ffn=512, L=2, D=2,
               W=96, S=48, mlp="gelu", dtype="bf16", seed=23, film=False),
    CoreConfig("edge_one_token", batch=1, n=1, d=128, n_heads=2, d_ffn=128, L=2, D=2, W=4, S=1,
               mlp="swiglu", dtype="bf16", seed=24),
    CoreConfig("edge_window_longer_than_doc", batch=3, n=50, d=128, n_heads=4, d_ffn=256, L=4,
               D=3, W=64, S=40, mlp="swiglu", dtype="bf16", seed=25),
    CoreConfig("edge_stride_zero_L1", batch=2, n=96, d=64, n_heads=1, d_ffn=64, L=1, D=3, W=32,
               S=0, mlp="gelu", dtype="fp32", seed=26, rope_theta=0.0),
    CoreConfig("edge_stride_ge_window", batch=2, n=100, d=128, n_heads=2, d_ffn=128, L=3, D=3,
               W=16, S=37, mlp="swiglu", dtype="bf16", seed=27),
    CoreConfig("edge_dh32_bf16", batch=2, n=130, d=128, n_heads=4, d_ffn=384, L=5, D=2, W=64,
               S=32, mlp="swiglu", dtype="bf16", seed=28),
    # at the limits: 64 experts (all used) and 64 documents x 128 window
    # slots = 8,192 windows per depth, the most one bucketing pass takes;
    # windows of 1 and 2 tokens, so nearly every M tile is partial (among 64
    # experts most top-1 margins fall under the near-tie threshold, so most
    # windows run forced to the oracle's choice; ids are compared on the rest)
    CoreConfig("edge_limit_experts_slots", batch=64, n=254, d=128, n_heads=2, d_ffn=128, L=64,
               D=2, W=2, S=1, mlp="swiglu", dtype="bf16", seed=41),
    # a wide model: d = 4,096 (64 heads), on a short document
    CoreConfig("edge_limit_wide_d", batch=1, n=40, d=4096, n_heads=64, d_ffn=256, L=2, D=2,
               W=16, S=8, mlp="swiglu", dtype="bf16", seed=42),
]


# the untied router (one W_r, b_r per routed depth) and per-(depth, expert)
# FiLM, on the fused bf16 path (d = 512 and 1024), the unfused bf16 path
# (d = 128) and fp32
VARIANTS = [
    CONFIG_BY_NAME["small_bf16"].scaled(2, 384).with_(
        name="variant_small_untied_expertfilm", router="per_depth", film_mode="depth_expert"),
    CONFIG_BY_NAME["mid_bf16"].scaled(1, 640).with_(
        name="variant_mid_untied_expertfilm", router="per_depth", film_mode="depth_expert"),
    CoreConfig("variant_bf16_d128_untied", batch=2, n=150, d=128, n_heads=2, d_ffn=256, L=3, D=3,
               W=40, S=13, mlp="swiglu", dtype="bf16", seed=31, router="per_depth",
               film_mode="depth_expert"),
    CoreConfig("variant_fp32_untied_expertfilm", batch=2, n=37, d=64, n_heads=2, d_ffn=128, L=3,
               D=4, W=5, S=3, mlp="swiglu", dtype="fp32", seed=32, router="per_depth",
               film_mode="depth_expert"),
]


@pytest.mark.parametrize("cfg", VARIANTS, ids=lambda c: c.name)
def test_parity_variants(cfg):
    print(f"[parity-variant] {cfg.name}", flush=True)
    _report(parity.run(parity.prepare(cfg)))


@pytest.mark.parametrize("cfg", EDGE, ids=lambda c: c.name)
def test_parity_edge_cases(cfg):
    print(f"[parity-edge] {cfg.name}", flush=True)
    _report(parity.run(parity.prepare(cfg)))


def test_parity_short_k_shapes():
    """K = 512 with every expert's row count a multiple of 256 (d = d_ffn =
    512, full 256-token windows, no shift): QKV (with RoPE) and gate/up run
    on two 256 x 128 workgroups per CU, the shape chosen for 16 stages of K
    or fewer; compared on the first and last documents."""
    cfg = CoreConfig("short_k_2x2", batch=8, n=2048, d=512, n_heads=8, d_ffn=512, L=4, D=2,
                     W=256, S=0, mlp="swiglu", dtype="bf16", seed=44)
    print(f"[parity] {cfg.name}", flush=True)
    _report(parity.run(parity.prepare(cfg), rows=[0, cfg.batch - 1], n_tokens=3 * cfg.W + cfg.W // 2))


def test_parity_activations_beyond_2_gib():
    """T x d_ffn bf16 values above 2 GiB (131,200 tokens, d_ffn 8,192): the
    gate/up output and the down projection's input stay row-major, because
    the GEMMs step through k panels with 32-bit offsets; compared on the
    first and last documents."""
    cfg = CoreConfig("acts_beyond_2gib", batch=2, n=65600, d=128, n_heads=2, d_ffn=8192, L=2, D=2,
                     W=64, S=32, mlp="swiglu", dtype="bf16", seed=46)
    assert cfg.tokens * cfg.d_ffn * 2 > 2 ** 31
    print(f"[parity] {cfg.name}", flush=True)
    _report(parity.run(parity.prepare(cfg), rows=[0, cfg.batch - 1], n_tokens=3 * cfg.W + cfg.W // 2))


def test_parity_many_experts_clear_margins():
    """Free routing over 32 experts with every route clear of the near-tie
    threshold: W_r drawn with std 1.0 instead of 0.02 makes the router's
    probabilities peaked (at 0.02 most margins among 32 experts fall under
    1e-3 and those windows run forced).  All 144 windows' ids, gates and
    margins are compared and none is forced; 16 to 19 experts are used per
    depth.  The 50x larger router weights carry the bf16 states' rounding
    50x into the later depths' logits, so those gates get 50x the usual
    bound; depth 1, which routes the same s^(0) on both sides, keeps 1e-5."""
    cfg = CoreConfig("free_L32_clear_margins", batch=8, n=1024, d=1024, n_heads=16, d_ffn=4096,
                     L=32, D=4, W=256, S=128, mlp="swiglu", dtype="bf16", seed=43, router_std=1.0)
    print(f"[parity] {cfg.name}", flush=True)
    rep = parity.run(parity.prepare(cfg), gate_tol_scale=1.0 / 0.02)
    _report(rep)
    assert rep.forced_windows == 0 and rep.ids_compared == 144, str(rep)


def test_gate_zero_identity_and_determinism_and_inplace():
    import torch
    from runtime_routed_transformer_amd.core import DeviceCore
    cfg = CONFIG_BY_NAME["small_bf16"].scaled(2, 256)
    inp = parity.prepare(cfg)
    core = DeviceCore(inp)
    core.set_forcing(forced_gate=np.zeros((cfg.D, cfg.batch, core.k_max), np.float32))
    out = core.forward().cpu().numpy()
    np.testing.assert_array_equal(out, inp.s0)
    core.set_forcing()
    a = core.forward().clone()
    b = core.forward().clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b), "two runs differ"
    # out of place, the first depth reads s0 directly: it must stay untouched
    np.testing.assert_array_equal(core.s0.cpu().numpy(), inp.s0)
    s = core.s0.clone()
    core.forward(s_in=s, s_out=s)
    torch.cuda.synchronize()
    assert torch.equal(s, a), "in-place run differs"


@pytest.mark.parametrize("name", ["mid_bf16", "small_bf16", "tiny_bf16_gelu"])
def test_prepared_weight_panels_give_the_row_major_result(name):
    """The grouped GEMMs reading wqkv, w_gu and w_down from the 32-k panels of
    lol_prepare_weight_panels compute bit for bit what they compute from the
    row-major matrices (only addresses differ), at every tile shape the
    workload's depths use, for SwiGLU and GELU."""
    import torch
    from runtime_routed_transformer_amd.core import DeviceCore
    if name == "tiny_bf16_gelu":
        cfg = CONFIG_BY_NAME["tiny_fp32"].with_(name=name, dtype="bf16", d=128, d_ffn=256)
    else:
        cfg = CONFIG_BY_NAME[name]
    inp = parity.prepare(cfg)
    core = DeviceCore(inp)
    assert core.weight_panels is not None and core.lib.weight_panels
    with_panels = core.forward().clone()
    core.lib.weight_panels = None
    row_major = core.forward().clone()
    torch.cuda.synchronize()
    assert torch.equal(with_panels, row_major)


def test_forced_own_path_and_bad_forced_id_flag():
    import torch
    from runtime_routed_transformer_amd import binding
    from runtime_routed_transformer_amd.core import DeviceCore
    cfg = CONFIG_BY_NAME["mid_bf16"].scaled(1, 512)
    inp = parity.prepare(cfg)
    core = DeviceCore(inp)
    free = core.forward().clone()
    pe, _, _ = core.path_numpy()
    core.set_forcing(forced_expert=pe)
    again = core.forward().clone()
    torch.cuda.synchronize()
    assert torch.equal(free, again)
    assert core.flags() == 0
    bad = np.full_like(pe, -1)
    bad[0, 0, 0] = cfg.L + 3
    core.set_forcing(forced_expert=bad)
    out = core.forward().clone()
    assert core.flags() & binding.LOL_FLAG_BAD_FORCED_ID
    assert torch.equal(out, free)    # the bad id was treated as free
    assert core.flags() == 0         # reading clears the flag


def test_forward_replays_from_a_hip_graph():
    """The whole forward captured once into a HIP graph (no memsets, no host
    synchronisation, no allocation inside it) and replayed: every replay,
    with eager work and synchronisations between them, equals the eager run."""
    import torch
    from runtime_routed_transformer_amd.core import DeviceCore
    cfg = CONFIG_BY_NAME["mid_bf16"].scaled(2, 512)
    inp = parity.prepare(cfg)
    core = DeviceCore(inp)
    eager = core.forward().clone()
    path_eager = [t.clone() for t in (core.path_expert, core.path_gate, core.path_margin)]
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        core.forward(s_out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, capture_error_mode="relaxed"):
        core.forward(s_out=out)
    for i in range(4):
        out.zero_()
        core.path_expert.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager forward"
        assert torch.equal(core.path_expert, path_eager[0]), f"replay {i}: path differs"
        assert torch.equal(core.path_gate, path_eager[1])
