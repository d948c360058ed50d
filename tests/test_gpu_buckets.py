"""Expert bucketing as a checked result.

A forward groups each depth's windows by chosen expert (the explainer
"Library of Layers: a transformer that picks its own layer order", What it
costs: a batch becomes a grouped dispatch, as in a mixture of experts) and
hands the grouped rows to the expert GEMMs in 128- and 256-row tiles.  Given
the routes, that grouping is unique: windows of expert e in (document,
window) order, one grouped row per token, experts in index order, every
expert's full tiles first and the partial last tiles after them.  This test
reads the last depth's tables through ``lol_core_read_buckets`` and the
per-depth expert counts ``util`` through the path, recomputes all of them on
the CPU from the path's ids and the window lengths of the partition, and
requires them to be equal, entry for entry.
"""
import sys

import numpy as np
import pytest

import oracle
from runtime_routed_transformer_amd.workloads import (CONFIG_BY_NAME, PACKED_BY_NAME, CoreConfig,
                                                      generate_packed)
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def expected_tables(ids, lens, L, T):
    """ids, lens: [slots] expert (-1 = no window) and tokens of each window
    slot, slots in (document, window) order; T = batch n."""
    counts = np.zeros(L, np.int64)
    tok = np.zeros(L, np.int64)
    for e, ln in zip(ids, lens):
        if e >= 0:
            counts[e] += 1
            tok[e] += ln
    row_off = np.concatenate([[0], np.cumsum(tok)])
    win_row0 = np.full(len(ids), -1, np.int64)
    nxt = row_off[:-1].copy()
    for slot, (e, ln) in enumerate(zip(ids, lens)):
        if e >= 0:
            win_row0[slot] = nxt[e]
            nxt[e] += ln

    def tiles(H):
        full = [(e, row_off[e] + i * H) for e in range(L) for i in range(tok[e] // H)]
        part = [(e, row_off[e] + (tok[e] // H) * H) for e in range(L) if tok[e] % H]
        used = full + part
        M = -(-T // H) + L
        return len(used), np.array(used + [(-1, 0)] * (M - len(used)), np.int64).reshape(M, 2)

    n128, t128 = tiles(128)
    n256, t256 = tiles(256)
    return {"counts": counts, "row_off": row_off, "win_row0": win_row0,
            "n_tiles": np.array([n128, n256]), "tiles128": t128, "tiles256": t256}


def _check(core, lens_of_doc, n_docs, cfg):
    """lens_of_doc(b, depth) -> window lengths of document b at that depth."""
    pe, _, _ = core.path_numpy()
    util = core.path_util.cpu().numpy()
    D, L, K_max = cfg.D, cfg.L, core.k_max
    for l in range(D):
        ids = pe[l][pe[l] >= 0]
        np.testing.assert_array_equal(util[l], np.bincount(ids, minlength=L),
                                      err_msg=f"util of depth {l + 1}")
    ids = pe[D - 1].reshape(-1)
    lens = np.zeros(n_docs * K_max, np.int64)
    for b in range(n_docs):
        ln = lens_of_doc(b, D)
        lens[b * K_max:b * K_max + len(ln)] = ln
    assert ((ids >= 0) == (lens > 0)).all(), "a window slot and its route disagree"
    want = expected_tables(ids, lens, L, cfg.batch * cfg.n)
    got = core.read_buckets()
    for name, w in want.items():
        np.testing.assert_array_equal(got[name], w, err_msg=f"{cfg.name}: {name}")
    print(f"{cfg.name}: last depth {D}, {int((ids >= 0).sum())} windows on "
          f"{int((want['counts'] > 0).sum())} experts, tiles {want['n_tiles'].tolist()}; "
          f"all tables equal", flush=True)
    sys.stdout.flush()


def _row_lens(cfg):
    return lambda b, depth: [e - s + 1 for s, e in oracle.partition(cfg.n, cfg.W, cfg.S, depth)]


# the limits: 64 documents x 128 window slots = 8,192 windows per depth on
# 64 experts, windows of 1 and 2 tokens
LIMIT = CoreConfig("limit_experts_slots", batch=64, n=254, d=128, n_heads=2, d_ffn=128, L=64,
                   D=2, W=2, S=1, mlp="swiglu", dtype="bf16", seed=41)
CASES = [
    CONFIG_BY_NAME["mid_bf16"],                            # last depth 8: shifted windows
    CONFIG_BY_NAME["mid_bf16"].with_(name="mid_bf16_D7", D=7),   # last depth 7: aligned
    CONFIG_BY_NAME["sparse_bf16"],                         # 32 experts, skewed load
    CONFIG_BY_NAME["sparse_bf16"].with_(name="sparse_bf16_D5", D=5),
    CONFIG_BY_NAME["forced_bf16"],                         # 64-token windows, 512 per depth
    LIMIT,                                                 # 8,192 window slots, 64 experts
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_bucketing_tables_equal_their_recomputation(cfg):
    import torch
    from runtime_routed_transformer_amd.core import DeviceCore
    print(f"[buckets] {cfg.name}", flush=True)
    inp = parity.prepare(cfg)
    core = DeviceCore(inp)
    core.set_forcing(forced_expert=inp.forced_expert)
    core.path_util.fill_(-7)
    core.forward()
    torch.cuda.synchronize(core.device)
    _check(core, _row_lens(cfg), cfg.batch, cfg)


def test_bucketing_tables_of_packed_documents():
    """Ragged documents: every expert's row count is arbitrary, so both tile
    tables end with partial tiles."""
    import torch
    from runtime_routed_transformer_amd.core import DeviceCore
    packed = generate_packed(PACKED_BY_NAME["mid_bf16_packed"])
    cfg = packed.core.cfg
    print(f"[buckets] {cfg.name} ({cfg.batch} documents)", flush=True)
    core = DeviceCore(packed.core)
    core.path_util.fill_(-7)
    s_in = torch.from_numpy(packed.stream()).to(core.device)
    s_out = torch.empty_like(s_in)
    core.forward_docs(s_in, s_out, torch.from_numpy(packed.start).to(core.device),
                      torch.from_numpy(packed.length).to(core.device))
    torch.cuda.synchronize(core.device)
    lens = lambda b, depth: [e - s + 1 for s, e in
                             oracle.partition(int(packed.length[b]), cfg.W, cfg.S, depth)]
    _check(core, lens, cfg.batch, cfg)
