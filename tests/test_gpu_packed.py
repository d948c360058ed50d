"""GPU parity of packed documents (``lol_core_forward_docs``): documents of
different lengths back to back in one token stream, each compared with the
oracle's run of that document alone (its own windows, router prefix and
attention; paper App. A document-blocked attention, the explainer's router
prefix restarting at every document).  Lengths cover one token, a window
minus one, a window plus one and the longest allowed; some streams leave
unused rows between documents, which must come back untouched."""
import sys

import numpy as np
import pytest

from runtime_routed_transformer_amd.workloads import (CONFIG_BY_NAME, PACKED_BY_NAME, CoreConfig,
                                                      PackedConfig, generate_packed)
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from runtime_routed_transformer_amd import binding
    binding.load()


def _report(rep):
    print(rep, flush=True)
    sys.stdout.flush()
    assert rep.ok, str(rep)


def _prepare(cfg, lengths=None):
    packed = generate_packed(cfg, lengths)
    from oracle.calibrate import apply_skew
    apply_skew(packed.core)
    return packed


CASES = [
    (PackedConfig("packed_fp32_ragged",
                  CoreConfig("c", batch=1, n=37, d=64, n_heads=2, d_ffn=128, L=3, D=4, W=5, S=3,
                             mlp="swiglu", dtype="fp32", seed=61), 0, 1, 3, 61),
     [37, 1, 6, 20, 4, 37, 2]),
    (PackedConfig("packed_bf16_d128",
                  CoreConfig("c", batch=1, n=150, d=128, n_heads=2, d_ffn=256, L=3, D=3, W=40,
                             S=13, mlp="swiglu", dtype="bf16", seed=62), 0, 1, 0, 62),
     [150, 39, 41, 1, 80]),
    (PackedConfig("packed_small_bf16", CONFIG_BY_NAME["small_bf16"].with_(n=384, seed=63),
                  0, 1, 2, 63),
     [384, 129, 1, 64, 255, 300, 7, 384]),
    (PackedConfig("packed_mid_bf16", CONFIG_BY_NAME["mid_bf16"].with_(n=640, seed=64), 0, 1, 0, 64),
     [640, 257, 100, 383]),
    (PackedConfig("packed_sparse_bf16", CONFIG_BY_NAME["sparse_bf16"].with_(n=600, seed=65),
                  0, 1, 5, 65),
     [600, 31, 256, 257, 44]),
]


@pytest.mark.parametrize("cfg,lengths", CASES, ids=lambda c: getattr(c, "name", ""))
def test_packed_documents_match_the_oracle_per_document(cfg, lengths):
    print(f"[packed] {cfg.name} lengths={lengths}", flush=True)
    _report(parity.run_docs(_prepare(cfg, lengths)))


def test_packed_mid_full_size_sampled():
    """The packed mid workload the benchmark times (16,384 tokens), compared
    on three documents' first 3.5 windows."""
    cfg = PACKED_BY_NAME["mid_bf16_packed"]
    packed = _prepare(cfg)
    B = packed.core.cfg.batch
    short = int(np.argmin(packed.length))
    docs = sorted({0, short, B - 1})
    print(f"[packed-full] {cfg.name} docs={B} compared={docs}", flush=True)
    _report(parity.run_docs(packed, docs=docs, prefix=3 * cfg.core.W + cfg.core.W // 2))


def test_packed_mid_full_size_every_document():
    """The same 16,384-token stream compared on every token of every
    document.  Its ragged expert row counts leave the down projection's
    persistent 256 x 256 tiles a short last round, which runs cut along K
    into pieces summed by a second kernel; the rows of those tiles are
    compared here like every other."""
    cfg = PACKED_BY_NAME["mid_bf16_packed"]
    packed = _prepare(cfg)
    print(f"[packed-full-all] {cfg.name} docs={packed.core.cfg.batch}", flush=True)
    _report(parity.run_docs(packed))


def test_packed_mid_full_size_repeats_bit_for_bit():
    """Two forwards of the 16,384-token packed stream give the same bits:
    the K-split tail's pieces are summed in a fixed order, whatever order
    the workgroups that made them finished in."""
    import torch
    from runtime_routed_transformer_amd.core import DeviceCore
    packed = _prepare(PACKED_BY_NAME["mid_bf16_packed"])
    core = DeviceCore(packed.core)
    s_in = torch.from_numpy(packed.stream()).to(core.device)
    d_start = torch.from_numpy(packed.start).to(core.device)
    d_len = torch.from_numpy(packed.length).to(core.device)
    outs = []
    for _ in range(3):
        s_out = torch.empty_like(s_in)
        core.forward_docs(s_in, s_out, d_start, d_len)
        outs.append(s_out)
    torch.cuda.synchronize(core.device)
    assert core.flags() == 0
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2]), "packed forwards differ"


def test_rows_as_documents_equal_the_row_layout_and_bad_tables_raise_a_flag():
    """A table naming the rows of the [batch][n] layout reproduces
    lol_core_forward bit for bit; a table with overlapping documents or a
    length above n raises LOL_FLAG_BAD_DOC (its entries are clamped into the
    stream, so nothing is accessed outside it)."""
    import torch
    from runtime_routed_transformer_amd import binding as B
    from runtime_routed_transformer_amd.core import DeviceCore

    cfg = CONFIG_BY_NAME["small_bf16"].scaled(3, 300, name="rows_as_docs")
    inp = parity.prepare(cfg)
    core = DeviceCore(inp)
    print(f"[packed-rows] {cfg.name}", flush=True)
    ref = core.forward().clone()
    torch.cuda.synchronize()
    assert core.flags() == 0
    dev = core.device
    start = torch.arange(cfg.batch, dtype=torch.int32, device=dev) * cfg.n
    length = torch.full((cfg.batch,), cfg.n, dtype=torch.int32, device=dev)
    s_in = core.s0.reshape(cfg.batch * cfg.n, cfg.d)
    out = torch.empty_like(s_in)
    core.forward_docs(s_in, out, start, length)
    torch.cuda.synchronize()
    assert core.flags() == 0
    assert torch.equal(out.reshape(ref.shape), ref)
    # overlapping documents and a document longer than n
    bad_start = torch.tensor([0, 10, 400], dtype=torch.int32, device=dev)
    bad_len = torch.tensor([300, 300, cfg.n + 50], dtype=torch.int32, device=dev)
    core.forward_docs(s_in, out, bad_start, bad_len)
    torch.cuda.synchronize()
    assert core.flags() & B.LOL_FLAG_BAD_DOC
    # host-side checks
    with pytest.raises(ValueError):
        core.forward_docs(s_in, out, start[:2], length[:2])
    st = B.lol_core_forward_docs(core.ccfg, cfg.batch * cfg.n, start.data_ptr(), None,
                                 s_in.data_ptr(), core.lib, core.rt, None, None, out.data_ptr(),
                                 core.path, core.workspace.data_ptr(), core.ws_bytes,
                                 torch.cuda.current_stream().cuda_stream)
    assert st == B.LOL_EINVAL
    st = B.lol_core_forward_docs(core.ccfg, 0, start.data_ptr(), length.data_ptr(),
                                 s_in.data_ptr(), core.lib, core.rt, None, None, out.data_ptr(),
                                 core.path, core.workspace.data_ptr(), core.ws_bytes,
                                 torch.cuda.current_stream().cuda_stream)
    assert st == B.LOL_EINVAL
