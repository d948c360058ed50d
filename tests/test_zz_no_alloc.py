"""The routed-core forward without a workspace argument.

``lol_core_forward_static`` runs the same kernels as ``lol_core_forward`` on
a buffer inside the library (one per GPU) instead of a caller workspace, for
callers that cannot allocate.  Two calls in a row, the second on a smaller
input, must each give exactly what ``lol_core_forward`` gives for the same
inputs: s^(D) and the whole path, bit for bit.
"""
import numpy as np
import pytest

from runtime_routed_transformer_amd import binding as B
from runtime_routed_transformer_amd.core import make_config
from runtime_routed_transformer_amd.workloads import CONFIG_BY_NAME
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(cfg):
    """(workspace forward, static forward) outputs and paths for cfg."""
    import torch
    from runtime_routed_transformer_amd.core import DeviceCore
    inp = parity.prepare(cfg)
    core = DeviceCore(inp)
    want = core.forward().clone()
    want_path = [t.clone() for t in (core.path_expert, core.path_gate, core.path_margin,
                                     core.path_util)]
    out = torch.full_like(want, -3.0)
    pe = torch.full_like(core.path_expert, -7)
    pg = torch.full_like(core.path_gate, 7.0)
    pm = torch.full_like(core.path_margin, 7.0)
    pu = torch.full_like(core.path_util, -7)
    path = B.lol_path(expert=pe.data_ptr(), gate=pg.data_ptr(), margin=pm.data_ptr(),
                      util=pu.data_ptr())
    st = torch.cuda.current_stream(core.device).cuda_stream
    status = B.lol_core_forward_static(core.ccfg, core.s0.data_ptr(), core.lib, core.rt, None,
                                       None, out.data_ptr(), path, st)
    assert status == B.LOL_OK, B.status_str(status)
    torch.cuda.synchronize(core.device)
    return (want, want_path), (out, [pe, pg, pm, pu])


def test_static_forward_equals_the_workspace_forward_twice_second_smaller():
    import torch
    first = CONFIG_BY_NAME["mid_bf16"].scaled(1, 512)
    second = CONFIG_BY_NAME["mid_bf16"].scaled(1, 300)
    assert (B.lol_core_workspace_size(make_config(second))
            < B.lol_core_workspace_size(make_config(first)) <= B.LOL_STATIC_SCRATCH_BYTES)
    for cfg in (first, second):
        print(f"[static forward] {cfg.name}", flush=True)
        (want, want_path), (got, got_path) = _both(cfg)
        assert torch.equal(got, want), f"{cfg.name}: s^(D) differs"
        for name, a, b in zip(("expert", "gate", "margin", "util"), got_path, want_path):
            assert torch.equal(a, b), f"{cfg.name}: path {name} differs"
        print(f"{cfg.name}: s^(D) and path identical", flush=True)


def test_static_forward_refuses_a_config_beyond_its_buffer():
    cfg = make_config(CONFIG_BY_NAME["mid_bf16"])
    assert B.lol_core_workspace_size(cfg) > B.LOL_STATIC_SCRATCH_BYTES
    lib, rt, path = B.lol_library(), B.lol_router(), B.lol_path()
    assert B.lol_core_forward_static(cfg, 4096, lib, rt, None, None, 4096, path,
                                     None) == B.LOL_EWORKSPACE
    np.testing.assert_equal(B.LOL_STATIC_SCRATCH_BYTES, 64 << 20)
