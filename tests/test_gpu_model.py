"""GPU parity of the whole forward of Algorithm 1 (paper Appendix A):
token embedding, causal prelude stack, routed core, causal coda stack and
vocabulary readout, through the C ABI, against the oracle's composition."""
import sys

import pytest

from runtime_routed_transformer_amd.workloads import (CONFIG_BY_NAME, FULL_BY_NAME, CoreConfig,
                                                      FullConfig, generate_full)
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = [
    # bf16, fused output projection (d = 512), vocabulary 1,024
    FullConfig("full_small_bf16", CONFIG_BY_NAME["small_bf16"].scaled(2, 256), vocab=1024,
               prelude=2, coda=2, seed=51),
    # bf16, unfused path (d = 128), ragged windows, vocabulary 384 (not a multiple of 256)
    FullConfig("full_d128_bf16", CoreConfig("c", batch=2, n=150, d=128, n_heads=2, d_ffn=256, L=3,
                                            D=3, W=40, S=13, mlp="swiglu", dtype="bf16", seed=52),
               vocab=384, prelude=1, coda=2, seed=53),
    # fp32 (tiny workload's shapes), vocabulary 192
    FullConfig("full_tiny_fp32", CONFIG_BY_NAME["tiny_fp32"], vocab=192, prelude=2, coda=1, seed=54),
    # the benchmark's full model at one document of 512 tokens (d = 1024, 4 + 8 + 4 layers,
    # vocabulary 32,768)
    FullConfig("full_mid_bf16@1x512", CONFIG_BY_NAME["mid_bf16"].scaled(1, 512), vocab=32768,
               prelude=4, coda=4, seed=FULL_BY_NAME["full_mid_bf16"].seed),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_full_forward_parity(cfg):
    print(f"[parity-full-model] {cfg.name}", flush=True)
    rep = parity.run_full(generate_full(cfg))
    print(rep, flush=True)
    sys.stdout.flush()
    assert rep.ok, str(rep)
