"""The measurement call behind the benchmark's matrix-core ceiling runs and
returns plausible numbers (it is not a parity test: nothing is computed
that the oracle could check)."""
import pytest

from runtime_routed_transformer_amd import binding as B

pytestmark = pytest.mark.gpu


def test_mfma_ceiling_measurement_is_plausible():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nbytes = B.load().lol_measure_mfma_bf16_scratch_size()
    assert nbytes > 0
    scratch = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    for shape in (16, 32):
        for rnd in (False, True):
            tf, ghz = B.lol_measure_mfma_bf16(shape, rnd, 2000, scratch.data_ptr(), nbytes, st)
            print(f"{shape}x{shape} random operands={rnd}: {tf:.0f} TFLOP/s at {ghz:.2f} GHz",
                  flush=True)
            assert 100.0 < tf < 3000.0 and 0.5 < ghz < 3.5
    assert B.load().lol_measure_mfma_bf16(16, 1, 10, scratch.data_ptr(), 16, None, None,
                                          st) == B.LOL_EINVAL
