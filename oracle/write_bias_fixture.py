"""Writes the skewed workloads' balancing bias to a fixture.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``): it runs the oracle's
calibration (``oracle.calibrate``) and nothing else, so that ``bench.py``
can read the calibrated bias, an input of the skewed workloads, without
running the oracle's router itself.

    python -m oracle.write_bias_fixture

For every workload with bias_mode "skewed" among the benchmark workloads it
stores the config it was calibrated for and the bias as float32 bit
patterns (exact).  ``tests/test_oracle_pins.py`` checks that the stored
bias still equals a fresh calibration.
"""
from __future__ import annotations

import dataclasses
import json
import os

import numpy as np

from runtime_routed_transformer_amd import workloads
from .calibrate import apply_skew

FIXTURE = os.path.join(os.path.dirname(workloads.__file__), "data", "skewed_bias.json")


def fixture_configs():
    return [c for c in workloads.CONFIG_BY_NAME.values() if c.bias_mode == "skewed"]


def calibrated(cfg) -> np.ndarray:
    inp = workloads.generate(cfg)
    apply_skew(inp)
    return np.asarray(inp.expert_bias, np.float32)


def main() -> None:
    out = {}
    for cfg in fixture_configs():
        bias = calibrated(cfg)
        out[cfg.name] = {"config": dataclasses.asdict(cfg),
                         "bias_f32_bits": [f"{int(u):08x}" for u in bias.view(np.uint32)]}
    with open(FIXTURE, "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(f"wrote {FIXTURE}: {', '.join(out)}")


if __name__ == "__main__":
    main()
