"""Skewed expert-bias calibration for the sparse large-library workload.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The workload asks for a frozen balancing bias b under which about 60% of
depth-1 windows pick one expert and the rest spread Zipf(1.2) over the other
experts.  b is found with the loss-free balancing update the pages describe
(blog, "How the order is chosen": every expert's bias moves by a fixed step
against the sign of its load minus its target; paper App. A: the bias enters
the choice only), run here against fixed targets with a shrinking step on the
depth-1 router scores, which depend only on s^(0).  The achieved per-depth
load is whatever the forward then produces and is reported, not assumed.
"""
from __future__ import annotations

import numpy as np

from .lol_oracle import partition, router_inputs, route


def target_counts(L: int, n_windows: int, seed: int, dominant_share: float = 0.6,
                  zipf_s: float = 1.2) -> np.ndarray:
    order = np.random.default_rng([seed, 1]).permutation(L)
    share = np.zeros(L)
    share[order[0]] = dominant_share
    ranks = np.arange(1, L)
    z = ranks ** (-zipf_s)
    share[order[1:]] = (1.0 - dominant_share) * z / z.sum()
    raw = share * n_windows
    cnt = np.floor(raw).astype(np.int64)
    rem = n_windows - cnt.sum()
    cnt[np.argsort(-(raw - cnt), kind="stable")[:rem]] += 1   # largest remainder
    return cnt


def depth1_probs(inp) -> np.ndarray:
    cfg = inp.cfg
    wins = partition(cfg.n, cfg.W, cfg.S, 1)
    probs = []
    for b in range(cfg.batch):
        r = router_inputs(np.asarray(inp.s0[b], np.float64), wins,
                          np.asarray(inp.e_depth[0], np.float64))
        for k in range(len(wins)):
            probs.append(route(r[k], inp.w_r, inp.b_r, np.zeros(cfg.L, np.float32)).probs)
    return np.stack(probs).astype(np.float32)


def calibrate_bias(inp, iters: int = 4000) -> np.ndarray:
    cfg = inp.cfg
    a = depth1_probs(inp)
    target = target_counts(cfg.L, a.shape[0], cfg.seed)
    b = np.zeros(cfg.L, np.float32)
    best, best_err = b.copy(), None
    step0 = float(a.max() - a.min()) / 8.0 + 1e-6
    for it in range(iters):
        load = np.bincount(np.argmax(a + b, axis=1), minlength=cfg.L)
        err = int(np.abs(load - target).sum())
        if best_err is None or err < best_err:
            best, best_err = b.copy(), err
            if err == 0:
                break
        step = np.float32(step0 * (1.0 - it / iters) + 1e-7)
        b = (b - step * np.sign(load - target).astype(np.float32)).astype(np.float32)
    return best


def apply_skew(inp) -> None:
    """Set ``inp.expert_bias`` in place for a workload with bias_mode 'skewed'."""
    if inp.cfg.bias_mode == "skewed":
        inp.expert_bias = calibrate_bias(inp)
