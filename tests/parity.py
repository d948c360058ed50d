"""GPU-vs-oracle parity harness (used by the GPU tests and smoke()).

Procedure: the oracle runs the workload with free routing (plus the
workload's own forced path); every window whose top-1 margin is at most
MARGIN is then forced on the GPU to the oracle's choice (several experts
are correct there), the GPU runs the same inputs, and the two are compared
on the whole path the ABI returns:

  * s^(D) and the update s^(D) - s^(0) within the mode's normwise tolerance;
  * the chosen id of every window whose margin clears MARGIN;
  * the gate of every window (the unbiased probability of the applied
    expert, review "Library of Layers: Routing Whole Transformer Blocks at
    Runtime", Eq. 5 example) within GATE_TOL;
  * the margin of every window (top-1 minus top-2 of the biased scores of
    the free router) within MARGIN_TOL, +inf where the oracle's is +inf;
  * every slot past a depth's last window reads (expert -1, gate 0,
    margin 0); the path buffers are filled with other values beforehand.

The router works in fp32 on both sides, but at later depths it reads states
that differ by the mode's rounding, so gates and margins carry that error:
GATE_TOL is 1e-5 in fp32 and 2e-3 in bf16 (as in the decode tests), and a
margin, a difference of two biased probabilities, gets twice that.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

import oracle
from oracle.calibrate import apply_skew
from runtime_routed_transformer_amd.workloads import generate

MARGIN = 1e-3
# normwise max relative error of s^(D) (the contract) and of the update s^(D) - s^(0)
TOL = {"fp32": 1e-4, "bf16": 2e-2}
UPDATE_TOL = {"fp32": 1e-4, "bf16": 2e-2}
# absolute error of the path's gates and margins
GATE_TOL = {"fp32": 1e-5, "bf16": 2e-3}
MARGIN_TOL = {"fp32": 2e-5, "bf16": 4e-3}
# depth 1 routes s^(0), the same fp32 input on both sides: only the order of
# the fp32 sums differs there
FIRST_DEPTH_GATE_TOL = 1e-5
# values the path buffers hold before a forward (every slot must be written)
JUNK_EXPERT, JUNK_VALUE = -7, 7.0


def margin_error(m_gpu: np.ndarray, m_ref: np.ndarray) -> float:
    """Max |m_gpu - m_ref| over finite oracle margins; inf if an infinite
    oracle margin (one-expert library) is not infinite on the GPU too."""
    m_gpu = np.asarray(m_gpu, np.float64)
    m_ref = np.asarray(m_ref, np.float64)
    fin = np.isfinite(m_ref)
    if not (np.isposinf(m_gpu[~fin]).all() and np.isposinf(m_ref[~fin]).all()):
        return math.inf
    return float(np.abs(m_gpu[fin] - m_ref[fin]).max()) if fin.any() else 0.0


def padding_ok(pe, pg, pm, n: int, cfg, rows) -> bool:
    """Slots k >= K_l of every depth read (-1, 0, 0) for the given rows of a
    [D][B][K_max] path computed on documents of n tokens."""
    ok = True
    for depth in range(1, cfg.D + 1):
        K = len(oracle.partition(n, cfg.W, cfg.S, depth))
        for b in rows:
            ok &= bool((pe[depth - 1, b, K:] == -1).all() and (pg[depth - 1, b, K:] == 0).all()
                       and (pm[depth - 1, b, K:] == 0).all())
    return ok


def fill_path_with_junk(core) -> None:
    core.path_expert.fill_(JUNK_EXPERT)
    core.path_gate.fill_(JUNK_VALUE)
    core.path_margin.fill_(JUNK_VALUE)


@dataclass
class ParityReport:
    name: str
    rel_err: float
    update_err: float
    id_mismatch: int
    ids_compared: int
    forced_windows: int
    gate_err: float
    margin_err: float
    pad_ok: bool
    tol: float
    update_tol: float
    gate_tol: float
    margin_tol: float
    gate_err_first: float = 0.0    # depth 1 only: both sides route the same s^(0)

    @property
    def ok(self) -> bool:
        return (self.rel_err <= self.tol and self.update_err <= self.update_tol
                and self.id_mismatch == 0 and self.gate_err <= self.gate_tol
                and self.margin_err <= self.margin_tol and self.pad_ok
                and self.gate_err_first <= FIRST_DEPTH_GATE_TOL)

    def __str__(self):
        return (f"{self.name}: rel_err={self.rel_err:.3e} (tol {self.tol:g}) update_err="
                f"{self.update_err:.3e} (tol {self.update_tol:g}) ids {self.ids_compared - self.id_mismatch}/"
                f"{self.ids_compared} equal, forced {self.forced_windows}, gate_err={self.gate_err:.2e} "
                f"(tol {self.gate_tol:g}; depth 1: {self.gate_err_first:.1e}) margin_err="
                f"{self.margin_err:.2e} (tol {self.margin_tol:g}) padding ok={self.pad_ok}")


def prepare(cfg):
    inp = generate(cfg)
    apply_skew(inp)
    return inp


def forced_for_gpu(inp, ref, rows, n_tokens):
    """The workload's forcing plus the oracle's id on every near-tie window."""
    cfg = inp.cfg
    forced = (inp.forced_expert.copy() if inp.forced_expert is not None
              else np.full((cfg.D, cfg.batch, cfg.k_max), -1, np.int32))
    compared = np.zeros((cfg.D, cfg.batch, cfg.k_max), bool)
    for depth in range(1, cfg.D + 1):
        wins = oracle.partition(n_tokens, cfg.W, cfg.S, depth)
        for ri, b in enumerate(rows):
            for k in range(len(wins)):
                if ref.margin[depth - 1, ri, k] <= MARGIN:
                    forced[depth - 1, b, k] = ref.expert[depth - 1, ri, k]
                compared[depth - 1, b, k] = True
    return forced, compared


def run(inp, rows=None, n_tokens=None, device="cuda:0", core=None,
        gate_tol_scale: float = 1.0) -> ParityReport:
    """gate_tol_scale: factor on GATE_TOL and MARGIN_TOL for routers whose
    weights are larger than the workloads' N(0, 0.02^2): a logit moves by
    W_r times the change of its input, so the later depths' gates inherit
    the states' rounding error multiplied by the weights' scale."""
    import torch
    from runtime_routed_transformer_amd.core import DeviceCore

    cfg = inp.cfg
    rows = list(range(cfg.batch)) if rows is None else list(rows)
    n_tokens = cfg.n if n_tokens is None else int(n_tokens)
    ref = oracle.forward(inp, forced_expert=inp.forced_expert, rows=rows, n_tokens=n_tokens)
    forced, compared = forced_for_gpu(inp, ref, rows, n_tokens)
    core = core or DeviceCore(inp, device)
    core.set_forcing(forced_expert=forced)
    fill_path_with_junk(core)
    core.forward()
    torch.cuda.synchronize(core.device)
    s_gpu = core.s_out.cpu().numpy()[rows, :n_tokens]
    pe, pg, pm = core.path_numpy()
    s_ref = ref.s64
    s0 = inp.s0[rows, :n_tokens].astype(np.float64)
    rel = float(np.abs(s_gpu - s_ref).max() / np.abs(s_ref).max())
    upd = float(np.abs((s_gpu - s0) - (s_ref - s0)).max() / np.abs(s_ref - s0).max())
    free_cmp = compared[:, rows] & (ref.margin > MARGIN)
    if inp.forced_expert is not None:
        free_cmp &= inp.forced_expert[:, rows] < 0
    gpu_ids = pe[:, rows]
    mism = int(np.count_nonzero(free_cmp & (gpu_ids != ref.expert)))
    cmp_all = compared[:, rows]
    gate_err = float(np.abs(pg[:, rows] - ref.gate)[cmp_all].max())
    marg_err = margin_error(pm[:, rows][cmp_all], ref.margin[cmp_all])
    pad = padding_ok(pe, pg, pm, cfg.n, cfg, rows)
    n_forced = int(np.count_nonzero(cmp_all & (ref.margin <= MARGIN)))
    gate_first = float(np.abs(pg[0, rows] - ref.gate[0])[cmp_all[0]].max())
    return ParityReport(cfg.name, rel, upd, mism, int(np.count_nonzero(free_cmp)), n_forced,
                        gate_err, marg_err, pad, TOL[cfg.dtype], UPDATE_TOL[cfg.dtype],
                        GATE_TOL[cfg.dtype] * gate_tol_scale,
                        MARGIN_TOL[cfg.dtype] * gate_tol_scale, gate_first)


@dataclass
class FullReport:
    name: str
    logit_err: float
    hidden_err: float
    id_mismatch: int
    ids_compared: int
    forced_windows: int
    gate_err: float
    margin_err: float
    pad_ok: bool
    tol: float
    gate_tol: float
    margin_tol: float

    @property
    def ok(self) -> bool:
        return (self.logit_err <= self.tol and self.hidden_err <= self.tol and self.id_mismatch == 0
                and self.gate_err <= self.gate_tol and self.margin_err <= self.margin_tol
                and self.pad_ok)

    def __str__(self):
        return (f"{self.name}: logit_err={self.logit_err:.3e} coda_out_err={self.hidden_err:.3e} "
                f"(tol {self.tol:g}) core ids {self.ids_compared - self.id_mismatch}/"
                f"{self.ids_compared} equal, forced {self.forced_windows}, core gate_err="
                f"{self.gate_err:.2e} (tol {self.gate_tol:g}) margin_err={self.margin_err:.2e} "
                f"(tol {self.margin_tol:g}) padding ok={self.pad_ok}")


def run_full(full, device="cuda:0") -> FullReport:
    """Algorithm 1 end to end (embedding, prelude, routed core, coda,
    readout) on the GPU against the oracle; near-tie core windows are forced
    to the oracle's choice as in ``run``."""
    import torch
    from runtime_routed_transformer_amd.model import DeviceModel

    core_cfg = full.core.cfg
    ref = oracle.full_forward(full, core_forced_expert=full.core.forced_expert)
    rows = list(range(core_cfg.batch))
    forced, compared = forced_for_gpu(full.core, ref.core, rows, core_cfg.n)
    model = DeviceModel(full, device)
    model.set_core_forcing(forced)
    fill_path_with_junk(model.core)
    logits = model.forward()
    torch.cuda.synchronize(model.device)
    lg = logits.cpu().numpy().astype(np.float64)
    hid = model.s.cpu().numpy().astype(np.float64)
    logit_err = float(np.abs(lg - ref.logits).max() / np.abs(ref.logits).max())
    hidden_err = float(np.abs(hid - ref.coda_out).max() / np.abs(ref.coda_out).max())
    pe, pg, pm = model.core.path_numpy()
    free_cmp = compared & (ref.core.margin > MARGIN)
    if full.core.forced_expert is not None:
        free_cmp &= full.core.forced_expert < 0
    mism = int(np.count_nonzero(free_cmp & (pe != ref.core.expert)))
    n_forced = int(np.count_nonzero(compared & (ref.core.margin <= MARGIN)))
    gate_err = float(np.abs(pg - ref.core.gate)[compared].max())
    marg_err = margin_error(pm[compared], ref.core.margin[compared])
    pad = padding_ok(pe, pg, pm, core_cfg.n, core_cfg, rows)
    dt = core_cfg.dtype
    return FullReport(full.cfg.name, logit_err, hidden_err, mism, int(np.count_nonzero(free_cmp)),
                      n_forced, gate_err, marg_err, pad, TOL[dt], GATE_TOL[dt], MARGIN_TOL[dt])


@dataclass
class DocsReport:
    name: str
    docs: int
    rel_err: float
    update_err: float
    id_mismatch: int
    ids_compared: int
    forced_windows: int
    gate_err: float
    margin_err: float
    gaps_untouched: bool
    pad_slots_ok: bool
    tol: float
    update_tol: float
    gate_tol: float
    margin_tol: float

    @property
    def ok(self) -> bool:
        return (self.rel_err <= self.tol and self.update_err <= self.update_tol
                and self.id_mismatch == 0 and self.gate_err <= self.gate_tol
                and self.margin_err <= self.margin_tol and self.gaps_untouched
                and self.pad_slots_ok)

    def __str__(self):
        return (f"{self.name}: {self.docs} docs rel_err={self.rel_err:.3e} (tol {self.tol:g}) "
                f"update_err={self.update_err:.3e} (tol {self.update_tol:g}) ids "
                f"{self.ids_compared - self.id_mismatch}/{self.ids_compared} equal, forced "
                f"{self.forced_windows}, gate_err={self.gate_err:.2e} (tol {self.gate_tol:g}) "
                f"margin_err={self.margin_err:.2e} (tol {self.margin_tol:g}), gaps untouched="
                f"{self.gaps_untouched}, padding slots ok={self.pad_slots_ok}")


def run_docs(packed, docs=None, prefix=None, device="cuda:0") -> DocsReport:
    """Packed documents on the GPU (``lol_core_forward_docs``) against the
    oracle run on each document alone.  ``docs``: the documents compared
    (default all); ``prefix``: compare only each document's first ``prefix``
    tokens (by the core's causality they equal a run of that prefix alone).
    Near-tie windows are forced to the oracle's choice as in ``run``."""
    import torch
    from runtime_routed_transformer_amd.core import DeviceCore

    inp = packed.core
    cfg = inp.cfg
    docs = list(range(cfg.batch)) if docs is None else list(docs)
    forced = (inp.forced_expert.copy() if inp.forced_expert is not None
              else np.full((cfg.D, cfg.batch, cfg.k_max), -1, np.int32))
    refs, ns = {}, {}
    for b in docs:
        n_b = int(packed.length[b]) if prefix is None else min(int(packed.length[b]), prefix)
        ns[b] = n_b
        refs[b] = oracle.forward(inp, forced_expert=inp.forced_expert, rows=[b], n_tokens=n_b)
        for depth in range(1, cfg.D + 1):
            for k in range(len(oracle.partition(n_b, cfg.W, cfg.S, depth))):
                if refs[b].margin[depth - 1, 0, k] <= MARGIN:
                    forced[depth - 1, b, k] = refs[b].expert[depth - 1, 0, k]
    core = DeviceCore(inp, device)
    core.set_forcing(forced_expert=forced)
    fill_path_with_junk(core)
    stream = packed.stream()
    s_in = torch.from_numpy(stream).to(core.device)
    s_out = torch.full_like(s_in, -7.0)
    d_start = torch.from_numpy(packed.start).to(core.device)
    d_len = torch.from_numpy(packed.length).to(core.device)
    core.forward_docs(s_in, s_out, d_start, d_len)
    torch.cuda.synchronize(core.device)
    flags = core.flags()
    out = s_out.cpu().numpy()
    pe, pg, pm = core.path_numpy()
    del core
    inside = np.zeros(packed.n_tokens, bool)
    for a, ln in zip(packed.start, packed.length):
        inside[a:a + ln] = True
    gaps_ok = bool((out[~inside] == -7.0).all()) and flags == 0
    err = ref_max = upd_err = upd_max = 0.0
    mism = cmp = n_forced = 0
    gate_err = 0.0
    m_gpu, m_ref = [], []
    pad_ok = True
    for b in docs:
        a, n_b, ref = int(packed.start[b]), ns[b], refs[b]
        s0_b = inp.s0[b, :n_b].astype(np.float64)
        err = max(err, float(np.abs(out[a:a + n_b] - ref.s64[0]).max()))
        ref_max = max(ref_max, float(np.abs(ref.s64[0]).max()))
        upd_err = max(upd_err, float(np.abs((out[a:a + n_b] - s0_b) - (ref.s64[0] - s0_b)).max()))
        upd_max = max(upd_max, float(np.abs(ref.s64[0] - s0_b).max()))
        for depth in range(1, cfg.D + 1):
            K_full = len(oracle.partition(int(packed.length[b]), cfg.W, cfg.S, depth))
            K_b = len(oracle.partition(n_b, cfg.W, cfg.S, depth))
            # slots past the document's last window: expert -1, gate 0
            pad_ok &= bool((pe[depth - 1, b, K_full:] == -1).all()
                           and (pg[depth - 1, b, K_full:] == 0).all()
                           and (pm[depth - 1, b, K_full:] == 0).all())
            # a window's route reads only earlier (complete) windows, so a
            # prefix run routes its windows as the whole document does
            for k in range(K_b):
                free = (ref.margin[depth - 1, 0, k] > MARGIN
                        and (inp.forced_expert is None or inp.forced_expert[depth - 1, b, k] < 0))
                if free:
                    cmp += 1
                    mism += int(pe[depth - 1, b, k] != ref.expert[depth - 1, 0, k])
                else:
                    n_forced += int(ref.margin[depth - 1, 0, k] <= MARGIN)
                gate_err = max(gate_err,
                               abs(float(pg[depth - 1, b, k]) - float(ref.gate[depth - 1, 0, k])))
                m_gpu.append(pm[depth - 1, b, k])
                m_ref.append(ref.margin[depth - 1, 0, k])
    dt = cfg.dtype
    return DocsReport(packed.cfg.name, len(docs), err / ref_max, upd_err / upd_max, mism, cmp,
                      n_forced, gate_err, margin_error(np.array(m_gpu), np.array(m_ref)), gaps_ok,
                      pad_ok, TOL[dt], UPDATE_TOL[dt], GATE_TOL[dt], MARGIN_TOL[dt])
