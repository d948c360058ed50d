"""The whole forward of Algorithm 1 on the device, through the C ABI.

Paper "Library of Layers (LoL)", Appendix A, Algorithm 1: the causal
prelude on the token sequence, the routed core, then the causal coda and the
vocabulary readout.  Prelude and coda are fixed-order stacks of decoder
layers with full causal attention (paper Sec. 3.1); each runs as one
``lol_core_forward`` call with one window per document (W = n, S = 0) and
the forced path "layer l at depth l, gate 1", so every block is applied in
full.  The token embedding and the readout are ``lol_embed`` and
``lol_lm_head``.  Every step runs in the library's kernels; PyTorch only
holds device memory and streams.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import binding as B
from .core import DeviceCore
from .workloads import FullInputs, bf16_bits


class DeviceModel:
    def __init__(self, full: FullInputs, device: str = "cuda:0"):
        self.full = full
        self.cfg = full.cfg
        core_cfg = full.core.cfg
        self.device = torch.device(device)
        self.dtype = B.LOL_BF16 if core_cfg.dtype == "bf16" else B.LOL_FP32
        self.prelude = DeviceCore(full.prelude, device)
        self.core = DeviceCore(full.core, device)
        self.coda = DeviceCore(full.coda, device)
        ones = lambda c: np.ones((c.cfg.D, c.cfg.batch, c.k_max), np.float32)
        self.prelude.set_forcing(forced_expert=full.prelude.forced_expert, forced_gate=ones(self.prelude))
        self.coda.set_forcing(forced_expert=full.coda.forced_expert, forced_gate=ones(self.coda))
        self.core.set_forcing(forced_expert=full.core.forced_expert)
        dev = self.device

        def weight(a):
            if core_cfg.dtype == "bf16":
                return torch.from_numpy(bf16_bits(a).view(np.int16)).to(dev)
            return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

        self.tokens = torch.from_numpy(np.ascontiguousarray(full.tokens, np.int32)).to(dev)
        self.embedding = weight(full.embedding)
        self.w_vocab = weight(full.w_vocab)
        self.g_final = torch.from_numpy(np.ascontiguousarray(full.g_final, np.float32)).to(dev)
        self.T, self.d, self.V = core_cfg.tokens, core_cfg.d, self.cfg.vocab
        self.s = torch.empty((core_cfg.batch, core_cfg.n, core_cfg.d), dtype=torch.float32, device=dev)
        self.logits = torch.empty((core_cfg.batch, core_cfg.n, self.V), dtype=torch.float32, device=dev)
        self.head_ws_bytes = B.load().lol_lm_head_workspace_size(self.T, self.d, self.V, self.dtype)
        if self.head_ws_bytes == 0:
            raise B.LolError(B.LOL_EINVAL, "lol_lm_head sizes")
        self.head_ws = torch.empty(self.head_ws_bytes, dtype=torch.uint8, device=dev)

    def set_core_forcing(self, forced_expert=None) -> None:
        self.core.set_forcing(forced_expert=forced_expert)

    STEPS = ("embed", "prelude", "core", "coda", "lm_head")

    def forward(self, stream: Optional[torch.cuda.Stream] = None, after=None) -> torch.Tensor:
        """Queue the whole forward on ``stream``; returns the logits [B][n][V].
        ``after(step)``, if given, is called once each step is queued (the
        benchmark records events there)."""
        lib = B.load()
        st = (stream or torch.cuda.current_stream(self.device)).cuda_stream
        status = lib.lol_embed(self.tokens.data_ptr(), self.T, self.embedding.data_ptr(), self.V,
                               self.d, self.dtype, self.s.data_ptr(), st)
        if status != B.LOL_OK:
            raise B.LolError(status, "lol_embed")
        if after:
            after("embed")
        for name, part in (("prelude", self.prelude), ("core", self.core), ("coda", self.coda)):
            part.forward(s_in=self.s, s_out=self.s, stream=stream)
            if after:
                after(name)
        status = lib.lol_lm_head(self.s.data_ptr(), self.T, self.d, self.g_final.data_ptr(),
                                 self.full.core.cfg.rms_eps, self.w_vocab.data_ptr(), self.V,
                                 self.dtype, self.logits.data_ptr(), self.head_ws.data_ptr(),
                                 self.head_ws_bytes, st)
        if status != B.LOL_OK:
            raise B.LolError(status, "lol_lm_head")
        if after:
            after("lm_head")
        return self.logits
