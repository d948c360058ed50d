"""Device-resident routed core: PyTorch holds device memory and streams, the
HIP library (through ``binding``) does all of the computation."""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import binding as B
from .workloads import CoreConfig, CoreInputs, bf16_bits


def make_config(cfg: CoreConfig) -> B.lol_core_config:
    return B.lol_core_config(
        batch=cfg.batch, n=cfg.n, d=cfg.d, n_heads=cfg.n_heads, d_ffn=cfg.d_ffn, L=cfg.L,
        D=cfg.D, W=cfg.W, S=cfg.S,
        mlp=B.LOL_MLP_SWIGLU if cfg.mlp == "swiglu" else B.LOL_MLP_GELU,
        dtype=B.LOL_BF16 if cfg.dtype == "bf16" else B.LOL_FP32,
        rms_eps=cfg.rms_eps, rope_theta=cfg.rope_theta)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


class DeviceCore:
    """Uploads one workload's inputs and runs ``lol_core_forward`` on them."""

    def __init__(self, inp: CoreInputs, device: str = "cuda:0"):
        self.inp = inp
        self.cfg = inp.cfg
        self.device = torch.device(device)
        self.ccfg = make_config(self.cfg)
        status = B.lol_core_validate(self.ccfg)
        if status != B.LOL_OK:
            raise B.LolError(status, f"config {self.cfg.name}")
        dev = self.device

        def f32(a):
            return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

        def weight(a):
            if self.cfg.dtype == "bf16":
                return torch.from_numpy(bf16_bits(a).view(np.int16)).to(dev)
            return f32(a)

        self.s0 = f32(inp.s0)
        self.w = {k: weight(getattr(inp, k)) for k in ("wqkv", "wo", "w_gu", "w_down")}
        self.g_attn, self.g_ffn = f32(inp.g_attn), f32(inp.g_ffn)
        self.film_gamma, self.film_beta = f32(inp.film_gamma), f32(inp.film_beta)
        self.w_r, self.b_r = f32(inp.w_r), f32(inp.b_r)
        self.e_depth, self.expert_bias = f32(inp.e_depth), f32(inp.expert_bias)
        # W_o in the fused output projection's panel layout, rearranged once
        # here rather than in every forward (None where the config does not
        # use it)
        self.wo_panels = None
        panel_bytes = B.lol_prepare_wo_panels_size(self.ccfg)
        if panel_bytes:
            self.wo_panels = torch.empty(panel_bytes, dtype=torch.uint8, device=dev)
            status = B.lol_prepare_wo_panels(self.ccfg, _ptr(self.w["wo"]), _ptr(self.wo_panels),
                                             torch.cuda.current_stream(dev).cuda_stream)
            if status != B.LOL_OK:
                raise B.LolError(status, "lol_prepare_wo_panels")
        self.lib = B.lol_library(
            wqkv=_ptr(self.w["wqkv"]), wo=_ptr(self.w["wo"]), w_gu=_ptr(self.w["w_gu"]),
            w_down=_ptr(self.w["w_down"]), g_attn=_ptr(self.g_attn), g_ffn=_ptr(self.g_ffn),
            film_gamma=_ptr(self.film_gamma), film_beta=_ptr(self.film_beta),
            film_per_expert=1 if self.cfg.film_mode == "depth_expert" else 0,
            wo_panels=_ptr(self.wo_panels))
        # the QKV, gate/up and down weights in 32-k panels (bf16), likewise
        # rearranged once
        self.weight_panels = None
        panel_bytes = B.lol_prepare_weight_panels_size(self.ccfg)
        if panel_bytes:
            self.weight_panels = torch.empty(panel_bytes, dtype=torch.uint8, device=dev)
            status = B.lol_prepare_weight_panels(self.ccfg, self.lib, _ptr(self.weight_panels),
                                                 torch.cuda.current_stream(dev).cuda_stream)
            if status != B.LOL_OK:
                raise B.LolError(status, "lol_prepare_weight_panels")
            self.lib.weight_panels = _ptr(self.weight_panels)
        self.rt = B.lol_router(w_r=_ptr(self.w_r), b_r=_ptr(self.b_r), e_depth=_ptr(self.e_depth),
                               expert_bias=_ptr(self.expert_bias),
                               per_depth=1 if self.cfg.router == "per_depth" else 0)
        self.k_max = B.lol_core_k_max(self.ccfg)
        self.ws_bytes = B.lol_core_workspace_size(self.ccfg)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        shape = (self.cfg.D, self.cfg.batch, self.k_max)
        self.path_expert = torch.empty(shape, dtype=torch.int32, device=dev)
        self.path_gate = torch.empty(shape, dtype=torch.float32, device=dev)
        self.path_margin = torch.empty(shape, dtype=torch.float32, device=dev)
        self.path_util = torch.empty((self.cfg.D, self.cfg.L), dtype=torch.int32, device=dev)
        self.path = B.lol_path(expert=_ptr(self.path_expert), gate=_ptr(self.path_gate),
                               margin=_ptr(self.path_margin), util=_ptr(self.path_util))
        self.s_out = torch.empty_like(self.s0)
        self.forced_expert = None
        self.forced_gate = None

    def set_forcing(self, forced_expert=None, forced_gate=None) -> None:
        shape = (self.cfg.D, self.cfg.batch, self.k_max)
        self.forced_expert = None if forced_expert is None else torch.from_numpy(
            np.array(np.broadcast_to(forced_expert, shape), np.int32)).to(self.device)
        self.forced_gate = None if forced_gate is None else torch.from_numpy(
            np.array(np.broadcast_to(forced_gate, shape), np.float32)).to(self.device)

    def forward(self, s_in: Optional[torch.Tensor] = None, s_out: Optional[torch.Tensor] = None,
                stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """Queue one forward on ``stream`` (default: torch's current stream)."""
        s_in = self.s0 if s_in is None else s_in
        s_out = self.s_out if s_out is None else s_out
        st = (stream or torch.cuda.current_stream(self.device)).cuda_stream
        status = B.lol_core_forward(self.ccfg, s_in.data_ptr(), self.lib, self.rt,
                                    _ptr(self.forced_expert), _ptr(self.forced_gate),
                                    s_out.data_ptr(), self.path, self.workspace.data_ptr(),
                                    self.ws_bytes, st)
        if status != B.LOL_OK:
            raise B.LolError(status, "lol_core_forward")
        return s_out

    def forward_docs(self, s_in: torch.Tensor, s_out: torch.Tensor, doc_start: torch.Tensor,
                     doc_len: torch.Tensor, stream: Optional[torch.cuda.Stream] = None
                     ) -> torch.Tensor:
        """Queue one forward over packed documents: ``s_in`` / ``s_out`` are
        [n_tokens][d] fp32 streams, ``doc_start`` / ``doc_len`` int32 [batch]
        device tensors (document b = rows doc_start[b] .. + doc_len[b] - 1)."""
        if (s_in.dim() != 2 or s_in.shape != s_out.shape or s_in.shape[1] != self.cfg.d
                or s_in.dtype != torch.float32 or s_out.dtype != torch.float32
                or not (s_in.is_contiguous() and s_out.is_contiguous())):
            raise ValueError("s_in / s_out must be contiguous fp32 [n_tokens][d]")
        for t in (doc_start, doc_len):
            if t.dtype != torch.int32 or t.numel() != self.cfg.batch or not t.is_contiguous():
                raise ValueError("doc_start / doc_len must be contiguous int32 [batch]")
        st = (stream or torch.cuda.current_stream(self.device)).cuda_stream
        status = B.lol_core_forward_docs(self.ccfg, s_in.shape[0], doc_start.data_ptr(),
                                         doc_len.data_ptr(), s_in.data_ptr(), self.lib, self.rt,
                                         _ptr(self.forced_expert), _ptr(self.forced_gate),
                                         s_out.data_ptr(), self.path, self.workspace.data_ptr(),
                                         self.ws_bytes, st)
        if status != B.LOL_OK:
            raise B.LolError(status, "lol_core_forward_docs")
        return s_out

    def read_buckets(self, stream: Optional[torch.cuda.Stream] = None) -> dict:
        """The last routed depth's expert bucketing of the most recent forward
        (``lol_core_read_buckets``), split into its named tables (numpy)."""
        n = B.lol_core_buckets_size(self.ccfg)
        out = torch.empty(n, dtype=torch.int32, device=self.device)
        st = (stream or torch.cuda.current_stream(self.device)).cuda_stream
        status = B.lol_core_read_buckets(self.ccfg, self.workspace.data_ptr(), self.ws_bytes,
                                         out.data_ptr(), st)
        if status != B.LOL_OK:
            raise B.LolError(status, "lol_core_read_buckets")
        torch.cuda.synchronize(self.device)
        a = out.cpu().numpy()
        L, slots = self.cfg.L, self.cfg.batch * self.k_max
        m128 = -(-self.cfg.batch * self.cfg.n // 128) + L
        m256 = -(-self.cfg.batch * self.cfg.n // 256) + L
        sizes = (("counts", L), ("row_off", L + 1), ("win_row0", slots), ("n_tiles", 2),
                 ("tiles128", 2 * m128), ("tiles256", 2 * m256))
        if sum(sz for _, sz in sizes) != n:
            raise RuntimeError("lol_core_buckets_size disagrees with the documented layout")
        res, off = {}, 0
        for name, sz in sizes:
            res[name] = a[off:off + sz].copy()
            off += sz
        res["tiles128"] = res["tiles128"].reshape(m128, 2)
        res["tiles256"] = res["tiles256"].reshape(m256, 2)
        return res

    def flags(self, stream: Optional[torch.cuda.Stream] = None) -> int:
        st = (stream or torch.cuda.current_stream(self.device)).cuda_stream
        return B.lol_core_read_flags(self.workspace.data_ptr(), st)

    def path_numpy(self):
        return (self.path_expert.cpu().numpy(), self.path_gate.cpu().numpy(),
                self.path_margin.cpu().numpy())


class DeviceDecoder:
    """Incremental decode on the GPU: ``step(pos, x)`` feeds token ``pos`` of
    every document (x: [batch][d] fp32 device tensor) through the routed
    depths with ``lol_decode_step`` and returns s^(D) of those tokens.  The
    library and router are those of a ``DeviceCore`` (shared device memory)."""

    def __init__(self, core: DeviceCore):
        self.core = core
        self.cfg = core.cfg
        self.state_bytes = B.lol_decode_state_size(core.ccfg)
        if self.state_bytes == 0:
            raise B.LolError(B.LOL_EUNSUPPORTED, f"decode of config {self.cfg.name}")
        self.state = torch.empty(self.state_bytes, dtype=torch.uint8, device=core.device)
        self.y = torch.empty((self.cfg.batch, self.cfg.d), dtype=torch.float32,
                             device=core.device)
        self.reset()

    def _stream(self, stream):
        return (stream or torch.cuda.current_stream(self.core.device)).cuda_stream

    def reset(self, stream: Optional[torch.cuda.Stream] = None) -> None:
        status = B.lol_decode_reset(self.core.ccfg, self.state.data_ptr(), self.state_bytes,
                                    self._stream(stream))
        if status != B.LOL_OK:
            raise B.LolError(status, "lol_decode_reset")

    def reset_row(self, row: int, stream: Optional[torch.cuda.Stream] = None) -> None:
        """Start a new document in one row; the other rows continue."""
        status = B.lol_decode_reset_row(self.core.ccfg, self.state.data_ptr(), self.state_bytes,
                                        row, self._stream(stream))
        if status != B.LOL_OK:
            raise B.LolError(status, "lol_decode_reset_row")

    def step(self, pos: Optional[int], x: torch.Tensor, y: Optional[torch.Tensor] = None,
             stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """pos: every row's position (lockstep), or None for each row's own
        next position held by the state."""
        pos = -1 if pos is None else pos
        y = self.y if y is None else y
        for t in (x, y):
            if (t.shape != (self.cfg.batch, self.cfg.d) or t.dtype != torch.float32
                    or not t.is_contiguous()):
                raise ValueError("x / y must be contiguous fp32 [batch][d]")
        c = self.core
        status = B.lol_decode_step(c.ccfg, pos, x.data_ptr(), c.lib, c.rt,
                                   _ptr(c.forced_expert), _ptr(c.forced_gate), y.data_ptr(),
                                   c.path, self.state.data_ptr(), self.state_bytes,
                                   self._stream(stream))
        if status != B.LOL_OK:
            raise B.LolError(status, "lol_decode_step")
        return y

    def flags(self, stream: Optional[torch.cuda.Stream] = None) -> int:
        return B.lol_decode_read_flags(self.state.data_ptr(), self._stream(stream))
