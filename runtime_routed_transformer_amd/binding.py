"""ctypes binding of liblol_core (include/lol_core.h), names as in the C ABI.

Argument marshalling only: every step of the routed core runs in the HIP
kernels of ``csrc/``.  Loading fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int32, c_size_t, c_uint32, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "liblol_core.so")

LOL_OK, LOL_EINVAL, LOL_EUNSUPPORTED, LOL_EWORKSPACE, LOL_EHIP = range(5)
LOL_FP32, LOL_BF16 = 0, 1
LOL_MLP_SWIGLU, LOL_MLP_GELU = 0, 1
LOL_FLAG_BAD_FORCED_ID = 1
LOL_FLAG_BAD_DOC = 2
LOL_FLAG_BAD_POS = 4
LOL_KERNEL_KINDS = 12
LOL_TIMING_ALL = (1 << LOL_KERNEL_KINDS) - 1

# every function the header declares, with (restype, argtypes)
_SIGNATURES = {}


class LolError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} (status {status})")
        self.status = status


class lol_core_config(ctypes.Structure):
    _fields_ = [(name, c_int32) for name in
                ("batch", "n", "d", "n_heads", "d_ffn", "L", "D", "W", "S", "mlp", "dtype")] + \
               [("rms_eps", c_float), ("rope_theta", c_float)]


class lol_library(ctypes.Structure):
    _fields_ = [(name, c_void_p) for name in
                ("wqkv", "wo", "w_gu", "w_down", "g_attn", "g_ffn", "film_gamma", "film_beta")] + \
               [("film_per_expert", c_int32), ("wo_panels", c_void_p), ("weight_panels", c_void_p)]


class lol_router(ctypes.Structure):
    _fields_ = [(name, c_void_p) for name in ("w_r", "b_r", "e_depth", "expert_bias")] + \
               [("per_depth", c_int32)]


class lol_path(ctypes.Structure):
    _fields_ = [(name, c_void_p) for name in ("expert", "gate", "margin", "util")]


_SIGNATURES.update({
    "lol_core_k_max": (c_int32, [POINTER(lol_core_config)]),
    "lol_core_validate": (c_int32, [POINTER(lol_core_config)]),
    "lol_core_workspace_size": (c_size_t, [POINTER(lol_core_config)]),
    "lol_core_forward": (c_int32, [POINTER(lol_core_config), c_void_p, POINTER(lol_library),
                                   POINTER(lol_router), c_void_p, c_void_p, c_void_p,
                                   POINTER(lol_path), c_void_p, c_size_t, c_void_p]),
    "lol_core_forward_docs": (c_int32, [POINTER(lol_core_config), ctypes.c_int64, c_void_p,
                                        c_void_p, c_void_p, POINTER(lol_library),
                                        POINTER(lol_router), c_void_p, c_void_p, c_void_p,
                                        POINTER(lol_path), c_void_p, c_size_t, c_void_p]),
    "lol_core_read_flags": (c_int32, [c_void_p, POINTER(c_uint32), c_void_p]),
    "lol_core_forward_static": (c_int32, [POINTER(lol_core_config), c_void_p,
                                          POINTER(lol_library), POINTER(lol_router), c_void_p,
                                          c_void_p, c_void_p, POINTER(lol_path), c_void_p]),
    "lol_prepare_wo_panels_size": (c_size_t, [POINTER(lol_core_config)]),
    "lol_prepare_wo_panels": (c_int32, [POINTER(lol_core_config), c_void_p, c_void_p, c_void_p]),
    "lol_prepare_weight_panels_size": (c_size_t, [POINTER(lol_core_config)]),
    "lol_prepare_weight_panels": (c_int32, [POINTER(lol_core_config), POINTER(lol_library), c_void_p,
                                            c_void_p]),
    "lol_core_buckets_size": (c_size_t, [POINTER(lol_core_config)]),
    "lol_core_read_buckets": (c_int32, [POINTER(lol_core_config), c_void_p, c_size_t, c_void_p,
                                        c_void_p]),
    "lol_core_timing_enable": (c_int32, [c_uint32]),
    "lol_core_timing_depth": (c_int32, [c_int32]),
    "lol_embed": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_int32, c_void_p,
                            c_void_p]),
    "lol_lm_head_workspace_size": (c_size_t, [c_int32, c_int32, c_int32, c_int32]),
    "lol_lm_head": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_float, c_void_p, c_int32,
                              c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "lol_decode_state_size": (c_size_t, [POINTER(lol_core_config)]),
    "lol_decode_reset": (c_int32, [POINTER(lol_core_config), c_void_p, c_size_t, c_void_p]),
    "lol_decode_reset_row": (c_int32, [POINTER(lol_core_config), c_void_p, c_size_t, c_int32,
                                       c_void_p]),
    "lol_decode_step": (c_int32, [POINTER(lol_core_config), c_int32, c_void_p,
                                  POINTER(lol_library), POINTER(lol_router), c_void_p, c_void_p,
                                  c_void_p, POINTER(lol_path), c_void_p, c_size_t, c_void_p]),
    "lol_decode_read_flags": (c_int32, [c_void_p, POINTER(c_uint32), c_void_p]),
    "lol_core_timing_collect": (c_int32, [POINTER(c_double), POINTER(c_int32)]),
    "lol_core_kernel_name": (c_char_p, [c_int32]),
    "lol_measure_mfma_bf16_scratch_size": (c_size_t, []),
    "lol_measure_mfma_bf16": (c_int32, [c_int32, c_int32, c_int32, c_void_p, c_size_t, POINTER(c_double),
                                        POINTER(c_double), c_void_p]),
    "lol_status_str": (c_char_p, [c_int32]),
})

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liblol_core.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m runtime_routed_transformer_amd.build_lib` "
                "(there is no fallback implementation)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def exported_symbols():
    return sorted(_SIGNATURES)


def status_str(status: int) -> str:
    return load().lol_status_str(status).decode()


def _check(status: int, what: str) -> None:
    if status != LOL_OK:
        raise LolError(status, what)


def lol_core_k_max(cfg: lol_core_config) -> int:
    return load().lol_core_k_max(ctypes.byref(cfg))


def lol_core_validate(cfg: lol_core_config) -> int:
    return load().lol_core_validate(ctypes.byref(cfg))


def lol_core_workspace_size(cfg: lol_core_config) -> int:
    return load().lol_core_workspace_size(ctypes.byref(cfg))


def lol_core_forward(cfg, s0, lib, rt, forced_expert, forced_gate, s_out, path, workspace,
                     workspace_bytes, stream) -> int:
    """Pointers are ints (device addresses) or None; lib/rt/path are structs."""
    return load().lol_core_forward(ctypes.byref(cfg), s0, ctypes.byref(lib), ctypes.byref(rt),
                                   forced_expert, forced_gate, s_out,
                                   ctypes.byref(path) if path is not None else None,
                                   workspace, workspace_bytes, stream)


def lol_core_forward_docs(cfg, n_tokens, doc_start, doc_len, s0, lib, rt, forced_expert,
                          forced_gate, s_out, path, workspace, workspace_bytes, stream) -> int:
    """Packed documents: doc_start / doc_len are device int32 [batch] arrays (ints)."""
    return load().lol_core_forward_docs(ctypes.byref(cfg), int(n_tokens), doc_start, doc_len, s0,
                                        ctypes.byref(lib), ctypes.byref(rt), forced_expert,
                                        forced_gate, s_out,
                                        ctypes.byref(path) if path is not None else None,
                                        workspace, workspace_bytes, stream)


LOL_STATIC_SCRATCH_BYTES = 64 << 20


def lol_core_forward_static(cfg, s0, lib, rt, forced_expert, forced_gate, s_out, path,
                            stream) -> int:
    """The forward without a workspace argument (the library's own buffer)."""
    return load().lol_core_forward_static(ctypes.byref(cfg), s0, ctypes.byref(lib),
                                          ctypes.byref(rt), forced_expert, forced_gate, s_out,
                                          ctypes.byref(path) if path is not None else None,
                                          stream)


def lol_core_read_flags(workspace, stream) -> int:
    out = c_uint32(0)
    _check(load().lol_core_read_flags(workspace, ctypes.byref(out), stream), "lol_core_read_flags")
    return int(out.value)


def lol_prepare_wo_panels_size(cfg: lol_core_config) -> int:
    return load().lol_prepare_wo_panels_size(ctypes.byref(cfg))


def lol_prepare_wo_panels(cfg, wo, wo_panels, stream) -> int:
    return load().lol_prepare_wo_panels(ctypes.byref(cfg), wo, wo_panels, stream)


def lol_prepare_weight_panels_size(cfg: lol_core_config) -> int:
    return load().lol_prepare_weight_panels_size(ctypes.byref(cfg))


def lol_prepare_weight_panels(cfg, lib, weight_panels, stream) -> int:
    return load().lol_prepare_weight_panels(ctypes.byref(cfg), None if lib is None else ctypes.byref(lib),
                                            weight_panels, stream)


def lol_core_buckets_size(cfg: lol_core_config) -> int:
    return load().lol_core_buckets_size(ctypes.byref(cfg))


def lol_core_read_buckets(cfg, workspace, workspace_bytes, out, stream) -> int:
    return load().lol_core_read_buckets(ctypes.byref(cfg), workspace, workspace_bytes, out, stream)


def lol_decode_state_size(cfg: lol_core_config) -> int:
    return load().lol_decode_state_size(ctypes.byref(cfg))


def lol_decode_reset(cfg, state, state_bytes, stream) -> int:
    return load().lol_decode_reset(ctypes.byref(cfg), state, state_bytes, stream)


def lol_decode_reset_row(cfg, state, state_bytes, row, stream) -> int:
    return load().lol_decode_reset_row(ctypes.byref(cfg), state, state_bytes, int(row), stream)


def lol_decode_step(cfg, pos, x, lib, rt, forced_expert, forced_gate, y, path, state,
                    state_bytes, stream) -> int:
    """One token per document: x / y are device [batch][d] fp32 addresses;
    pos = -1 takes each row's own next position from the state."""
    return load().lol_decode_step(ctypes.byref(cfg), int(pos), x, ctypes.byref(lib),
                                  ctypes.byref(rt), forced_expert, forced_gate, y,
                                  ctypes.byref(path) if path is not None else None, state,
                                  state_bytes, stream)


def lol_decode_read_flags(state, stream) -> int:
    out = c_uint32(0)
    _check(load().lol_decode_read_flags(state, ctypes.byref(out), stream), "lol_decode_read_flags")
    return int(out.value)


def lol_core_timing_enable(mask: int) -> None:
    """Bit k of ``mask`` times kernel kind k; 0 disables, LOL_TIMING_ALL times all."""
    _check(load().lol_core_timing_enable(int(mask)), "lol_core_timing_enable")


def lol_core_timing_depth(depth: int) -> None:
    """Time only the launches of depth index ``depth`` (-1: every depth)."""
    _check(load().lol_core_timing_depth(int(depth)), "lol_core_timing_depth")


def kernel_kind(name: str) -> int:
    for k in range(LOL_KERNEL_KINDS):
        if lol_core_kernel_name(k) == name:
            return k
    raise KeyError(name)


def lol_core_timing_collect():
    ms = (c_double * LOL_KERNEL_KINDS)()
    cnt = (c_int32 * LOL_KERNEL_KINDS)()
    _check(load().lol_core_timing_collect(ms, cnt), "lol_core_timing_collect")
    return {lol_core_kernel_name(k): (float(ms[k]), int(cnt[k])) for k in range(LOL_KERNEL_KINDS)}


def lol_measure_mfma_bf16(shape: int, random_operands: bool, iters: int, scratch, scratch_bytes,
                          stream):
    """(TFLOP/s, GHz) of the register-only bf16 MFMA loop (measurement only);
    shape 32 = 32x32x16, 16 = 16x16x32."""
    tf, ghz = c_double(0.0), c_double(0.0)
    _check(load().lol_measure_mfma_bf16(int(shape), 1 if random_operands else 0, int(iters), scratch,
                                        scratch_bytes, ctypes.byref(tf), ctypes.byref(ghz), stream),
           "lol_measure_mfma_bf16")
    return float(tf.value), float(ghz.value)


def lol_core_kernel_name(kind: int):
    name = load().lol_core_kernel_name(kind)
    return None if name is None else name.decode()
