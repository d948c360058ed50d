"""CPU checks of the C ABI: the built library loads, exports every function
include/lol_core.h declares, and rejects invalid configurations and
arguments on the host before anything is launched."""
import ctypes
import os
import re

import pytest

from runtime_routed_transformer_amd import binding as B
from runtime_routed_transformer_amd.core import make_config
from runtime_routed_transformer_amd.workloads import CONFIG_BY_NAME, CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lol_core.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lol_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("liblol_core.so is not built (run __graft_entry__.build())")
    return B.load()


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert declared == B.exported_symbols()
    for name in declared:
        assert hasattr(lib, name), name


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        B._lib_saved = B._lib
        try:
            B._lib = None
            B.load(str(tmp_path / "nope.so"))
        finally:
            B._lib = B._lib_saved


def test_sizes_and_validation(lib):
    for cfg in CONFIGS:
        c = make_config(cfg)
        assert B.lol_core_validate(c) == B.LOL_OK, cfg.name
        assert B.lol_core_k_max(c) == -(-cfg.n // cfg.W) + 1
        assert B.lol_core_workspace_size(c) > 0
    base = CONFIG_BY_NAME["small_bf16"]
    bad = {
        "W": 0, "S": -1, "n_heads": 3, "L": 0, "D": 0, "batch": 0, "n": 0, "d_ffn": 0,
    }
    for k, v in bad.items():
        c = make_config(base)
        setattr(c, k, v)
        assert B.lol_core_validate(c) == B.LOL_EINVAL, k
        assert B.lol_core_workspace_size(c) == 0
    c = make_config(base); c.L = 65
    assert B.lol_core_validate(c) == B.LOL_EUNSUPPORTED
    # documents x window slots: 64 x 128 = 8,192 is the most one depth takes
    c = make_config(base); c.L = 64; c.batch = 64; c.n = 254; c.W = 2; c.S = 1
    assert B.lol_core_k_max(c) == 128 and B.lol_core_validate(c) == B.LOL_OK
    c.batch = 65
    assert B.lol_core_validate(c) == B.LOL_EUNSUPPORTED
    c = make_config(base); c.n_heads = 4      # d_head 128
    assert B.lol_core_validate(c) == B.LOL_EUNSUPPORTED
    c = make_config(base); c.d_ffn = 192       # bf16 needs multiples of 128
    assert B.lol_core_validate(c) == B.LOL_EUNSUPPORTED
    c = make_config(base); c.mlp = 7
    assert B.lol_core_validate(c) == B.LOL_EINVAL
    c = make_config(base); c.rms_eps = 0.0
    assert B.lol_core_validate(c) == B.LOL_EINVAL


def test_forward_rejects_bad_arguments_before_launch(lib):
    c = make_config(CONFIG_BY_NAME["tiny_fp32"])
    libw = B.lol_library(wqkv=16, wo=16, w_gu=16, w_down=16, g_attn=16, g_ffn=16)
    rt = B.lol_router(w_r=16, e_depth=16)
    ws = B.lol_core_workspace_size(c)
    # NULL s0
    assert B.lol_core_forward(c, None, libw, rt, None, None, 16, None, 256, ws, None) == B.LOL_EINVAL
    # NULL weight
    libn = B.lol_library(wqkv=None, wo=16, w_gu=16, w_down=16, g_attn=16, g_ffn=16)
    assert B.lol_core_forward(c, 16, libn, rt, None, None, 16, None, 256, ws, None) == B.LOL_EINVAL
    # FiLM half given
    libf = B.lol_library(wqkv=16, wo=16, w_gu=16, w_down=16, g_attn=16, g_ffn=16, film_gamma=16)
    assert B.lol_core_forward(c, 16, libf, rt, None, None, 16, None, 256, ws, None) == B.LOL_EINVAL
    # workspace too small / missing
    assert B.lol_core_forward(c, 16, libw, rt, None, None, 16, None, 256, ws - 1, None) == B.LOL_EWORKSPACE
    assert B.lol_core_forward(c, 16, libw, rt, None, None, 16, None, None, ws, None) == B.LOL_EWORKSPACE
    # invalid config
    c.W = 0
    assert B.lol_core_forward(c, 16, libw, rt, None, None, 16, None, 256, ws, None) == B.LOL_EINVAL


def test_status_and_kernel_names(lib):
    assert B.status_str(B.LOL_OK) == "ok"
    assert "workspace" in B.status_str(B.LOL_EWORKSPACE)
    names = [B.lol_core_kernel_name(k) for k in range(B.LOL_KERNEL_KINDS)]
    assert all(names) and len(set(names)) == len(names)
    assert B.lol_core_kernel_name(B.LOL_KERNEL_KINDS) is None


def test_timing_controls_validate(lib):
    # host-only calls: the kind mask and the depth filter
    assert lib.lol_core_timing_enable(1 << B.LOL_KERNEL_KINDS) == B.LOL_EINVAL
    assert lib.lol_core_timing_depth(-2) == B.LOL_EINVAL
    for depth in (0, 5, -1):
        assert lib.lol_core_timing_depth(depth) == B.LOL_OK
    assert lib.lol_core_timing_enable(0) == B.LOL_OK


def test_forward_rejects_unknown_variant_flags(lib):
    # router tying and FiLM layout flags are 0 or 1; anything else is rejected
    # before any launch
    c = make_config(CONFIG_BY_NAME["tiny_fp32"])
    ws = B.lol_core_workspace_size(c)
    for lib_flag, rt_flag in ((2, 0), (0, 2), (-1, 0)):
        libw = B.lol_library(wqkv=16, wo=16, w_gu=16, w_down=16, g_attn=16, g_ffn=16,
                             film_per_expert=lib_flag)
        rt = B.lol_router(w_r=16, e_depth=16, per_depth=rt_flag)
        assert B.lol_core_forward(c, 16, libw, rt, None, None, 16, None, 256, ws, None) == B.LOL_EINVAL


def test_embedding_and_readout_reject_bad_arguments(lib):
    # host-checked before any launch
    assert lib.lol_lm_head_workspace_size(64, 128, 256, B.LOL_BF16) > 0
    assert lib.lol_lm_head_workspace_size(64, 96, 256, B.LOL_BF16) == 0    # d % 128
    assert lib.lol_lm_head_workspace_size(64, 128, 200, B.LOL_BF16) == 0   # V % 128
    assert lib.lol_lm_head_workspace_size(64, 64, 64, B.LOL_FP32) > 0
    assert lib.lol_lm_head_workspace_size(0, 64, 64, B.LOL_FP32) == 0
    ws = lib.lol_lm_head_workspace_size(64, 128, 256, B.LOL_BF16)
    args = dict(s=16, T=64, d=128, g=16, eps=1e-6, w=16, V=256, dt=B.LOL_BF16, out=16)
    def head(**kw):
        a = {**args, **kw}
        return lib.lol_lm_head(a["s"], a["T"], a["d"], a["g"], a["eps"], a["w"], a["V"], a["dt"],
                               a["out"], kw.get("ws", 256), kw.get("wsb", ws), None)
    assert head(s=None) == B.LOL_EINVAL
    assert head(eps=0.0) == B.LOL_EINVAL
    assert head(V=200) == B.LOL_EINVAL
    assert head(dt=7) == B.LOL_EINVAL
    assert head(wsb=ws - 1) == B.LOL_EWORKSPACE
    assert head(ws=None) == B.LOL_EWORKSPACE
    assert lib.lol_embed(None, 4, 16, 10, 64, B.LOL_FP32, 16, None) == B.LOL_EINVAL
    assert lib.lol_embed(16, 4, 16, 10, 62, B.LOL_FP32, 16, None) == B.LOL_EINVAL
    assert lib.lol_embed(16, 0, 16, 10, 64, B.LOL_FP32, 16, None) == B.LOL_EINVAL
    assert lib.lol_embed(16, 4, 16, 10, 64, 5, 16, None) == B.LOL_EINVAL


def test_decode_sizes_and_host_checks(lib):
    # decode state sizes, supported range and host-side rejections (no launch)
    for cfg in CONFIGS:
        c = make_config(cfg)
        size = B.lol_decode_state_size(c)
        # keys and values of one open window per depth, document and head dominate
        act = 2 if cfg.dtype == "bf16" else 4
        assert size >= 2 * cfg.D * cfg.batch * cfg.W * cfg.d * act, cfg.name
    c = make_config(CONFIG_BY_NAME["small_bf16"]); c.batch = 65
    assert B.lol_decode_state_size(c) == 0
    c = make_config(CONFIG_BY_NAME["small_bf16"]); c.W = 0
    assert B.lol_decode_state_size(c) == 0
    c = make_config(CONFIG_BY_NAME["tiny_fp32"])
    size = B.lol_decode_state_size(c)
    libw = B.lol_library(wqkv=16, wo=16, w_gu=16, w_down=16, g_attn=16, g_ffn=16)
    rt = B.lol_router(w_r=16, e_depth=16)

    def step(pos=0, x=16, y=16, state=256, nbytes=size, libx=libw, rtx=rt):
        return B.lol_decode_step(c, pos, x, libx, rtx, None, None, y, None, state, nbytes, None)
    assert step(x=None) == B.LOL_EINVAL
    assert step(y=None) == B.LOL_EINVAL
    assert step(pos=-2) == B.LOL_EINVAL
    assert step(pos=c.n) == B.LOL_EINVAL
    assert step(nbytes=size - 1) == B.LOL_EWORKSPACE
    assert step(state=None) == B.LOL_EWORKSPACE
    assert step(state=256 + 16) == B.LOL_EWORKSPACE       # not 256-byte aligned
    assert step(libx=B.lol_library(wqkv=16, wo=16, w_gu=16, w_down=None, g_attn=16,
                                   g_ffn=16)) == B.LOL_EINVAL
    assert step(rtx=B.lol_router(w_r=16, e_depth=16, per_depth=3)) == B.LOL_EINVAL
    assert B.lol_decode_reset(c, None, size, None) == B.LOL_EWORKSPACE
    assert B.lol_decode_reset(c, 256, size - 1, None) == B.LOL_EWORKSPACE
    big = make_config(CONFIG_BY_NAME["tiny_fp32"]); big.d = 8192; big.n_heads = 128
    assert B.lol_decode_reset(big, 256, 1 << 40, None) == B.LOL_EUNSUPPORTED
    assert lib.lol_decode_read_flags(None, None, None) == B.LOL_EINVAL
    for row in (-1, c.batch):
        assert B.lol_decode_reset_row(c, 256, size, row, None) == B.LOL_EINVAL
    assert B.lol_decode_reset_row(c, None, size, 0, None) == B.LOL_EWORKSPACE


def test_prepared_wo_panels_sizes_and_rejections(lib):
    """lol_prepare_wo_panels: a buffer of L d d bf16 values where the fused
    output projection is used (bf16, d a multiple of 256 up to 1024), none
    elsewhere; bad arguments are refused before anything is launched."""
    for cfg in CONFIGS:
        c = make_config(cfg)
        want = cfg.L * cfg.d * cfg.d * 2 if (cfg.dtype == "bf16" and cfg.d % 256 == 0
                                             and cfg.d <= 1024) else 0
        assert B.lol_prepare_wo_panels_size(c) == want, cfg.name
    tiny = make_config(CONFIG_BY_NAME["tiny_fp32"])
    assert B.lol_prepare_wo_panels(tiny, 4096, 1 << 20, None) == B.LOL_EUNSUPPORTED
    mid = make_config(CONFIG_BY_NAME["mid_bf16"])
    size = B.lol_prepare_wo_panels_size(mid)
    assert B.lol_prepare_wo_panels(mid, None, 4096, None) == B.LOL_EINVAL
    assert B.lol_prepare_wo_panels(mid, 4096, None, None) == B.LOL_EINVAL
    assert B.lol_prepare_wo_panels(mid, 4096 + 8, 1 << 40, None) == B.LOL_EINVAL   # misaligned
    assert B.lol_prepare_wo_panels(mid, 4096, 4096 + size - 16, None) == B.LOL_EINVAL  # overlap
    bad = make_config(CONFIG_BY_NAME["mid_bf16"]); bad.W = 0
    assert B.lol_prepare_wo_panels_size(bad) == 0
    assert B.lol_prepare_wo_panels(bad, 4096, 1 << 40, None) == B.LOL_EINVAL


def test_prepared_weight_panels_sizes_and_rejections(lib):
    """lol_prepare_weight_panels: the three GEMM matrices' bytes in bf16 mode,
    nothing in fp32 mode; bad arguments are refused before anything is
    launched, and a forward refuses weight panels in fp32 mode or
    misaligned."""
    for cfg in CONFIGS:
        c = make_config(cfg)
        n_gu = (2 if cfg.mlp == "swiglu" else 1) * cfg.d_ffn
        want = (cfg.L * (3 * cfg.d * cfg.d + n_gu * cfg.d + cfg.d * cfg.d_ffn) * 2
                if cfg.dtype == "bf16" else 0)
        assert B.lol_prepare_weight_panels_size(c) == want, cfg.name
    tiny = make_config(CONFIG_BY_NAME["tiny_fp32"])
    libw = B.lol_library(wqkv=4096, wo=4096, w_gu=1 << 36, w_down=1 << 37, g_attn=16, g_ffn=16)
    assert B.lol_prepare_weight_panels(tiny, libw, 1 << 40, None) == B.LOL_EUNSUPPORTED
    mid = make_config(CONFIG_BY_NAME["mid_bf16"])
    size = B.lol_prepare_weight_panels_size(mid)
    assert B.lol_prepare_weight_panels(mid, None, 1 << 40, None) == B.LOL_EINVAL
    assert B.lol_prepare_weight_panels(mid, libw, None, None) == B.LOL_EINVAL
    assert B.lol_prepare_weight_panels(mid, libw, (1 << 40) + 8, None) == B.LOL_EINVAL  # misaligned
    assert B.lol_prepare_weight_panels(mid, libw, 4096 + 16, None) == B.LOL_EINVAL  # overlaps wqkv
    assert B.lol_prepare_weight_panels(mid, libw, (1 << 37) - size + 16, None) == B.LOL_EINVAL  # w_down
    libm = B.lol_library(wqkv=4096, wo=4096, w_gu=None, w_down=1 << 37, g_attn=16, g_ffn=16)
    assert B.lol_prepare_weight_panels(mid, libm, 1 << 40, None) == B.LOL_EINVAL
    bad = make_config(CONFIG_BY_NAME["mid_bf16"]); bad.W = 0
    assert B.lol_prepare_weight_panels_size(bad) == 0
    assert B.lol_prepare_weight_panels(bad, libw, 1 << 40, None) == B.LOL_EINVAL
    # a forward with weight panels: fp32 mode and misaligned panels are
    # refused (before the workspace check, which a one-byte-short workspace
    # would fail: nothing can be launched)
    rt = B.lol_router(w_r=16, e_depth=16)
    for cfg, panels in ((CONFIG_BY_NAME["tiny_fp32"], 1 << 40), (CONFIG_BY_NAME["mid_bf16"], (1 << 40) + 8)):
        c = make_config(cfg)
        lw = B.lol_library(wqkv=16, wo=16, w_gu=16, w_down=16, g_attn=16, g_ffn=16, weight_panels=panels)
        ws = B.lol_core_workspace_size(c)
        assert B.lol_core_forward(c, 16, lw, rt, None, None, 16, None, 256, ws - 1, None) == B.LOL_EINVAL


def test_buckets_size_matches_the_documented_layout(lib):
    """counts [L], row_off [L + 1], win_row0 [batch K_max], n_tiles [2],
    tiles128 [ceil(T / 128) + L][2], tiles256 [ceil(T / 256) + L][2]."""
    for cfg in CONFIGS:
        c = make_config(cfg)
        T = cfg.batch * cfg.n
        want = (cfg.L + cfg.L + 1 + cfg.batch * cfg.k_max + 2 + 2 * (-(-T // 128) + cfg.L)
                + 2 * (-(-T // 256) + cfg.L))
        assert B.lol_core_buckets_size(c) == want, cfg.name
    mid = make_config(CONFIG_BY_NAME["mid_bf16"])
    ws = B.lol_core_workspace_size(mid)
    assert B.lol_core_read_buckets(mid, 1 << 20, ws, None, None) == B.LOL_EINVAL
    assert B.lol_core_read_buckets(mid, None, ws, 4096, None) == B.LOL_EWORKSPACE
    assert B.lol_core_read_buckets(mid, 1 << 20, ws - 1, 4096, None) == B.LOL_EWORKSPACE
    assert B.lol_core_read_buckets(mid, (1 << 20) + 16, ws, 4096, None) == B.LOL_EWORKSPACE
    bad = make_config(CONFIG_BY_NAME["mid_bf16"]); bad.D = 0
    assert B.lol_core_buckets_size(bad) == 0
    assert B.lol_core_read_buckets(bad, 1 << 20, ws, 4096, None) == B.LOL_EINVAL


def test_mfma_measurement_rejects_bad_arguments(lib):
    import ctypes
    tf, ghz = ctypes.c_double(), ctypes.c_double()
    f = lib.lol_measure_mfma_bf16
    assert f(16, 2, 10, 4096, 1 << 20, ctypes.byref(tf), ctypes.byref(ghz), None) == B.LOL_EINVAL
    assert f(16, 1, 0, 4096, 1 << 20, ctypes.byref(tf), ctypes.byref(ghz), None) == B.LOL_EINVAL
    assert f(16, 1, 10, None, 1 << 20, ctypes.byref(tf), ctypes.byref(ghz), None) == B.LOL_EINVAL
    assert f(16, 1, 10, 4096 + 16, 1 << 20, ctypes.byref(tf), ctypes.byref(ghz), None) == B.LOL_EINVAL
    assert f(16, 1, 10, 4096, 1 << 20, None, ctypes.byref(ghz), None) == B.LOL_EINVAL
    assert f(8, 1, 10, 4096, 1 << 20, ctypes.byref(tf), ctypes.byref(ghz), None) == B.LOL_EINVAL
    assert f(64, 1, 10, 4096, 1 << 20, ctypes.byref(tf), ctypes.byref(ghz), None) == B.LOL_EINVAL
