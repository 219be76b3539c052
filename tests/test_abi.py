"""The C ABI, checked on the host without a GPU.

The library must load, export every function include/latentmoe.h declares,
and reject bad arguments before anything is enqueued.  Every call here fails
validation (the workspace check comes last and is always given too few
bytes), so no kernel is ever launched with the placeholder pointers.
"""
import ctypes
import os
import re
import subprocess

import pytest

from sparse_moe_layer_06_amd import binding as B
from sparse_moe_layer_06_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "latentmoe.h")

FAKE = 0x100000  # aligned placeholder, never dereferenced
MIS = FAKE + 8   # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    fns = declared_functions()
    assert sorted(B.EXPORTED) == fns


def test_library_exports_every_declared_symbol():
    L = B.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def dims(**kw):
    cfg = synth.CONFIGS["mid_bf16"].with_(**kw) if kw else synth.CONFIGS["mid_bf16"]
    return B.dims_of(cfg)


def test_validate_accepts_every_workload():
    for cfg in synth.CONFIGS.values():
        assert B.validate_dims(B.dims_of(cfg)) == B.LMOE_OK, cfg.name
        assert B.workspace_bytes(cfg) > 0


@pytest.mark.parametrize("field,value,code", [
    ("l", 1000, B.LMOE_ERR_SHAPE),      # l != d/4
    ("d", 4000, B.LMOE_ERR_SHAPE),      # d not a multiple of 256
    ("T", 0, B.LMOE_ERR_SHAPE),
    ("E", 1025, B.LMOE_ERR_SHAPE),
    ("E", 0, B.LMOE_ERR_SHAPE),
    ("k", 0, B.LMOE_ERR_SHAPE),
    ("k", 129, B.LMOE_ERR_SHAPE),       # k > E
    ("f", 100, B.LMOE_ERR_SHAPE),
    ("f_s", 32, B.LMOE_ERR_SHAPE),
    ("act_dtype", 7, B.LMOE_ERR_DTYPE),
    ("expert_dtype", B.LMOE_F32, B.LMOE_ERR_DTYPE),  # fp32 experts with bf16 activations
    ("shared_dtype", 7, B.LMOE_ERR_DTYPE),
    ("shared_dtype", B.LMOE_F32, B.LMOE_ERR_DTYPE),  # fp32 shared weights with bf16 activations
    ("router_latent", 2, B.LMOE_ERR_SHAPE),
    ("proj_dtype", 7, B.LMOE_ERR_DTYPE),
    ("proj_dtype", B.LMOE_F32, B.LMOE_ERR_DTYPE),  # fp32 projections with bf16 activations
])
def test_validate_rejects(field, value, code):
    d = dims()
    setattr(d, field, value)
    assert B.validate_dims(d) == code
    assert B.lib().lmoe_workspace_bytes(ctypes.byref(d)) == 0


def test_workspace_grows_with_tokens():
    cfg = synth.CONFIGS["mid_bf16"]
    assert B.workspace_bytes(cfg, 1) < B.workspace_bytes(cfg, 64) < B.workspace_bytes(cfg, 2048)


def _forward(d, *, x=FAKE, W_down=FAKE, W_r=FAKE, bias=None, experts=None, W_up=FAKE, shared="auto",
             k=None, out=FAKE, ws=FAKE, ws_bytes=None, dbg=None):
    L = B.lib()
    ex = experts if experts is not None else B.Experts(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    if shared == "auto":
        shared = B.Shared(FAKE, FAKE) if d.f_s > 0 else None
    need = L.lmoe_workspace_bytes(ctypes.byref(d))
    ws_bytes = need - 1 if ws_bytes is None else ws_bytes
    assert ws_bytes < max(need, 1)  # guard: validation can never pass
    return L.latentmoe_forward(ctypes.byref(d), x, W_down, W_r, bias, ctypes.byref(ex), W_up,
                               ctypes.byref(shared) if shared is not None else None,
                               d.k if k is None else k, out, ws, ws_bytes,
                               ctypes.byref(dbg) if dbg is not None else None, None)


def test_forward_error_paths():
    d = dims()
    assert _forward(d) == B.LMOE_ERR_WORKSPACE
    assert _forward(d, ws=None, ws_bytes=0) == B.LMOE_ERR_WORKSPACE
    assert _forward(d, x=None) == B.LMOE_ERR_NULL
    assert _forward(d, out=None) == B.LMOE_ERR_NULL
    assert _forward(d, W_up=MIS) == B.LMOE_ERR_ALIGN
    assert _forward(d, bias=MIS) == B.LMOE_ERR_ALIGN
    assert _forward(d, k=d.k + 1) == B.LMOE_ERR_SHAPE
    assert _forward(d, shared=None) == B.LMOE_ERR_SHAPE  # f_s > 0 but no shared weights
    assert _forward(d, experts=B.Experts(FAKE, None, None, None, None, None, None, None)) == B.LMOE_ERR_NULL
    dbg = B.Debug(z=MIS)
    assert _forward(d, dbg=dbg) == B.LMOE_ERR_ALIGN
    bad = dims()
    bad.l = 1
    assert _forward(bad) == B.LMOE_ERR_SHAPE


def test_forward_nvfp4_requires_codes():
    d = B.dims_of(synth.CONFIGS["prefill_nvfp4"])
    ex = B.Experts(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert _forward(d, experts=ex) == B.LMOE_ERR_NULL


def test_staged_error_paths():
    L = B.lib()
    d = dims()
    need = L.lmoe_workspace_bytes(ctypes.byref(d))
    sh = B.Shared(FAKE, FAKE)
    assert L.lmoe_project_route(ctypes.byref(d), FAKE, FAKE, FAKE, None, ctypes.byref(sh), FAKE, FAKE, FAKE,
                                FAKE, None, FAKE, need - 1, None) == B.LMOE_ERR_NULL  # hs missing
    assert L.lmoe_project_route(ctypes.byref(d), FAKE, FAKE, FAKE, None, ctypes.byref(sh), FAKE, FAKE, FAKE,
                                FAKE, FAKE, FAKE, need - 1, None) == B.LMOE_ERR_WORKSPACE
    assert L.lmoe_permute(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, need - 1, None) == B.LMOE_ERR_NULL
    assert L.lmoe_permute(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == B.LMOE_ERR_WORKSPACE
    ex = B.Experts(FAKE, FAKE, None, None, None, None, None, None)
    assert L.lmoe_experts_ffn(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(ex), MIS, FAKE, need - 1,
                              None) == B.LMOE_ERR_ALIGN
    assert L.lmoe_combine_up(ctypes.byref(d), FAKE, FAKE, None, FAKE, ctypes.byref(sh), FAKE, None, FAKE, FAKE,
                             need - 1, None) == B.LMOE_ERR_NULL  # gate missing
    assert L.lmoe_combine_up(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE, need - 1,
                             None) == B.LMOE_ERR_SHAPE  # f_s > 0 without shared weights
    assert L.lmoe_combine_up(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, ctypes.byref(sh), FAKE, None, FAKE, FAKE,
                             need - 1, None) == B.LMOE_ERR_WORKSPACE


def test_strerror_and_last_error():
    L = B.lib()
    for code in range(-6, 1):
        assert L.lmoe_strerror(code)
    assert L.lmoe_last_hip_error() == 0


def test_pack_error_paths():
    L = B.lib()
    far = FAKE + (1 << 30)  # disjoint placeholder
    assert L.lmoe_pack_expert_weights(2, 100, 64, FAKE, far, None) == B.LMOE_ERR_SHAPE
    assert L.lmoe_pack_expert_weights(2, 64, 96, FAKE, far, None) == B.LMOE_ERR_SHAPE
    assert L.lmoe_pack_expert_weights(0, 64, 64, FAKE, far, None) == B.LMOE_ERR_SHAPE
    assert L.lmoe_pack_expert_weights(2, 64, 64, None, far, None) == B.LMOE_ERR_NULL
    assert L.lmoe_pack_expert_weights(2, 64, 64, MIS, far, None) == B.LMOE_ERR_ALIGN
    assert L.lmoe_pack_expert_weights(2, 64, 64, FAKE, FAKE + 4096, None) == B.LMOE_ERR_SHAPE  # overlap


def test_tiled_experts_need_bf16_activations():
    d = dims()
    d.expert_dtype = B.LMOE_BF16_TILED
    assert B.validate_dims(d) == B.LMOE_OK
    d.act_dtype = B.LMOE_F32
    assert B.validate_dims(d) == B.LMOE_ERR_DTYPE


def test_fp8_shared_rules():
    d = dims()  # bf16 activations, f_s = 4096
    d.shared_dtype = B.LMOE_FP8_E4M3
    assert B.validate_dims(d) == B.LMOE_OK
    d.f_s = 4096 + 64  # the fp8 K step is 128
    assert B.validate_dims(d) == B.LMOE_ERR_SHAPE
    f = B.dims_of(synth.CONFIGS["tiny_f32"])
    f.shared_dtype = B.LMOE_FP8_E4M3  # fp8 shared weights need bf16 activations
    assert B.validate_dims(f) == B.LMOE_ERR_DTYPE
    # the per-row scales are required with fp8 weights
    d = dims()
    d.shared_dtype = B.LMOE_FP8_E4M3
    assert _forward(d, shared=B.Shared(FAKE, FAKE, None, FAKE)) == B.LMOE_ERR_NULL
    assert _forward(d, shared=B.Shared(FAKE, FAKE, FAKE, MIS)) == B.LMOE_ERR_ALIGN
    assert _forward(d, shared=B.Shared(FAKE, FAKE, FAKE, FAKE)) == B.LMOE_ERR_WORKSPACE
    assert B.lib().lmoe_workspace_bytes(ctypes.byref(d)) > B.lib().lmoe_workspace_bytes(ctypes.byref(dims()))


def test_fp8_projection_rules():
    d = dims(proj_fp8=True)  # bf16 activations, l = 1024
    assert B.validate_dims(d) == B.LMOE_OK
    f = B.dims_of(synth.CONFIGS["tiny_f32"])
    f.proj_dtype = B.LMOE_FP8_E4M3  # fp8 projections need bf16 activations
    assert B.validate_dims(f) == B.LMOE_ERR_DTYPE
    std = dims(standard_moe=True, l=4096, proj_fp8=True)  # a standard MoE has no projections
    assert B.validate_dims(std) == B.LMOE_ERR_DTYPE
    assert B.validate_dims(dims(d=512, l=128, proj_fp8=True)) == B.LMOE_OK
    assert B.validate_dims(dims(d=256, l=64, proj_fp8=True)) == B.LMOE_ERR_SHAPE  # fp8 K step of W_up

    def mat(codes, scales):  # host lmoe_fp8_matrix naming device arrays
        m = B.Fp8Matrix(codes, scales)
        return m, ctypes.cast(ctypes.pointer(m), ctypes.c_void_p)

    good, pg = mat(FAKE, FAKE)
    no_scales, pn = mat(FAKE, None)
    mis, pm = mat(MIS, FAKE)
    assert _forward(d, W_down=pg, W_up=pg) == B.LMOE_ERR_WORKSPACE
    assert _forward(d, W_down=None, W_up=pg) == B.LMOE_ERR_NULL
    assert _forward(d, W_down=pg, W_up=pn) == B.LMOE_ERR_NULL
    assert _forward(d, W_down=pm, W_up=pg) == B.LMOE_ERR_ALIGN
    L = B.lib()
    assert L.lmoe_workspace_bytes(ctypes.byref(d)) > L.lmoe_workspace_bytes(ctypes.byref(dims()))
    need = L.lmoe_workspace_bytes(ctypes.byref(d))
    sh = B.Shared(FAKE, FAKE)
    assert L.lmoe_project_route(ctypes.byref(d), FAKE, pn, FAKE, None, ctypes.byref(sh), FAKE, FAKE, FAKE,
                                FAKE, FAKE, FAKE, need - 1, None) == B.LMOE_ERR_NULL
    assert L.lmoe_combine_up(ctypes.byref(d), FAKE, FAKE, FAKE, pm, ctypes.byref(sh), FAKE, None, FAKE, FAKE,
                             need - 1, None) == B.LMOE_ERR_ALIGN
    assert L.lmoe_combine_up(ctypes.byref(d), FAKE, FAKE, FAKE, pg, ctypes.byref(sh), FAKE, None, FAKE, FAKE,
                             need - 1, None) == B.LMOE_ERR_WORKSPACE


def test_mxfp8_projection_rules():
    d = dims(proj_mxfp8=True)
    assert d.proj_dtype == B.LMOE_MXFP8 and B.validate_dims(d) == B.LMOE_OK
    f = B.dims_of(synth.CONFIGS["tiny_f32"])
    f.proj_dtype = B.LMOE_MXFP8  # 8-bit projections need bf16 activations
    assert B.validate_dims(f) == B.LMOE_ERR_DTYPE
    assert B.validate_dims(dims(standard_moe=True, l=4096, proj_mxfp8=True)) == B.LMOE_ERR_DTYPE
    assert B.validate_dims(dims(d=256, l=64, proj_mxfp8=True)) == B.LMOE_ERR_SHAPE
    good = B.Fp8Matrix(FAKE, FAKE)
    bad = B.Fp8Matrix(FAKE, MIS)
    pg = ctypes.cast(ctypes.pointer(good), ctypes.c_void_p)
    pb = ctypes.cast(ctypes.pointer(bad), ctypes.c_void_p)
    assert _forward(d, W_down=pg, W_up=pg) == B.LMOE_ERR_WORKSPACE
    assert _forward(d, W_down=pg, W_up=pb) == B.LMOE_ERR_ALIGN
    L = B.lib()
    assert L.lmoe_workspace_bytes(ctypes.byref(d)) > L.lmoe_workspace_bytes(ctypes.byref(dims()))


def test_quantize_rows_mxfp8_error_paths():
    L = B.lib()
    assert L.lmoe_quantize_rows_mxfp8(0, 64, FAKE, FAKE, FAKE, None) == B.LMOE_ERR_SHAPE
    assert L.lmoe_quantize_rows_mxfp8(4, 48, FAKE, FAKE, FAKE, None) == B.LMOE_ERR_SHAPE  # not a multiple of 32
    assert L.lmoe_quantize_rows_mxfp8(4, 1 << 21, FAKE, FAKE, FAKE, None) == B.LMOE_ERR_SHAPE
    assert L.lmoe_quantize_rows_mxfp8(4, 64, FAKE, None, FAKE, None) == B.LMOE_ERR_NULL
    assert L.lmoe_quantize_rows_mxfp8(4, 64, FAKE, FAKE, MIS, None) == B.LMOE_ERR_ALIGN


def test_quantize_rows_error_paths():
    L = B.lib()
    assert L.lmoe_quantize_rows_fp8(0, 64, FAKE, FAKE, FAKE, None) == B.LMOE_ERR_SHAPE
    assert L.lmoe_quantize_rows_fp8(4, 60, FAKE, FAKE, FAKE, None) == B.LMOE_ERR_SHAPE
    assert L.lmoe_quantize_rows_fp8(4, 1 << 21, FAKE, FAKE, FAKE, None) == B.LMOE_ERR_SHAPE
    assert L.lmoe_quantize_rows_fp8(4, 64, None, FAKE, FAKE, None) == B.LMOE_ERR_NULL
    assert L.lmoe_quantize_rows_fp8(4, 64, FAKE, FAKE, MIS, None) == B.LMOE_ERR_ALIGN


def test_context_error_paths():
    # host-side argument checks; creating a context needs the device to exist
    # (on a machine without one, or for device -1, LMOE_ERR_HIP)
    L = B.lib()
    assert L.lmoe_create(None, 0) == B.LMOE_ERR_NULL
    assert L.lmoe_destroy(None) == B.LMOE_OK
    assert L.lmoe_ctx_reserve(None, ctypes.byref(dims())) == B.LMOE_ERR_NULL
    assert L.lmoe_ctx_workspace_bytes(None) == 0
    h = ctypes.c_void_p()
    assert L.lmoe_create(ctypes.byref(h), -1) == B.LMOE_ERR_HIP and not h.value
    ex = B.Experts(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    d = dims()
    assert L.lmoe_ctx_forward(None, ctypes.byref(d), FAKE, FAKE, FAKE, None, ctypes.byref(ex), FAKE, None, d.k,
                              FAKE, None, None) == B.LMOE_ERR_NULL


def test_static_forward_rejects_layers_beyond_its_scratch_before_any_launch():
    # the allocation-free entry point: a layer whose workspace exceeds the
    # library's per-GPU scratch array is refused on the host
    big = synth.CONFIGS["prefill_bf16"]
    assert B.workspace_bytes(big) > B.LMOE_STATIC_SCRATCH_BYTES
    d = B.dims_of(big)
    rc = B.lib().lmoe_static_forward(ctypes.byref(d), None, None, None, None, None, None, None, big.k, None,
                                     None, None)
    assert rc == B.LMOE_ERR_WORKSPACE
    # the decode workloads fit
    for name in ("decode_bf16_zipf",):
        c = synth.CONFIGS[name]
        for v in (c, c.with_(router_latent=True), c.with_(proj_fp8=True), c.with_(proj_mxfp8=True),
                  c.with_(l=c.d, E=128, k=6, standard_moe=True)):
            assert B.workspace_bytes(v) <= B.LMOE_STATIC_SCRATCH_BYTES


def test_static_scratch_size_matches_header():
    with open(os.path.join(ROOT, "include", "latentmoe.h")) as fh:
        m = re.search(r"#define LMOE_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", fh.read())
    assert m and int(m.group(1)) << int(m.group(2)) == B.LMOE_STATIC_SCRATCH_BYTES
