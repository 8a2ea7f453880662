"""The C ABI library on the host (no GPU needed): it loads, exports every entry point the header
declares, and rejects bad arguments before touching a device."""
import ctypes
import os
import re

import pytest

from expert_ffn_canvas_amd import dgmoe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", n) for n in sorted(os.listdir(os.path.join(ROOT, "include")))
           if n.endswith(".h")]


def declared_functions():
    names = set()
    for hdr in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(hdr).read(), flags=re.S)
        names |= set(re.findall(r"\b(dg_\w+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("dg_moe_create", "dg_moe_forward", "dg_moe_destroy", "dg_head_create", "dg_head_forward",
              "dg_head_destroy"):
        assert n in names
    assert set(names) == set(dgmoe.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(dgmoe.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported"


def test_struct_layouts_match_the_header():
    # dg_moe_config: 11 four-byte fields; dg_moe_weights: 8 pointers; dg_moe_debug: 8 pointers
    assert ctypes.sizeof(dgmoe.dg_moe_config) == 44
    assert ctypes.sizeof(dgmoe.dg_moe_weights) == 64
    assert ctypes.sizeof(dgmoe.dg_moe_debug) == 64


def test_version_and_status_strings():
    assert dgmoe.dg_moe_abi_version() == 2
    assert dgmoe.dg_moe_status_string(dgmoe.DG_OK) == "ok"
    for st in range(-7, 0):
        assert dgmoe.dg_moe_status_string(st) not in ("", "unknown status")
    assert dgmoe.dg_moe_status_string(-99) == "unknown status"


def test_workspace_bytes():
    good = dgmoe.make_config(max_tokens=256)
    ws = dgmoe.dg_moe_workspace_bytes(good)
    # at least act and the bf16 per-slot outputs, plus the router weight in fp32
    T, K, D, F, E = 256, 8, 2816, 704, 128
    assert ws >= K * T * F * 2 + K * T * D * 2 + E * D * 4
    assert dgmoe.dg_moe_workspace_bytes(dgmoe.make_config(D=100)) == 0
    q8 = dgmoe.make_config(max_tokens=256, experts=dgmoe.DG_Q8_0, flags=dgmoe.DG_MOE_PACK_WEIGHTS)
    assert dgmoe.dg_moe_workspace_bytes(q8) >= K * T * F * 2 + K * T * D * 2 + E * D * 4
    assert dgmoe.dg_moe_workspace_bytes(dgmoe.make_config(experts=dgmoe.DG_Q8_0)) == 0


def _weights(align=16):
    base = 1 << 20
    return dgmoe.dg_moe_weights(base, base + 1 * 4096, 0, base + 2 * 4096, base + 3 * 4096, base + 4 * 4096,
                                0, 0) if align == 16 else \
        dgmoe.dg_moe_weights(base + 8, base + 4096, 0, base + 2 * 4096, base + 3 * 4096, base + 4 * 4096, 0, 0)


@pytest.mark.parametrize("field,value,status", [
    ("n_experts", 0, dgmoe.DG_ERR_SHAPE),
    ("n_experts", 300, dgmoe.DG_ERR_SHAPE),
    ("top_k", 9, dgmoe.DG_ERR_SHAPE),
    ("top_k", 0, dgmoe.DG_ERR_SHAPE),
    ("d_model", 2800, dgmoe.DG_ERR_SHAPE),
    ("d_ff", 700, dgmoe.DG_ERR_SHAPE),
    ("max_tokens", 0, dgmoe.DG_ERR_SHAPE),
    ("rms_eps", 0.0, dgmoe.DG_ERR_INVALID_ARG),
    ("act_dtype", dgmoe.DG_F16, dgmoe.DG_ERR_DTYPE),
    ("router_w_dtype", dgmoe.DG_I4G128, dgmoe.DG_ERR_DTYPE),
    ("expert_w_dtype", dgmoe.DG_F32, dgmoe.DG_ERR_DTYPE),
    ("expert_w_dtype", 7, dgmoe.DG_ERR_DTYPE),
    # Q8_0 and MX blocks are read from the packed copy only: without DG_MOE_PACK_WEIGHTS they are refused
    ("expert_w_dtype", dgmoe.DG_Q8_0, dgmoe.DG_ERR_DTYPE),
    ("expert_w_dtype", dgmoe.DG_MXFP4, dgmoe.DG_ERR_DTYPE),
    ("expert_w_dtype", dgmoe.DG_MXFP8, dgmoe.DG_ERR_DTYPE),
    ("flags", 0x80, dgmoe.DG_ERR_INVALID_ARG),
    ("struct_size", 12, dgmoe.DG_ERR_INVALID_ARG),
])
def test_create_rejects_bad_config(field, value, status):
    cfg = dgmoe.make_config()
    setattr(cfg, field, value)
    st, h = dgmoe.dg_moe_create(cfg, _weights(), 0)
    assert st == status
    assert not h.value
    assert dgmoe.dg_moe_last_error() != ""


def test_create_rejects_null_and_misaligned_weights():
    cfg = dgmoe.make_config()
    w = _weights()
    w.w_down = None
    st, _ = dgmoe.dg_moe_create(cfg, w, 0)
    assert st == dgmoe.DG_ERR_INVALID_ARG
    st, _ = dgmoe.dg_moe_create(cfg, _weights(align=8), 0)
    assert st == dgmoe.DG_ERR_ALIGN
    cfg4 = dgmoe.make_config(experts=dgmoe.DG_I4G128)
    st, _ = dgmoe.dg_moe_create(cfg4, _weights(), 0)  # int4 without scales
    assert st == dgmoe.DG_ERR_INVALID_ARG
    h = ctypes.c_void_p()
    assert dgmoe._lib.dg_moe_create(None, ctypes.byref(w), None, ctypes.byref(h)) == dgmoe.DG_ERR_INVALID_ARG


def test_forward_and_destroy_with_null_handle():
    assert dgmoe.dg_moe_forward(None, 16, 32, 4, None, 0, 0) == dgmoe.DG_ERR_INVALID_ARG
    dbg = dgmoe.dg_moe_debug()
    assert dgmoe.dg_moe_forward_debug(None, 16, 32, 4, dbg, 0) == dgmoe.DG_ERR_INVALID_ARG
    assert dgmoe.dg_moe_destroy(None) == dgmoe.DG_OK


# ----------------------------------------------------------------------------- canvas output stage

def test_head_struct_layout_and_workspace():
    assert ctypes.sizeof(dgmoe.dg_head_config) == 28
    cfg = dgmoe.make_head_config(V=262144, D=2816, max_tokens=256)
    # five arrays of (V / 256) x max_tokens four-byte partials
    assert dgmoe.dg_head_workspace_bytes(cfg) == 5 * 1024 * 256 * 4
    assert dgmoe.dg_head_workspace_bytes(dgmoe.make_head_config(D=100)) == 0


@pytest.mark.parametrize("field,value,status", [
    ("vocab", 0, dgmoe.DG_ERR_SHAPE),
    ("vocab", (1 << 24) + 1, dgmoe.DG_ERR_SHAPE),
    ("d_model", 2800, dgmoe.DG_ERR_SHAPE),
    ("d_model", 0, dgmoe.DG_ERR_SHAPE),
    ("max_tokens", 0, dgmoe.DG_ERR_SHAPE),
    ("h_dtype", dgmoe.DG_F32, dgmoe.DG_ERR_DTYPE),
    ("emb_dtype", dgmoe.DG_MXFP8, dgmoe.DG_ERR_DTYPE),
    ("flags", 1, dgmoe.DG_ERR_INVALID_ARG),
    ("struct_size", 12, dgmoe.DG_ERR_INVALID_ARG),
])
def test_head_create_rejects_bad_config(field, value, status):
    cfg = dgmoe.make_head_config()
    setattr(cfg, field, value)
    st, h = dgmoe.dg_head_create(cfg, 1 << 20)
    assert st == status and not h.value
    assert dgmoe.dg_moe_last_error() != ""


def test_head_create_rejects_null_and_misaligned_table():
    cfg = dgmoe.make_head_config()
    st, h = dgmoe.dg_head_create(cfg, 0)
    assert st == dgmoe.DG_ERR_INVALID_ARG and not h.value
    st, h = dgmoe.dg_head_create(cfg, (1 << 20) + 8)
    assert st == dgmoe.DG_ERR_ALIGN and not h.value


def test_head_forward_and_destroy_with_null_handle():
    assert dgmoe.dg_head_forward(None, 16, 4, 1.0, None, 32, 48, None, 0) == dgmoe.DG_ERR_INVALID_ARG
    assert dgmoe.dg_head_forward_profiled(None, 16, 4, 1.0, None, 32, 48, None, [1] * 6, 0) == \
        dgmoe.DG_ERR_INVALID_ARG
    assert dgmoe.dg_head_destroy(None) == dgmoe.DG_OK
