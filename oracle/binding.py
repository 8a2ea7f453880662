"""ctypes binding of the C++ oracle (test infrastructure only).

All arrays are numpy arrays on the host. bf16 tensors are passed as their raw
uint16 bit patterns, fp16 scales as uint16 bit patterns, int4 weights as the
packed uint8 bytes, Q8_0, MXFP4 and MXFP8 weights as their 34-, 17- and 33-byte blocks (uint8).
"""
import ctypes
import os

import numpy as np

from .build import LIB, SOURCES, build

_lib = None

DT_F32, DT_BF16, DT_F16, DT_I4G128, DT_Q8_0, DT_MXFP4, DT_MXFP8 = 0, 1, 2, 3, 4, 5, 6

_p = ctypes.c_void_p
_i = ctypes.c_int
_d = ctypes.c_double


def load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("DG_ORACLE_LIB")  # a sanitized build (oracle.build --sanitize), else the plain one
    if not path:
        path = LIB
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < max(os.path.getmtime(s) for s in SOURCES):
            build()
    lib = ctypes.CDLL(path)
    lib.oracle_gelu_tanh_f32.restype = ctypes.c_float
    lib.oracle_gelu_tanh_f32.argtypes = [ctypes.c_float]
    lib.oracle_gelu_tanh_f64.restype = ctypes.c_double
    lib.oracle_gelu_tanh_f64.argtypes = [ctypes.c_double]
    lib.oracle_half_to_float.restype = ctypes.c_float
    lib.oracle_half_to_float.argtypes = [ctypes.c_uint16]
    lib.oracle_float_to_bf16.restype = ctypes.c_uint16
    lib.oracle_float_to_bf16.argtypes = [ctypes.c_float]
    lib.oracle_dequant_i4.restype = None
    lib.oracle_dequant_i4.argtypes = [_p, _p, ctypes.c_int64, _i, _p]
    lib.oracle_dequant_q8_0.restype = None
    lib.oracle_dequant_q8_0.argtypes = [_p, ctypes.c_int64, _i, _p]
    lib.oracle_dequant_mxfp4.restype = None
    lib.oracle_dequant_mxfp4.argtypes = [_p, ctypes.c_int64, _i, _p]
    lib.oracle_dequant_mxfp8.restype = None
    lib.oracle_dequant_mxfp8.argtypes = [_p, ctypes.c_int64, _i, _p]
    lib.oracle_route.restype = _i
    lib.oracle_route.argtypes = [_i, _i, _i, _i, _d, _i, _p, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i]
    lib.oracle_permute.restype = _i
    lib.oracle_permute.argtypes = [_i, _i, _i, _p, _p, _p, _p, _p]
    lib.oracle_moe_forward.restype = _i
    lib.oracle_moe_forward.argtypes = [_i, _i, _i, _i, _i, _d, _i, _p, _i, _p, _p, _p, _p, _i, _p, _p,
                                       _p, _p, _p, _p, _i, _i, _p, _p, _p, _p, _p, _i]
    lib.oracle_expert_ffn.restype = _i
    lib.oracle_expert_ffn.argtypes = [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _i, _p]
    lib.oracle_canvas_head.restype = _i
    lib.oracle_canvas_head.argtypes = [_i, _i, _i, _p, _p, _d, _p, _i, _p, _p, _p, _p, _i]
    lib.oracle_round_bf16.restype = None
    lib.oracle_round_bf16.argtypes = [_p, _p, ctypes.c_int64]
    _lib = lib
    return lib


def _ptr(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle takes C-contiguous numpy arrays"
    return a.ctypes.data


def _dtype_code(a):
    if a.dtype == np.float32:
        return DT_F32
    if a.dtype == np.uint16:  # raw bf16 bits
        return DT_BF16
    raise TypeError(f"unsupported array dtype {a.dtype}")


def gelu_tanh_f32(z):
    return load().oracle_gelu_tanh_f32(float(z))


def gelu_tanh_f64(z):
    return load().oracle_gelu_tanh_f64(float(z))


def half_to_float(bits):
    return load().oracle_half_to_float(int(bits))


def float_to_bf16_bits(f):
    return load().oracle_float_to_bf16(float(f))


def dequant_i4(q, s, K):
    """q: uint8 [rows, ceil(K/2)], s: uint16 fp16 bits [rows, ceil(K/128)] -> fp32 [rows, K]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint16)
    rows = q.shape[0]
    out = np.empty((rows, K), dtype=np.float32)
    load().oracle_dequant_i4(_ptr(q), _ptr(s), rows, K, _ptr(out))
    return out


def dequant_q8_0(blocks, K):
    """blocks: uint8 [rows, K/32 * 34] (or [rows, K/32, 34]) -> fp32 [rows, K]."""
    rows = blocks.shape[0]
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(rows, -1)
    assert b.shape[1] == K // 32 * 34
    out = np.empty((rows, K), dtype=np.float32)
    load().oracle_dequant_q8_0(_ptr(b), rows, K, _ptr(out))
    return out


def dequant_mxfp4(blocks, K):
    """blocks: uint8 [rows, K/32 * 17] (or [rows, K/32, 17]) -> fp32 [rows, K]."""
    rows = blocks.shape[0]
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(rows, -1)
    assert b.shape[1] == K // 32 * 17
    out = np.empty((rows, K), dtype=np.float32)
    load().oracle_dequant_mxfp4(_ptr(b), rows, K, _ptr(out))
    return out


def dequant_mxfp8(blocks, K):
    """blocks: uint8 [rows, K/32 * 33] (or [rows, K/32, 33]) -> fp32 [rows, K]."""
    rows = blocks.shape[0]
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(rows, -1)
    assert b.shape[1] == K // 32 * 33
    out = np.empty((rows, K), dtype=np.float32)
    load().oracle_dequant_mxfp8(_ptr(b), rows, K, _ptr(out))
    return out


def _expert_arrays(w):
    """(dtype code, gate_up, down, gate_up scales, down scales, F) of a weight dict."""
    if "q_gate_up" in w:
        gu = w["q_gate_up"]
        return DT_I4G128, gu, w["q_down"], w["s_gate_up"], w["s_down"], gu.shape[1] // 2
    if "q8_gate_up" in w:
        gu = w["q8_gate_up"]
        return DT_Q8_0, np.ascontiguousarray(gu), np.ascontiguousarray(w["q8_down"]), None, None, gu.shape[1] // 2
    if "mx4_gate_up" in w:
        gu = w["mx4_gate_up"]
        return DT_MXFP4, np.ascontiguousarray(gu), np.ascontiguousarray(w["mx4_down"]), None, None, gu.shape[1] // 2
    if "mx8_gate_up" in w:
        gu = w["mx8_gate_up"]
        return DT_MXFP8, np.ascontiguousarray(gu), np.ascontiguousarray(w["mx8_down"]), None, None, gu.shape[1] // 2
    gu = w["w_gate_up"]
    return DT_BF16, gu, w["w_down"], None, None, gu.shape[1] // 2


def route(x, router_w, router_gamma, router_bias, k, eps, forced=None, n_threads=0):
    """Router only. Returns dict(idx [T,k] int32, w [T,k] f64, logits [T,E] f64, gap [T], r [T])."""
    T, D = x.shape
    E = router_w.shape[0]
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    logits = np.empty((T, E), dtype=np.float64)
    gap = np.empty((T,), dtype=np.float64)
    r = np.empty((T,), dtype=np.float64)
    forced_arr = None if forced is None else np.ascontiguousarray(forced, dtype=np.int32)
    rc = load().oracle_route(T, D, E, k, eps, _dtype_code(x), _ptr(x), _dtype_code(router_w), _ptr(router_w),
                             _ptr(router_gamma), _ptr(router_bias), _ptr(forced_arr), _ptr(idx), _ptr(w),
                             _ptr(logits), _ptr(gap), _ptr(r), n_threads)
    if rc != 0:
        raise ValueError("oracle_route rejected its arguments")
    return dict(idx=idx, w=w, logits=logits, gap=gap, r=r)


def permute(idx, n_experts):
    T, k = idx.shape
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    counts = np.empty((n_experts,), dtype=np.int32)
    offsets = np.empty((n_experts + 1,), dtype=np.int32)
    sorted_token = np.empty((T * k,), dtype=np.int32)
    row_of_slot = np.empty((T * k,), dtype=np.int32)
    rc = load().oracle_permute(T, k, n_experts, _ptr(idx), _ptr(counts), _ptr(offsets), _ptr(sorted_token),
                               _ptr(row_of_slot))
    if rc != 0:
        raise ValueError("oracle_permute: expert id out of range")
    return dict(counts=counts, offsets=offsets, sorted_token=sorted_token, row_of_slot=row_of_slot)


def moe_forward(w, x, k, eps, forced=None, tokens=None, add_input=False, addend=None, n_threads=0):
    """The whole layer on the host.

    `w` is a dict of numpy arrays: router_w (f32 or uint16 bf16 bits) [E,D], router_gamma f32 [D],
    router_bias f32 [E] or None, ffn_gamma f32 [D], and either w_gate_up / w_down as uint16 bf16 bits
    ([E,2F,D] / [E,D,F]) or, for int4, q_gate_up uint8 [E,2F,D/2], s_gate_up uint16 [E,2F,D/128],
    q_down uint8 [E,D,F/2], s_down uint16 [E,D,ceil(F/128)], or, for Q8_0, q8_gate_up uint8
    [E,2F,D/32,34] and q8_down uint8 [E,D,F/32,34], or, for MXFP4, mx4_gate_up uint8 [E,2F,D/32,17] and
    mx4_down uint8 [E,D,F/32,17], or, for MXFP8, mx8_gate_up uint8 [E,2F,D/32,33] and mx8_down uint8
    [E,D,F/32,33].
    Returns dict(out [n,D] f32, idx [n,k], w [n,k] f64, gap [n]).
    """
    T, D = x.shape
    E = w["router_w"].shape[0]
    ew, gu, dn, sgu, sdn, F = _expert_arrays(w)
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    n = T if tok is None else len(tok)
    out = np.empty((n, D), dtype=np.float32)
    idx = np.empty((n, k), dtype=np.int32)
    wts = np.empty((n, k), dtype=np.float64)
    gap = np.empty((n,), dtype=np.float64)
    forced_arr = None if forced is None else np.ascontiguousarray(forced, dtype=np.int32)
    if addend is not None:
        assert addend.dtype == x.dtype and addend.shape == x.shape
    rc = load().oracle_moe_forward(
        T, D, F, E, k, eps, _dtype_code(x), _ptr(x), _dtype_code(w["router_w"]), _ptr(w["router_w"]),
        _ptr(w["router_gamma"]), _ptr(w.get("router_bias")), _ptr(w["ffn_gamma"]), ew, _ptr(gu), _ptr(dn),
        _ptr(sgu), _ptr(sdn), _ptr(forced_arr), _ptr(tok), n, int(bool(add_input)), _ptr(addend), _ptr(out),
        _ptr(idx), _ptr(wts), _ptr(gap), n_threads)
    if rc != 0:
        raise ValueError("oracle_moe_forward rejected its arguments")
    return dict(out=out, idx=idx, w=wts, gap=gap)


def expert_ffn(w, e, h):
    """FFN of expert e on fp32 rows h [n, D] -> [n, D]."""
    h = np.ascontiguousarray(h, dtype=np.float32)
    n, D = h.shape
    E = w["router_w"].shape[0]
    ew, gu, dn, sgu, sdn, F = _expert_arrays(w)
    y = np.empty((n, D), dtype=np.float32)
    rc = load().oracle_expert_ffn(D, F, E, e, ew, _ptr(gu), _ptr(dn), _ptr(sgu), _ptr(sdn), _ptr(h), n, _ptr(y))
    if rc != 0:
        raise ValueError("bad expert id")
    return y


def canvas_head(h, emb, beta=1.0, tokens=None, want_logits=False, n_threads=0):
    """Canvas output stage on the host: h uint16 bf16 bits [T, D], emb uint16 bf16 bits [V, D].

    Returns dict(entropy [n] f64, argmax [n] int32, gap [n] f64, logits [n, V] f64 or None) for the
    positions `tokens` (all T if None).
    """
    h = np.ascontiguousarray(h, dtype=np.uint16)
    emb = np.ascontiguousarray(emb, dtype=np.uint16)
    T, D = h.shape
    V = emb.shape[0]
    assert emb.shape[1] == D
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    n = T if tok is None else len(tok)
    ent = np.empty(n, dtype=np.float64)
    am = np.empty(n, dtype=np.int32)
    gap = np.empty(n, dtype=np.float64)
    lg = np.empty((n, V), dtype=np.float64) if want_logits else None
    rc = load().oracle_canvas_head(T, V, D, _ptr(h), _ptr(emb), float(beta), _ptr(tok), n, _ptr(lg), _ptr(ent),
                                   _ptr(am), _ptr(gap), n_threads)
    if rc != 0:
        raise ValueError("oracle_canvas_head: bad argument")
    return {"entropy": ent, "argmax": am, "gap": gap, "logits": lg}
