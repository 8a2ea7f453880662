"""ctypes binding of libdgmoe.so (include/dg_moe.h, include/dg_head.h): argument marshalling only.

The C entry points are exposed under their own names. `MoELayer` and
`CanvasHead` are small convenience wrappers that keep torch tensors (device
memory) alive next to a handle; every step runs in the HIP library.

Importing this module loads the library and fails loudly if it has not been
built: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdgmoe.so")

DG_F32, DG_BF16, DG_F16, DG_I4G128, DG_Q8_0, DG_MXFP4, DG_MXFP8 = 0, 1, 2, 3, 4, 5, 6
DG_OK = 0
DG_ERR_INVALID_ARG, DG_ERR_SHAPE, DG_ERR_DTYPE, DG_ERR_ALIGN = -1, -2, -3, -4
DG_ERR_OOM, DG_ERR_HIP, DG_ERR_UNSUPPORTED = -5, -6, -7
DG_MOE_PACK_WEIGHTS = 0x1
DG_FWD_ADD_INPUT = 0x1
DG_FWD_ROUTER_NO_WAIT = 0x2
DG_FWD_GEMM_NO_WAIT = 0x4
ABI_VERSION = 2
DG_DEV_QUEUE_OVERFLOW, DG_DEV_XCD_ROUTER, DG_DEV_XCD_GEMM, DG_DEV_WAIT_TIMEOUT = 0x1, 0x2, 0x4, 0x8

EXPORTED = ("dg_moe_create", "dg_moe_forward", "dg_moe_forward_debug", "dg_moe_forward_profiled", "dg_moe_destroy",
            "dg_moe_status_string", "dg_moe_last_error", "dg_moe_abi_version", "dg_moe_workspace_bytes",
            "dg_head_create", "dg_head_forward", "dg_head_forward_profiled", "dg_head_destroy",
            "dg_head_workspace_bytes", "dg_head_forward_noalloc")
DG_HEAD_NOALLOC_SCRATCH_BYTES = 8 << 20


class dg_moe_config(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("act_dtype", ctypes.c_int32), ("router_w_dtype", ctypes.c_int32),
                ("expert_w_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class dg_moe_weights(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_gamma", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("ffn_gamma", ctypes.c_void_p), ("w_gate_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("s_gate_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p)]


class dg_moe_debug(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("sorted_slot", ctypes.c_void_p), ("row_of_slot", ctypes.c_void_p),
                ("queue_len", ctypes.c_void_p), ("dev_flags", ctypes.c_void_p)]


class dg_head_config(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("vocab", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("h_dtype", ctypes.c_int32), ("emb_dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m expert_ffn_canvas_amd.build` "
                          "(there is no CPU fallback for the MoE layer)")
    # Load torch first: its HIP runtime then owns the process, and the library (which needs the same
    # soname, libamdhip64.so.7) binds to that one runtime, the one that made the caller's streams and memory.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32
    lib.dg_moe_create.argtypes = [ctypes.POINTER(dg_moe_config), ctypes.POINTER(dg_moe_weights), vp,
                                  ctypes.POINTER(vp)]
    lib.dg_moe_create.restype = i32
    lib.dg_moe_forward.argtypes = [vp, vp, vp, i32, vp, u32, vp]
    lib.dg_moe_forward.restype = i32
    lib.dg_moe_forward_debug.argtypes = [vp, vp, vp, i32, ctypes.POINTER(dg_moe_debug), vp]
    lib.dg_moe_forward_debug.restype = i32
    lib.dg_moe_forward_profiled.argtypes = [vp, vp, vp, i32, vp, u32, ctypes.POINTER(vp), vp]
    lib.dg_moe_forward_profiled.restype = i32
    lib.dg_moe_destroy.argtypes = [vp]
    lib.dg_moe_destroy.restype = i32
    lib.dg_moe_status_string.argtypes = [i32]
    lib.dg_moe_status_string.restype = ctypes.c_char_p
    lib.dg_moe_last_error.argtypes = []
    lib.dg_moe_last_error.restype = ctypes.c_char_p
    lib.dg_moe_abi_version.argtypes = []
    lib.dg_moe_abi_version.restype = i32
    lib.dg_moe_workspace_bytes.argtypes = [ctypes.POINTER(dg_moe_config)]
    lib.dg_moe_workspace_bytes.restype = ctypes.c_uint64
    f32 = ctypes.c_float
    lib.dg_head_create.argtypes = [ctypes.POINTER(dg_head_config), vp, ctypes.POINTER(vp)]
    lib.dg_head_create.restype = i32
    lib.dg_head_forward.argtypes = [vp, vp, i32, f32, vp, vp, vp, vp, vp]
    lib.dg_head_forward.restype = i32
    lib.dg_head_forward_profiled.argtypes = [vp, vp, i32, f32, vp, vp, vp, vp, ctypes.POINTER(vp), vp]
    lib.dg_head_forward_profiled.restype = i32
    lib.dg_head_destroy.argtypes = [vp]
    lib.dg_head_destroy.restype = i32
    lib.dg_head_workspace_bytes.argtypes = [ctypes.POINTER(dg_head_config)]
    lib.dg_head_workspace_bytes.restype = ctypes.c_uint64
    lib.dg_head_forward_noalloc.argtypes = [ctypes.POINTER(dg_head_config), vp, vp, i32, f32, vp, vp, vp, vp, vp]
    lib.dg_head_forward_noalloc.restype = i32
    if lib.dg_moe_abi_version() != ABI_VERSION:
        raise ImportError("libdgmoe.so ABI version mismatch")
    return lib


_lib = _load()


class DgMoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        detail = _lib.dg_moe_last_error().decode()
        super().__init__(f"{where}: {_lib.dg_moe_status_string(status).decode()} ({status}): {detail}")


def _check(status, where):
    if status != DG_OK:
        raise DgMoeError(status, where)


# --- the C entry points under their own names -------------------------------------------------------------

def dg_moe_create(cfg: dg_moe_config, weights: dg_moe_weights, stream: int):
    """Returns (status, handle)."""
    h = ctypes.c_void_p()
    st = _lib.dg_moe_create(ctypes.byref(cfg), ctypes.byref(weights), ctypes.c_void_p(stream), ctypes.byref(h))
    return st, h


def dg_moe_forward(handle, x: int, out: int, T: int, addend: int | None, flags: int, stream: int) -> int:
    return _lib.dg_moe_forward(handle, x, out, T, addend, flags, ctypes.c_void_p(stream))


def dg_moe_forward_debug(handle, x: int, out: int, T: int, dbg: dg_moe_debug, stream: int) -> int:
    return _lib.dg_moe_forward_debug(handle, x, out, T, ctypes.byref(dbg), ctypes.c_void_p(stream))


def dg_moe_forward_profiled(handle, x: int, out: int, T: int, addend: int | None, flags: int, events,
                            stream: int) -> int:
    """events: sequence of twelve hipEvent_t handles (ints): start/stop of each of the six kernels."""
    if len(events) != 12:
        raise ValueError("dg_moe_forward_profiled takes 12 events")
    arr = (ctypes.c_void_p * 12)(*events)
    return _lib.dg_moe_forward_profiled(handle, x, out, T, addend, flags, arr, ctypes.c_void_p(stream))


def dg_moe_destroy(handle) -> int:
    return _lib.dg_moe_destroy(handle)


def dg_moe_status_string(status: int) -> str:
    return _lib.dg_moe_status_string(status).decode()


def dg_moe_last_error() -> str:
    return _lib.dg_moe_last_error().decode()


def dg_moe_abi_version() -> int:
    return _lib.dg_moe_abi_version()


def dg_moe_workspace_bytes(cfg: dg_moe_config) -> int:
    return _lib.dg_moe_workspace_bytes(ctypes.byref(cfg))


def dg_head_create(cfg: dg_head_config, emb: int):
    """Returns (status, handle)."""
    h = ctypes.c_void_p()
    st = _lib.dg_head_create(ctypes.byref(cfg), ctypes.c_void_p(emb), ctypes.byref(h))
    return st, h


def dg_head_forward(handle, h: int, T: int, beta: float, logits: int | None, entropy: int, argmax: int,
                    mean_entropy: int | None, stream: int) -> int:
    return _lib.dg_head_forward(handle, h, T, beta, logits, entropy, argmax, mean_entropy, ctypes.c_void_p(stream))


def dg_head_forward_profiled(handle, h: int, T: int, beta: float, logits: int | None, entropy: int, argmax: int,
                             mean_entropy: int | None, events, stream: int) -> int:
    """events: six hipEvent_t handles (ints): start/stop of each of the three kernels."""
    if len(events) != 6:
        raise ValueError("dg_head_forward_profiled takes 6 events")
    arr = (ctypes.c_void_p * 6)(*events)
    return _lib.dg_head_forward_profiled(handle, h, T, beta, logits, entropy, argmax, mean_entropy, arr,
                                         ctypes.c_void_p(stream))


def dg_head_destroy(handle) -> int:
    return _lib.dg_head_destroy(handle)


def dg_head_workspace_bytes(cfg: dg_head_config) -> int:
    return _lib.dg_head_workspace_bytes(ctypes.byref(cfg))


def dg_head_forward_noalloc(cfg: dg_head_config, emb: int, h: int, T: int, beta: float, logits: int | None,
                            entropy: int, argmax: int, mean_entropy: int | None, stream: int) -> int:
    return _lib.dg_head_forward_noalloc(ctypes.byref(cfg), emb, h, T, beta, logits, entropy, argmax, mean_entropy,
                                        ctypes.c_void_p(stream))


def make_head_config(V=262144, D=2816, max_tokens=256, h_dtype=DG_BF16, emb_dtype=DG_BF16, flags=0) -> dg_head_config:
    return dg_head_config(ctypes.sizeof(dg_head_config), V, D, max_tokens, h_dtype, emb_dtype, flags)


def make_config(E=128, K=8, D=2816, F=704, max_tokens=256, eps=1e-6, act=DG_BF16, router_w=DG_BF16,
                experts=DG_BF16, flags=0) -> dg_moe_config:
    return dg_moe_config(ctypes.sizeof(dg_moe_config), E, K, D, F, max_tokens, eps, act, router_w, experts, flags)


# --- torch convenience wrapper (device memory and streams only) -------------------------------------------

def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype_code(t):
    import torch
    return {torch.float32: DG_F32, torch.bfloat16: DG_BF16, torch.float16: DG_F16}[t.dtype]


class MoELayer:
    """One MoE layer handle over device tensors in the synth weight-dict format."""

    def __init__(self, weights: dict, max_tokens: int, act_dtype, top_k: int = 8, eps: float = 1e-6,
                 pack: bool = False, stream=None):
        import torch
        self.w = weights  # keep the borrowed device tensors alive
        rw = weights["router_w"]
        i4 = "q_gate_up" in weights
        q8 = "q8_gate_up" in weights  # Q8_0 blocks [E, rows, K/32, 34]; read from the packed copy only
        mx4 = "mx4_gate_up" in weights  # MXFP4 blocks [E, rows, K/32, 17]; read from the packed copy only
        mx8 = "mx8_gate_up" in weights  # MXFP8 blocks [E, rows, K/32, 33]; read from the packed copy only
        E, D = rw.shape
        key = "q_" if i4 else "q8_" if q8 else "mx4_" if mx4 else "mx8_" if mx8 else "w_"
        gu, dn = weights[key + "gate_up"], weights[key + "down"]
        F = gu.shape[1] // 2
        self.E, self.D, self.F = E, D, F
        self.K = top_k
        self.act_dtype = act_dtype
        cfg = make_config(E=E, K=self.K, D=D, F=F, max_tokens=max_tokens, eps=eps, act=_dtype_code(
            torch.empty((), dtype=act_dtype)), router_w=_dtype_code(rw),
            experts=DG_I4G128 if i4 else DG_Q8_0 if q8 else DG_MXFP4 if mx4 else DG_MXFP8 if mx8 else DG_BF16,
            flags=DG_MOE_PACK_WEIGHTS if pack else 0)
        wts = dg_moe_weights(
            _ptr(rw), _ptr(weights["router_gamma"]), _ptr(weights.get("router_bias")), _ptr(weights["ffn_gamma"]),
            _ptr(gu), _ptr(dn),
            _ptr(weights.get("s_gate_up")), _ptr(weights.get("s_down")))
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        st, h = dg_moe_create(cfg, wts, self.stream.cuda_stream)
        _check(st, "dg_moe_create")
        self.handle = h
        self.max_tokens = max_tokens
        # bf16 activations with packed bf16 experts: the expert norm rides on the gate_up weight and r, and the
        # forward runs no norm kernel (its two profiling events are then recorded back to back)
        self.expert_norm_folded = bool(pack and not (i4 or q8 or mx4 or mx8) and act_dtype == torch.bfloat16)
        # both GEMMs run in one launch, except for int4 experts read in place (the fused launch's profiling
        # events are the gate_up pair; the down pair is recorded back to back after it)
        self.gemms_fused = bool(pack or not i4)

    def forward(self, x, out=None, addend=None, add_input=False, router_no_wait=False):
        import torch
        T = x.shape[0]
        if out is None:
            out = torch.empty((T, self.D), dtype=x.dtype, device=x.device)
        flags = (DG_FWD_ADD_INPUT if add_input else 0) | (DG_FWD_ROUTER_NO_WAIT if router_no_wait else 0)
        st = dg_moe_forward(self.handle, _ptr(x), _ptr(out), T, _ptr(addend), flags, self.stream.cuda_stream)
        _check(st, "dg_moe_forward")
        return out

    def forward_debug(self, x, out=None):
        """Forward plus routing/permutation outputs (device tensors): the routing, counts, offsets, the sorted
        slots, queue_len (8 gate_up and 8 down queue lengths, then the two capacities) and the handle's
        sticky device status word dev_flags (DG_DEV_* bits)."""
        import torch
        T = x.shape[0]
        dev = x.device
        if out is None:
            out = torch.empty((T, self.D), dtype=x.dtype, device=dev)
        r = dict(
            topk_idx=torch.empty((T, self.K), dtype=torch.int32, device=dev),
            topk_w=torch.empty((T, self.K), dtype=torch.float32, device=dev),
            counts=torch.empty((self.E,), dtype=torch.int32, device=dev),
            offsets=torch.empty((self.E + 1,), dtype=torch.int32, device=dev),
            sorted_slot=torch.empty((T * self.K,), dtype=torch.int32, device=dev),
            row_of_slot=torch.empty((T * self.K,), dtype=torch.int32, device=dev),
            queue_len=torch.empty((18,), dtype=torch.int32, device=dev),
            dev_flags=torch.empty((1,), dtype=torch.int32, device=dev),
        )
        dbg = dg_moe_debug(*(_ptr(r[k]) for k in ("topk_idx", "topk_w", "counts", "offsets", "sorted_slot",
                                                   "row_of_slot", "queue_len", "dev_flags")))
        st = dg_moe_forward_debug(self.handle, _ptr(x), _ptr(out), T, dbg, self.stream.cuda_stream)
        _check(st, "dg_moe_forward_debug")
        r["out"] = out
        return r

    def close(self):
        if getattr(self, "handle", None):
            _check(dg_moe_destroy(self.handle), "dg_moe_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class CanvasHead:
    """The canvas output stage over a borrowed bf16 embedding table emb [V, D] (a torch device tensor)."""

    def __init__(self, emb, max_tokens: int, stream=None):
        import torch
        if emb.dtype != torch.bfloat16:
            raise TypeError("the embedding table must be bf16")
        self.emb = emb  # borrowed: kept alive with the handle
        self.V, self.D = emb.shape
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        st, h = dg_head_create(make_head_config(self.V, self.D, max_tokens), _ptr(emb))
        _check(st, "dg_head_create")
        self.handle = h
        self.max_tokens = max_tokens

    def forward(self, h, beta: float = 1.0, want_logits: bool = True, out=None):
        """Returns dict(logits [T, V] f32 or None, entropy [T] f32, argmax [T] int32, mean_entropy [1] f32)."""
        import torch
        T = h.shape[0]
        dev = h.device
        r = out if out is not None else {
            "logits": torch.empty((T, self.V), dtype=torch.float32, device=dev) if want_logits else None,
            "entropy": torch.empty((T,), dtype=torch.float32, device=dev),
            "argmax": torch.empty((T,), dtype=torch.int32, device=dev),
            "mean_entropy": torch.empty((1,), dtype=torch.float32, device=dev),
        }
        st = dg_head_forward(self.handle, _ptr(h), T, beta, _ptr(r["logits"]), _ptr(r["entropy"]), _ptr(r["argmax"]),
                             _ptr(r["mean_entropy"]), self.stream.cuda_stream)
        _check(st, "dg_head_forward")
        return r

    def close(self):
        if getattr(self, "handle", None):
            _check(dg_head_destroy(self.handle), "dg_head_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
