"""ctypes binding of libpoetx (include/poetx.h).

Argument marshalling only: each function below has the name of the C entry point
it calls and forwards raw device pointers, sizes and the HIP stream.  Every step
of the layer runs in the library's HIP kernels; there is no fallback path, and a
missing or unloadable library raises.

Tensors are torch tensors on the GPU (torch provides device memory and
streams).  bfloat16 data may be passed as torch.bfloat16 or as 16-bit integer
tensors holding the bit patterns.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# POETX_LIBRARY names another build of the library (e.g. to compare two builds in one process tree)
LIB_PATH = os.environ.get("POETX_LIBRARY") or os.path.join(HERE, "libpoetx.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "poetx.h")

POETX_OK, POETX_E_NULL, POETX_E_SHAPE, POETX_E_DTYPE, POETX_E_WORKSPACE, POETX_E_PERM, POETX_E_HIP, POETX_E_UNSUPPORTED = range(8)
POETX_F32, POETX_BF16, POETX_I8 = 0, 1, 2
POETX_OP_CNP, POETX_OP_FWD, POETX_OP_BWD, POETX_OP_MERGE = 0, 1, 2, 3
POETX_KC_NONE, POETX_KC_GEMM, POETX_KC_APPLY, POETX_KC_DGRAD, POETX_KC_CNP, POETX_KC_PERMUTE, POETX_KC_OPTIM = range(7)

DTYPES = {"f32": POETX_F32, "bf16": POETX_BF16, "i8": POETX_I8}
# what the forward saves: H and Xt; Xt only (H recomputed from it); Xt only (H taken back from Y)
POETX_XFAST, POETX_XMEM, POETX_XOUT = 0, 1, 2
POETX_MAX_SIDES = 64  # most sides one batched call accepts
POETX_MAX_GROUP = 8  # most linears one group call accepts
MODES = {"xfast": POETX_XFAST, "xmem": POETX_XMEM, "xout": POETX_XOUT}


class PoetxError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libpoetx status {status}: {msg}")
        self.status = status


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("m", ctypes.c_int32),
        ("n", ctypes.c_int32),
        ("b", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32),
        ("w_dtype", ctypes.c_int32),
        ("mode", ctypes.c_int32),
    ]


POETX_SPO_BLOCK, POETX_SPO_FULL = 0, 1
SPO_KINDS = {"block": POETX_SPO_BLOCK, "full": POETX_SPO_FULL}


class SpoDesc(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int32),
        ("b", ctypes.c_int32),
        ("kind", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32),
    ]


class GradSide(ctypes.Structure):
    _fields_ = [
        ("A", ctypes.c_void_p),
        ("lda", ctypes.c_int64),
        ("B", ctypes.c_void_p),
        ("ldb", ctypes.c_int64),
        ("d", ctypes.c_int32),
    ]


class FwdCall(ctypes.Structure):
    _fields_ = [
        ("desc", ctypes.POINTER(LayerDesc)),
        ("X", ctypes.c_void_p),
        ("perm_R", ctypes.c_void_p),
        ("perm_P", ctypes.c_void_p),
        ("Wt", ctypes.c_void_p),
        ("g_R", ctypes.c_void_p),
        ("g_P", ctypes.c_void_p),
        ("Y", ctypes.c_void_p),
        ("H_save", ctypes.c_void_p),
        ("ws", ctypes.c_void_p),
        ("ws_bytes", ctypes.c_size_t),
    ]


class BwdCall(ctypes.Structure):
    _fields_ = [
        ("desc", ctypes.POINTER(LayerDesc)),
        ("Y", ctypes.c_void_p),
        ("dZ", ctypes.c_void_p),
        ("perm_R", ctypes.c_void_p),
        ("perm_P", ctypes.c_void_p),
        ("Wt", ctypes.c_void_p),
        ("g_R", ctypes.c_void_p),
        ("g_P", ctypes.c_void_p),
        ("H_save", ctypes.c_void_p),
        ("dX", ctypes.c_void_p),
        ("ws", ctypes.c_void_p),
        ("ws_bytes", ctypes.c_size_t),
    ]


class AdamParams(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float),
        ("beta1", ctypes.c_float),
        ("beta2", ctypes.c_float),
        ("eps", ctypes.c_float),
        ("weight_decay", ctypes.c_float),
        ("t", ctypes.c_int64),
    ]


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_SIG = {
    "poetx_version": (ctypes.c_char_p, []),
    "poetx_last_error": (ctypes.c_char_p, []),
    "poetx_packed_len": (ctypes.c_int64, [ctypes.c_int32]),
    "poetx_g_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    "poetx_weight_bytes": (ctypes.c_size_t, [ctypes.POINTER(LayerDesc)]),
    "poetx_saved_bytes": (ctypes.c_size_t, [ctypes.POINTER(LayerDesc), ctypes.c_int64]),
    "poetx_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(LayerDesc), ctypes.c_int64, ctypes.c_int32]),
    "poetx_perm_from_seed": (ctypes.c_int, [ctypes.c_uint64, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]),
    "poetx_cnp_build": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_size_t, _P]),
    "poetx_cnp_build_noalloc": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P]),
    "poetx_premerge": (ctypes.c_int, [ctypes.POINTER(LayerDesc), _P, ctypes.c_int64, _P, _P, _P, _P, _P]),
    "poetx_linear_fwd": (
        ctypes.c_int,
        [ctypes.POINTER(LayerDesc), ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    ),
    "poetx_linear_bwd": (
        ctypes.c_int,
        [ctypes.POINTER(LayerDesc), ctypes.c_int64] + [_P] * 14 + [ctypes.c_size_t, _P],
    ),
    "poetx_timer_enable": (ctypes.c_int, [ctypes.c_int32]),
    "poetx_timer_read": (
        ctypes.c_int,
        [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
         ctypes.POINTER(ctypes.c_double)],
    ),
    "poetx_merge_reinit": (
        ctypes.c_int,
        [ctypes.POINTER(LayerDesc), _P, _P, _P, _P, _P, _P, _P, ctypes.c_uint64, ctypes.c_uint64, _P, ctypes.c_size_t, _P],
    ),
    "poetx_cnp_batch_workspace_size": (
        ctypes.c_size_t, [ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, ctypes.c_int32]
    ),
    "poetx_cnp_build_batch": (
        ctypes.c_int,
        [ctypes.c_int32, ctypes.POINTER(_P), ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, ctypes.c_int32,
         ctypes.POINTER(_P), _P, ctypes.c_size_t, _P],
    ),
    "poetx_cnp_grad_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]),
    "poetx_linear_bwd_dx": (
        ctypes.c_int,
        [ctypes.POINTER(LayerDesc), ctypes.c_int64] + [_P] * 12 + [ctypes.c_int64, ctypes.c_int64, _P, ctypes.c_size_t, _P],
    ),
    "poetx_cnp_backward_batch": (
        ctypes.c_int,
        [ctypes.c_int32, ctypes.POINTER(_P), ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, ctypes.c_int32, _P,
         ctypes.c_size_t, ctypes.POINTER(_P), _P],
    ),
    "poetx_cnp_backward_batch_reuse": (
        ctypes.c_int,
        [ctypes.c_int32, ctypes.POINTER(_P), ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, ctypes.c_int32, _P,
         ctypes.c_size_t, _P, ctypes.c_size_t, ctypes.POINTER(_P), _P],
    ),
    "poetx_linear_bwd_dx_sides": (
        ctypes.c_int,
        [ctypes.POINTER(LayerDesc), ctypes.c_int64] + [_P] * 9 + [ctypes.POINTER(GradSide), _P, ctypes.c_size_t, _P],
    ),
    "poetx_linear_fwd_group": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(FwdCall), ctypes.c_int64, _P]),
    "poetx_linear_bwd_dx_group": (
        ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(BwdCall), ctypes.c_int64, ctypes.POINTER(GradSide), _P]
    ),
    "poetx_block_grads_workspace_size": (
        ctypes.c_size_t, [ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
    ),
    "poetx_block_grads_batch": (
        ctypes.c_int,
        [ctypes.c_int32, ctypes.POINTER(GradSide), ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_size_t,
         _P, ctypes.c_size_t, _P],
    ),
    "poetx_spo_saved_bytes": (ctypes.c_size_t, [ctypes.POINTER(SpoDesc), ctypes.c_int64]),
    "poetx_spo_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(SpoDesc), ctypes.c_int64, ctypes.c_int32]),
    "poetx_spo_fwd": (ctypes.c_int, [ctypes.POINTER(SpoDesc), ctypes.c_int64] + [_P] * 6 + [ctypes.c_size_t, _P]),
    "poetx_spo_bwd": (ctypes.c_int, [ctypes.POINTER(SpoDesc), ctypes.c_int64] + [_P] * 8 + [ctypes.c_size_t, _P]),
    "poetx_fold_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(LayerDesc), ctypes.c_int32, ctypes.POINTER(SpoDesc)]),
    "poetx_fold_factor": (
        ctypes.c_int,
        [ctypes.POINTER(LayerDesc), ctypes.c_int32, ctypes.POINTER(SpoDesc), _P, _P, _P, _P, ctypes.c_int64, _P,
         ctypes.c_size_t, _P],
    ),
    "poetx_store_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(LayerDesc)]),
    "poetx_store_weight": (ctypes.c_int, [ctypes.POINTER(LayerDesc), _P, ctypes.c_int64, _P, _P, ctypes.c_size_t, _P]),
    "poetx_wc_state_bytes": (ctypes.c_size_t, [ctypes.POINTER(LayerDesc), ctypes.c_int64]),
    "poetx_wc_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(LayerDesc), ctypes.c_int64, ctypes.c_int32]),
    "poetx_wc_fwd": (ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.c_int64] + [_P] * 9 + [ctypes.c_size_t, _P]),
    "poetx_wc_bwd": (ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.c_int64] + [_P] * 12 + [ctypes.c_size_t, _P]),
    "poetx_adam_step_batch": (
        ctypes.c_int,
        [ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(_P), ctypes.POINTER(_P), ctypes.POINTER(_P),
         ctypes.POINTER(_P), ctypes.POINTER(AdamParams), _P],
    ),
}


def lib() -> ctypes.CDLL:
    """Load libpoetx.so (after torch, so that both share one HIP runtime)."""
    global _lib
    if _lib is None:
        try:
            import torch  # noqa: F401  (loads the HIP runtime the library must share)
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run orthogonal_reparameterized_cnp_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def header_symbols() -> list:
    """Names of the functions include/poetx.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(poetx_\w+)\s*\(", text, re.M)))


def _check(st: int):
    if st != POETX_OK:
        raise PoetxError(st, lib().poetx_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def desc(m: int, n: int, b: int, act: str, w: str, mode: str = "xfast") -> LayerDesc:
    return LayerDesc(m, n, b, DTYPES[act], DTYPES[w], MODES[mode])


# ---------------------------------------------------------------- helpers ---
def poetx_version() -> str:
    return lib().poetx_version().decode()


def poetx_last_error() -> str:
    return lib().poetx_last_error().decode()


def poetx_packed_len(b: int) -> int:
    return lib().poetx_packed_len(b)


def poetx_g_bytes(d: int, b: int, dtype: int) -> int:
    return lib().poetx_g_bytes(d, b, dtype)


def poetx_weight_bytes(dsc: LayerDesc) -> int:
    return lib().poetx_weight_bytes(ctypes.byref(dsc))


def poetx_saved_bytes(dsc: LayerDesc, T: int) -> int:
    return lib().poetx_saved_bytes(ctypes.byref(dsc), T)


def poetx_workspace_size(dsc: LayerDesc, T: int, op: int) -> int:
    return lib().poetx_workspace_size(ctypes.byref(dsc), T, op)


def poetx_perm_from_seed(seed: int, d: int):
    import numpy as np

    out = np.empty(d, dtype=np.int32)
    _check(lib().poetx_perm_from_seed(seed, d, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
    return out


def poetx_timer_enable(kernel_class: int):
    _check(lib().poetx_timer_enable(kernel_class))


def poetx_timer_read():
    """(launches, total_ms, flops, bytes) of the enabled class since the last read."""
    n, ms, fl, by = ctypes.c_int64(), ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _check(lib().poetx_timer_read(ctypes.byref(n), ctypes.byref(ms), ctypes.byref(fl), ctypes.byref(by)))
    return n.value, ms.value, fl.value, by.value


# ------------------------------------------------------------- the calls ---
def poetx_cnp_build(q, d: int, b: int, dtype: int, g, ws, ws_bytes: int, stream=None):
    _check(lib().poetx_cnp_build(_ptr(q), d, b, dtype, _ptr(g), _ptr(ws), ws_bytes, _stream(stream)))


def poetx_cnp_build_noalloc(q, d: int, b: int, dtype: int, g, stream=None):
    _check(lib().poetx_cnp_build_noalloc(_ptr(q), d, b, dtype, _ptr(g), _stream(stream)))


def poetx_premerge(dsc: LayerDesc, W0, ld_w0: int, w0_scale, perm_R, perm_P, Wt, stream=None):
    _check(
        lib().poetx_premerge(
            ctypes.byref(dsc), _ptr(W0), ld_w0, _ptr(w0_scale), _ptr(perm_R), _ptr(perm_P), _ptr(Wt), _stream(stream)
        )
    )


def poetx_linear_fwd(dsc: LayerDesc, T: int, X, perm_R, perm_P, Wt, g_R, g_P, Y, H_save, ws, ws_bytes: int, stream=None):
    _check(
        lib().poetx_linear_fwd(
            ctypes.byref(dsc), T, _ptr(X), _ptr(perm_R), _ptr(perm_P), _ptr(Wt), _ptr(g_R), _ptr(g_P), _ptr(Y),
            _ptr(H_save), _ptr(ws), ws_bytes, _stream(stream),
        )
    )


def poetx_linear_bwd(dsc: LayerDesc, T: int, Y, dZ, perm_R, perm_P, Wt, g_R, g_P, q_R, q_P, H_save, dX, dq_R, dq_P,
                     ws, ws_bytes: int, stream=None):
    _check(
        lib().poetx_linear_bwd(
            ctypes.byref(dsc), T, _ptr(Y), _ptr(dZ), _ptr(perm_R), _ptr(perm_P), _ptr(Wt), _ptr(g_R), _ptr(g_P),
            _ptr(q_R), _ptr(q_P), _ptr(H_save), _ptr(dX), _ptr(dq_R), _ptr(dq_P), _ptr(ws), ws_bytes, _stream(stream),
        )
    )


def poetx_merge_reinit(dsc: LayerDesc, Wt, perm_R, perm_P, g_R, g_P, q_R, q_P, seed_R: int, seed_P: int, ws,
                       ws_bytes: int, stream=None):
    _check(
        lib().poetx_merge_reinit(
            ctypes.byref(dsc), _ptr(Wt), _ptr(perm_R), _ptr(perm_P), _ptr(g_R), _ptr(g_P), _ptr(q_R), _ptr(q_P),
            seed_R & ((1 << 64) - 1), seed_P & ((1 << 64) - 1), _ptr(ws), ws_bytes, _stream(stream),
        )
    )


# ------------------------------------------------- batched CNP (one layer) ---
def _ptr_array(ts):
    return (_P * len(ts))(*[_ptr(t) for t in ts])


def _i32_array(xs):
    return (ctypes.c_int32 * len(xs))(*xs)


def poetx_cnp_batch_workspace_size(d, b: int, dtype: int) -> int:
    return lib().poetx_cnp_batch_workspace_size(len(d), _i32_array(d), b, dtype)


def poetx_cnp_build_batch(q, d, b: int, dtype: int, g, ws, ws_bytes: int, stream=None):
    """q, d, g: per-side lists (device tensors / ints), marshalled into host arrays."""
    _check(lib().poetx_cnp_build_batch(len(d), _ptr_array(q), _i32_array(d), b, dtype, _ptr_array(g), _ptr(ws),
                                       ws_bytes, _stream(stream)))


def poetx_cnp_grad_bytes(blocks: int, b: int, dtype: int) -> int:
    return lib().poetx_cnp_grad_bytes(blocks, b, dtype)


def poetx_linear_bwd_dx(dsc: LayerDesc, T: int, Y, dZ, perm_R, perm_P, Wt, g_R, g_P, q_R, q_P, H_save, dX, dg,
                        dg_first: int, dg_blocks: int, ws, ws_bytes: int, stream=None):
    _check(
        lib().poetx_linear_bwd_dx(
            ctypes.byref(dsc), T, _ptr(Y), _ptr(dZ), _ptr(perm_R), _ptr(perm_P), _ptr(Wt), _ptr(g_R), _ptr(g_P),
            _ptr(q_R), _ptr(q_P), _ptr(H_save), _ptr(dX), _ptr(dg), dg_first, dg_blocks, _ptr(ws), ws_bytes,
            _stream(stream),
        )
    )


def poetx_cnp_backward_batch_reuse(q, d, b: int, dtype: int, build_ws, build_ws_bytes: int, dg, dg_bytes: int, dq,
                                   stream=None):
    _check(lib().poetx_cnp_backward_batch_reuse(len(d), _ptr_array(q), _i32_array(d), b, dtype, _ptr(build_ws),
                                                build_ws_bytes, _ptr(dg), dg_bytes, _ptr_array(dq), _stream(stream)))


def poetx_linear_bwd_dx_sides(dsc: LayerDesc, T: int, Y, dZ, perm_R, perm_P, Wt, g_R, g_P, H_save, dX, ws,
                              ws_bytes: int, stream=None):
    """dX into `dX`; returns the two sides' block-gradient operands (R, P) as GradSide records."""
    sides = (GradSide * 2)()
    _check(
        lib().poetx_linear_bwd_dx_sides(
            ctypes.byref(dsc), T, _ptr(Y), _ptr(dZ), _ptr(perm_R), _ptr(perm_P), _ptr(Wt), _ptr(g_R), _ptr(g_P),
            _ptr(H_save), _ptr(dX), sides, _ptr(ws), ws_bytes, _stream(stream),
        )
    )
    return [sides[0], sides[1]]


def poetx_linear_fwd_group(calls, T: int, stream=None):
    """calls: list of dicts with the keyword arguments of poetx_linear_fwd (dsc, X, perm_R, perm_P, Wt, g_R, g_P,
    Y, H_save, ws, ws_bytes), marshalled into a host array of FwdCall records."""
    descs = [c["dsc"] for c in calls]  # kept alive through the call
    arr = (FwdCall * len(calls))(*[
        FwdCall(ctypes.pointer(dsc), _ptr(c["X"]), _ptr(c["perm_R"]), _ptr(c["perm_P"]), _ptr(c["Wt"]), _ptr(c["g_R"]),
                _ptr(c["g_P"]), _ptr(c["Y"]), _ptr(c["H_save"]), _ptr(c["ws"]), c["ws_bytes"])
        for c, dsc in zip(calls, descs)
    ])
    _check(lib().poetx_linear_fwd_group(len(calls), arr, T, _stream(stream)))


def poetx_linear_bwd_dx_group(calls, T: int, stream=None):
    """calls: list of dicts with the keyword arguments of poetx_linear_bwd_dx_sides (dsc, Y, dZ, perm_R, perm_P, Wt,
    g_R, g_P, H_save, dX, ws, ws_bytes); returns the block-gradient operands of every linear as pairs (R, P) of
    GradSide records."""
    descs = [c["dsc"] for c in calls]
    arr = (BwdCall * len(calls))(*[
        BwdCall(ctypes.pointer(dsc), _ptr(c["Y"]), _ptr(c["dZ"]), _ptr(c["perm_R"]), _ptr(c["perm_P"]), _ptr(c["Wt"]),
                _ptr(c["g_R"]), _ptr(c["g_P"]), _ptr(c["H_save"]), _ptr(c["dX"]), _ptr(c["ws"]), c["ws_bytes"])
        for c, dsc in zip(calls, descs)
    ])
    sides = (GradSide * (2 * len(calls)))()
    _check(lib().poetx_linear_bwd_dx_group(len(calls), arr, T, sides, _stream(stream)))
    return [[sides[2 * i], sides[2 * i + 1]] for i in range(len(calls))]


def poetx_block_grads_workspace_size(d, rows: int, b: int, dtype: int) -> int:
    return lib().poetx_block_grads_workspace_size(len(d), _i32_array(d), rows, b, dtype)


def poetx_block_grads_batch(sides, rows: int, b: int, dtype: int, dg, dg_bytes: int, ws, ws_bytes: int, stream=None):
    """sides: list of GradSide records (from poetx_linear_bwd_dx_sides), marshalled into a host array."""
    arr = (GradSide * len(sides))(*sides)
    _check(lib().poetx_block_grads_batch(len(sides), arr, rows, b, dtype, _ptr(dg), dg_bytes, _ptr(ws), ws_bytes,
                                         _stream(stream)))


def poetx_cnp_backward_batch(q, d, b: int, dtype: int, dg, dg_bytes: int, dq, stream=None):
    _check(lib().poetx_cnp_backward_batch(len(d), _ptr_array(q), _i32_array(d), b, dtype, _ptr(dg), dg_bytes,
                                          _ptr_array(dq), _stream(stream)))


# ------------------------------------------------- optimiser step on packed q ---
def poetx_adam_step_batch(q, dq, m1, m2, lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
                          t: int, lens=None, stream=None):
    """q, dq, m1, m2: per-side lists of fp32 device tensors; lens defaults to each q's numel()."""
    if lens is None:
        lens = [x.numel() for x in q]
    hp = AdamParams(lr, beta1, beta2, eps, weight_decay, t)
    _check(lib().poetx_adam_step_batch(len(lens), (ctypes.c_int64 * len(lens))(*lens), _ptr_array(q), _ptr_array(dq),
                                       _ptr_array(m1), _ptr_array(m2), ctypes.byref(hp), _stream(stream)))


# ------------------------------------------------------------ one SPO factor ---
def spo_desc(d: int, b: int, kind: str, act: str) -> SpoDesc:
    return SpoDesc(d, b, SPO_KINDS[kind], DTYPES[act])


def poetx_spo_saved_bytes(dsc: SpoDesc, T: int) -> int:
    return lib().poetx_spo_saved_bytes(ctypes.byref(dsc), T)


def poetx_spo_workspace_size(dsc: SpoDesc, T: int, op: int) -> int:
    return lib().poetx_spo_workspace_size(ctypes.byref(dsc), T, op)


def poetx_spo_fwd(dsc: SpoDesc, T: int, X, idx, G, Y, saved, ws, ws_bytes: int, stream=None):
    _check(lib().poetx_spo_fwd(ctypes.byref(dsc), T, _ptr(X), _ptr(idx), _ptr(G), _ptr(Y), _ptr(saved), _ptr(ws),
                               ws_bytes, _stream(stream)))


def poetx_spo_bwd(dsc: SpoDesc, T: int, dY, idx, G, q, saved, dX, dq, ws, ws_bytes: int, stream=None):
    _check(lib().poetx_spo_bwd(ctypes.byref(dsc), T, _ptr(dY), _ptr(idx), _ptr(G), _ptr(q), _ptr(saved), _ptr(dX),
                               _ptr(dq), _ptr(ws), ws_bytes, _stream(stream)))


# --------------------------------------------------- weight-centric baseline ---
def poetx_wc_state_bytes(dsc: LayerDesc, T: int) -> int:
    return lib().poetx_wc_state_bytes(ctypes.byref(dsc), T)


def poetx_wc_workspace_size(dsc: LayerDesc, T: int, op: int) -> int:
    return lib().poetx_wc_workspace_size(ctypes.byref(dsc), T, op)


def poetx_wc_fwd(dsc: LayerDesc, T: int, X, perm_R, perm_P, Wt, g_R, g_P, Y, state, ws, ws_bytes: int, stream=None):
    _check(lib().poetx_wc_fwd(ctypes.byref(dsc), T, _ptr(X), _ptr(perm_R), _ptr(perm_P), _ptr(Wt), _ptr(g_R), _ptr(g_P),
                              _ptr(Y), _ptr(state), _ptr(ws), ws_bytes, _stream(stream)))


def poetx_wc_bwd(dsc: LayerDesc, T: int, dZ, perm_R, perm_P, g_R, g_P, q_R, q_P, state, dX, dq_R, dq_P, ws,
                 ws_bytes: int, stream=None):
    _check(lib().poetx_wc_bwd(ctypes.byref(dsc), T, _ptr(dZ), _ptr(perm_R), _ptr(perm_P), _ptr(g_R), _ptr(g_P),
                              _ptr(q_R), _ptr(q_P), _ptr(state), _ptr(dX), _ptr(dq_R), _ptr(dq_P), _ptr(ws), ws_bytes,
                              _stream(stream)))


# ---------------------------------------- merging a chain's outer factors ---
def poetx_fold_workspace_size(dsc: LayerDesc, side: int, f: SpoDesc) -> int:
    return lib().poetx_fold_workspace_size(ctypes.byref(dsc), side, ctypes.byref(f))


def poetx_fold_factor(dsc: LayerDesc, side: int, f: SpoDesc, idx, G, perm, W, ldw: int, ws, ws_bytes: int,
                      stream=None):
    _check(lib().poetx_fold_factor(ctypes.byref(dsc), side, ctypes.byref(f), _ptr(idx), _ptr(G), _ptr(perm), _ptr(W),
                                   ldw, _ptr(ws), ws_bytes, _stream(stream)))


def poetx_store_workspace_size(dsc: LayerDesc) -> int:
    return lib().poetx_store_workspace_size(ctypes.byref(dsc))


def poetx_store_weight(dsc: LayerDesc, W, ldw: int, Wt, ws, ws_bytes: int, stream=None):
    _check(lib().poetx_store_weight(ctypes.byref(dsc), _ptr(W), ldw, _ptr(Wt), _ptr(ws), ws_bytes, _stream(stream)))
