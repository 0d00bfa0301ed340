"""ctypes binding of libikbo.so (argument marshalling only).

Every function has the name of the C entry point it calls (include/ikbo.h).
Tensor arguments are torch tensors on the current HIP device (or, for the
``*_host`` arguments, numpy int32 arrays); they are passed as raw pointers.
A negative status raises :class:`IkboError` carrying the library's message.
All computation happens in the library's HIP kernels; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libikbo.so")

IKBO_OK = 0
IKBO_ERR_INVALID_ARG = -1
IKBO_ERR_BAD_OFFSETS = -2
IKBO_ERR_BAD_MAPPING = -3
IKBO_ERR_UNSUPPORTED = -4
IKBO_ERR_HIP = -5
IKBO_ERR_NOMEM = -6
IKBO_DTYPE_BF16 = 0
IKBO_DTYPE_F32 = 1

# Every symbol include/ikbo.h declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_IP = ctypes.POINTER(ctypes.c_int32)
_LP = ctypes.POINTER(ctypes.c_int64)
SIGNATURES = {
    "ikbo_version": (ctypes.c_int, []),
    "ikbo_last_error": (ctypes.c_char_p, []),
    "ikbo_group_csr": (ctypes.c_int, [_IP, _I, _I, _I, _I, _IP, _IP, _IP, _IP, _I, _IP]),
    "ikbo_attn_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P]),
    "ikbo_attn_fwd_ex": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _P]),
    "ikbo_self_target_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _P, _P]),
    "ikbo_attn_fwd_materialized": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _P]),
    "ikbo_plan_create": (ctypes.c_int, [ctypes.POINTER(_P)]),
    "ikbo_plan_build": (ctypes.c_int, [_P, _IP, _IP, _I, _I, _I, _I, _I, _I, _I, _P]),
    "ikbo_attn_fwd_planned": (ctypes.c_int, [_P, _P, _P, _P, _P, _F, _P, _P, _P]),
    "ikbo_plan_destroy": (None, [_P]),
    "ikbo_plan_info": (ctypes.c_int, [_P, _LP, _I]),
    "ikbo_plan_timing": (ctypes.c_int, [_P, _I]),
    "ikbo_plan_trace": (ctypes.c_int, [_P, _I]),
    "ikbo_plan_trace_read": (ctypes.c_int, [_P, _LP, _I, _IP]),
    "ikbo_plan_timing_read": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float),
                                             _I, _IP]),
    "ikbo_lce_create": (ctypes.c_int, [ctypes.POINTER(_P), _P, _I, _I, _I, _I, _P]),
    "ikbo_lce_fwd": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _I, _P, _P]),
    "ikbo_lce_errors": (ctypes.c_int, [_P, _LP]),
    "ikbo_lce_timing": (ctypes.c_int, [_P, _I]),
    "ikbo_lce_timing_read": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float),
                                            _I, _IP]),
    "ikbo_lce_destroy": (None, [_P]),
    "ikbo_lce3_create": (ctypes.c_int, [ctypes.POINTER(_P), _P, _I, _I, _I, _I, _I, _P]),
    "ikbo_lce3_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "ikbo_bwd_create": (ctypes.c_int, [ctypes.POINTER(_P)]),
    "ikbo_attn_bwd": (ctypes.c_int, [_P, _IP, _IP, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "ikbo_bwd_info": (ctypes.c_int, [_P, _LP, _I]),
    "ikbo_bwd_timing": (ctypes.c_int, [_P, _I]),
    "ikbo_bwd_timing_read": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float),
                                            _I, _IP]),
    "ikbo_bwd_destroy": (None, [_P]),
    "ikbo_mx_create": (ctypes.c_int, [ctypes.POINTER(_P)]),
    "ikbo_attn_fwd_mxfp8": (ctypes.c_int, [_P, _IP, _IP, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P, _P, _P]),
    "ikbo_mx_info": (ctypes.c_int, [_P, _LP, _I]),
    "ikbo_mx_timing": (ctypes.c_int, [_P, _I]),
    "ikbo_mx_timing_read": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float),
                                           _I, _IP]),
    "ikbo_mx_destroy": (None, [_P]),
}

_lib = None


class IkboError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"ikbo status {status}: {msg}")
        self.status = status


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Loads libikbo.so (built in-tree by broadcast_free_target_amd._build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python -m broadcast_free_target_amd._build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(status: int) -> int:
    if status < 0:
        raise IkboError(status, load_library().ikbo_last_error().decode())
    return status


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _i32(a: np.ndarray):
    assert a.dtype == np.int32 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_IP)


def ikbo_version() -> int:
    return load_library().ikbo_version()


def ikbo_last_error() -> str:
    return load_library().ikbo_last_error().decode()


def ikbo_group_csr(cand_to_user_host: np.ndarray, n_users: int, n_q: int, bm: int):
    """Host CSR grouping.  Returns (counts, cand_offsets, cand_perm, tiles[T, 3])."""
    lib = load_library()
    c2u = np.ascontiguousarray(cand_to_user_host, dtype=np.int32)
    n_cand = int(c2u.shape[0])
    counts = np.zeros(max(n_users, 1), np.int32)
    offs = np.zeros(n_users + 1, np.int32)
    perm = np.zeros(max(n_cand, 1), np.int32)
    nt = ctypes.c_int32(0)
    rc = lib.ikbo_group_csr(_i32(c2u), n_cand, n_users, n_q, bm, _i32(counts), _i32(offs), _i32(perm),
                            None, 0, ctypes.byref(nt))
    if rc == IKBO_ERR_INVALID_ARG and nt.value > 0:
        pass  # size query: tiles buffer too small
    elif rc < 0:
        _check(rc)
    tiles = np.zeros((max(nt.value, 1), 3), np.int32)
    _check(lib.ikbo_group_csr(_i32(c2u), n_cand, n_users, n_q, bm, _i32(counts), _i32(offs), _i32(perm),
                              _i32(tiles), nt.value, ctypes.byref(nt)))
    return counts[:n_users], offs, perm[:n_cand], tiles[:nt.value]


def ikbo_attn_fwd(q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, H, d, scale, out,
                  stream=None) -> int:
    return _check(load_library().ikbo_attn_fwd(
        _ptr(q_cand), _ptr(k_user), _ptr(v_user), _ptr(user_offsets), _ptr(cand_to_user),
        n_users, n_cand, H, d, float(scale), _ptr(out), _stream(stream)))


def ikbo_attn_fwd_ex(q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, n_q, H, d, scale,
                     dtype, out, stream=None) -> int:
    return _check(load_library().ikbo_attn_fwd_ex(
        _ptr(q_cand), _ptr(k_user), _ptr(v_user), _ptr(user_offsets), _ptr(cand_to_user),
        n_users, n_cand, n_q, H, d, float(scale), dtype, _ptr(out), _stream(stream)))


def ikbo_self_target_fwd(q_user, q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, H, d,
                         scale, dtype, out_user, out_cand, stream=None) -> int:
    return _check(load_library().ikbo_self_target_fwd(
        _ptr(q_user), _ptr(q_cand), _ptr(k_user), _ptr(v_user), _ptr(user_offsets), _ptr(cand_to_user),
        n_users, n_cand, H, d, float(scale), dtype, _ptr(out_user), _ptr(out_cand), _stream(stream)))


def ikbo_attn_fwd_materialized(q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, n_q, H, d,
                               scale, dtype, out, stream=None) -> int:
    return _check(load_library().ikbo_attn_fwd_materialized(
        _ptr(q_cand), _ptr(k_user), _ptr(v_user), _ptr(user_offsets), _ptr(cand_to_user),
        n_users, n_cand, n_q, H, d, float(scale), dtype, _ptr(out), _stream(stream)))


def ikbo_plan_create() -> int:
    h = _P()
    _check(load_library().ikbo_plan_create(ctypes.byref(h)))
    return h.value


def ikbo_plan_build(plan, user_offsets_host, cand_to_user_host, n_users, n_cand, n_q, H, d, dtype,
                    with_self=0, stream=None) -> int:
    offs = np.ascontiguousarray(user_offsets_host, dtype=np.int32)
    c2u = np.ascontiguousarray(cand_to_user_host, dtype=np.int32)
    return _check(load_library().ikbo_plan_build(
        plan, _i32(offs), _i32(c2u) if c2u.size else None, n_users, n_cand, n_q, H, d, dtype,
        int(with_self), _stream(stream)))


def ikbo_attn_fwd_planned(plan, q_cand, q_user, k_user, v_user, scale, out_cand, out_user=None,
                          stream=None) -> int:
    return _check(load_library().ikbo_attn_fwd_planned(
        plan, _ptr(q_cand), _ptr(q_user), _ptr(k_user), _ptr(v_user), float(scale), _ptr(out_cand),
        _ptr(out_user), _stream(stream)))


def ikbo_plan_destroy(plan) -> None:
    load_library().ikbo_plan_destroy(plan)


def ikbo_plan_info(plan) -> dict:
    info = (ctypes.c_int64 * 9)()
    _check(load_library().ikbo_plan_info(plan, info, 9))
    keys = ("n_items", "grid", "n_groups", "n_slots", "partial_bytes", "n_target_tiles", "n_self_tiles", "n_cu",
            "kernel")
    return dict(zip(keys, list(info)))


def ikbo_plan_timing(plan, enable: bool) -> int:
    return _check(load_library().ikbo_plan_timing(plan, 1 if enable else 0))


def ikbo_plan_timing_read(plan, max_n: int = 4096):
    """Per-launch (attention, merge) kernel durations in ms of the timed launches."""
    a = (ctypes.c_float * max(max_n, 1))()
    m = (ctypes.c_float * max(max_n, 1))()
    n = ctypes.c_int32(0)
    _check(load_library().ikbo_plan_timing_read(plan, a, m, max_n, ctypes.byref(n)))
    return list(a[:n.value]), list(m[:n.value])


def ikbo_plan_trace(plan, enable: bool) -> int:
    return _check(load_library().ikbo_plan_trace(plan, 1 if enable else 0))


def ikbo_plan_trace_read(plan, max_items: int = 1 << 20) -> np.ndarray:
    """Per-item trace records of the last launch: int64 [n_items, 6]."""
    buf = np.zeros((max(max_items, 1), 6), dtype=np.int64)
    n = ctypes.c_int32(0)
    _check(load_library().ikbo_plan_trace_read(plan, buf.ctypes.data_as(_LP), max_items, ctypes.byref(n)))
    return buf[:n.value]


def ikbo_lce_create(w, M, K_u, K_c, ldw=None, stream=None) -> int:
    """Packs W [M, ldw] (device bf16, user columns first) into a library handle."""
    h = _P()
    _check(load_library().ikbo_lce_create(ctypes.byref(h), _ptr(w), M, K_u, K_c, K_u + K_c if ldw is None else ldw,
                                          _stream(stream)))
    return h.value


def ikbo_lce_fwd(lce, x_user, x_cand, cand_to_user, n_users, n_cand, N, out, stream=None) -> int:
    return _check(load_library().ikbo_lce_fwd(lce, _ptr(x_user), _ptr(x_cand), _ptr(cand_to_user), n_users, n_cand,
                                              N, _ptr(out), _stream(stream)))


def ikbo_lce_errors(lce) -> int:
    c = ctypes.c_int64(0)
    _check(load_library().ikbo_lce_errors(lce, ctypes.byref(c)))
    return c.value


def ikbo_lce_timing(lce, enable: bool) -> int:
    return _check(load_library().ikbo_lce_timing(lce, 1 if enable else 0))


def ikbo_lce_timing_read(lce, max_n: int = 4096):
    """Per-call (user GEMM, candidate GEMM) durations in ms of the timed calls."""
    a = (ctypes.c_float * max(max_n, 1))()
    b = (ctypes.c_float * max(max_n, 1))()
    n = ctypes.c_int32(0)
    _check(load_library().ikbo_lce_timing_read(lce, a, b, max_n, ctypes.byref(n)))
    return list(a[:n.value]), list(b[:n.value])


def ikbo_lce_destroy(lce) -> None:
    load_library().ikbo_lce_destroy(lce)


def ikbo_bwd_create() -> int:
    h = _P()
    _check(load_library().ikbo_bwd_create(ctypes.byref(h)))
    return h.value


def ikbo_attn_bwd(bwd, user_offsets_host, cand_to_user_host, n_users, n_cand, n_q, H, d, scale, q_cand, k_user,
                  v_user, out, dout, dq_cand, dk_user, dv_user, stream=None) -> int:
    """Gradients of target attention; the mapping arrays are host int32 arrays."""
    offs = np.ascontiguousarray(user_offsets_host, dtype=np.int32)
    c2u = np.ascontiguousarray(cand_to_user_host, dtype=np.int32)
    return _check(load_library().ikbo_attn_bwd(
        bwd, _i32(offs), _i32(c2u) if c2u.size else None, n_users, n_cand, n_q, H, d, float(scale), _ptr(q_cand),
        _ptr(k_user), _ptr(v_user), _ptr(out), _ptr(dout), _ptr(dq_cand), _ptr(dk_user), _ptr(dv_user),
        _stream(stream)))


def ikbo_bwd_info(bwd) -> dict:
    a = (ctypes.c_int64 * 3)()
    _check(load_library().ikbo_bwd_info(bwd, a, 3))
    return {"dq_items": a[0], "dkv_items": a[1], "dq_split_groups": a[2]}


def ikbo_bwd_timing(bwd, enable: bool) -> int:
    return _check(load_library().ikbo_bwd_timing(bwd, 1 if enable else 0))


def ikbo_bwd_timing_read(bwd, max_n: int = 4096):
    """Per-call (dQ kernel, dK/dV kernel) durations in ms of the timed calls."""
    a = (ctypes.c_float * max(max_n, 1))()
    b = (ctypes.c_float * max(max_n, 1))()
    n = ctypes.c_int32(0)
    _check(load_library().ikbo_bwd_timing_read(bwd, a, b, max_n, ctypes.byref(n)))
    return list(a[:n.value]), list(b[:n.value])


def ikbo_bwd_destroy(bwd) -> None:
    load_library().ikbo_bwd_destroy(bwd)


def ikbo_mx_create() -> int:
    h = _P()
    _check(load_library().ikbo_mx_create(ctypes.byref(h)))
    return h.value


def ikbo_attn_fwd_mxfp8(mx, user_offsets_host, cand_to_user_host, n_users, n_cand, n_q, H, d, scale, q_codes,
                        q_scales, k_codes, k_scales, v_codes, v_scales, out, stream=None) -> int:
    """MXFP8 target attention; the mapping arrays are host int32 arrays, the
    codes and scales uint8 device tensors, out a bf16 device tensor."""
    offs = np.ascontiguousarray(user_offsets_host, dtype=np.int32)
    c2u = np.ascontiguousarray(cand_to_user_host, dtype=np.int32)
    return _check(load_library().ikbo_attn_fwd_mxfp8(
        mx, _i32(offs), _i32(c2u) if c2u.size else None, n_users, n_cand, n_q, H, d, float(scale), _ptr(q_codes),
        _ptr(q_scales), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales), _ptr(out), _stream(stream)))


def ikbo_mx_info(mx) -> dict:
    a = (ctypes.c_int64 * 3)()
    _check(load_library().ikbo_mx_info(mx, a, 3))
    return {"n_items": a[0], "n_groups": a[1], "grid": a[2]}


def ikbo_mx_timing(mx, enable: bool) -> int:
    return _check(load_library().ikbo_mx_timing(mx, 1 if enable else 0))


def ikbo_mx_timing_read(mx, max_n: int = 4096):
    """Per-call (attention kernel, merge kernel) durations in ms of the timed calls."""
    a = (ctypes.c_float * max(max_n, 1))()
    b = (ctypes.c_float * max(max_n, 1))()
    n = ctypes.c_int32(0)
    _check(load_library().ikbo_mx_timing_read(mx, a, b, max_n, ctypes.byref(n)))
    return list(a[:n.value]), list(b[:n.value])


def ikbo_mx_destroy(mx) -> None:
    load_library().ikbo_mx_destroy(mx)


def ikbo_lce3_create(w, M, K_u, K_v, K_c, ldw=None, stream=None) -> int:
    """Packs W [M, ldw] (device bf16; user, vendor, item columns) for three levels."""
    h = _P()
    _check(load_library().ikbo_lce3_create(ctypes.byref(h), _ptr(w), M, K_u, K_v, K_c,
                                           K_u + K_v + K_c if ldw is None else ldw, _stream(stream)))
    return h.value


def ikbo_lce3_fwd(lce, x_user, x_vendor, x_cand, vendor_to_user, cand_to_vendor, n_users, n_vendors, n_cand, N, out,
                  stream=None) -> int:
    return _check(load_library().ikbo_lce3_fwd(lce, _ptr(x_user), _ptr(x_vendor), _ptr(x_cand), _ptr(vendor_to_user),
                                               _ptr(cand_to_vendor), n_users, n_vendors, n_cand, N, _ptr(out),
                                               _stream(stream)))

