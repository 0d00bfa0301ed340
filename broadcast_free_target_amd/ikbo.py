"""ctypes binding of libikbo.so (argument marshalling only).

Every function has the name of the C entry point it calls (include/ikbo.h).
Tensor arguments are torch tensors on the current HIP device (or, for the
``*_host`` arguments, numpy int32 arrays); they are passed as raw pointers.
A negative status raises :class:`IkboError` carrying the library's message.
All computation happens in the library's HIP kernels; there is no fallback.
"""

from __future__ import annotations

import ctypes
from collections import OrderedDict
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
    "ikbo_attn_fwd_f32": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P]),
    "ikbo_attn_fwd_mt": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _I, _I]),
    "ikbo_attn_fwd_mt_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _I, _I]),
    "ikbo_attn_fwd_ex": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _P]),
    "ikbo_self_target_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _P, _P]),
    "ikbo_attn_fwd_materialized": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _I, _I]),
    "ikbo_plan_create": (ctypes.c_int, [_P, _P, _I, _I, _I, _I, _I, _I, _I, _P, ctypes.POINTER(_P)]),
    "ikbo_plan_build": (ctypes.c_int, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "ikbo_attn_fwd_planned": (ctypes.c_int, [_P, _P, _P, _P, _P, _F, _P, _P, _P]),
    "ikbo_attn_fwd_hostmap": (ctypes.c_int, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _F, _P, _P,
                                             _P]),
    "ikbo_attn_fwd_train": (ctypes.c_int, [_P, _P, _P, _P, _F, _P, _P, _P]),
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
    "ikbo_attn_bwd": (ctypes.c_int, [_P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                     _P]),
    "ikbo_bwd_info": (ctypes.c_int, [_P, _LP, _I]),
    "ikbo_bwd_timing": (ctypes.c_int, [_P, _I]),
    "ikbo_bwd_timing_read": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float),
                                            _I, _IP]),
    "ikbo_bwd_destroy": (None, [_P]),
    "ikbo_mx_create": (ctypes.c_int, [ctypes.POINTER(_P)]),
    "ikbo_attn_fwd_mxfp8": (ctypes.c_int, [_P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P, _P, _P]),
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
    if t is None or isinstance(t, int):
        return t
    return t.data_ptr()


def _bad(msg: str):
    return IkboError(IKBO_ERR_INVALID_ARG, msg)


def _need(t, nbytes: int, name: str, elem: Optional[int] = None) -> None:
    """Checks a device tensor argument against the extent the call will touch.

    The C ABI receives bare pointers and cannot see a buffer's size, so a
    mismatched dtype or shape would let the kernels read or write past the
    allocation.  Tensors are checked here (device-resident, contiguous, element
    size, at least nbytes); a raw integer pointer is the caller's to size."""
    if t is None or isinstance(t, int):
        return
    if not getattr(t, "is_cuda", False):
        raise _bad(f"{name}: expected a device tensor")
    if elem is not None and t.element_size() != elem:
        raise _bad(f"{name}: element size {t.element_size()}, expected {elem} (dtype {t.dtype})")
    if not t.is_contiguous():
        raise _bad(f"{name}: tensor must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise _bad(f"{name}: {have} bytes, the call needs {nbytes}")


def _es(dtype: int) -> int:
    return 2 if dtype == IKBO_DTYPE_BF16 else 4


# dimensions each built plan / created handle was given, for _need
_PLAN_DIMS: dict = {}
_LCE_DIMS: dict = {}


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


# Addresses of the last few host mapping arrays.  Reading an ndarray's address
# through numpy's ctypes interface costs microseconds, a sizeable part of a
# small request's host time when the same arrays come back call after call.
# Each entry holds a reference to its array, so the array cannot be freed and
# its id reused while the entry exists, and an ndarray's buffer does not move
# while referenced.
_HOST_PTRS: "OrderedDict[int, tuple]" = OrderedDict()


def _host_i32(a: np.ndarray) -> Optional[int]:
    """Address of a contiguous int32 host array, read by the C side during the call."""
    if a.size == 0:
        return None
    e = _HOST_PTRS.get(id(a))
    if e is not None and e[0] is a:
        return e[1]
    if a.dtype != np.int32 or not a.flags["C_CONTIGUOUS"]:
        raise _bad("host mapping arrays must be contiguous int32")
    ptr = a.ctypes.data
    _HOST_PTRS[id(a)] = (a, ptr)
    if len(_HOST_PTRS) > 8:
        _HOST_PTRS.popitem(last=False)
    return ptr


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


def _total_len(user_offsets, n_users) -> Optional[int]:
    """user_offsets[n_users] of a device offsets tensor (one 4-byte copy; the
    device-mapping calls synchronise on the mapping anyway), or None for a raw
    pointer or an offsets tensor too short to hold it."""
    if user_offsets is None or isinstance(user_offsets, int) or user_offsets.numel() < n_users + 1 or n_users < 0:
        return None
    return int(user_offsets[n_users].item())


def _check_common(q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, n_q, H, d, es, out):
    """Checks every tensor against the extent the call touches.  Returns the
    total key count user_offsets[n_users] when it could be read, else None."""
    rows = n_cand * n_q * H * d * es
    _need(q_cand, rows, "q_cand", es)
    _need(out, rows, "out", es)
    _need(user_offsets, (n_users + 1) * 4, "user_offsets", 4)
    _need(cand_to_user, n_cand * 4, "cand_to_user", 4)
    total = _total_len(user_offsets, n_users)
    kv = 0 if total is None or total < 0 else total * H * d * es
    _need(k_user, kv, "k_user", es)
    _need(v_user, kv, "v_user", es)
    return total


def ikbo_attn_fwd(q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, H, d, scale, out,
                  stream=None) -> int:
    _check_common(q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, 1, H, d, 2, out)
    return _check(load_library().ikbo_attn_fwd(
        _ptr(q_cand), _ptr(k_user), _ptr(v_user), _ptr(user_offsets), _ptr(cand_to_user),
        n_users, n_cand, H, d, float(scale), _ptr(out), _stream(stream)))


def ikbo_attn_fwd_f32(q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, H, d, scale, out,
                      stream=None) -> int:
    _check_common(q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, 1, H, d, 4, out)
    return _check(load_library().ikbo_attn_fwd_f32(
        _ptr(q_cand), _ptr(k_user), _ptr(v_user), _ptr(user_offsets), _ptr(cand_to_user),
        n_users, n_cand, H, d, float(scale), _ptr(out), _stream(stream)))


def ikbo_attn_fwd_mt(q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, H, d, scale, out,
                     stream=None, n_q=1, dtype=IKBO_DTYPE_BF16) -> int:
    _check_common(q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, n_q, H, d, _es(dtype), out)
    return _check(load_library().ikbo_attn_fwd_mt(
        _ptr(q_cand), _ptr(k_user), _ptr(v_user), _ptr(user_offsets), _ptr(cand_to_user),
        n_users, n_cand, H, d, float(scale), _ptr(out), _stream(stream), n_q, dtype))


def ikbo_attn_fwd_mt_noalloc(q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, H, d, scale, out,
                             stream=None, n_q=1, dtype=IKBO_DTYPE_BF16) -> int:
    _check_common(q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, n_q, H, d, _es(dtype), out)
    return _check(load_library().ikbo_attn_fwd_mt_noalloc(
        _ptr(q_cand), _ptr(k_user), _ptr(v_user), _ptr(user_offsets), _ptr(cand_to_user),
        n_users, n_cand, H, d, float(scale), _ptr(out), _stream(stream), n_q, dtype))


def ikbo_attn_fwd_ex(q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, n_q, H, d, scale,
                     dtype, out, stream=None) -> int:
    _check_common(q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, n_q, H, d, _es(dtype), out)
    return _check(load_library().ikbo_attn_fwd_ex(
        _ptr(q_cand), _ptr(k_user), _ptr(v_user), _ptr(user_offsets), _ptr(cand_to_user),
        n_users, n_cand, n_q, H, d, float(scale), dtype, _ptr(out), _stream(stream)))


def ikbo_self_target_fwd(q_user, q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, H, d,
                         scale, dtype, out_user, out_cand, stream=None) -> int:
    es = _es(dtype)
    total = _check_common(q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, 1, H, d, es, out_cand)
    kv = 0 if total is None or total < 0 else total * H * d * es
    _need(q_user, kv, "q_user", es)
    _need(out_user, kv, "out_user", es)
    return _check(load_library().ikbo_self_target_fwd(
        _ptr(q_user), _ptr(q_cand), _ptr(k_user), _ptr(v_user), _ptr(user_offsets), _ptr(cand_to_user),
        n_users, n_cand, H, d, float(scale), dtype, _ptr(out_user), _ptr(out_cand), _stream(stream)))


def ikbo_attn_fwd_materialized(q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, H, d, scale,
                               out, stream=None, n_q=1, dtype=IKBO_DTYPE_BF16) -> int:
    _check_common(q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, n_q, H, d, _es(dtype), out)
    return _check(load_library().ikbo_attn_fwd_materialized(
        _ptr(q_cand), _ptr(k_user), _ptr(v_user), _ptr(user_offsets), _ptr(cand_to_user),
        n_users, n_cand, H, d, float(scale), _ptr(out), _stream(stream), n_q, dtype))


def ikbo_plan_create(user_offsets_host, cand_to_user_host, n_users, n_cand, n_q, H, d, dtype, with_self=0,
                     stream=None) -> int:
    """A plan built for the request the host mapping arrays describe."""
    offs = np.ascontiguousarray(user_offsets_host, dtype=np.int32)
    c2u = np.ascontiguousarray(cand_to_user_host, dtype=np.int32)
    h = _P()
    _check(load_library().ikbo_plan_create(_host_i32(offs), _host_i32(c2u), n_users, n_cand, n_q, H, d, dtype,
                                           int(with_self), _stream(stream), ctypes.byref(h)))
    _PLAN_DIMS[h.value] = _plan_dims(offs, n_users, n_cand, n_q, H, d, dtype, with_self)
    return h.value


def _plan_dims(offs, n_users, n_cand, n_q, H, d, dtype, with_self):
    """(element size, q/out bytes, k/v bytes, with_self, lse bytes) of a request."""
    es = _es(dtype)
    return (es, n_cand * n_q * H * d * es, int(offs[n_users]) * H * d * es, bool(with_self), n_cand * n_q * H * 4)


def ikbo_plan_build(plan, user_offsets_host, cand_to_user_host, n_users, n_cand, n_q, H, d, dtype,
                    with_self=0, stream=None) -> int:
    offs = np.ascontiguousarray(user_offsets_host, dtype=np.int32)
    c2u = np.ascontiguousarray(cand_to_user_host, dtype=np.int32)
    _PLAN_DIMS.pop(plan, None)
    rc = _check(load_library().ikbo_plan_build(
        plan, _host_i32(offs), _host_i32(c2u), n_users, n_cand, n_q, H, d, dtype, int(with_self), _stream(stream)))
    _PLAN_DIMS[plan] = _plan_dims(offs, n_users, n_cand, n_q, H, d, dtype, with_self)
    return rc


def ikbo_attn_fwd_planned(plan, q_cand, q_user, k_user, v_user, scale, out_cand, out_user=None,
                          stream=None) -> int:
    dims = _PLAN_DIMS.get(plan)
    if dims is not None:
        es, cand_bytes, kv_bytes, with_self, _ = dims
        _need(q_cand, cand_bytes, "q_cand", es)
        _need(out_cand, cand_bytes, "out_cand", es)
        _need(k_user, kv_bytes, "k_user", es)
        _need(v_user, kv_bytes, "v_user", es)
        if with_self:
            _need(q_user, kv_bytes, "q_user", es)
            _need(out_user, kv_bytes, "out_user", es)
    return _check(load_library().ikbo_attn_fwd_planned(
        plan, _ptr(q_cand), _ptr(q_user), _ptr(k_user), _ptr(v_user), float(scale), _ptr(out_cand),
        _ptr(out_user), _stream(stream)))


def ikbo_attn_fwd_hostmap(plan, user_offsets_host, cand_to_user_host, n_users, n_cand, n_q, H, d, dtype, with_self,
                          q_cand, q_user, k_user, v_user, scale, out_cand, out_user=None, stream=None) -> int:
    """Rebuilds the plan for the request the host mapping arrays describe and
    launches it, in one library call."""
    offs = np.ascontiguousarray(user_offsets_host, dtype=np.int32)
    c2u = np.ascontiguousarray(cand_to_user_host, dtype=np.int32)
    dims = _plan_dims(offs, n_users, n_cand, n_q, H, d, dtype, with_self) if offs.size > n_users >= 0 else None
    if dims is not None:
        es, cand_bytes, kv_bytes, _, _ = dims
        _need(q_cand, cand_bytes, "q_cand", es)
        _need(out_cand, cand_bytes, "out_cand", es)
        _need(k_user, kv_bytes, "k_user", es)
        _need(v_user, kv_bytes, "v_user", es)
        if with_self:
            _need(q_user, kv_bytes, "q_user", es)
            _need(out_user, kv_bytes, "out_user", es)
    _PLAN_DIMS.pop(plan, None)
    rc = _check(load_library().ikbo_attn_fwd_hostmap(
        plan, _host_i32(offs), _host_i32(c2u), n_users, n_cand, n_q, H, d, dtype, int(with_self), _ptr(q_cand),
        _ptr(q_user), _ptr(k_user), _ptr(v_user), float(scale), _ptr(out_cand), _ptr(out_user), _stream(stream)))
    _PLAN_DIMS[plan] = dims
    return rc


def ikbo_attn_fwd_train(plan, q_cand, k_user, v_user, scale, out_cand, lse, stream=None) -> int:
    """The planned launch that also writes each row's log-sum-exp (fp32 [n_cand, n_q, H])."""
    dims = _PLAN_DIMS.get(plan)
    if dims is not None:
        es, cand_bytes, kv_bytes, _, lse_bytes = dims
        _need(q_cand, cand_bytes, "q_cand", es)
        _need(out_cand, cand_bytes, "out_cand", es)
        _need(k_user, kv_bytes, "k_user", es)
        _need(v_user, kv_bytes, "v_user", es)
        _need(lse, lse_bytes, "lse", 4)
    return _check(load_library().ikbo_attn_fwd_train(
        plan, _ptr(q_cand), _ptr(k_user), _ptr(v_user), float(scale), _ptr(out_cand), _ptr(lse), _stream(stream)))


def ikbo_plan_destroy(plan) -> None:
    _PLAN_DIMS.pop(plan, None)
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
    ld = K_u + K_c if ldw is None else ldw
    _need(w, M * ld * 2, "w", 2)
    _check(load_library().ikbo_lce_create(ctypes.byref(h), _ptr(w), M, K_u, K_c, ld, _stream(stream)))
    _LCE_DIMS[h.value] = (M, K_u, K_c)
    return h.value


def ikbo_lce_fwd(lce, x_user, x_cand, cand_to_user, n_users, n_cand, N, out, stream=None) -> int:
    dims = _LCE_DIMS.get(lce)
    if dims is not None and len(dims) == 3:
        M, K_u, K_c = dims
        _need(x_user, n_users * K_u * N * 2, "x_user", 2)
        _need(x_cand, n_cand * K_c * N * 2, "x_cand", 2)
        _need(out, n_cand * M * N * 2, "out", 2)
        _need(cand_to_user, n_cand * 4, "cand_to_user", 4)
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
    _LCE_DIMS.pop(lce, None)
    load_library().ikbo_lce_destroy(lce)


def ikbo_bwd_create() -> int:
    h = _P()
    _check(load_library().ikbo_bwd_create(ctypes.byref(h)))
    return h.value


def ikbo_attn_bwd(bwd, user_offsets_host, cand_to_user_host, n_users, n_cand, n_q, H, d, scale, q_cand, k_user,
                  v_user, out, dout, dq_cand, dk_user, dv_user, stream=None, lse=None) -> int:
    """Gradients of target attention; the mapping arrays are host int32 arrays.
    lse (optional): the forward's log-sum-exp, fp32 [n_cand, n_q, H]."""
    _need(lse, n_cand * n_q * H * 4, "lse", 4)
    offs = np.ascontiguousarray(user_offsets_host, dtype=np.int32)
    c2u = np.ascontiguousarray(cand_to_user_host, dtype=np.int32)
    if offs.size >= n_users + 1:
        rows = n_cand * n_q * H * d * 2
        kv = int(offs[n_users]) * H * d * 2
        for t, nm in ((q_cand, "q_cand"), (out, "out"), (dout, "dout"), (dq_cand, "dq_cand")):
            _need(t, rows, nm, 2)
        for t, nm in ((k_user, "k_user"), (v_user, "v_user"), (dk_user, "dk_user"), (dv_user, "dv_user")):
            _need(t, kv, nm, 2)
    return _check(load_library().ikbo_attn_bwd(
        bwd, _host_i32(offs), _host_i32(c2u), n_users, n_cand, n_q, H, d, float(scale), _ptr(q_cand),
        _ptr(k_user), _ptr(v_user), _ptr(out), _ptr(dout), _ptr(dq_cand), _ptr(dk_user), _ptr(dv_user), _ptr(lse),
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
    if offs.size >= n_users + 1 and d % 32 == 0:
        T = int(offs[n_users])
        nvb = int(((offs[1:n_users + 1] - offs[:n_users] + 31) // 32).sum())
        _need(q_codes, n_cand * n_q * H * d, "q_codes", 1)
        _need(q_scales, n_cand * n_q * H * (d // 32), "q_scales", 1)
        _need(k_codes, T * H * d, "k_codes", 1)
        _need(k_scales, T * H * (d // 32), "k_scales", 1)
        _need(v_codes, T * H * d, "v_codes", 1)
        _need(v_scales, nvb * H * d, "v_scales", 1)
        _need(out, n_cand * n_q * H * d * 2, "out", 2)
    return _check(load_library().ikbo_attn_fwd_mxfp8(
        mx, _host_i32(offs), _host_i32(c2u), n_users, n_cand, n_q, H, d, float(scale), _ptr(q_codes),
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
    ld = K_u + K_v + K_c if ldw is None else ldw
    _need(w, M * ld * 2, "w", 2)
    _check(load_library().ikbo_lce3_create(ctypes.byref(h), _ptr(w), M, K_u, K_v, K_c, ld, _stream(stream)))
    _LCE_DIMS[h.value] = (M, K_u, K_v, K_c)
    return h.value


def ikbo_lce3_fwd(lce, x_user, x_vendor, x_cand, vendor_to_user, cand_to_vendor, n_users, n_vendors, n_cand, N, out,
                  stream=None) -> int:
    dims = _LCE_DIMS.get(lce)
    if dims is not None and len(dims) == 4:
        M, K_u, K_v, K_c = dims
        _need(x_user, n_users * K_u * N * 2, "x_user", 2)
        _need(x_vendor, n_vendors * K_v * N * 2, "x_vendor", 2)
        _need(x_cand, n_cand * K_c * N * 2, "x_cand", 2)
        _need(out, n_cand * M * N * 2, "out", 2)
        _need(vendor_to_user, n_vendors * 4, "vendor_to_user", 4)
        _need(cand_to_vendor, n_cand * 4, "cand_to_vendor", 4)
    return _check(load_library().ikbo_lce3_fwd(lce, _ptr(x_user), _ptr(x_vendor), _ptr(x_cand), _ptr(vendor_to_user),
                                               _ptr(cand_to_vendor), n_users, n_vendors, n_cand, N, _ptr(out),
                                               _stream(stream)))

