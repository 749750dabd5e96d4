"""Python binding of libwkv7 (ctypes): argument marshalling only.

Each function has the name of the C entry point it calls and the same
argument order. Device buffers are passed as torch tensors (their
data_ptr() is handed over), host int32 arrays as numpy arrays or sequences,
streams as torch streams (or None for the current stream). A non-zero status
raises `Wkv7Error` carrying the library's message. Every computation happens
in the library's HIP kernels; nothing here computes.

The library must have been built (`python -m linear_attention_rnn_amd.build`);
importing this module without it raises ImportError.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwkv7.so")

WKV7_OK = 0
WKV7_ERR_INVALID_ARG = -1
WKV7_ERR_OUT_OF_RANGE = -2
WKV7_ERR_DUPLICATE_SLOT = -3
WKV7_ERR_POOL_FULL = -4
WKV7_ERR_UNSUPPORTED = -5
WKV7_ERR_OOM = -6
WKV7_ERR_HIP = -7

WKV7_F32 = 0
WKV7_BF16 = 1

WKV7_OPT_PREFILL_MIN_LEN = 1
WKV7_OPT_CHUNK_PRECISE = 2
WKV7_OPT_SEGMENT_LEN = 3

# Every symbol include/wkv7.h declares.
EXPORTS = (
    "wkv7_last_error", "wkv7_version", "wkv7_pool_create", "wkv7_pool_destroy",
    "wkv7_slot_bytes", "wkv7_pool_state_ptr", "wkv7_pool_shape",
    "wkv7_pool_device", "wkv7_pool_set_option", "wkv7_slot_alloc",
    "wkv7_slot_free",
    "wkv7_forward", "wkv7_forward_noalloc", "wkv7_snapshot", "wkv7_fork", "wkv7_reset",
    "wkv7_hibernate", "wkv7_resume", "wkv7_plan_create", "wkv7_plan_tokens",
    "wkv7_forward_plan", "wkv7_plan_destroy", "wkv7_migrate",
    "wkv7_image_header_init", "wkv7_image_header_check",
    "wkv7_sessions_create", "wkv7_sessions_destroy", "wkv7_session_begin",
    "wkv7_session_end", "wkv7_session_abort", "wkv7_session_drop_chat",
    "wkv7_sessions_stats", "wkv7_q8_quantize", "wkv7_q8_matmul",
    "wkv7_q8_linear",
)

# session outcomes and flags (include/wkv7_session.h)
WKV7_SESSION_HIT = 0
WKV7_SESSION_NEW = 1
WKV7_SESSION_RESTART_EDIT = 2
WKV7_SESSION_RESTART_PARENT = 3
WKV7_SESSION_RESTART_EVICTED = 4
WKV7_SESSIONS_KEEP_PARENT = 1


class wkv7_turn_key(ctypes.Structure):
    _fields_ = [("model", ctypes.c_uint64), ("user", ctypes.c_uint64),
                ("chat", ctypes.c_uint64), ("parent", ctypes.c_uint64)]


class wkv7_session_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "hits", "news", "restarts_edit", "restarts_parent",
        "restarts_evicted", "resets", "forks", "hibernates", "resumes",
        "drops")] + [(n, ctypes.c_int32) for n in (
            "active", "parked_device", "parked_host", "free_host_images")]

WKV7_IMAGE_MAGIC = b"WKV7SLOT"
WKV7_IMAGE_VERSION = 1


class wkv7_image_header(ctypes.Structure):
    """The 64-byte versioned header in front of serialized slot images."""
    _fields_ = [("magic", ctypes.c_char * 8), ("version", ctypes.c_uint32),
                ("header_bytes", ctypes.c_uint32), ("H", ctypes.c_uint32),
                ("N", ctypes.c_uint32), ("state_dtype", ctypes.c_uint32),
                ("n_slots", ctypes.c_uint32), ("slot_bytes", ctypes.c_uint64),
                ("reserved", ctypes.c_uint64 * 3)]


class Wkv7Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libwkv7 status {status}: {message}")
        self.status = status
        self.message = message


def _load() -> ctypes.CDLL:
    # One HIP runtime per process: torch ships its own libamdhip64 (same
    # soname as the system one). Loading torch first makes the library bind
    # to that already-loaded runtime instead of pulling in a second copy.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m linear_attention_rnn_amd.build` (there is no fallback)")
    return ctypes.CDLL(LIB_PATH)


lib = _load()

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_vp = ctypes.c_void_p
_pi32 = ctypes.POINTER(ctypes.c_int32)

lib.wkv7_last_error.restype = ctypes.c_char_p
lib.wkv7_last_error.argtypes = []
lib.wkv7_version.restype = _i32
lib.wkv7_version.argtypes = []
lib.wkv7_pool_create.restype = _i32
lib.wkv7_pool_create.argtypes = [_i32, _i32, _i32, ctypes.POINTER(_vp)]
lib.wkv7_pool_destroy.restype = _i32
lib.wkv7_pool_destroy.argtypes = [_vp]
lib.wkv7_slot_bytes.restype = _sz
lib.wkv7_slot_bytes.argtypes = [_vp]
lib.wkv7_pool_state_ptr.restype = _vp
lib.wkv7_pool_state_ptr.argtypes = [_vp]
lib.wkv7_pool_shape.restype = _i32
lib.wkv7_pool_shape.argtypes = [_vp, _pi32, _pi32, _pi32]
lib.wkv7_pool_device.restype = _i32
lib.wkv7_pool_device.argtypes = [_vp, _pi32]
lib.wkv7_pool_set_option.restype = _i32
lib.wkv7_pool_set_option.argtypes = [_vp, _i32, _i64]
lib.wkv7_slot_alloc.restype = _i32
lib.wkv7_slot_alloc.argtypes = [_vp, _i32, _pi32]
lib.wkv7_slot_free.restype = _i32
lib.wkv7_slot_free.argtypes = [_vp, _pi32, _i32]
lib.wkv7_forward.restype = _i32
lib.wkv7_forward.argtypes = [_vp, _pi32, _pi32, _i32, _i32, _vp, _vp, _vp,
                             _vp, _vp, _vp, _vp, _vp]
lib.wkv7_forward_noalloc.restype = _i32
lib.wkv7_forward_noalloc.argtypes = [_vp, _pi32, _pi32, _i32, _i32, _vp, _vp,
                                     _vp, _vp, _vp, _vp, _vp, _vp]
lib.wkv7_snapshot.restype = _i32
lib.wkv7_snapshot.argtypes = [_vp, _i32, _vp, _vp]
lib.wkv7_fork.restype = _i32
lib.wkv7_fork.argtypes = [_vp, _pi32, _pi32, _i32, _vp]
lib.wkv7_reset.restype = _i32
lib.wkv7_reset.argtypes = [_vp, _pi32, _i32, _vp]
lib.wkv7_hibernate.restype = _i32
lib.wkv7_hibernate.argtypes = [_vp, _pi32, _i32, _vp, _sz, _vp]
lib.wkv7_resume.restype = _i32
lib.wkv7_resume.argtypes = [_vp, _pi32, _i32, _vp, _sz, _vp]
lib.wkv7_plan_create.restype = _i32
lib.wkv7_plan_create.argtypes = [_vp, _pi32, _pi32, _i32, ctypes.POINTER(_vp)]
lib.wkv7_plan_tokens.restype = _i64
lib.wkv7_plan_tokens.argtypes = [_vp]
lib.wkv7_forward_plan.restype = _i32
lib.wkv7_forward_plan.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _vp, _vp]
lib.wkv7_plan_destroy.restype = _i32
lib.wkv7_plan_destroy.argtypes = [_vp]
lib.wkv7_migrate.restype = _i32
lib.wkv7_migrate.argtypes = [_vp, _pi32, _vp, _pi32, _i32, _vp]
lib.wkv7_image_header_init.restype = _i32
lib.wkv7_image_header_init.argtypes = [ctypes.POINTER(wkv7_image_header),
                                       _i32, _i32, _i32]
lib.wkv7_sessions_create.restype = _i32
lib.wkv7_sessions_create.argtypes = [_vp, _i32, _i32, _i32, ctypes.POINTER(_vp)]
lib.wkv7_sessions_destroy.restype = _i32
lib.wkv7_sessions_destroy.argtypes = [_vp]
lib.wkv7_session_begin.restype = _i32
lib.wkv7_session_begin.argtypes = [_vp, ctypes.POINTER(wkv7_turn_key), _pi32,
                                   _i64, _vp, _pi32,
                                   ctypes.POINTER(_i64), _pi32]
lib.wkv7_session_end.restype = _i32
lib.wkv7_session_end.argtypes = [_vp, _i32, ctypes.c_uint64, _pi32, _i64]
lib.wkv7_session_abort.restype = _i32
lib.wkv7_session_abort.argtypes = [_vp, _i32]
lib.wkv7_session_drop_chat.restype = _i32
lib.wkv7_session_drop_chat.argtypes = [_vp, ctypes.c_uint64, ctypes.c_uint64,
                                       ctypes.c_uint64]
lib.wkv7_sessions_stats.restype = _i32
lib.wkv7_sessions_stats.argtypes = [_vp, ctypes.POINTER(wkv7_session_stats)]
lib.wkv7_q8_quantize.restype = _i32
lib.wkv7_q8_quantize.argtypes = [_vp, _i32, _i64, _i64, _vp, _vp, _vp]
lib.wkv7_q8_matmul.restype = _i32
lib.wkv7_q8_matmul.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp]
lib.wkv7_q8_linear.restype = _i32
lib.wkv7_q8_linear.argtypes = [_vp, _vp, _i64, _i64, _vp, _i32, _i64, _vp, _vp,
                               _vp, _vp]
lib.wkv7_image_header_check.restype = _i32
lib.wkv7_image_header_check.argtypes = [ctypes.POINTER(wkv7_image_header),
                                        _i32, _i32]


def _check(status: int) -> None:
    if status != WKV7_OK:
        raise Wkv7Error(status, lib.wkv7_last_error().decode(errors="replace"))


def _ids(x) -> np.ndarray:
    """Host int32 array (contiguous) from a sequence or numpy array."""
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32).reshape(-1))


def _iptr(a: np.ndarray):
    return a.ctypes.data_as(_pi32) if a.size else None


def _dptr(t) -> Optional[int]:
    """Address of a tensor's storage (device or pinned host), or None."""
    if t is None:
        return None
    return int(t.data_ptr()) if t.numel() else None


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream) or None
    if isinstance(stream, int):
        return stream or None
    return int(stream.cuda_stream) or None


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return WKV7_F32
    if t.dtype == torch.bfloat16:
        return WKV7_BF16
    return -1  # the library reports WKV7_ERR_UNSUPPORTED


def _check_io(T_tot: Optional[int], H: Optional[int], dtype: Optional[int],
              ins, o, device: Optional[int] = None) -> None:
    """Argument checks the library cannot make on raw pointers, raised as
    ValueError before any call: r..b must be contiguous tensors of one dtype,
    o a contiguous float32 tensor, all on one GPU (the pool's, `device`,
    when given), each with at least T_tot * H * 64 elements (the rows the
    call reads or writes), and a dtype code given explicitly must match the
    inputs' element width. An unsupported dtype, a misaligned pointer or a
    NULL tensor is left to the library, which rejects it with its own
    status. T_tot/H/device None: not yet known (checked by the caller's
    second call, after it has queried the pool).
    """
    import torch
    named = list(zip(("r", "w", "k", "v", "a", "b"), ins)) + [("o", o)]
    present = [(n, t) for n, t in named if t is not None]
    for n, t in present:
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{n} must be a torch.Tensor, not {type(t)!r}")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    ins_present = [(n, t) for n, t in present if n != "o"]
    if ins_present:
        d0 = ins_present[0][1].dtype
        supported = (torch.float32, torch.bfloat16)
        if d0 in supported:
            for n, t in ins_present:
                if t.dtype != d0:
                    raise ValueError(f"r..b must share one dtype: {n} is "
                                     f"{t.dtype}, r is {d0}")
            code = WKV7_F32 if d0 == torch.float32 else WKV7_BF16
            if dtype is not None and dtype in (WKV7_F32, WKV7_BF16) and \
                    dtype != code:
                raise ValueError(f"dtype code {dtype} does not match the "
                                 f"inputs' {d0}")
    if o is not None and o.dtype != torch.float32:
        raise ValueError(f"o must be float32, not {o.dtype}")
    if T_tot is not None and H is not None:
        need = T_tot * H * 64
        for n, t in present:
            if t.numel() < need:
                raise ValueError(f"{n} has {t.numel()} elements; the call "
                                 f"needs [{T_tot}, {H}, 64] = {need}")
    devs = {(t.device.type, t.device.index) for _, t in present}
    for n, t in present:
        if t.device.type != "cuda":
            raise ValueError(f"{n} is on {t.device}, not on a GPU")
    if len(devs) > 1:
        raise ValueError("r..b and o must be on one GPU")
    if device is not None:
        for n, t in present:
            if t.device.index != device:
                raise ValueError(f"{n} is on {t.device}; the pool's memory is "
                                 f"on device {device}")


def wkv7_version() -> int:
    return int(lib.wkv7_version())


def wkv7_last_error() -> str:
    return lib.wkv7_last_error().decode(errors="replace")


def wkv7_pool_create(n_slots: int, H: int, N: int) -> int:
    handle = _vp()
    _check(lib.wkv7_pool_create(n_slots, H, N, ctypes.byref(handle)))
    return int(handle.value)


def wkv7_pool_destroy(pool: int) -> None:
    _check(lib.wkv7_pool_destroy(pool))


def wkv7_slot_bytes(pool: int) -> int:
    return int(lib.wkv7_slot_bytes(pool))


def wkv7_pool_state_ptr(pool: int) -> int:
    return int(lib.wkv7_pool_state_ptr(pool) or 0)


def wkv7_pool_shape(pool: int):
    n, h, d = _i32(), _i32(), _i32()
    _check(lib.wkv7_pool_shape(pool, ctypes.byref(n), ctypes.byref(h),
                               ctypes.byref(d)))
    return n.value, h.value, d.value


def wkv7_pool_device(pool: int) -> int:
    d = _i32()
    _check(lib.wkv7_pool_device(pool, ctypes.byref(d)))
    return d.value


def wkv7_pool_set_option(pool: int, opt: int, val: int) -> None:
    _check(lib.wkv7_pool_set_option(pool, opt, val))


def wkv7_slot_alloc(pool: int, n: int) -> np.ndarray:
    out = np.zeros(max(n, 0), dtype=np.int32)
    _check(lib.wkv7_slot_alloc(pool, n, _iptr(out)))
    return out


def wkv7_slot_free(pool: int, ids: Sequence[int]) -> None:
    a = _ids(ids)
    _check(lib.wkv7_slot_free(pool, _iptr(a), a.size))


def wkv7_forward(pool: int, slot_ids, cu_seqlens, r, w, k, v, a, b, o,
                 stream=None, dtype: Optional[int] = None) -> None:
    """o[T_tot, H, N] fp32 <- recurrence over the packed batch (in place)."""
    ids = _ids(slot_ids)
    cu = _ids(cu_seqlens)
    if cu.size != ids.size + 1:
        raise ValueError("cu_seqlens must have len(slot_ids) + 1 entries")
    _check_io(None, None, dtype, (r, w, k, v, a, b), o)
    _check_io(int(cu[-1]), wkv7_pool_shape(pool)[1], dtype,
              (r, w, k, v, a, b), o, wkv7_pool_device(pool))
    code = _dtype_code(r) if dtype is None else dtype
    _check(lib.wkv7_forward(pool, _iptr(ids), _iptr(cu), ids.size, code,
                            _dptr(r), _dptr(w), _dptr(k), _dptr(v), _dptr(a),
                            _dptr(b), _dptr(o), _stream(stream)))


def wkv7_forward_noalloc(pool: int, slot_ids, cu_seqlens, r, w, k, v, a, b,
                         o, stream=None, dtype: Optional[int] = None) -> None:
    """wkv7_forward with the kernels' scratch in the library's static array."""
    ids = _ids(slot_ids)
    cu = _ids(cu_seqlens)
    if cu.size != ids.size + 1:
        raise ValueError("cu_seqlens must have len(slot_ids) + 1 entries")
    _check_io(None, None, dtype, (r, w, k, v, a, b), o)
    _check_io(int(cu[-1]), wkv7_pool_shape(pool)[1], dtype,
              (r, w, k, v, a, b), o, wkv7_pool_device(pool))
    code = _dtype_code(r) if dtype is None else dtype
    _check(lib.wkv7_forward_noalloc(pool, _iptr(ids), _iptr(cu), ids.size,
                                    code, _dptr(r), _dptr(w), _dptr(k),
                                    _dptr(v), _dptr(a), _dptr(b), _dptr(o),
                                    _stream(stream)))


def wkv7_plan_create(pool: int, slot_ids, cu_seqlens) -> int:
    """Validate and upload a batch's metadata once; returns the plan handle."""
    ids = _ids(slot_ids)
    cu = _ids(cu_seqlens)
    if cu.size != ids.size + 1:
        raise ValueError("cu_seqlens must have len(slot_ids) + 1 entries")
    out = _vp()
    _check(lib.wkv7_plan_create(pool, _iptr(ids), _iptr(cu), ids.size,
                                ctypes.byref(out)))
    return out.value


def wkv7_plan_tokens(plan: int) -> int:
    return int(lib.wkv7_plan_tokens(plan))


def wkv7_forward_plan(pool: int, plan: int, r, w, k, v, a, b, o, stream=None,
                      dtype: Optional[int] = None) -> None:
    """wkv7_forward over a plan's batch: kernel launches only (capturable)."""
    _check_io(None, None, dtype, (r, w, k, v, a, b), o)
    if plan:
        _check_io(wkv7_plan_tokens(plan), wkv7_pool_shape(pool)[1], dtype,
                  (r, w, k, v, a, b), o, wkv7_pool_device(pool))
    code = _dtype_code(r) if dtype is None else dtype
    _check(lib.wkv7_forward_plan(pool, plan, code, _dptr(r), _dptr(w),
                                 _dptr(k), _dptr(v), _dptr(a), _dptr(b),
                                 _dptr(o), _stream(stream)))


def wkv7_plan_destroy(plan: int) -> None:
    _check(lib.wkv7_plan_destroy(plan))


def wkv7_migrate(src_pool: int, src_ids, dst_pool: int, dst_ids,
                 stream=None) -> None:
    s, d = _ids(src_ids), _ids(dst_ids)
    if s.size != d.size:
        raise ValueError("migrate: src_ids and dst_ids differ in length")
    _check(lib.wkv7_migrate(src_pool, _iptr(s), dst_pool, _iptr(d), s.size,
                            _stream(stream)))


def wkv7_image_header_init(H: int, N: int, n_slots: int) -> wkv7_image_header:
    hdr = wkv7_image_header()
    _check(lib.wkv7_image_header_init(ctypes.byref(hdr), H, N, n_slots))
    return hdr


def wkv7_image_header_check(hdr: wkv7_image_header, H: int, N: int) -> None:
    _check(lib.wkv7_image_header_check(ctypes.byref(hdr), H, N))


def wkv7_sessions_create(pool: Optional[int], dry_slots: int = 0,
                         host_images: int = 0, flags: int = 0) -> int:
    out = _vp()
    _check(lib.wkv7_sessions_create(pool, dry_slots, host_images, flags,
                                    ctypes.byref(out)))
    return out.value


def wkv7_sessions_destroy(s: int) -> None:
    _check(lib.wkv7_sessions_destroy(s))


def wkv7_session_begin(s: int, model: int, user: int, chat: int, parent: int,
                       tokens, stream=None):
    """Returns (slot, n_reuse, outcome)."""
    t = _ids(tokens)
    key = wkv7_turn_key(model, user, chat, parent)
    slot, reuse, oc = _i32(), _i64(), _i32()
    # NULL (the null stream) unless a stream is given: a host-only manager
    # must not touch the GPU
    hs = None if stream is None else _stream(stream)
    _check(lib.wkv7_session_begin(s, ctypes.byref(key), _iptr(t), t.size, hs,
                                  ctypes.byref(slot), ctypes.byref(reuse),
                                  ctypes.byref(oc)))
    return slot.value, reuse.value, oc.value


def wkv7_session_end(s: int, slot: int, message: int, tokens) -> None:
    t = _ids(tokens)
    _check(lib.wkv7_session_end(s, slot, message, _iptr(t), t.size))


def wkv7_session_abort(s: int, slot: int) -> None:
    _check(lib.wkv7_session_abort(s, slot))


def wkv7_session_drop_chat(s: int, model: int, user: int, chat: int) -> None:
    _check(lib.wkv7_session_drop_chat(s, model, user, chat))


def wkv7_sessions_stats(s: int) -> dict:
    out = wkv7_session_stats()
    _check(lib.wkv7_sessions_stats(s, ctypes.byref(out)))
    return {n: getattr(out, n) for n, _ in wkv7_session_stats._fields_}


def wkv7_q8_quantize(x, q, scale, stream=None, dtype: Optional[int] = None):
    """Per-row INT8 codes of the 2-D device tensor x into q (int8, same
    shape) and scale (float32 [rows])."""
    rows, cols = x.shape
    code = _dtype_code(x) if dtype is None else dtype
    _check(lib.wkv7_q8_quantize(_dptr(x), code, rows, cols, _dptr(q),
                                _dptr(scale), _stream(stream)))


def wkv7_q8_matmul(wq, w_scale, xq, x_scale, y, stream=None) -> None:
    """y[B, out] = INT8 product of codes wq [out, in] and xq [B, in]."""
    out, inn = wq.shape
    B = xq.shape[0]
    _check(lib.wkv7_q8_matmul(_dptr(wq), _dptr(w_scale), out, inn, _dptr(xq),
                              _dptr(x_scale), B, _dptr(y), _stream(stream)))


def wkv7_q8_linear(wq, w_scale, x, xq, x_scale, y, stream=None) -> None:
    """Quantize x [B, in] (float32 or bfloat16) into xq, x_scale and
    y[B, out] = INT8 product of wq [out, in] with them."""
    out, inn = wq.shape
    B = x.shape[0]
    _check(lib.wkv7_q8_linear(_dptr(wq), _dptr(w_scale), out, inn, _dptr(x),
                              _dtype_code(x),
                              B, _dptr(xq), _dptr(x_scale), _dptr(y),
                              _stream(stream)))


def wkv7_snapshot(pool: int, slot: int, dst, stream=None) -> None:
    _check(lib.wkv7_snapshot(pool, slot, _dptr(dst), _stream(stream)))


def wkv7_fork(pool: int, src, dst, stream=None) -> None:
    s, d = _ids(src), _ids(dst)
    if s.size != d.size:
        raise ValueError("fork: src and dst differ in length")
    _check(lib.wkv7_fork(pool, _iptr(s), _iptr(d), s.size, _stream(stream)))


def wkv7_reset(pool: int, ids, stream=None) -> None:
    a = _ids(ids)
    _check(lib.wkv7_reset(pool, _iptr(a), a.size, _stream(stream)))


def wkv7_hibernate(pool: int, ids, host_dst, stream=None) -> None:
    """host_dst: pinned CPU tensor of at least len(ids) * slot_bytes bytes."""
    a = _ids(ids)
    nbytes = host_dst.numel() * host_dst.element_size()
    _check(lib.wkv7_hibernate(pool, _iptr(a), a.size, _dptr(host_dst), nbytes,
                              _stream(stream)))


def wkv7_resume(pool: int, ids, src, stream=None) -> None:
    """src: pinned CPU tensor or device tensor of slot images."""
    a = _ids(ids)
    nbytes = src.numel() * src.element_size()
    _check(lib.wkv7_resume(pool, _iptr(a), a.size, _dptr(src), nbytes,
                           _stream(stream)))


def pool_state(pool: int):
    """The pool's state as a torch float32 tensor view [n_slots, H, N, N].

    A zero-copy view of the library-owned device buffer (valid until the
    pool is destroyed); for inspection and set-up by tests and benchmarks.
    """
    import torch
    n, h, d = wkv7_pool_shape(pool)
    ptr = wkv7_pool_state_ptr(pool)
    return _device_view(ptr, (n, h, d, d), torch.float32)


def _device_view(ptr: int, shape, dtype):
    import torch

    class _Iface:
        __cuda_array_interface__ = {
            "shape": tuple(shape), "typestr": "<f4", "data": (ptr, False),
            "version": 2, "strides": None,
        }
    return torch.as_tensor(_Iface(), device="cuda")
