"""Python side of the plain-C float64 oracle (oracle/wkv7_ref.c).

TEST INFRASTRUCTURE. Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module. The product path never
calls it; it shares no code with the HIP kernels or their host library.

The C library computes the same per-element recurrence as
oracle/wkv7_oracle.py (page "RWKV-X Architecture", section "WKV-7 Kernel
(Generalized Delta Rule)", product form
S_t = S_{t-1}(diag(w_t) + a_t b_t^T) + v_t k_t^T, o_t = S_t r_t), token by
token in float64, and is pinned by the same pins. It exists so that the
full-size workloads (millions of token-heads) can be compared element by
element: its loops keep one head's state in cache, and independent heads run
on worker threads (ctypes releases the interpreter lock during the call).

Inputs may be float64 or float32 arrays, or bfloat16 torch tensors; the C
side widens each value exactly, so no float64 copy of a large input is made.
"""
from __future__ import annotations

import concurrent.futures as cf
import ctypes
import os
import subprocess
import threading
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "wkv7_ref.c")
LIB = os.path.join(HERE, "libwkv7ref.so")
NAMES = ("r", "w", "k", "v", "a", "b")
CFLAGS = ["-O3", "-fPIC", "-shared", "-std=c99", "-ffp-contract=off",
          "-fno-fast-math"]

_F64, _F32, _BF16 = 0, 1, 2
_lib = None
_lock = threading.Lock()


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the C oracle with gcc (a few hundred milliseconds)."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, src, "-o", tmp], check=True,
                   capture_output=True, text=True)
    os.replace(tmp, out)
    return out


def load_lib(path: str) -> ctypes.CDLL:
    lib = ctypes.CDLL(path)
    fn = lib.wkv7_ref_run
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                   ctypes.c_int, ctypes.POINTER(ctypes.c_void_p),
                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                   ctypes.c_int64]
    return lib


def lib() -> ctypes.CDLL:
    """The built oracle library (compiled here first if it is missing)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB) or \
                    os.path.getmtime(LIB) < os.path.getmtime(SRC):
                build()
            _lib = load_lib(LIB)
    return _lib


MAX_THREADS = 16   # the host share one GPU's jobs may use


def default_threads() -> int:
    """Worker threads: the process's CPU set, at most MAX_THREADS."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, MAX_THREADS))


def _as_input(x):
    """(keep-alive object, pointer, dtype code, shape) for one input array."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach()
            if x.device.type != "cpu":
                x = x.cpu()
            x = x.contiguous()
            if x.dtype == torch.bfloat16:
                return x, x.data_ptr(), _BF16, tuple(x.shape)
            if x.dtype == torch.float32:
                return x, x.data_ptr(), _F32, tuple(x.shape)
            x = x.to(torch.float64).numpy()
    except ImportError:
        pass
    a = np.asarray(x)
    if a.dtype == np.float32:
        a = np.ascontiguousarray(a)
        return a, a.ctypes.data, _F32, a.shape
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data, _F64, a.shape


def run_heads(S: np.ndarray, inputs: Dict[str, object], T: int,
              n_heads: int, N: int, threads: Optional[int] = None,
              fn=None) -> np.ndarray:
    """The recurrence over T tokens for n_heads independent heads.

    S: float64 [n_heads, N, N] (C-contiguous), updated in place to the final
    states. inputs[name]: [T, n_heads, N] (any leading shape with that many
    elements), all of one dtype. Returns o: float64 [T, n_heads, N].
    """
    assert S.dtype == np.float64 and S.flags.c_contiguous
    assert S.size == n_heads * N * N
    held, ptrs, dt = [], [], None
    for n in NAMES:
        keep, p, d, shape = _as_input(inputs[n])
        if int(np.prod(shape)) != T * n_heads * N:
            raise ValueError(f"input {n}: shape {shape} is not "
                             f"[{T}, {n_heads}, {N}]")
        if dt is not None and d != dt:
            raise ValueError("inputs must share one dtype")
        dt = d
        held.append(keep)
        ptrs.append(p)
    o = np.empty((T, n_heads, N), dtype=np.float64)
    arr = (ctypes.c_void_p * 6)(*ptrs)
    call = fn if fn is not None else lib().wkv7_ref_run
    nt = threads or default_threads()
    parts = min(nt, n_heads) if T * n_heads > 64 else 1
    bounds = [n_heads * i // parts for i in range(parts + 1)]

    def work(i):
        rc = call(T, n_heads, N, dt, arr, S.ctypes.data, o.ctypes.data,
                  bounds[i], bounds[i + 1])
        if rc != 0:
            raise ValueError("wkv7_ref_run rejected its arguments")

    if parts == 1:
        work(0)
    else:
        with cf.ThreadPoolExecutor(max_workers=parts) as ex:
            list(ex.map(work, range(parts)))
    del held
    return o


def sequence(S0, r, w, k, v, a, b, threads: Optional[int] = 1, fn=None
             ) -> Tuple[np.ndarray, np.ndarray]:
    """Same signature and result as oracle.wkv7_oracle.wkv7_sequence.

    S0: [..., N, N]; r..b: [T, ..., N]. Returns (o [T, ..., N], S_T).
    """
    S0 = np.asarray(S0, dtype=np.float64)
    N = S0.shape[-1]
    lead = S0.shape[:-2]
    n_heads = int(np.prod(lead)) if lead else 1
    x = {"r": r, "w": w, "k": k, "v": v, "a": a, "b": b}
    T = int(r.shape[0]) if hasattr(r, "shape") else len(r)
    S = np.array(S0, dtype=np.float64, copy=True).reshape(n_heads, N, N)
    S = np.ascontiguousarray(S)
    o = run_heads(S, x, T, n_heads, N, threads=threads, fn=fn)
    return o.reshape((T,) + lead + (N,)), S.reshape(lead + (N, N))


def forward(states: Dict[int, np.ndarray], slot_ids: Sequence[int],
            cu_seqlens: Sequence[int], inputs: Dict[str, object], H: int,
            N: int, threads: Optional[int] = None
            ) -> Tuple[np.ndarray, Dict[int, np.ndarray]]:
    """Same contract as oracle.wkv7_oracle.wkv7_forward (packed batch)."""
    ids = [int(x) for x in slot_ids]
    if len(set(ids)) != len(ids):
        raise ValueError("a slot may appear once per call")
    T_tot = int(cu_seqlens[-1])
    o = np.zeros((T_tot, H, N), dtype=np.float64)
    out = {}
    for s, slot in enumerate(ids):
        lo, hi = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        S0 = states.get(slot)
        S = (np.zeros((H, N, N)) if S0 is None
             else np.array(S0, dtype=np.float64, copy=True))
        S = np.ascontiguousarray(S.reshape(H, N, N))
        if hi > lo:
            o[lo:hi] = run_heads(S, {n: inputs[n][lo:hi] for n in NAMES},
                                 hi - lo, H, N, threads=threads)
        out[slot] = S
    return o, out
