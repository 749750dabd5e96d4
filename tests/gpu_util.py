"""Helpers for the GPU tests: move states in and out of a pool through the
C ABI, and compare against the float64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from linear_attention_rnn_amd import wkv7 as W
from oracle import rel_max_err
from wkv7_inputs import NAMES, as_f64

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(batch):
    return {n: batch.inputs[n].to(DEV).contiguous() for n in NAMES}


def set_states(pool, ids, states_cpu):
    """Write fp32 states [n, H, N, N] into slots `ids` (resume from device)."""
    if len(ids) == 0:
        return
    src = states_cpu.to(DEV).contiguous()
    W.wkv7_resume(pool, ids, src)
    torch.cuda.synchronize()


def get_states(pool, ids):
    """Read slots `ids` as float32 [n, H, N, N] (CPU) via hibernate."""
    n, H, N = W.wkv7_pool_shape(pool)
    out = torch.empty((len(ids), H, N, N), dtype=torch.float32,
                      pin_memory=True)
    if len(ids):
        W.wkv7_hibernate(pool, ids, out)
    torch.cuda.synchronize()
    return out.clone()


def run_forward(pool, batch, stream=None):
    x = to_dev(batch)
    o = torch.full((batch.T_tot, batch.H, batch.N), float("nan"),
                   dtype=torch.float32, device=DEV)
    W.wkv7_forward(pool, batch.slot_ids, batch.cu_seqlens, x["r"], x["w"],
                   x["k"], x["v"], x["a"], x["b"], o, stream=stream)
    torch.cuda.synchronize()
    return o.cpu()


def rel_err(got, ref):
    """The parity metric, max |got - ref| / rms(ref) (oracle.rel_max_err)."""
    return rel_max_err(got, ref)


def tol_for(dtype):
    return 1e-3 if dtype == "f32" else 2e-2
