"""Seeded synthetic inputs for the WKV-7 state-slot path.

This module is shared by the float64 oracle and the HIP path. It only draws
random numbers and rounds them to the dtype the device receives; it holds none
of the recurrence's arithmetic.

Input recipe (the distributions the workloads are drawn from):

* r, k, v ~ N(0, 1) per channel;
* w = exp(-exp(x)) with x ~ N(-0.6, 0.5) (second parameter = standard
  deviation), so w lies in (0, 1];
* kk = z / ||z||_2 with z ~ N(0, I_N) drawn per (token, head), independently
  of k;
* a = -kk;  b = kk * alpha with alpha = sigmoid(N(0, 1)) per channel;
* initial states: zero for fresh requests, N(0, 0.1) for resident ones.

Every array is drawn in float64 and rounded once, round-to-nearest-even, to
the dtype the device receives (bf16 through torch on the CPU, or fp32). The
oracle consumes exactly those rounded values, upcast back to float64.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

NAMES = ("r", "w", "k", "v", "a", "b")

F32 = "f32"
BF16 = "bf16"


def _torch_dtype(dtype: str) -> torch.dtype:
    if dtype == F32:
        return torch.float32
    if dtype == BF16:
        return torch.bfloat16
    raise ValueError(f"unknown dtype {dtype!r}")


def round_to(x64: np.ndarray, dtype: str) -> torch.Tensor:
    """Round a float64 array once (RNE) to `dtype`; returns a CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(x64)).to(_torch_dtype(dtype))


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a CPU or device tensor (bf16/fp32 upcast exactly)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def draw_tokens64(rng: np.random.Generator, T: int, H: int, N: int,
                  alpha_scalar: bool = False,
                  w_override: Optional[float] = None) -> Dict[str, np.ndarray]:
    """float64 draws of r,w,k,v,a,b with shape [T, H, N] (before rounding).

    `alpha_scalar` draws one alpha per (token, head) instead of per channel.
    """
    shape = (T, H, N)
    r = rng.standard_normal(shape)
    k = rng.standard_normal(shape)
    v = rng.standard_normal(shape)
    x = rng.normal(-0.6, 0.5, size=shape)
    w = np.exp(-np.exp(x))
    if w_override is not None:
        w = np.full(shape, float(w_override))
    z = rng.standard_normal(shape)
    nrm = np.sqrt((z * z).sum(axis=-1, keepdims=True))
    kk = z / nrm
    if alpha_scalar:
        alpha = _sigmoid(rng.standard_normal((T, H, 1)))
    else:
        alpha = _sigmoid(rng.standard_normal(shape))
    return {"r": r, "w": w, "k": k, "v": v, "a": -kk, "b": kk * alpha}


@dataclasses.dataclass
class Batch:
    """One packed call: tokens of all sequences concatenated along dim 0."""
    dtype: str
    H: int
    N: int
    slot_ids: np.ndarray            # int32 [n_seq]
    cu_seqlens: np.ndarray          # int32 [n_seq + 1]
    inputs: Dict[str, torch.Tensor]  # CPU tensors [T_tot, H, N] in `dtype`

    @property
    def T_tot(self) -> int:
        return int(self.cu_seqlens[-1])

    def inputs64(self) -> Dict[str, np.ndarray]:
        return {n: as_f64(self.inputs[n]) for n in NAMES}


def make_batch(rng: np.random.Generator, slot_ids: Sequence[int],
               lengths: Sequence[int], H: int, N: int, dtype: str,
               **draw_kw) -> Batch:
    lengths = [int(x) for x in lengths]
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    raw = draw_tokens64(rng, T, H, N, **draw_kw)
    inputs = {n: round_to(raw[n], dtype) for n in NAMES}
    return Batch(dtype, H, N, np.asarray(slot_ids, dtype=np.int32), cu, inputs)


def draw_states(rng: np.random.Generator, n: int, H: int, N: int,
                std: float = 0.1) -> torch.Tensor:
    """fp32 states N(0, std) with shape [n, H, N, N] (CPU)."""
    return round_to(rng.normal(0.0, std, size=(n, H, N, N)), F32)


# --------------------------------------------------------------------------
# The five workloads. Each returns plain data; nothing here touches a device.
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    n_slots: int
    H: int
    N: int
    dtype: str
    batch: Batch
    init_ids: np.ndarray             # slots given a non-zero initial state
    init_states: Optional[torch.Tensor]  # [len(init_ids), H, N, N] fp32


def cfg_small(seed: int = 0) -> Workload:
    """One layer, H=2, N=64, one sequence of T=64, fp32 inputs, zero state."""
    rng = np.random.default_rng(seed)
    b = make_batch(rng, [0], [64], 2, 64, F32)
    return Workload("small_h2_t64_f32", 1, 2, 64, F32, b,
                    np.zeros(0, np.int32), None)


def cfg_decode(seed: int = 1, step: int = 0, n_slots: int = 1024,
               n_active: int = 256, H: int = 32, N: int = 64) -> Workload:
    """Decode step: 256 active ids of a 1024-slot pool, H=32, bf16 inputs.

    The active set (a random subset in random order) and the initial states
    depend only on `seed`; each `step` draws fresh token inputs.
    """
    rng = np.random.default_rng(seed)
    ids = rng.permutation(n_slots)[:n_active].astype(np.int32)
    states = draw_states(rng, n_active, H, N)
    step_rng = np.random.default_rng([seed, 1000 + step])
    b = make_batch(step_rng, ids, [1] * n_active, H, N, BF16)
    return Workload(f"decode_b{n_active}_h{H}_pool{n_slots}_bf16", n_slots, H,
                    N, BF16, b, ids, states)


def decode_step_inputs(seed: int, step: int, ids: np.ndarray, H: int,
                       N: int) -> Batch:
    step_rng = np.random.default_rng([seed, 1000 + step])
    return make_batch(step_rng, ids, [1] * len(ids), H, N, BF16)


def cfg_prefill(seed: int = 2, n_seq: int = 8, T: int = 4096, H: int = 32,
                N: int = 64, dtype: str = BF16) -> Workload:
    """Prefill: 8 fresh sequences of T=4096, H=32, zero state; bf16 inputs
    (the workload) or fp32 inputs of the same recipe."""
    rng = np.random.default_rng(seed)
    ids = np.arange(n_seq, dtype=np.int32)
    b = make_batch(rng, ids, [T] * n_seq, H, N, dtype)
    return Workload(f"prefill_b{n_seq}_t{T}_h{H}_{dtype}", n_seq, H, N, dtype,
                    b, np.zeros(0, np.int32), None)


@dataclasses.dataclass
class MixedLayer:
    batch: Batch
    decode_ids: np.ndarray
    prefill_ids: np.ndarray
    init_states: torch.Tensor        # decode slots' initial states


def cfg_mixed_layers(seed: int = 3, n_layers: int = 12, n_slots: int = 128,
                     H: int = 12, N: int = 64, n_decode: int = 64,
                     prefill_lens: Sequence[int] = (512, 1024, 2048, 2048),
                     shuffle: bool = False) -> List[MixedLayer]:
    """RWKV-X-0.2B-shaped stack: per layer 64 decode slots + 4 ragged prefills.

    Layers are independent recurrences (one pool per layer); every layer
    draws its own inputs. Decode entries come first in `cu_seqlens` unless
    `shuffle`.
    """
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_slots).astype(np.int32)
    dec_ids = perm[:n_decode]
    pre_ids = perm[n_decode:n_decode + len(prefill_lens)]
    layers = []
    for _ in range(n_layers):
        ids = np.concatenate([dec_ids, pre_ids])
        lens = [1] * n_decode + list(prefill_lens)
        if shuffle:
            order = rng.permutation(len(ids))
            ids = ids[order]
            lens = [lens[i] for i in order]
        states = draw_states(rng, n_decode, H, N)
        b = make_batch(rng, ids, lens, H, N, BF16)
        layers.append(MixedLayer(b, dec_ids.copy(), pre_ids.copy(), states))
    return layers


def cfg_large_pool(seed: int = 4, n_slots: int = 4096, H: int = 64,
                   N: int = 64, n_decode: int = 1024, n_prefill: int = 32,
                   min_len: int = 128, max_len: int = 8192):
    """Large pool: H=64, 4096 slots; 1024 decode ids plus 32 ragged prefills.

    Returns (decode Batch, decode initial states, prefill Batch). Decode and
    prefill ids are disjoint; prefill lengths are integer-uniform in
    [min_len, max_len] inclusive.
    """
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_slots).astype(np.int32)
    dec_ids = perm[:n_decode]
    pre_ids = perm[n_decode:n_decode + n_prefill]
    states = draw_states(rng, n_decode, H, N)
    dec = make_batch(rng, dec_ids, [1] * n_decode, H, N, BF16)
    lens = rng.integers(min_len, max_len + 1, size=n_prefill)
    pre = make_batch(rng, pre_ids, lens, H, N, BF16)
    return dec, states, pre


def draw_tokens_device(gen: "torch.Generator", T: int, H: int, N: int,
                       dtype: str, device) -> Dict[str, torch.Tensor]:
    """The same recipe drawn with a seeded torch generator on `device`.

    Used where many steps of fresh inputs are needed on the device (the
    benchmark); parity tests use the float64 draws above.
    """
    shape = (T, H, N)
    f = dict(dtype=torch.float32, device=device, generator=gen)
    r = torch.randn(shape, **f)
    k = torch.randn(shape, **f)
    v = torch.randn(shape, **f)
    x = torch.randn(shape, **f) * 0.5 - 0.6
    w = torch.exp(-torch.exp(x))
    z = torch.randn(shape, **f)
    kk = z / torch.linalg.vector_norm(z, dim=-1, keepdim=True)
    alpha = torch.sigmoid(torch.randn(shape, **f))
    td = _torch_dtype(dtype)
    out = {"r": r, "w": w, "k": k, "v": v, "a": -kk, "b": kk * alpha}
    return {n: out[n].to(td).contiguous() for n in NAMES}
