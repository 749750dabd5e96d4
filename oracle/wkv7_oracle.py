"""Float64 CPU oracle of the RWKV-7 WKV recurrence over state slots.

TEST INFRASTRUCTURE. Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module. The product path never
calls it, and it shares no code with the HIP kernels or their host library.

What it computes (page "RWKV-X Architecture", section "WKV-7 Kernel
(Generalized Delta Rule)"): per head, a [head_size, head_size] state is
updated once per timestep by a decay, a delta-rule term, and a key-value
outer product, and the timestep's output is read from the state.

The page's four pseudocode lines do not type-check as printed. The reading
taken here is the product form of the generalized delta rule

    S_t = S_{t-1} (diag(w_t) + a_t b_t^T) + v_t k_t^T,     o_t = S_t r_t,

with S[i][j]: i indexes the value (row), j the key (column). Written out per
element, for one head and one timestep:

    sa[i]   = sum_j S_{t-1}[i][j] * a_t[j]          (uses the state before
                                                     this step's decay)
    S_t[i][j] = S_{t-1}[i][j] * w_t[j] + sa[i] * b_t[j] + v_t[i] * k_t[j]
    o_t[i]  = sum_j S_t[i][j] * r_t[j]              (uses the updated state)

The state has the same size for every sequence length (the same section
says so). Heads, sequences and slots are independent. Nothing is clamped: w is used exactly as given.

Everything is float64; inputs are the exact dtype-rounded values the device
receives, upcast. Loops run over timesteps in Python and are vectorised over
any leading batch dimensions (heads, sequences), which does not change the
per-element arithmetic.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence, Tuple

import numpy as np

_NAMES = ("r", "w", "k", "v", "a", "b")


def wkv7_step(S: np.ndarray, r: np.ndarray, w: np.ndarray, k: np.ndarray,
              v: np.ndarray, a: np.ndarray, b: np.ndarray
              ) -> Tuple[np.ndarray, np.ndarray]:
    """One timestep for a batch of heads.

    S: [..., N, N] state before the step (not modified).
    r, w, k, v, a, b: [..., N].
    Returns (o [..., N], S_next [..., N, N]).
    """
    # delta-rule term: reads the state before this step's decay
    sa = (S * a[..., None, :]).sum(axis=-1)
    S_next = (S * w[..., None, :]
              + sa[..., :, None] * b[..., None, :]
              + v[..., :, None] * k[..., None, :])
    # readout from the updated state
    o = (S_next * r[..., None, :]).sum(axis=-1)
    return o, S_next


def wkv7_sequence(S0: np.ndarray, r: np.ndarray, w: np.ndarray,
                  k: np.ndarray, v: np.ndarray, a: np.ndarray, b: np.ndarray
                  ) -> Tuple[np.ndarray, np.ndarray]:
    """Run T timesteps from S0.

    S0: [..., N, N]; r..b: [T, ..., N] (time first).
    Returns (o [T, ..., N], S_T [..., N, N]), both float64.
    """
    S = np.array(S0, dtype=np.float64, copy=True)
    T = r.shape[0]
    o = np.empty(r.shape, dtype=np.float64)
    for t in range(T):
        o[t], S = wkv7_step(S, r[t], w[t], k[t], v[t], a[t], b[t])
    return o, S


def wkv7_forward(states: Dict[int, np.ndarray], slot_ids: Sequence[int],
                 cu_seqlens: Sequence[int], inputs: Dict[str, np.ndarray],
                 H: int, N: int) -> Tuple[np.ndarray, Dict[int, np.ndarray]]:
    """Packed batch over slots: the semantics of one pool forward call.

    states: slot id -> [H, N, N] state (slots absent from the dict are zero).
    slot_ids[s], tokens cu_seqlens[s] : cu_seqlens[s+1] of `inputs[name]`
    ([T_tot, H, N]) form sequence s. Each sequence runs from its slot's state;
    the final state is returned for every slot named. A zero-length sequence
    leaves its slot unchanged.
    Returns (o [T_tot, H, N], {slot id: final state}).
    """
    ids = [int(x) for x in slot_ids]
    if len(set(ids)) != len(ids):
        raise ValueError("a slot may appear once per call")
    x = {n: np.asarray(inputs[n], dtype=np.float64) for n in _NAMES}
    T_tot = int(cu_seqlens[-1])
    o = np.zeros((T_tot, H, N), dtype=np.float64)
    out_states = {}
    for s, slot in enumerate(ids):
        lo, hi = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        S0 = states.get(slot)
        if S0 is None:
            S0 = np.zeros((H, N, N), dtype=np.float64)
        seq = {n: x[n][lo:hi] for n in _NAMES}
        o_s, S_T = wkv7_sequence(S0, **seq)
        o[lo:hi] = o_s
        out_states[slot] = S_T
    return o, out_states


def wkv7_decode_batch(S0: np.ndarray, inputs: Dict[str, np.ndarray]
                      ) -> Tuple[np.ndarray, np.ndarray]:
    """One token for each of B slots at once.

    S0: [B, H, N, N]; inputs[name]: [B, H, N] (token b belongs to slot b).
    Returns (o [B, H, N], S_1 [B, H, N, N]).
    """
    x = {n: np.asarray(inputs[n], dtype=np.float64) for n in _NAMES}
    return wkv7_step(np.asarray(S0, dtype=np.float64), **x)


def rel_max_err(got: np.ndarray, ref: np.ndarray,
                scale: Optional[np.ndarray] = None) -> float:
    """max |got - ref| / rms(scale or ref), in float64 (the parity metric)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return 0.0
    sc = ref if scale is None else np.asarray(scale, dtype=np.float64)
    rms = float(np.sqrt(np.mean(sc * sc)))
    if rms == 0.0:
        return float(np.max(np.abs(got - ref)))
    return float(np.max(np.abs(got - ref)) / rms)
