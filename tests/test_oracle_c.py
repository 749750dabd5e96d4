"""The plain-C float64 oracle (oracle/wkv7_ref.c) against the same pins as
the numpy oracle, plus planted mistakes in copies of its source (CPU only).

The C oracle is what the full-size GPU parity tests compare against, so it
is pinned on its own, not only through agreement with the numpy oracle.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest
import torch

from oracle import wkv7_cref as C
from oracle import wkv7_sequence, wkv7_forward
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_c_oracle_pin(pin):
    pin(C.sequence)


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
def test_c_oracle_agrees_with_numpy_oracle(dtype):
    """Same per-element arithmetic in float64: the two agree to rounding of
    the sums' order (numpy sums pairwise, the C loops left to right)."""
    rng = np.random.default_rng(30)
    T, H, N = 37, 3, 64
    x = P._draw(rng, T, N, H=H)
    if dtype == "f32":
        xin = {n: x[n].astype(np.float32) for n in P.NAMES}
        x64 = {n: xin[n].astype(np.float64) for n in P.NAMES}
    elif dtype == "bf16":
        xin = {n: torch.from_numpy(x[n]).to(torch.bfloat16) for n in P.NAMES}
        x64 = {n: xin[n].to(torch.float64).numpy() for n in P.NAMES}
    else:
        xin, x64 = x, x
    S0 = rng.standard_normal((H, N, N)) * 0.1
    o_ref, S_ref = wkv7_sequence(S0, **x64)
    o, S = C.sequence(S0, **xin, threads=2)
    assert P._rel(o, o_ref) < 1e-13 and P._rel(S, S_ref) < 1e-13


def test_c_oracle_threads_do_not_change_bits():
    rng = np.random.default_rng(31)
    T, H, N = 20, 7, 64
    x = P._draw(rng, T, N, H=H)
    S0 = rng.standard_normal((H, N, N))
    o1, S1 = C.sequence(S0, **x, threads=1)
    o4, S4 = C.sequence(S0, **x, threads=4)
    assert np.array_equal(o1, o4) and np.array_equal(S1, S4)


def test_c_forward_packs_sequences_and_slots():
    rng = np.random.default_rng(32)
    H, N = 2, 64
    lens = [3, 0, 5, 1]
    ids = [7, 2, 4, 0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    x = P._draw(rng, T, N, H=H)
    states = {7: rng.standard_normal((H, N, N)),
              0: rng.standard_normal((H, N, N))}
    o, out = C.forward(states, ids, cu, x, H, N, threads=2)
    o_ref, out_ref = wkv7_forward(states, ids, cu, x, H, N)
    assert P._rel(o, o_ref) < 1e-13
    for s in ids:
        assert P._rel(out[s], out_ref[s]) < 1e-13 or not np.any(out_ref[s])
    assert np.array_equal(out[2], np.zeros((H, N, N)))
    with pytest.raises(ValueError):
        C.forward(states, [1, 1], [0, 1, 2], {n: x[n][:2] for n in P.NAMES},
                  H, N)


def test_c_oracle_rejects_bad_arguments():
    lib = C.lib()
    S = np.zeros((1, 4, 4))
    o = np.zeros((1, 1, 4))
    x = np.zeros(4)
    arr = (ctypes.c_void_p * 6)(*([x.ctypes.data] * 6))
    f = lib.wkv7_ref_run
    assert f(1, 1, 4, 0, arr, S.ctypes.data, o.ctypes.data, 0, 1) == 0
    assert f(1, 1, 4, 7, arr, S.ctypes.data, o.ctypes.data, 0, 1) == -1
    assert f(1, 1, 0, 0, arr, S.ctypes.data, o.ctypes.data, 0, 1) == -1
    assert f(1, 1, 4, 0, arr, S.ctypes.data, o.ctypes.data, 0, 2) == -1
    assert f(-1, 1, 4, 0, arr, S.ctypes.data, o.ctypes.data, 0, 1) == -1
    nul = (ctypes.c_void_p * 6)(*([None] * 6))
    assert f(1, 1, 4, 0, nul, S.ctypes.data, o.ctypes.data, 0, 1) == -1


# Planted mistakes: each is one plausible slip in the C source, compiled into
# a library of its own; every one must fail at least one pin.
C_MUTANTS = {
    "drop_delta_term": (" + sa * b[j] ", " "),
    "delta_sign": (" + sa * b[j] ", " - sa * b[j] "),
    "decay_before_delta": ("sa += row[j] * a[j];",
                           "sa += row[j] * w[j] * a[j];"),
    "k_in_place_of_b": ("sa * b[j]", "sa * k[j]"),
    "a_b_swapped": ("sa += row[j] * a[j];", "sa += row[j] * b[j];"),
    "sa_transposed": ("sa += row[j] * a[j];", "sa += Sh[j * N + i] * a[j];"),
    "outer_product_transposed": ("v[i] * k[j]", "v[j] * k[i]"),
    "decay_on_rows": ("row[j] * w[j]", "row[j] * w[i]"),
    "readout_transposed": ("acc += row[j] * r[j];",
                           "acc += Sh[j * N + i] * r[j];"),
    "readout_before_update": ("acc += row[j] * r[j];",
                              "acc += (row[j] - v[i] * k[j] - sa * b[j]) "
                              "/ w[j] * r[j];"),
    "stale_decay_index": ("w[c] = widen(in[1], dtype, base + c);",
                          "w[c] = widen(in[1], dtype, (t > 0 ? base - "
                          "n_heads * N : base) + c);"),
    "heads_time_major_swapped": ("int64_t base = (t * n_heads + h) * N;",
                                 "int64_t base = (h * T + t) * N;"),
    "bf16_low_half": ("(uint32_t)((const uint16_t *)p)[idx] << 16",
                      "(uint32_t)((const uint16_t *)p)[idx]"),
}


def _build_mutant(name, tmp_path):
    with open(C.SRC) as f:
        src = f.read()
    old, new = C_MUTANTS[name]
    assert old in src, f"mutation anchor for {name} not found"
    path = os.path.join(tmp_path, f"mut_{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new, 1))
    lib = os.path.join(tmp_path, f"libmut_{name}.so")
    subprocess.run(["gcc", *C.CFLAGS, path, "-o", lib], check=True,
                   capture_output=True)
    return C.load_lib(lib)


def _bf16_pin(seq):
    """bf16 inputs are widened exactly: the same values as float64 inputs."""
    rng = np.random.default_rng(33)
    x = P._draw(rng, 5, 8, H=2)
    xb = {n: torch.from_numpy(x[n]).to(torch.bfloat16) for n in P.NAMES}
    x64 = {n: xb[n].to(torch.float64).numpy() for n in P.NAMES}
    S0 = rng.standard_normal((2, 8, 8))
    o1, S1 = seq(S0, **xb)
    o2, S2 = seq(S0, **x64)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2), "bf16 widening"


@pytest.mark.parametrize("name", sorted(C_MUTANTS))
def test_c_mutant_is_caught(name, tmp_path):
    lib = _build_mutant(name, str(tmp_path))

    def seq(S0, r, w, k, v, a, b):
        return C.sequence(S0, r, w, k, v, a, b, fn=lib.wkv7_ref_run)

    failures = []
    for pin in P.ALL_PINS + [_bf16_pin]:
        try:
            with np.errstate(all="ignore"):
                pin(seq)
        except (AssertionError, FloatingPointError, ValueError,
                np.linalg.LinAlgError):
            failures.append(pin.__name__)
    assert failures, f"C mutant {name} passed every pin"
