"""Pins for the float64 oracle: each checks it against something other than
itself (closed forms, brute-force matrix products, exact rationals, a
hand-worked example, invariants, and an independent chunked algorithm).

Every pin takes `seq`, a callable with the oracle's `wkv7_sequence`
signature: seq(S0 [..., N, N], r, w, k, v, a, b [T, ..., N]) -> (o, S_T).
The mutation test feeds deliberately broken copies of the oracle through the
same pins; each copy must fail at least one.

The operation is the generalized delta rule of page "RWKV-X Architecture",
section "WKV-7 Kernel (Generalized Delta Rule)", in product form
S_t = S_{t-1}(diag(w_t) + a_t b_t^T) + v_t k_t^T, o_t = S_t r_t.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

from tests.chunk_form64 import chunked_sequence64

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NAMES = ("r", "w", "k", "v", "a", "b")


def _draw(rng, T, N, H=None, alpha_scalar=False):
    shape = (T, N) if H is None else (T, H, N)
    r = rng.standard_normal(shape)
    k = rng.standard_normal(shape)
    v = rng.standard_normal(shape)
    w = np.exp(-np.exp(rng.normal(-0.6, 0.5, size=shape)))
    z = rng.standard_normal(shape)
    kk = z / np.linalg.norm(z, axis=-1, keepdims=True)
    if alpha_scalar:
        al = 1 / (1 + np.exp(-rng.standard_normal(shape[:-1] + (1,))))
    else:
        al = 1 / (1 + np.exp(-rng.standard_normal(shape)))
    return dict(r=r, w=w, k=k, v=v, a=-kk, b=kk * al)


def _rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.sqrt(np.mean(ref * ref)),
                                                 1e-300))


# -- P1: a = b = 0 gives decayed linear attention (closed form, O(T^2)) ----

def pin_decayed_linear_attention(seq, seed=11, T=9, N=5):
    rng = np.random.default_rng(seed)
    x = _draw(rng, T, N)
    x["a"][:] = 0.0
    x["b"][:] = 0.0
    S0 = rng.standard_normal((N, N))
    o, ST = seq(S0, **x)
    w, k, v, r = x["w"], x["k"], x["v"], x["r"]
    o_ref = np.zeros((T, N))
    for t in range(T):
        lam_t = np.prod(w[:t + 1], axis=0)            # decay since the start
        for i in range(N):
            acc = sum(S0[i, j] * lam_t[j] * r[t, j] for j in range(N))
            for s in range(t + 1):
                dec = np.prod(w[s + 1:t + 1], axis=0)  # empty product = 1
                acc += v[s, i] * sum(k[s, j] * dec[j] * r[t, j]
                                     for j in range(N))
            o_ref[t, i] = acc
    S_ref = S0 * np.prod(w, axis=0)[None, :]
    for s in range(T):
        dec = np.prod(w[s + 1:], axis=0)
        S_ref = S_ref + np.outer(v[s], k[s] * dec)
    assert _rel(o, o_ref) < 1e-12, "a=b=0 closed form: o"
    assert _rel(ST, S_ref) < 1e-12, "a=b=0 closed form: S_T"


# -- P2: w = 1, a = b = 0 gives a cumulative outer-product sum -------------

def pin_cumulative_outer_sum(seq, seed=12, T=17, N=6):
    rng = np.random.default_rng(seed)
    x = _draw(rng, T, N)
    x["w"][:] = 1.0
    x["a"][:] = 0.0
    x["b"][:] = 0.0
    S0 = rng.standard_normal((N, N))
    o, ST = seq(S0, **x)
    outer = x["v"][:, :, None] * x["k"][:, None, :]        # [T, N, N]
    S_all = S0[None] + np.cumsum(outer, axis=0)
    o_ref = np.matmul(S_all, x["r"][:, :, None])[..., 0]
    assert _rel(o, o_ref) < 1e-13, "cumulative sum: o"
    assert _rel(ST, S_all[-1]) < 1e-13, "cumulative sum: S_T"


# -- P3: brute-force matrix products on tiny T, N ----------------------------

def _transition(w, a, b):
    return np.diag(w) + np.outer(a, b)


def pin_bruteforce_products(seq, seed=13, T=6, N=4):
    rng = np.random.default_rng(seed)
    x = _draw(rng, T, N)
    S0 = rng.standard_normal((N, N))
    o, ST = seq(S0, **x)
    G = [_transition(x["w"][t], x["a"][t], x["b"][t]) for t in range(T)]

    def chain(lo, hi):            # G_lo ... G_{hi-1}; identity if empty
        M = np.eye(N)
        for t in range(lo, hi):
            M = M @ G[t]
        return M

    for t in range(T):
        S_t = S0 @ chain(0, t + 1)
        for s in range(t + 1):
            S_t = S_t + np.outer(x["v"][s], x["k"][s]) @ chain(s + 1, t + 1)
        assert _rel(o[t], S_t @ x["r"][t]) < 1e-12, f"brute force: o[{t}]"
        if t == T - 1:
            assert _rel(ST, S_t) < 1e-12, "brute force: S_T"


# -- exact rationals: dyadic inputs, float64 must reproduce exactly ---------

def pin_exact_rationals(seq, seed=14, T=3, N=3):
    rng = np.random.default_rng(seed)
    # small dyadic values keep every float64 operation exact
    def dy(shape, lo, hi):
        return rng.integers(lo, hi, size=shape) / 8.0
    x = dict(r=dy((T, N), -8, 9), k=dy((T, N), -8, 9), v=dy((T, N), -8, 9),
             a=dy((T, N), -8, 9), b=dy((T, N), -8, 9), w=dy((T, N), 1, 9))
    S0 = dy((N, N), -8, 9)
    o, ST = seq(S0, **x)
    F = lambda M: [[Fraction(float(e)) for e in row] for row in M]
    S = F(S0)
    for t in range(T):
        w = [Fraction(float(e)) for e in x["w"][t]]
        a = [Fraction(float(e)) for e in x["a"][t]]
        b = [Fraction(float(e)) for e in x["b"][t]]
        k = [Fraction(float(e)) for e in x["k"][t]]
        v = [Fraction(float(e)) for e in x["v"][t]]
        r = [Fraction(float(e)) for e in x["r"][t]]
        Gt = [[(w[i] if i == j else 0) + a[i] * b[j] for j in range(N)]
              for i in range(N)]
        S = [[sum(S[i][m] * Gt[m][j] for m in range(N)) + v[i] * k[j]
              for j in range(N)] for i in range(N)]
        o_t = [sum(S[i][j] * r[j] for j in range(N)) for i in range(N)]
        for i in range(N):
            assert float(o_t[i]) == o[t][i], f"exact rationals: o[{t}][{i}]"
    for i in range(N):
        for j in range(N):
            assert float(S[i][j]) == ST[i][j], "exact rationals: S_T"


# -- hand-worked example (text fixture) --------------------------------------

def load_handworked():
    vals = {}
    with open(os.path.join(GOLDEN, "wkv7_n2_t2_handworked.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, t, *nums = line.split()
            vals[(name, int(t))] = np.array([float(z) for z in nums])
    return vals


def pin_handworked(seq):
    g = load_handworked()
    x = {n: np.stack([g[(n, 1)], g[(n, 2)]]) for n in NAMES}
    o, ST = seq(np.zeros((2, 2)), **x)
    assert np.array_equal(o[0], g[("o", 1)]), "hand-worked o1"
    assert np.array_equal(o[1], g[("o", 2)]), "hand-worked o2"
    assert np.array_equal(ST.reshape(-1), g[("S", 2)]), "hand-worked S2"


# -- P4: a single token from a zero state -----------------------------------

def pin_single_token(seq, seed=15, N=7):
    rng = np.random.default_rng(seed)
    x = _draw(rng, 1, N)
    o, ST = seq(np.zeros((N, N)), **x)
    k, v, r = x["k"][0], x["v"][0], x["r"][0]
    assert _rel(o[0], v * float(k @ r)) < 1e-14, "T=1: o = v (k.r)"
    assert _rel(ST, np.outer(v, k)) < 1e-15, "T=1: S = v k^T"


# -- P5: delta-rule write recalls the value exactly --------------------------

def pin_delta_rule_recall(seq, seed=16, T=12, N=8):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((T, N))
    kh = z / np.linalg.norm(z, axis=1, keepdims=True)
    x = dict(r=kh.copy(), w=np.ones((T, N)), k=kh.copy(),
             v=rng.standard_normal((T, N)), a=-kh, b=kh.copy())
    S0 = rng.standard_normal((N, N))
    o, _ = seq(S0, **x)
    assert np.max(np.abs(o - x["v"])) < 1e-12, "delta-rule recall: o_t = v_t"


# -- P6: the two-step expansion fixes which state the a-term reads ----------

def pin_two_step_order(seq, seed=17, N=6):
    rng = np.random.default_rng(seed)
    x = _draw(rng, 2, N)
    o, ST = seq(np.zeros((N, N)), **x)
    k1, v1 = x["k"][0], x["v"][0]
    w2, a2, b2, k2, v2, r2 = (x[n][1] for n in ("w", "a", "b", "k", "v", "r"))
    # S2 = v1 (k1*w2)^T + v1 (k1.a2) b2^T + v2 k2^T
    S2 = np.outer(v1, k1 * w2) + float(k1 @ a2) * np.outer(v1, b2) \
        + np.outer(v2, k2)
    o2 = v1 * float((k1 * w2) @ r2) + v1 * float(k1 @ a2) * float(b2 @ r2) \
        + v2 * float(k2 @ r2)
    assert _rel(ST, S2) < 1e-14, "two steps: S2"
    assert _rel(o[1], o2) < 1e-14, "two steps: o2"


# -- P7: state size does not depend on T ------------------------------------

def pin_state_size(seq, seed=18, H=3, N=8):
    rng = np.random.default_rng(seed)
    for T in (1, 2048):
        x = _draw(rng, T, N, H=H)
        o, ST = seq(np.zeros((H, N, N)), **x)
        assert ST.shape == (H, N, N), "state shape independent of T"
        assert o.shape == (T, H, N)
        assert np.all(np.isfinite(ST)) and np.all(np.isfinite(o))


# -- P8: fork-then-continue equals a fresh run, bit for bit ------------------

def pin_fork_continue(seq, seed=19, T=40, T1=17, H=2, N=8):
    rng = np.random.default_rng(seed)
    x = _draw(rng, T, N, H=H)
    S0 = rng.standard_normal((H, N, N))
    o_full, S_full = seq(S0, **x)
    o_a, S_mid = seq(S0, **{n: x[n][:T1] for n in NAMES})
    fork = S_mid.copy()
    o_b, S_end = seq(fork, **{n: x[n][T1:] for n in NAMES})
    assert np.array_equal(np.concatenate([o_a, o_b]), o_full), "fork: o"
    assert np.array_equal(S_end, S_full), "fork: S_T"


# -- P9: linearity in (S0, v); value-index equivariance; head independence --

def pin_linearity_equivariance(seq, seed=20, T=10, H=2, N=6):
    rng = np.random.default_rng(seed)
    x = _draw(rng, T, N, H=H)
    S0, S1 = rng.standard_normal((2, H, N, N))
    v1 = rng.standard_normal((T, H, N))
    al, be = 0.7, -1.3
    o0, T0 = seq(S0, **x)
    x1 = dict(x, v=v1)
    o1, T1 = seq(S1, **x1)
    xm = dict(x, v=al * x["v"] + be * v1)
    om, Tm = seq(al * S0 + be * S1, **xm)
    assert _rel(om, al * o0 + be * o1) < 1e-12, "linearity: o"
    assert _rel(Tm, al * T0 + be * T1) < 1e-12, "linearity: S_T"
    perm = rng.permutation(N)
    xp = dict(x, v=x["v"][..., perm])
    op, Tp = seq(S0[:, perm, :], **xp)
    assert np.array_equal(op, o0[..., perm]), "value permutation: o"
    assert np.array_equal(Tp, T0[:, perm, :]), "value permutation: S_T"
    # each head alone equals the same head run together with the others
    for h in range(H):
        oh, Th = seq(S0[h], **{n: x[n][:, h] for n in NAMES})
        assert np.array_equal(oh, o0[:, h]), "head independence: o"
        assert np.array_equal(Th, T0[h]), "head independence: S_T"


# -- P10: contraction bound on every step ------------------------------------

def pin_contraction_bound(seq, seed=21, T=300, N=16):
    """||S_t||_F <= ||G_t||_2 ||S_{t-1}||_F + ||v_t|| ||k_t|| at every t."""
    rng = np.random.default_rng(seed)
    x = _draw(rng, T, N, alpha_scalar=True)
    S = rng.standard_normal((N, N))
    prev = np.linalg.norm(S)
    for t in range(T):
        _, S = seq(S, **{n: x[n][t:t + 1] for n in NAMES})
        G = _transition(x["w"][t], x["a"][t], x["b"][t])
        g2 = np.linalg.norm(G, 2)
        bound = g2 * prev + np.linalg.norm(x["v"][t]) * np.linalg.norm(x["k"][t])
        cur = np.linalg.norm(S)
        assert cur <= bound * (1 + 1e-12), f"contraction bound at t={t}"
        # scalar alpha makes G symmetric with norm below one
        assert g2 < 1.0
        prev = cur


# -- P11: the chunked (WY/UT) algorithm, run independently, agrees ----------

def pin_chunked_algorithm(seq, seed=22, T=200, H=2, N=16, L=16):
    rng = np.random.default_rng(seed)
    x = _draw(rng, T, N, H=H)
    S0 = rng.standard_normal((H, N, N)) * 0.1
    o, ST = seq(S0, **x)
    for h in range(H):
        oc, Sc = chunked_sequence64(S0[h], **{n: x[n][:, h] for n in NAMES},
                                    L=L)
        assert _rel(oc, o[:, h]) < 1e-11, "chunked algorithm: o"
        assert _rel(Sc, ST[h]) < 1e-11, "chunked algorithm: S_T"


ALL_PINS = [
    pin_decayed_linear_attention,
    pin_cumulative_outer_sum,
    pin_bruteforce_products,
    pin_exact_rationals,
    pin_handworked,
    pin_single_token,
    pin_delta_rule_recall,
    pin_two_step_order,
    pin_state_size,
    pin_fork_continue,
    pin_linearity_equivariance,
    pin_contraction_bound,
    pin_chunked_algorithm,
]
