"""Chunked (WY/UT) form of the WKV-7 recurrence, float64, for testing.

An independent algorithm that reaches the same result as the sequential
recurrence S_t = S_{t-1}(diag(w_t) + a_t b_t^T) + v_t k_t^T, o_t = S_t r_t
(page "RWKV-X Architecture", section "WKV-7 Kernel (Generalized Delta
Rule)"; the chunked form is derived here, the page only names a batched
forward as a prefill optimisation).

Within a chunk starting from state S0, let c_t = sum_{u<=t} log w_u (per key
channel), Lambda_t = exp(c_t), and u_t = S_{t-1} a_t. Unrolling gives

    u_t = S0 (a_t * Lambda_{t-1}) + sum_{s<t} [u_s <a_t, b_s Lambda_{t-1}/Lambda_s>
                                               + v_s <a_t, k_s Lambda_{t-1}/Lambda_s>]
    o_t = S0 (r_t * Lambda_t)     + sum_{s<=t} [u_s <r_t, b_s Lambda_t/Lambda_s>
                                               + v_s <r_t, k_s Lambda_t/Lambda_s>]
    S_L = S0 diag(Lambda_L) + sum_s (u_s b_s^T + v_s k_s^T) diag(Lambda_L/Lambda_s)

so, stacking per-token rows, U = (I - A_ab)^-1 (Abar S0^T + A_ak V),
O = Rbar S0^T + M_rb U + M_rk V and S_L = S0 diag(Lambda_L) + U^T Bbar + V^T Kbar,
with the L x L matrices built from operands scaled about a mid-chunk
reference rho (A_* strictly lower, M_* lower including the diagonal).

This module is test infrastructure: it pins the oracle (in float64) and,
with reduced-precision products plugged in, models the operand precision of
the device kernels' plans on the CPU; it is not used by either at run time.
"""
from __future__ import annotations

import numpy as np


def chunk_step64(S0, r, w, k, v, a, b, mm=None):
    """One chunk (n rows) from S0 [N, N]; returns (O [n, N], S_L [N, N]).

    `mm(P, Q)`, if given, replaces every product P @ Q (to model a kernel's
    operand precision: rounded or split operands, rounded results).
    """
    if mm is None:
        def mm(P, Q):
            return P @ Q
    n = r.shape[0]
    c = np.cumsum(np.log(w), axis=0)                  # c_t, t = 1..n
    cprev = np.vstack([np.zeros((1, w.shape[1])), c[:-1]])
    rho = c[(n - 1) // 2]
    Ah, Rh = a * np.exp(cprev - rho), r * np.exp(c - rho)
    Bh, Kh = b * np.exp(rho - c), k * np.exp(rho - c)
    cL = c[-1]
    Ab, Rb = a * np.exp(cprev), r * np.exp(c)
    Bb, Kb = b * np.exp(cL - c), k * np.exp(cL - c)
    A_ab = np.tril(mm(Ah, Bh.T), -1)
    A_ak = np.tril(mm(Ah, Kh.T), -1)
    M_rb = np.tril(mm(Rh, Bh.T), 0)
    M_rk = np.tril(mm(Rh, Kh.T), 0)
    Tinv = np.linalg.inv(np.eye(n) - A_ab)
    X = mm(Ab, S0.T) + mm(A_ak, v)
    U = mm(Tinv, X)
    O = mm(Rb, S0.T) + mm(M_rb, U) + mm(M_rk, v)
    S_L = S0 * np.exp(cL)[None, :] + mm(U.T, Bb) + mm(v.T, Kb)
    return O, S_L


def chunked_sequence64(S0, r, w, k, v, a, b, L=64, mm=None):
    """Whole sequence in chunks of L (the last one may be shorter)."""
    S = np.array(S0, dtype=np.float64, copy=True)
    T = r.shape[0]
    outs = []
    for lo in range(0, T, L):
        hi = min(lo + L, T)
        O, S = chunk_step64(S, r[lo:hi], w[lo:hi], k[lo:hi], v[lo:hi],
                            a[lo:hi], b[lo:hi], mm=mm)
        outs.append(O)
    o = np.concatenate(outs) if outs else np.zeros_like(r)
    return o, S
