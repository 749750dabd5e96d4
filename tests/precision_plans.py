"""CPU models of the operand precision of the chunked kernels, for testing.

Each model runs the chunked (WY/UT) form of the recurrence (derived in
tests/chunk_form64.py; the page, "RWKV-X Architecture", section "WKV-7
Kernel (Generalized Delta Rule)", gives only the sequential recurrence) with
the device kernels' roundings applied to the operands and results of every
product, and float64 everywhere else. It is a model of where each kernel
rounds, not a bit-exact copy of its arithmetic (the accumulation order of
the matrix cores is not modelled); the tests compare it with the float64
oracle at the workloads' lengths to pin how much of the error bar each plan
spends and how that grows with the sequence length.

Plans:
* fp32 chunk form: every operand rounded to float32 (headroom of the form);
* split-bf16 with exact T, chunks of 64 (the earlier precise kernel):
  every product from bf16 hi + lo operand pairs, hi*hi + hi*lo + lo*hi,
  float32 results;
* the chunked kernel's fast plan (bf16 inputs; chunks of 32): split-bf16
  Gram products stored as fp16; T from the fp16 A_ab by the product
  (I + A)(I + A^2)(I + A^4)(I + A^8) per 16 x 16 diagonal block with fp16
  operands; every value-side product with single fp16 operands, the state,
  X and U scaled per 16-row block by a power of two first; the state
  carried in float32;
* the precise plan of the same kernel (fp32 inputs; chunks of 32): the
  same Gram products and T, every value-side product from split-bf16
  operands (T's fp16 values split exactly), nothing scaled.
"""
from __future__ import annotations

import numpy as np
import torch

from tests.chunk_form64 import chunked_sequence64


def f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32) \
        .astype(np.float16).astype(np.float64)


def bf16(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    return t.to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def split_bf16(x):
    x = f32(x)
    h = bf16(x)
    return h, bf16(f32(x - h))


def mm_split(P, Q):
    """P @ Q from split bf16 operands: three products, float32 result."""
    Ph, Pl = split_bf16(P)
    Qh, Ql = split_bf16(Q)
    return f32(Pl @ Qh + Ph @ Ql + Ph @ Qh)


def mm_f32(P, Q):
    return f32(f32(P) @ f32(Q))


def mm_bf16(P, Q):
    return f32(bf16(P) @ bf16(Q))


def pow2_f16(x, axis, block=16):
    """fp16 after scaling each block of `block` indices along `axis` by the
    power of two that brings its largest magnitude just below 2^14."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    n = x.shape[axis]
    for lo in range(0, n, block):
        sl = [slice(None)] * x.ndim
        sl[axis] = slice(lo, min(lo + block, n))
        sl = tuple(sl)
        m = float(np.max(np.abs(f32(x[sl])))) if x[sl].size else 0.0
        if m > 0.0 and np.isfinite(m):
            e = int(np.floor(np.log2(m)))
            s = 2.0 ** (13 - e)
        else:
            s = 1.0
        out[sl] = f16(f32(x[sl]) * s) / s
    return out


def _inverse_unit_lower16(A16):
    """(I - A)^-1 of a strictly lower 16 x 16 fp16 A as the kernel forms it:
    P = I + A; three times N <- N N, P <- P + P N, with fp16 operands and
    float32 results; returns the fp16 values of P."""
    n = A16.shape[0]
    N16 = A16
    P32 = f32(np.eye(n) + A16)
    P16 = f16(P32)
    for _ in range(3):
        N16 = f16(N16 @ N16)
        P32 = f32(P32 + P16 @ N16)
        P16 = f16(P32)
    return P16


def _key_side(r, w, k, v, a, b, L):
    """The part both plans of the chunked kernel share: padding of a short
    chunk (w = 1, everything else 0), the decay products, the decay-scaled
    operands (float32), the four Gram matrices (split-bf16 operands, float32
    results, masked) and T from the fp16 A_ab by the product form per
    16 x 16 diagonal block."""
    n, N = r.shape
    if n < L:                       # padding: w = 1, everything else 0
        pad = L - n
        z = np.zeros((pad, N))
        r, k, v, a, b = (np.vstack([x, z]) for x in (r, k, v, a, b))
        w = np.vstack([w, np.ones((pad, N))])
    w32 = f32(w)
    lam = np.cumprod(w32.astype(np.float32), axis=0).astype(np.float64)
    lamprev = np.vstack([np.ones((1, N)), lam[:-1]])
    lamL = lam[-1]
    suf = f32(lamL[None, :] / lam)
    Abar, Rbar = f32(a * lamprev), f32(r * lam)
    Bbar, Kbar = f32(b * suf), f32(k * suf)
    inv = f32(1.0 / lamL)
    Ahat, Rhat = f32(Abar * inv), f32(Rbar * inv)
    G_ab = np.tril(mm_split(Ahat, Bbar.T), -1)
    G_ak = np.tril(mm_split(Ahat, Kbar.T), -1)
    G_rb = np.tril(mm_split(Rhat, Bbar.T), 0)
    G_rk = np.tril(mm_split(Rhat, Kbar.T), 0)
    # T = [[D0, 0], [T10, D1]], D_p = (I - A_pp)^-1, T10 = D1 (A10 D0)
    A_ab = f16(G_ab)
    h = L // 2
    D0 = _inverse_unit_lower16(A_ab[:h, :h])
    D1 = _inverse_unit_lower16(A_ab[h:, h:])
    Y = f16(A_ab[h:, :h] @ D0)
    T10 = f16(D1 @ Y)
    T16 = np.zeros((L, L))
    T16[:h, :h], T16[h:, :h], T16[h:, h:] = D0, T10, D1
    return dict(n=n, v=v, lamL=lamL, Abar=Abar, Rbar=Rbar, Bbar=Bbar,
                Kbar=Kbar, G_ak=G_ak, G_rb=G_rb, G_rk=G_rk, T16=T16)


def fast_chunk(S0, r, w, k, v, a, b, L=32):
    """One chunk (n <= L rows) of the default bf16 kernel's plan.

    S0: [N, N] (float32 values in float64). Returns (O [n, N], S_L)."""
    K = _key_side(r, w, k, v, a, b, L)
    n, lamL, T16 = K["n"], K["lamL"], K["T16"]
    A_ak, M_rb, M_rk = f16(K["G_ak"]), f16(K["G_rb"]), f16(K["G_rk"])
    Sf = pow2_f16(S0, axis=0)                   # blocks of 16 state rows
    V16, Ab16, Rb16 = f16(K["v"]), f16(K["Abar"]), f16(K["Rbar"])
    Bb16, Kb16 = f16(K["Bbar"]), f16(K["Kbar"])
    X = f32(Ab16 @ Sf.T + A_ak @ V16)           # [t][i]
    U = f32(T16 @ pow2_f16(X, axis=1))
    Uf = pow2_f16(U, axis=1)
    O = f32(Rb16 @ Sf.T + M_rb @ Uf + M_rk @ V16)
    S_L = f32(lamL[None, :] * S0 + Uf.T @ Bb16 + V16.T @ Kb16)
    return O[:n], S_L


def precise_chunk(S0, r, w, k, v, a, b, L=32):
    """One chunk of the chunked kernel's precise plan (fp32 inputs, or bf16
    inputs on request): the same key side, then every value-side product
    from split-bf16 operands (the state, X, U, the decay-scaled operands, V
    and the Gram matrices all split; T's fp16 values split exactly), no
    scaling, float32 results."""
    K = _key_side(r, w, k, v, a, b, L)
    n, lamL, T16, V = K["n"], K["lamL"], K["T16"], f32(K["v"])
    X = f32(mm_split(K["Abar"], S0.T) + mm_split(K["G_ak"], V))
    U = mm_split(T16, X)
    O = f32(mm_split(K["Rbar"], S0.T) + mm_split(K["G_rk"], V)
            + mm_split(K["G_rb"], U))
    S_L = f32(lamL[None, :] * S0 + mm_split(V.T, K["Kbar"])
              + mm_split(U.T, K["Bbar"]))
    return O[:n], S_L


def _sequence(chunk, S0, r, w, k, v, a, b, L):
    S = f32(S0)
    outs = []
    for lo in range(0, r.shape[0], L):
        hi = min(lo + L, r.shape[0])
        O, S = chunk(S, r[lo:hi], w[lo:hi], k[lo:hi], v[lo:hi],
                     a[lo:hi], b[lo:hi], L=L)
        outs.append(O)
    return np.concatenate(outs), S


def fast_sequence(S0, r, w, k, v, a, b, L=32):
    return _sequence(fast_chunk, S0, r, w, k, v, a, b, L)


def precise_sequence(S0, r, w, k, v, a, b, L=32):
    return _sequence(precise_chunk, S0, r, w, k, v, a, b, L)


def split_sequence(S0, r, w, k, v, a, b, L=64):
    """Split-bf16 operands for every product, T exact, chunks of 64 (the
    plan of the 64-token kernel the precise plan replaced)."""
    return chunked_sequence64(S0, r, w, k, v, a, b, L=L, mm=mm_split)


def fp32_sequence(S0, r, w, k, v, a, b, L=64):
    return chunked_sequence64(S0, r, w, k, v, a, b, L=L, mm=mm_f32)


def bf16_sequence(S0, r, w, k, v, a, b, L=64):
    """Single bf16 operands everywhere (a plan the kernels do not use)."""
    return chunked_sequence64(S0, r, w, k, v, a, b, L=L, mm=mm_bf16)
