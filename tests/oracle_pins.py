"""Pins for the float64 oracle: checks against what the article and plain
mathematics fix, never against the oracle's own formula retyped.

Each ``pin_*`` function takes the loaded oracle library (so the same pins can
be run against copies of the oracle with planted mistakes) and raises
AssertionError on failure.  Citations are to the article "From GPT-2 to Kimi
K3, explained" (Chinese mirror on transcrab.onev.cat, German mirror on
youmind.com), by section.

Independent evaluations used:
* quadratic masked form of linear attention (chunk size = sequence length,
  section "DeltaNet (Parallelizing ...)", chunk-size interpolation remark),
  with the feature map from torch's ``F.elu`` + 1 as the article writes it;
* closed-form state sums (section "Linear Attention": S = S + k^T v, z = z + k);
* the convex-hull / running-mean property (section "Linear Attention",
  three-step description: non-negative scores, divided by their sum,
  weighted mean of v);
* the UT/WY form solved densely with a library triangular solve (section
  "DeltaNet (Parallelizing ...)", reparameterisation and chunked code, C = T);
* the generalised Householder form S_t = S_{t-1}(I - b k k^T) + b v k^T in the
  article's transposed convention (same section);
* the chunked algorithm of the same section at several chunk sizes;
* exact retrieval and replacement (section "DeltaNet (Fast Weight
  Programmers)": reading back with a unit key returns v exactly; writing a key
  again replaces the old association);
* gate limits (section "Gated Delta Net": decay 1 is the plain delta rule,
  decay 0 clears the memory), the scalar-gated Householder form, closed forms
  of pure decay, and the per-channel gated UT form;
* for the additive cache with a forgetting factor (section "Gated Delta Net",
  first step): its unrolled sum, i.e. the decayed masked quadratic form
  (tril(Q K^T) * e^{G_t - G_j}) V, and the limits a = 1 (plain additive
  linear attention, closed-form state) and a = 0 (only the newest write);
* for the delta rule's gradient (the training use the article gives the
  chunk form for): central finite differences of the forward oracle, and
  torch autograd through a plain float64 loop of the same recurrence.
"""
from __future__ import annotations

import numpy as np
import scipy.linalg
import torch
import torch.nn.functional as F

import oracle

RTOL = 1e-11


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol=RTOL, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    assert err <= tol * scale, f"{what}: max abs err {err:.3e} (scale {scale:.3e})"


def _phi(x):
    """Feature map as the article writes it: F.elu(x) + 1."""
    return (F.elu(torch.from_numpy(np.asarray(x, np.float64))) + 1.0).numpy()


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _delta_inputs(rng, B, H, T, dk, dv, gated=False, gate_scale=1.0 / 16):
    q = rng.standard_normal((B, H, T, dk))
    k = _unit_rows(rng.standard_normal((B, H, T, dk)))
    v = rng.standard_normal((B, H, T, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, T))))
    g = None
    if gated:
        x = rng.standard_normal((B, H, T, dk))
        g = -np.log1p(np.exp(x)) * gate_scale
    return q, k, v, beta, g


# --------------------------------------------------------------------------
# Linear attention
# --------------------------------------------------------------------------

def pin_la_quadratic_masked_form(lib):
    """Recurrence == (tril(phiQ phiK^T) V + phiQ S0) / (rowsum(tril(...)) + phiQ z0)."""
    rng = _rng(1)
    B, H, T, dk, dv = 2, 3, 37, 8, 5
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    S0 = 0.3 * rng.standard_normal((B, H, dk, dv))
    z0 = 0.5 + np.abs(rng.standard_normal((B, H, dk)))
    for init in (False, True):
        o, S, z = oracle.la_recurrent(q, k, v, S0 if init else None,
                                      z0 if init else None, lib=lib)
        fq, fk = _phi(q), _phi(k)
        for b in range(B):
            for h in range(H):
                A = np.tril(fq[b, h] @ fk[b, h].T)
                num = A @ v[b, h]
                den = A.sum(axis=1)
                if init:
                    num = num + fq[b, h] @ S0[b, h]
                    den = den + fq[b, h] @ z0[b, h]
                _close(o[b, h], num / den[:, None], what="la quadratic o")


def pin_la_closed_form_state(lib):
    """S_T = S0 + phi(K)^T V and z_T = z0 + sum phi(k_t), independent of token order."""
    rng = _rng(2)
    B, H, T, dk, dv = 1, 2, 29, 6, 7
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    S0 = rng.standard_normal((B, H, dk, dv))
    z0 = 1.0 + np.abs(rng.standard_normal((B, H, dk)))
    _, S, z = oracle.la_recurrent(q, k, v, S0, z0, lib=lib)
    fk = _phi(k)
    for h in range(H):
        _close(S[0, h], S0[0, h] + fk[0, h].T @ v[0, h], what="la closed S")
        _close(z[0, h], z0[0, h] + fk[0, h].sum(axis=0), what="la closed z")
    perm = rng.permutation(T)
    _, S2, z2 = oracle.la_recurrent(q[:, :, perm], k[:, :, perm], v[:, :, perm],
                                    S0, z0, lib=lib)
    _close(S2, S, what="la order-free S")
    _close(z2, z, what="la order-free z")


def pin_la_convex_hull_and_running_mean(lib):
    """Outputs are weighted means of past values with non-negative weights:
    one token returns v_1; identical keys and queries give the running mean;
    every coordinate stays within the range of the values seen so far."""
    rng = _rng(3)
    B, H, T, dk, dv = 1, 1, 40, 4, 3
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    o, _, _ = oracle.la_recurrent(q, k, v, lib=lib)
    _close(o[0, 0, 0], v[0, 0, 0], what="la first token")
    for t in range(T):
        lo = v[0, 0, :t + 1].min(axis=0) - 1e-12
        hi = v[0, 0, :t + 1].max(axis=0) + 1e-12
        assert np.all(o[0, 0, t] >= lo) and np.all(o[0, 0, t] <= hi), "hull"
    ksame = np.broadcast_to(rng.standard_normal((1, 1, 1, dk)), (B, H, T, dk)).copy()
    o2, _, _ = oracle.la_recurrent(q, ksame, v, lib=lib)
    mean = np.cumsum(v[0, 0], axis=0) / np.arange(1, T + 1)[:, None]
    _close(o2[0, 0], mean, what="la running mean")


def pin_la_elu_branches(lib):
    """phi(x) = x + 1 for x > 0 and exp(x) otherwise: with d_k = 1 and zero
    prior state the single-token normaliser equals phi(q) phi(k) exactly."""
    xs = np.array([-3.0, -0.5, 0.0, 0.25, 2.0])
    for xq in xs:
        for xk in xs:
            q = np.full((1, 1, 1, 1), xq)
            k = np.full((1, 1, 1, 1), xk)
            v = np.ones((1, 1, 1, 1))
            _, S, z = oracle.la_recurrent(q, k, v, lib=lib)
            _close(z[0, 0, 0], _phi(np.array([xk]))[0], what="phi(k)")
            _close(S[0, 0, 0, 0], _phi(np.array([xk]))[0], what="phi(k) v")


# --------------------------------------------------------------------------
# Delta rule
# --------------------------------------------------------------------------

def _ut_form(q, k, v, beta, S0):
    """Dense UT/WY form for one head at chunk size C = T:
    U = (I + tril(diag(beta) K K^T, -1))^{-1} diag(beta) (V - K S0),
    O = Q S0 + tril(Q K^T) U, S_T = S0 + K^T U."""
    T = k.shape[0]
    Lm = np.tril(beta[:, None] * (k @ k.T), -1)
    rhs = beta[:, None] * (v - k @ S0)
    U = scipy.linalg.solve_triangular(np.eye(T) + Lm, rhs, lower=True)
    O = q @ S0 + np.tril(q @ k.T) @ U
    return O, S0 + k.T @ U


def pin_delta_ut_form(lib):
    rng = _rng(4)
    B, H, T, dk, dv = 2, 2, 48, 8, 6
    q, k, v, beta, _ = _delta_inputs(rng, B, H, T, dk, dv)
    S0 = 0.5 * rng.standard_normal((B, H, dk, dv))
    for init in (False, True):
        o, S = oracle.delta_recurrent(q, k, v, beta, None, S0 if init else None, lib=lib)
        for b in range(B):
            for h in range(H):
                s0 = S0[b, h] if init else np.zeros((dk, dv))
                O, ST = _ut_form(q[b, h], k[b, h], v[b, h], beta[b, h], s0)
                _close(o[b, h], O, what="delta UT o")
                _close(S[b, h], ST, what="delta UT S")


def pin_delta_householder_form(lib):
    """Transposed convention: M_t = M_{t-1}(I - b k k^T) + b v k^T, o_t = M_t q_t
    with M = S^T (d_v x d_k)."""
    rng = _rng(5)
    B, H, T, dk, dv = 1, 2, 33, 7, 9
    q, k, v, beta, _ = _delta_inputs(rng, B, H, T, dk, dv)
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = oracle.delta_recurrent(q, k, v, beta, None, S0, lib=lib)
    for h in range(H):
        M = S0[0, h].T.copy()
        for t in range(T):
            kt = k[0, h, t][:, None]
            M = M @ (np.eye(dk) - beta[0, h, t] * (kt @ kt.T)) \
                + beta[0, h, t] * (v[0, h, t][:, None] @ kt.T)
            _close(o[0, h, t], M @ q[0, h, t], what="householder o")
        _close(S[0, h], M.T, what="householder S")


def _chunked_delta(q, k, v, beta, C):
    """The article's chunkwise delta rule for one head, written from its
    description: per chunk, T = (I + tril(diag(beta) K K^T, -1))^{-1} by forward
    substitution, W = T diag(beta) K, U = T diag(beta) V; then over chunks in
    order u = U - W S, o = Q S + tril(Q K^T) u, S += K^T u."""
    L, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv))
    O = np.empty((L, dv))
    for c0 in range(0, L, C):
        Q, K, V, b = q[c0:c0 + C], k[c0:c0 + C], v[c0:c0 + C], beta[c0:c0 + C]
        n = K.shape[0]
        A = np.tril(b[:, None] * (K @ K.T), -1)
        Tm = np.zeros((n, n))
        for i in range(n):              # row i of (I + A)^{-1}
            Tm[i, i] = 1.0
            for j in range(i):
                Tm[i, j] = -A[i, j:i] @ Tm[j:i, j]
        W = Tm @ (b[:, None] * K)
        U = Tm @ (b[:, None] * V)
        u = U - W @ S
        O[c0:c0 + n] = Q @ S + np.tril(Q @ K.T) @ u
        S = S + K.T @ u
    return O, S


def pin_delta_chunk_size_invariance(lib):
    """Any chunk size gives the recurrence's result (C = 1 is the recurrence,
    C = T the quadratic form)."""
    rng = _rng(6)
    B, H, T, dk, dv = 1, 1, 64, 8, 8
    q, k, v, beta, _ = _delta_inputs(rng, B, H, T, dk, dv)
    o, S = oracle.delta_recurrent(q, k, v, beta, lib=lib)
    for C in (1, 2, 4, 16, 64):
        O, ST = _chunked_delta(q[0, 0], k[0, 0], v[0, 0], beta[0, 0], C)
        _close(o[0, 0], O, tol=1e-10, what=f"chunk C={C} o")
        _close(S[0, 0], ST, tol=1e-10, what=f"chunk C={C} S")


def pin_delta_exact_retrieval(lib):
    """beta = 1 with orthonormal keys and a zero state stores every pair
    exactly: K S_T = V, and a query equal to an earlier key returns its value."""
    rng = _rng(7)
    dk = dv = 16
    T = 12
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:T][None, None]
    v = rng.standard_normal((1, 1, T, dv))
    beta = np.ones((1, 1, T))
    pick = rng.integers(0, np.arange(1, T + 1))       # earlier-or-same key
    q = k[0, 0, pick][None, None]
    o, S = oracle.delta_recurrent(q, k, v, beta, lib=lib)
    _close(k[0, 0] @ S[0, 0], v[0, 0], tol=1e-12, what="retrieval K S = V")
    _close(o[0, 0], v[0, 0, pick], tol=1e-12, what="retrieval q = k_j")


def pin_delta_replacement(lib):
    """Writing the same unit key twice with beta = 1 replaces the old value."""
    rng = _rng(8)
    dk, dv = 10, 4
    kk = _unit_rows(rng.standard_normal(dk))
    k = np.stack([kk, kk])[None, None]
    v = rng.standard_normal((1, 1, 2, dv))
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, S = oracle.delta_recurrent(k, k, v, np.ones((1, 1, 2)), None, S0, lib=lib)
    _close(o[0, 0, 0], v[0, 0, 0], tol=1e-12, what="replacement first")
    _close(o[0, 0, 1], v[0, 0, 1], tol=1e-12, what="replacement second")
    _close(kk @ S[0, 0], v[0, 0, 1], tol=1e-12, what="replacement state")


def pin_delta_one_step_identities(lib):
    """For a unit key: k S_1 = (1 - b) k S_0 + b v; beta = 0 leaves S unchanged
    and the output is q S_0; beta = 1 makes k read back v exactly."""
    rng = _rng(9)
    dk, dv = 12, 5
    for b in (0.0, 0.3, 1.0):
        k = _unit_rows(rng.standard_normal((1, 1, 1, dk)))
        q = rng.standard_normal((1, 1, 1, dk))
        v = rng.standard_normal((1, 1, 1, dv))
        S0 = rng.standard_normal((1, 1, dk, dv))
        o, S = oracle.delta_recurrent(q, k, v, np.full((1, 1, 1), b), None, S0, lib=lib)
        kv = k[0, 0, 0]
        _close(kv @ S[0, 0], (1 - b) * (kv @ S0[0, 0]) + b * v[0, 0, 0], tol=1e-12,
               what=f"one-step b={b}")
        if b == 0.0:
            _close(S, S0, tol=0, what="beta=0 state")
            _close(o[0, 0, 0], q[0, 0, 0] @ S0[0, 0], tol=1e-12, what="beta=0 out")


# --------------------------------------------------------------------------
# Gated delta rule (per key channel)
# --------------------------------------------------------------------------

def pin_gated_limits(lib):
    """Decay 1 (g = 0) is the plain delta rule; decay 0 (g = -inf) clears the
    memory before every write, so S_t = b_t k_t^T v_t and o_t = b_t (q_t.k_t) v_t."""
    rng = _rng(10)
    B, H, T, dk, dv = 1, 2, 20, 6, 4
    q, k, v, beta, _ = _delta_inputs(rng, B, H, T, dk, dv)
    S0 = rng.standard_normal((B, H, dk, dv))
    o1, S1 = oracle.delta_recurrent(q, k, v, beta, np.zeros((B, H, T, dk)), S0, lib=lib)
    o2, S2 = oracle.delta_recurrent(q, k, v, beta, None, S0, lib=lib)
    _close(o1, o2, tol=0, what="g=0 o")
    _close(S1, S2, tol=0, what="g=0 S")
    o3, S3 = oracle.delta_recurrent(q, k, v, beta, np.full((B, H, T, dk), -np.inf),
                                    S0, lib=lib)
    for h in range(H):
        _close(S3[0, h], beta[0, h, -1] * np.outer(k[0, h, -1], v[0, h, -1]),
               what="a=0 state")
        qk = np.sum(q[0, h] * k[0, h], axis=1)
        _close(o3[0, h], (beta[0, h] * qk)[:, None] * v[0, h], what="a=0 out")


def pin_gated_scalar_householder(lib):
    """The scalar-gated delta rule (one decay per token, given either as
    g [B,H,T] or equal across the channels of g [B,H,T,dk]) is
    M_t = a_t M_{t-1} (I - b k k^T) + b v k^T (transposed convention)."""
    rng = _rng(11)
    B, H, T, dk, dv = 1, 1, 30, 5, 6
    q, k, v, beta, _ = _delta_inputs(rng, B, H, T, dk, dv)
    alpha = np.exp(-np.abs(rng.standard_normal(T)) * 0.3)
    g_tok = np.log(alpha)[None, None, :].copy()
    g_chan = np.broadcast_to(g_tok[..., None], (B, H, T, dk)).copy()
    S0 = rng.standard_normal((B, H, dk, dv))
    M = S0[0, 0].T.copy()
    Ms = []
    for t in range(T):
        kt = k[0, 0, t][:, None]
        M = alpha[t] * M @ (np.eye(dk) - beta[0, 0, t] * (kt @ kt.T)) \
            + beta[0, 0, t] * (v[0, 0, t][:, None] @ kt.T)
        Ms.append(M.copy())
    for g in (g_chan, g_tok):
        o, S = oracle.delta_recurrent(q, k, v, beta, g, S0, lib=lib)
        for t in range(T):
            _close(o[0, 0, t], Ms[t] @ q[0, 0, t], what=f"scalar gate o {g.ndim}")
        _close(S[0, 0], Ms[-1].T, what=f"scalar gate S {g.ndim}")


def pin_gated_pure_decay_closed_forms(lib):
    """beta = 0: S_T = diag(prod_t a_t) S_0.  One write at t = 1 (beta_1 = 1,
    zero start) followed by decay-only steps: S_T = diag(prod_{t>=2} a_t) k_1^T v_1,
    i.e. a token written at step x and read at x + n carries a_{x+1} ... a_{x+n}."""
    rng = _rng(12)
    B, H, T, dk, dv = 1, 1, 15, 6, 3
    q, k, v, _, g = _delta_inputs(rng, B, H, T, dk, dv, gated=True, gate_scale=0.5)
    S0 = rng.standard_normal((B, H, dk, dv))
    _, S = oracle.delta_recurrent(q, k, v, np.zeros((B, H, T)), g, S0, lib=lib)
    decay = np.exp(g[0, 0].sum(axis=0))
    _close(S[0, 0], decay[:, None] * S0[0, 0], what="pure decay")
    beta = np.zeros((B, H, T))
    beta[0, 0, 0] = 1.0
    _, S = oracle.delta_recurrent(q, k, v, beta, g, None, lib=lib)
    decay = np.exp(g[0, 0, 1:].sum(axis=0))
    _close(S[0, 0], decay[:, None] * np.outer(k[0, 0, 0], v[0, 0, 0]),
           what="write then decay")


def pin_gated_ut_form(lib):
    """Per-channel gated UT form at C = T (cumulative decay G_t = prod_{s<=t} a_s):
    (I + tril(diag(b) (K*G)(K/G)^T, -1)) U = diag(b)(V - (K*G) S0),
    O = (Q*G) S0 + tril((Q*G)(K/G)^T) U,  S_T = diag(G_T) S0 + (K*G_T/G)^T U."""
    rng = _rng(13)
    B, H, T, dk, dv = 1, 2, 24, 6, 5
    q, k, v, beta, g = _delta_inputs(rng, B, H, T, dk, dv, gated=True, gate_scale=0.2)
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = oracle.delta_recurrent(q, k, v, beta, g, S0, lib=lib)
    for h in range(H):
        G = np.exp(np.cumsum(g[0, h], axis=0))
        Kt, Kh, Qt = k[0, h] * G, k[0, h] / G, q[0, h] * G
        Lm = np.tril(beta[0, h][:, None] * (Kt @ Kh.T), -1)
        rhs = beta[0, h][:, None] * (v[0, h] - Kt @ S0[0, h])
        U = scipy.linalg.solve_triangular(np.eye(T) + Lm, rhs, lower=True)
        O = Qt @ S0[0, h] + np.tril(Qt @ Kh.T) @ U
        ST = G[-1][:, None] * S0[0, h] + (k[0, h] * (G[-1] / G)).T @ U
        _close(o[0, h], O, tol=1e-10, what="gated UT o")
        _close(S[0, h], ST, tol=1e-10, what="gated UT S")


# --------------------------------------------------------------------------
# Gated linear attention (scalar decay, no normaliser)
# --------------------------------------------------------------------------

def _gla_inputs(rng, B, H, T, dk, dv, scale=0.3):
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    g = -np.abs(rng.standard_normal((B, H, T))) * scale
    return q, k, v, g


def pin_gla_decayed_quadratic_form(lib):
    """Unrolling S_t = a_t S_{t-1} + k_t^T v_t with G_t = sum_{s<=t} log a_s:
    S_t = e^{G_t} S_0 + sum_{j<=t} e^{G_t - G_j} k_j^T v_j, so
    O = diag(e^G) Q S_0 + (tril(Q K^T) * M) V with M_tj = e^{G_t - G_j}, and
    S_T = e^{G_T} S_0 + (K * e^{G_T - G})^T V."""
    rng = _rng(20)
    B, H, T, dk, dv = 1, 2, 25, 6, 5
    q, k, v, g = _gla_inputs(rng, B, H, T, dk, dv)
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = oracle.gla_recurrent(q, k, v, g, S0, lib=lib)
    for h in range(H):
        G = np.cumsum(g[0, h])
        M = np.tril(np.exp(G[:, None] - G[None, :]))
        Q, K, V = q[0, h], k[0, h], v[0, h]
        O = np.exp(G)[:, None] * (Q @ S0[0, h]) + (np.tril(Q @ K.T) * M) @ V
        ST = np.exp(G[-1]) * S0[0, h] + (K * np.exp(G[-1] - G)[:, None]).T @ V
        _close(o[0, h], O, tol=1e-10, what="gla quadratic o")
        _close(S[0, h], ST, tol=1e-10, what="gla quadratic S")


def pin_gla_limits(lib):
    """No decay (g None, or g = 0) is additive linear attention without a
    normaliser: S_T = S_0 + sum_j k_j^T v_j (in any order), o_t = q_t S_t.
    Decay 0 (g = -inf) keeps only the newest write: S_t = k_t^T v_t,
    o_t = (q_t . k_t) v_t."""
    rng = _rng(21)
    B, H, T, dk, dv = 1, 2, 18, 5, 4
    q, k, v, _ = _gla_inputs(rng, B, H, T, dk, dv)
    S0 = rng.standard_normal((B, H, dk, dv))
    o1, S1 = oracle.gla_recurrent(q, k, v, None, S0, lib=lib)
    o2, S2 = oracle.gla_recurrent(q, k, v, np.zeros((B, H, T)), S0, lib=lib)
    _close(o1, o2, tol=0, what="g=0 o")
    _close(S1, S2, tol=0, what="g=0 S")
    for h in range(H):
        K, V = k[0, h], v[0, h]
        perm = rng.permutation(T)
        _close(S1[0, h], S0[0, h] + K[perm].T @ V[perm], what="additive closed form")
        Sc = S0[0, h] + np.cumsum(K[:, :, None] * V[:, None, :], axis=0)
        _close(o1[0, h], np.einsum("td,tde->te", q[0, h], Sc), what="additive read")
    o3, S3 = oracle.gla_recurrent(q, k, v, np.full((B, H, T), -np.inf), S0, lib=lib)
    for h in range(H):
        _close(S3[0, h], np.outer(k[0, h, -1], v[0, h, -1]), what="a=0 state")
        qk = np.sum(q[0, h] * k[0, h], axis=1)
        _close(o3[0, h], qk[:, None] * v[0, h], what="a=0 out")


# --------------------------------------------------------------------------
# Gradient of the delta rule
# --------------------------------------------------------------------------

def _delta_loss(q, k, v, beta, S0, dO, dST, lib):
    o, S = oracle.delta_recurrent(q, k, v, beta, None, S0, lib=lib)
    return float(np.sum(o * dO) + np.sum(S * dST))


def pin_delta_backward_finite_differences(lib):
    """Every gradient the backward returns matches central differences of
    the forward oracle's loss sum(dO * o) + sum(dST * S_T) (float64)."""
    rng = _rng(30)
    B, H, T, dk, dv = 1, 2, 6, 3, 4
    q, k, v, beta, _ = _delta_inputs(rng, B, H, T, dk, dv)
    S0 = rng.standard_normal((B, H, dk, dv))
    dO = rng.standard_normal((B, H, T, dv))
    dST = rng.standard_normal((B, H, dk, dv))
    grads = oracle.delta_backward(q, k, v, beta, dO, S0, dST, lib=lib)
    names = ("q", "k", "v", "beta", "S0")
    args = dict(q=q, k=k, v=v, beta=beta, S0=S0)
    h = 1e-6
    for name, g in zip(names, grads):
        x = args[name]
        num = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            saved = x[idx]
            x[idx] = saved + h
            lp = _delta_loss(args["q"], args["k"], args["v"], args["beta"], args["S0"], dO, dST, lib)
            x[idx] = saved - h
            lm = _delta_loss(args["q"], args["k"], args["v"], args["beta"], args["S0"], dO, dST, lib)
            x[idx] = saved
            num[idx] = (lp - lm) / (2 * h)
        _close(g, num, tol=1e-6, what=f"d{name} vs finite differences")


def pin_delta_backward_autograd(lib):
    """The backward equals torch autograd through a plain float64 loop of the
    recurrence (read with k, correct with beta (v - r), write k^T u, read
    with q), at a size with several dozen tokens."""
    rng = _rng(31)
    B, H, T, dk, dv = 1, 2, 40, 8, 6
    q, k, v, beta, _ = _delta_inputs(rng, B, H, T, dk, dv)
    S0 = rng.standard_normal((B, H, dk, dv))
    dO = rng.standard_normal((B, H, T, dv))
    dST = rng.standard_normal((B, H, dk, dv))
    tq, tk, tv, tb, tS0 = (torch.tensor(x, dtype=torch.float64, requires_grad=True)
                           for x in (q, k, v, beta, S0))
    S = tS0
    outs = []
    for t in range(T):
        kt = tk[:, :, t]
        r = torch.einsum("bhi,bhij->bhj", kt, S)
        u = tb[:, :, t, None] * (tv[:, :, t] - r)
        S = S + kt[..., :, None] * u[..., None, :]
        outs.append(torch.einsum("bhi,bhij->bhj", tq[:, :, t], S))
    o = torch.stack(outs, 2)
    loss = (o * torch.from_numpy(dO)).sum() + (S * torch.from_numpy(dST)).sum()
    loss.backward()
    grads = oracle.delta_backward(q, k, v, beta, dO, S0, dST, lib=lib)
    for name, g, t in zip(("q", "k", "v", "beta", "S0"), grads, (tq, tk, tv, tb, tS0)):
        _close(g, t.grad.numpy(), tol=1e-11, what=f"d{name} vs autograd")


def _gated_loss(q, k, v, beta, g, S0, dO, dST, lib):
    o, S = oracle.delta_recurrent(q, k, v, beta, g, S0, lib=lib)
    return float(np.sum(o * dO) + np.sum(S * dST))


def pin_gated_backward_finite_differences(lib):
    """With either gate (one decay per token, one per key channel), every
    gradient the backward returns, dg included, matches central differences
    of the gated forward oracle's loss (float64)."""
    rng = _rng(32)
    B, H, T, dk, dv = 1, 2, 6, 3, 4
    for per_channel in (False, True):
        q, k, v, beta, g = _delta_inputs(rng, B, H, T, dk, dv, gated=True, gate_scale=0.5)
        g = np.ascontiguousarray(g if per_channel else g[..., 0])
        S0 = rng.standard_normal((B, H, dk, dv))
        dO = rng.standard_normal((B, H, T, dv))
        dST = rng.standard_normal((B, H, dk, dv))
        grads = oracle.delta_backward(q, k, v, beta, dO, S0, dST, g=g, lib=lib)
        args = dict(q=q, k=k, v=v, beta=beta, S0=S0, g=g)
        h = 1e-6
        for name, gr in zip(("q", "k", "v", "beta", "S0", "g"), grads):
            x = args[name]
            num = np.empty_like(x)
            for idx in np.ndindex(x.shape):
                saved = x[idx]
                x[idx] = saved + h
                lp = _gated_loss(q, k, v, beta, g, S0, dO, dST, lib)
                x[idx] = saved - h
                lm = _gated_loss(q, k, v, beta, g, S0, dO, dST, lib)
                x[idx] = saved
                num[idx] = (lp - lm) / (2 * h)
            _close(gr, num, tol=1e-6,
                   what=f"d{name} vs finite differences ({'channel' if per_channel else 'token'} gate)")


def pin_gated_backward_autograd(lib):
    """With a per-channel gate, the backward equals torch autograd through a
    plain float64 loop (decay the key rows of S, read with k, correct with
    beta (v - r), write k^T u, read with q) at a few dozen tokens."""
    rng = _rng(33)
    B, H, T, dk, dv = 1, 2, 40, 8, 6
    q, k, v, beta, g = _delta_inputs(rng, B, H, T, dk, dv, gated=True, gate_scale=0.25)
    S0 = rng.standard_normal((B, H, dk, dv))
    dO = rng.standard_normal((B, H, T, dv))
    dST = rng.standard_normal((B, H, dk, dv))
    tq, tk, tv, tb, tS0, tg = (torch.tensor(x, dtype=torch.float64, requires_grad=True)
                               for x in (q, k, v, beta, S0, g))
    S = tS0
    outs = []
    for t in range(T):
        S = torch.exp(tg[:, :, t])[..., :, None] * S
        kt = tk[:, :, t]
        r = (kt[..., :, None] * S).sum(-2)
        u = tb[:, :, t, None] * (tv[:, :, t] - r)
        S = S + kt[..., :, None] * u[..., None, :]
        outs.append((tq[:, :, t][..., :, None] * S).sum(-2))
    o = torch.stack(outs, 2)
    loss = (o * torch.from_numpy(dO)).sum() + (S * torch.from_numpy(dST)).sum()
    loss.backward()
    grads = oracle.delta_backward(q, k, v, beta, dO, S0, dST, g=g, lib=lib)
    for name, gr, t in zip(("q", "k", "v", "beta", "S0", "g"), grads, (tq, tk, tv, tb, tS0, tg)):
        _close(gr, t.grad.numpy(), tol=1e-11, what=f"d{name} vs autograd (channel gate)")


def pin_gated_backward_rescaling_identity(lib):
    """One decay per token: dividing S_t by the cumulative decay Gamma_t
    turns the gated rule into the ungated one with q_t scaled by Gamma_t and
    v_t divided by it (the erase I - beta k k^T is scale free), and the final
    state is Gamma_T times the rescaled one.  So the gradient of
    G_t = log Gamma_t is q_t . dq_t - v_t . dv_t (plus dST . S_T at t = T),
    and dg_t is the sum of those from t to the end.  With g = 0 both gates
    give the ungated gradients; a per-channel gate with equal channels gives
    the per-token one, and its dg summed over the channels."""
    rng = _rng(34)
    B, H, T, dk, dv = 2, 2, 50, 8, 5
    q, k, v, beta, g = _delta_inputs(rng, B, H, T, dk, dv, gated=True, gate_scale=0.3)
    gt = np.ascontiguousarray(g[..., 0])
    S0 = rng.standard_normal((B, H, dk, dv))
    dO = rng.standard_normal((B, H, T, dv))
    dST = rng.standard_normal((B, H, dk, dv))
    dq, dk_, dv_, db, dS0, dg = oracle.delta_backward(q, k, v, beta, dO, S0, dST, g=gt, lib=lib)
    _, ST = oracle.delta_recurrent(q, k, v, beta, gt, S0, lib=lib)
    dG = np.sum(q * dq, -1) - np.sum(v * dv_, -1)
    dG[..., -1] += np.sum(dST * ST, axis=(-2, -1))
    _close(dg, np.flip(np.cumsum(np.flip(dG, -1), -1), -1), tol=1e-10, what="dg vs rescaling identity")
    # equal channels: the per-channel gate is the per-token one
    gc = np.ascontiguousarray(np.repeat(gt[..., None], dk, -1))
    ch = oracle.delta_backward(q, k, v, beta, dO, S0, dST, g=gc, lib=lib)
    for name, a, b in zip(("q", "k", "v", "beta", "S0"), ch[:5], (dq, dk_, dv_, db, dS0)):
        _close(a, b, tol=1e-12, what=f"d{name}: equal channels vs per-token gate")
    _close(ch[5].sum(-1), dg, tol=1e-12, what="dg: channels summed vs per-token gate")
    # zero gate: the ungated gradients, and dg = dG summed as above
    ung = oracle.delta_backward(q, k, v, beta, dO, S0, dST, lib=lib)
    for gz in (np.zeros_like(gt), np.zeros_like(g)):
        z = oracle.delta_backward(q, k, v, beta, dO, S0, dST, g=gz, lib=lib)
        for name, a, b in zip(("q", "k", "v", "beta", "S0"), z[:5], ung):
            _close(a, b, tol=1e-12, what=f"d{name}: zero gate vs ungated")


# --------------------------------------------------------------------------
# The layer's prologue: q, k = normalize(silu(.)), beta = sigmoid(.)
# --------------------------------------------------------------------------

def pin_prologue_facts(lib):
    """Rows come out with norm `scale` and point along silu(x): silu is
    x * sigmoid(x), so silu(0) = 0, silu(x) -> x for large x and -> 0 for
    very negative x, and the ratio of two silu values at a, b is the ratio
    a s(a) / (b s(b)); a zero row stays zero (the 1e-12 floor).  sigmoid(0)
    = 1/2 and sigmoid(-z) = 1 - sigmoid(z); one-head logits give every head
    the same beta."""
    x = np.array([[0.0, 40.0, -40.0, 1.0], [0.5, -0.5, 2.0, -3.0], [0.0, 0.0, 0.0, 0.0]])
    out = oracle.qk_prologue(x, True, 2.5, lib=lib)
    _close(np.linalg.norm(out[:2], axis=1), np.array([2.5, 2.5]), tol=1e-14, what="row norms")
    _close(out[2], np.zeros(4), tol=0, what="zero row")
    r0 = out[0] / 2.5 * np.linalg.norm([0.0, 40.0, 0.0, 1.0 / (1.0 + np.exp(-1.0))])
    _close(r0[[0, 2]], np.zeros(2), tol=1e-15, what="silu(0), silu(-40)")
    _close(r0[1], 40.0, tol=1e-14, what="silu(40)")
    sg = lambda z: 1.0 / (1.0 + np.exp(-z))  # noqa: E731  (the logistic function's definition)
    ratio = out[1, 0] / out[1, 2]
    _close(ratio, (0.5 * sg(0.5)) / (2.0 * sg(2.0)), tol=1e-14, what="silu ratio")
    plain = oracle.qk_prologue(x[:2], False, 1.0, lib=lib)
    _close(plain, x[:2] / np.linalg.norm(x[:2], axis=1, keepdims=True), tol=1e-15, what="no silu")
    lg = np.array([[[0.0, 1.5, -1.5, 30.0]]])
    be = oracle.beta_sigmoid(lg, 3, lib=lib)
    _close(be[0, 0, 0], 0.5, tol=0, what="sigmoid(0)")
    _close(be[0, 0, 1] + be[0, 0, 2], 1.0, tol=1e-15, what="sigmoid symmetry")
    _close(be[0, 1], be[0, 0], tol=0, what="head broadcast")
    _close(be[0, 2], be[0, 0], tol=0, what="head broadcast")
    lg3 = np.random.default_rng(40).standard_normal((2, 3, 5))
    be3 = oracle.beta_sigmoid(lg3, 3, lib=lib)
    _close(be3 + oracle.beta_sigmoid(-lg3, 3, lib=lib), np.ones_like(be3), tol=1e-15,
           what="per-head symmetry")
    # per-head logits: head h reads its own logit (sigmoid is increasing, and
    # a zero logit gives exactly 1/2 in the head that holds it)
    lgh = np.array([[[0.0, -2.0], [1.0, 0.0], [3.0, 2.0]]])
    bh = oracle.beta_sigmoid(lgh, 3, lib=lib)
    assert np.all(np.diff(bh[0], axis=0) > 0), "beta must follow each head's own logit"
    _close(np.array([bh[0, 0, 0], bh[0, 1, 1]]), np.array([0.5, 0.5]), tol=0, what="own head")


# --------------------------------------------------------------------------
# Input handling and state carry
# --------------------------------------------------------------------------

def pin_stored_precision_widening(lib):
    """bf16 and fp32 inputs are widened exactly: the result equals the one on
    the same values given as float64 (widened by torch)."""
    gen = torch.Generator().manual_seed(14)
    q, k, v = (torch.randn(1, 2, 9, 8, generator=gen) for _ in range(3))
    beta = torch.sigmoid(torch.randn(1, 2, 9, generator=gen))
    g = -F.softplus(torch.randn(1, 2, 9, 8, generator=gen)) / 4
    for dt in (torch.bfloat16, torch.float32):
        args = [t.to(dt) for t in (q, k, v, beta, g)]
        o1, S1 = oracle.delta_recurrent(*args, lib=lib)
        o2, S2 = oracle.delta_recurrent(*[t.double() for t in args], lib=lib)
        _close(o1, o2, tol=0, what="widening delta o")
        _close(S1, S2, tol=0, what="widening delta S")
        la1 = oracle.la_recurrent(*args[:3], lib=lib)
        la2 = oracle.la_recurrent(*[t.double() for t in args[:3]], lib=lib)
        for a, b in zip(la1, la2):
            _close(a, b, tol=0, what="widening la")
        gs = args[4][..., 0].contiguous()
        gl1 = oracle.gla_recurrent(*args[:3], gs, lib=lib)
        gl2 = oracle.gla_recurrent(*[t.double() for t in args[:3]], gs.double(), lib=lib)
        for a, b in zip(gl1, gl2):
            _close(a, b, tol=0, what="widening gla")


def pin_state_carry(lib):
    """Two calls chained through the returned state equal one call over the
    concatenated tokens, and T one-token calls equal one T-token call."""
    rng = _rng(15)
    B, H, T, dk, dv = 1, 2, 20, 5, 4
    q, k, v, beta, g = _delta_inputs(rng, B, H, T, dk, dv, gated=True)
    o, S = oracle.delta_recurrent(q, k, v, beta, g, lib=lib)
    o1, S1 = oracle.delta_recurrent(q[:, :, :7], k[:, :, :7], v[:, :, :7],
                                    beta[:, :, :7], g[:, :, :7], lib=lib)
    o2, S2 = oracle.delta_recurrent(q[:, :, 7:], k[:, :, 7:], v[:, :, 7:],
                                    beta[:, :, 7:], g[:, :, 7:], S1, lib=lib)
    _close(np.concatenate([o1, o2], axis=2), o, what="carry o")
    _close(S2, S, what="carry S")
    St = None
    for t in range(T):
        ot, St = oracle.delta_recurrent(q[:, :, t:t + 1], k[:, :, t:t + 1],
                                        v[:, :, t:t + 1], beta[:, :, t:t + 1],
                                        g[:, :, t:t + 1], St, lib=lib)
        _close(ot[:, :, 0], o[:, :, t], what="step o")
    _close(St, S, what="step S")
    qa, ka, va = (rng.standard_normal((B, H, T, d)) for d in (dk, dk, dv))
    oa, Sa, za = oracle.la_recurrent(qa, ka, va, lib=lib)
    ob1, Sb1, zb1 = oracle.la_recurrent(qa[:, :, :11], ka[:, :, :11], va[:, :, :11], lib=lib)
    ob2, Sb2, zb2 = oracle.la_recurrent(qa[:, :, 11:], ka[:, :, 11:], va[:, :, 11:],
                                        Sb1, zb1, lib=lib)
    _close(np.concatenate([ob1, ob2], axis=2), oa, what="la carry o")
    _close(Sb2, Sa, what="la carry S")
    _close(zb2, za, what="la carry z")
    gg = -np.abs(rng.standard_normal((B, H, T))) * 0.2
    oc, Sc = oracle.gla_recurrent(qa, ka, va, gg, lib=lib)
    oc1, Sc1 = oracle.gla_recurrent(qa[:, :, :9], ka[:, :, :9], va[:, :, :9], gg[:, :, :9],
                                    lib=lib)
    oc2, Sc2 = oracle.gla_recurrent(qa[:, :, 9:], ka[:, :, 9:], va[:, :, 9:], gg[:, :, 9:],
                                    Sc1, lib=lib)
    _close(np.concatenate([oc1, oc2], axis=2), oc, what="gla carry o")
    _close(Sc2, Sc, what="gla carry S")


ALL_PINS = [
    pin_la_quadratic_masked_form,
    pin_la_closed_form_state,
    pin_la_convex_hull_and_running_mean,
    pin_la_elu_branches,
    pin_delta_ut_form,
    pin_delta_householder_form,
    pin_delta_chunk_size_invariance,
    pin_delta_exact_retrieval,
    pin_delta_replacement,
    pin_delta_one_step_identities,
    pin_gated_limits,
    pin_gated_scalar_householder,
    pin_gated_pure_decay_closed_forms,
    pin_gated_ut_form,
    pin_gla_decayed_quadratic_form,
    pin_gla_limits,
    pin_delta_backward_finite_differences,
    pin_delta_backward_autograd,
    pin_gated_backward_finite_differences,
    pin_gated_backward_autograd,
    pin_gated_backward_rescaling_identity,
    pin_prologue_facts,
    pin_stored_precision_widening,
    pin_state_carry,
]


def run_all(lib) -> list[str]:
    """Run every pin against ``lib``; return the names of the pins that fail."""
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(lib)
        except AssertionError:
            failed.append(pin.__name__)
    return failed


if __name__ == "__main__":   # used by the planted-mistake test in a subprocess
    import sys
    lib = oracle.load(sys.argv[1]) if len(sys.argv) > 1 else oracle.load()
    bad = run_all(lib)
    print("FAILED:" + ",".join(bad))
    sys.exit(1 if bad else 0)
