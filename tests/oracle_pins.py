"""Pins for the fp64 oracle: checks against things other than the oracle.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with what the pages or the mathematics fix. They are run
against the real oracle (all must pass) and against deliberately wrong
builds of it (each wrong build must fail at least one pin).

Sources of truth used here, none of which is the oracle itself:
  * hand-derived fixtures under tests/golden/ (exact rational answers);
  * torch's scaled_dot_product_attention in fp64 on the CPU, for the
    statement that W_R = 0 gives plain softmax attention (zubnet.ai news
    item, second paragraph; encorp.ai blog, section on keeping softmax);
  * numpy's weighted covariance (np.cov with aweights) for the closed form
    with affine values;
  * numpy's least-squares solver for the local-linear intercept: with the
    probe set to the exact local-linear solve, the output is the intercept
    of the softmax-weighted linear fit (pages describe Parallax as a
    parameterised local linear attention whose learned probe replaces the
    per-query solve: encorp.ai blog, sections on keeping softmax and on
    removing the conjugate-gradient solver);
  * invariances of a weighted mean and a covariance;
  * for the exact local-linear probe (conjugate gradient), numpy's least
    squares on the softmax-weighted fit with ridge rows appended, and the
    closed forms of identical keys and of a query at the key mean.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert np.all(np.isfinite(a)), f"{what}: non-finite output"
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def sdpa_f64(q, k, v, scale, causal):
    """q: [B,H,Nq,D], k/v: [B,H,Nk,D] numpy -> numpy, torch fp64 CPU."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    o = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), is_causal=causal, scale=scale)
    return o.numpy()


# --------------------------------------------------------------- fixtures

def pin_golden_causal(orc):
    with open(os.path.join(GOLDEN, "hand_causal_n3_d2.json")) as f:
        g = json.load(f)
    shp = (1, 3, 1, 2)
    arr = lambda key: np.array(g[key], dtype=np.float64).reshape(shp)
    o = orc.fwd(arr("q"), arr("k"), arr("v"), arr("rho"), scale=g["scale"],
                causal=True)
    _close(o.reshape(3, 2), g["expected"], g["tolerance"], "golden causal")


def pin_golden_decode(orc):
    with open(os.path.join(GOLDEN, "hand_decode_d1.json")) as f:
        g = json.load(f)
    q = np.array(g["q"]).reshape(1, 1, 1)
    k = np.array(g["k"]).reshape(1, 1, 2, 1)
    v = np.array(g["v"]).reshape(1, 1, 2, 1)
    rho = np.array(g["rho"]).reshape(1, 1, 1)
    o = orc.decode(q, rho, k, v, scale=g["scale"])
    _close(o.reshape(1), g["expected"], g["tolerance"], "golden decode")
    o0 = orc.decode(q, np.zeros_like(rho), k, v, scale=g["scale"])
    _close(o0.reshape(1), g["expected_rho_zero"], g["tolerance"],
           "golden decode rho=0")


# ---------------------------------------------------- softmax reduction

def pin_rho_zero_decode_is_sdpa(orc):
    r = _rng(11)
    B, H, L, D = 2, 3, 37, 8
    q = r.standard_normal((B, H, D))
    k = r.standard_normal((B, H, L, D))
    v = r.standard_normal((B, H, L, D))
    scale = 0.37
    seqlens = np.array([37, 19], dtype=np.int32)
    o = orc.decode(q, np.zeros_like(q), k, v, seqlens=seqlens, scale=scale)
    for b in range(B):
        n = seqlens[b]
        ref = sdpa_f64(q[b:b + 1, :, None, :], k[b:b + 1, :, :n],
                       v[b:b + 1, :, :n], scale, False)[:, :, 0, :]
        _close(o[b:b + 1], ref, 1e-12, f"rho=0 decode b={b}")


def pin_rho_zero_fwd_is_sdpa(orc):
    r = _rng(12)
    B, N, H, D = 2, 29, 2, 6
    q, k, v = (r.standard_normal((B, N, H, D)) for _ in range(3))
    scale = 1.3
    for causal in (True, False):
        o = orc.fwd(q, k, v, np.zeros_like(q), scale=scale, causal=causal)
        ref = sdpa_f64(q.transpose(0, 2, 1, 3), k.transpose(0, 2, 1, 3),
                       v.transpose(0, 2, 1, 3), scale, causal)
        _close(o, ref.transpose(0, 2, 1, 3), 1e-12, f"rho=0 fwd causal={causal}")


# ----------------------------------------------------------- closed forms

def pin_single_key(orc):
    r = _rng(13)
    D, Lmax = 5, 9
    q, rho = r.standard_normal((1, 1, D)), r.standard_normal((1, 1, D)) * 3
    k = r.standard_normal((1, 1, Lmax, D))
    v = r.standard_normal((1, 1, Lmax, D))
    k[:, :, 1:] = np.nan  # positions beyond the length must not be read
    v[:, :, 1:] = np.nan
    o = orc.decode(q, rho, k, v, seqlens=np.array([1], np.int32), scale=0.5)
    assert np.array_equal(o[0, 0], v[0, 0, 0]), "single key must return v_0"
    # causal row 0 of a prefill sees one key
    B, N, H = 1, 7, 2
    q2, k2, v2, rho2 = (r.standard_normal((B, N, H, D)) for _ in range(4))
    o2 = orc.fwd(q2, k2, v2, rho2 * 5, scale=0.7, causal=True)
    assert np.array_equal(o2[0, 0], v2[0, 0]), "causal row 0 must return v_0"


def pin_degenerate_keys_values(orc):
    r = _rng(14)
    D, L = 4, 11
    q, rho = r.standard_normal((1, 1, D)), r.standard_normal((1, 1, D)) * 2
    # identical keys: uniform weights, zero covariance -> mean of values
    k = np.broadcast_to(r.standard_normal(D), (1, 1, L, D)).copy()
    v = r.standard_normal((1, 1, L, D))
    o = orc.decode(q, rho, k, v, scale=0.9)
    _close(o[0, 0], v[0, 0].mean(axis=0), 1e-13, "identical keys")
    # constant values -> that constant
    k = r.standard_normal((1, 1, L, D))
    c = r.standard_normal(D)
    v = np.broadcast_to(c, (1, 1, L, D)).copy()
    o = orc.decode(q, rho, k, v, scale=0.9)
    _close(o[0, 0], c, 1e-13, "constant values")


def pin_affine_values(orc):
    """v_j = A k_j + b  =>  o = A kbar + b - A Sigma_kk rho."""
    r = _rng(15)
    D, L = 6, 23
    q, rho = r.standard_normal(D), r.standard_normal(D)
    K = r.standard_normal((L, D))
    A = r.standard_normal((D, D))
    b = r.standard_normal(D)
    V = K @ A.T + b
    scale = 0.45
    p = scipy.special.softmax(scale * (K @ q))
    kbar = np.average(K, axis=0, weights=p)
    S = np.cov(K.T, aweights=p, bias=True)
    expect = A @ kbar + b - A @ S @ rho
    o = orc.decode(q[None, None], rho[None, None], K[None, None], V[None, None],
                   scale=scale)
    _close(o[0, 0], expect, 1e-11, "affine values")


def pin_local_linear_intercept(orc):
    """rho = Sigma_kk^{-1}(kbar - q)  =>  o = weighted LS intercept at q."""
    r = _rng(16)
    D, L = 4, 40
    q = r.standard_normal(D)
    K = r.standard_normal((L, D))
    V = r.standard_normal((L, D))
    scale = 0.5
    p = scipy.special.softmax(scale * (K @ q))
    kbar = np.average(K, axis=0, weights=p)
    S = np.cov(K.T, aweights=p, bias=True)
    rho = np.linalg.solve(S, kbar - q)
    X = np.hstack([np.ones((L, 1)), K - q])
    w = np.sqrt(p)[:, None]
    coef, *_ = np.linalg.lstsq(w * X, w * V, rcond=None)
    o = orc.decode(q[None, None], rho[None, None], K[None, None], V[None, None],
                   scale=scale)
    _close(o[0, 0], coef[0], 1e-9, "local-linear intercept")
    # with affine values the intercept is the exact value at q
    A = r.standard_normal((D, D))
    b = r.standard_normal(D)
    Va = K @ A.T + b
    o = orc.decode(q[None, None], rho[None, None], K[None, None],
                   Va[None, None], scale=scale)
    _close(o[0, 0], A @ q + b, 1e-9, "local-linear intercept, affine values")


# ------------------------------------------------------------- invariances

def pin_invariances(orc):
    r = _rng(17)
    B, H, L, D = 1, 2, 21, 5
    q, rho = r.standard_normal((B, H, D)), r.standard_normal((B, H, D))
    k, v = r.standard_normal((B, H, L, D)), r.standard_normal((B, H, L, D))
    s = 0.6
    o = orc.decode(q, rho, k, v, scale=s)
    c = r.standard_normal(D)
    _close(orc.decode(q, rho, k + c, v, scale=s), o, 1e-12, "key translation")
    _close(orc.decode(q, rho, k, v + c, scale=s), o + c, 1e-12,
           "value translation")
    v2 = r.standard_normal((B, H, L, D))
    o2 = orc.decode(q, rho, k, v2, scale=s)
    _close(orc.decode(q, rho, k, 2.0 * v - 3.0 * v2, scale=s), 2 * o - 3 * o2,
           1e-12, "linear in V")
    rho2 = r.standard_normal((B, H, D))
    o0 = orc.decode(q, np.zeros_like(rho), k, v, scale=s)
    _close(orc.decode(q, rho + rho2, k, v, scale=s),
           o + orc.decode(q, rho2, k, v, scale=s) - o0, 1e-12, "affine in rho")
    perm = r.permutation(L)
    _close(orc.decode(q, rho, k[:, :, perm], v[:, :, perm], scale=s), o,
           1e-12, "key/value permutation")


# ----------------------------------------------- one-pass and split-merge

def pin_onepass_equals_twopass(orc, D=5, L=13, chunk=3, seed=18, scale=0.8):
    r = _rng(seed)
    q, rho = r.standard_normal((1, 1, D)), r.standard_normal((1, 1, D))
    k, v = r.standard_normal((1, 1, L, D)), r.standard_normal((1, 1, L, D))
    a = orc.decode(q, rho, k, v, scale=scale)
    b = orc.decode_onepass(q, rho, k, v, scale=scale, chunk=chunk)
    _close(b, a, 1e-12, "one-pass vs explicit covariance")


def pin_split_merge(orc):
    r = _rng(19)
    D, L = 7, 50
    q, rho = r.standard_normal(D), r.standard_normal(D)
    K, V = r.standard_normal((L, D)), r.standard_normal((L, D))
    s = 0.4
    whole = orc.decode(q[None, None], rho[None, None], K[None, None],
                       V[None, None], scale=s)[0, 0]
    cuts = [0, 3, 3, 17, 31, 50]  # includes an empty piece
    states = [orc.decode_partial(q, rho, K, V, a, b, s, chunk=4)
              for a, b in zip(cuts[:-1], cuts[1:])]
    _close(orc.merge(states), whole, 1e-12, "split-merge")
    _close(orc.merge(states[::-1]), whole, 1e-12, "split-merge reversed")


# ------------------------------------------------------- prefill structure

def pin_causal_row_is_prefix_decode(orc):
    r = _rng(20)
    B, N, H, D = 2, 17, 2, 4
    q, k, v, rho = (r.standard_normal((B, N, H, D)) for _ in range(4))
    s = 0.55
    o = orc.fwd(q, k, v, rho, scale=s, causal=True)
    full = orc.fwd(q, k, v, rho, scale=s, causal=False)
    kk = k.transpose(0, 2, 1, 3)
    vv = v.transpose(0, 2, 1, 3)
    for i in (0, 1, 8, N - 1):
        dec = orc.decode(q[:, i], rho[:, i], kk, vv,
                         seqlens=np.full(B, i + 1, np.int32), scale=s)
        _close(o[:, i], dec, 1e-12, f"causal row {i} vs prefix decode")
        dec = orc.decode(q[:, i], rho[:, i], kk, vv, scale=s)
        _close(full[:, i], dec, 1e-12, f"full row {i} vs decode")
    rows = [(0, 0, 1), (1, 16, 0), (1, 5, 1)]
    sel = orc.fwd_rows(q, k, v, rho, rows, scale=s, causal=True)
    for n, (b, i, h) in enumerate(rows):
        _close(sel[n], o[b, i, h], 0.0, "fwd_rows")


def pin_lengths(orc):
    r = _rng(21)
    B, H, L, D = 3, 2, 10, 3
    q, rho = r.standard_normal((B, H, D)), r.standard_normal((B, H, D))
    k, v = r.standard_normal((B, H, L, D)), r.standard_normal((B, H, L, D))
    sl = np.array([0, 4, 10], np.int32)
    kp, vp = k.copy(), v.copy()
    for b in range(B):
        kp[b, :, sl[b]:] = np.nan
        vp[b, :, sl[b]:] = np.nan
    o = orc.decode(q, rho, kp, vp, seqlens=sl, scale=0.5)
    assert np.array_equal(o[0], np.zeros((H, D))), "empty context -> zeros"
    ref = orc.decode(q[1:2], rho[1:2], k[1:2, :, :4], v[1:2, :, :4], scale=0.5)
    _close(o[1:2], ref, 0.0, "length 4 == truncated cache")
    op = orc.decode_onepass(q, rho, kp, vp, seqlens=sl, scale=0.5, chunk=3)
    _close(op, o, 1e-12, "one-pass with lengths")


# --------------------------------------------------------------- backward

def _loss_fd(orc, x, dout, scale, causal, h=1e-6):
    """Central differences of L = sum(dout * fwd(q, k, v, rho)) w.r.t. each
    element of each input, from the forward oracle alone."""
    grads = []
    for idx in range(4):
        g = np.zeros_like(x[idx])
        it = np.nditer(x[idx], flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            xp = [a.copy() for a in x]
            xm = [a.copy() for a in x]
            xp[idx][mi] += h
            xm[idx][mi] -= h
            lp = float(np.sum(dout * orc.fwd(*xp, scale=scale, causal=causal)))
            lm = float(np.sum(dout * orc.fwd(*xm, scale=scale, causal=causal)))
            g[mi] = (lp - lm) / (2.0 * h)
        grads.append(g)
    return grads


def pin_bwd_finite_differences(orc):
    """Each gradient equals central differences of the forward output
    (the pages define only the forward; its derivative is unique)."""
    r = _rng(31)
    for causal, scale in ((True, 0.7), (False, 1.3)):
        B, N, H, D = 1, 4, 2, 3
        x = [r.standard_normal((B, N, H, D)) for _ in range(4)]
        dout = r.standard_normal((B, N, H, D))
        got = orc.bwd(*x, dout, scale=scale, causal=causal)
        ref = _loss_fd(orc, x, dout, scale, causal)
        for name, a, e in zip(("dq", "dk", "dv", "drho"), got, ref):
            _close(a, e, 1e-7, f"{name} vs finite differences (causal={causal})")


def pin_bwd_drho_is_minus_cov_t_g(orc):
    """o_i = vbar_i - C_i rho_i is linear in rho_i, so
    d rho_i = -C_i^T g_i with C_i the softmax-weighted covariance."""
    r = _rng(32)
    B, N, H, D = 2, 6, 1, 4
    q, k, v, rho, dout = (r.standard_normal((B, N, H, D)) for _ in range(5))
    scale = 0.9
    _, _, _, drho = orc.bwd(q, k, v, rho, dout, scale=scale, causal=True)
    for b in range(B):
        for i in range(N):
            K, V = k[b, :i + 1, 0], v[b, :i + 1, 0]
            w = scipy.special.softmax(scale * (K @ q[b, i, 0]))
            C = np.cov(V.T, K.T, aweights=w, bias=True)[:D, D:] if i > 0 else np.zeros((D, D))
            _close(drho[b, i, 0], -C.T @ dout[b, i, 0], 1e-12, f"drho row {i}")


def pin_bwd_shift_invariances(orc):
    """Adding one vector to every key leaves every output unchanged (the
    softmax sees a per-query constant, the covariance is centred), so the
    key gradients sum to zero; adding one vector to every value adds it to
    every output, so the value gradients sum to the summed output grads."""
    r = _rng(33)
    B, N, H, D = 2, 7, 3, 5
    x = [r.standard_normal((B, N, H, D)) for _ in range(4)]
    dout = r.standard_normal((B, N, H, D))
    for causal in (True, False):
        dq, dk, dv, drho = orc.bwd(*x, dout, scale=0.6, causal=causal)
        _close(dk.sum(axis=1), np.zeros((B, H, D)), 1e-12, "sum_j dk_j")
        _close(dv.sum(axis=1), dout.sum(axis=1), 1e-12, "sum_j dv_j")
        # linear in rho: rho_i . drho_i = g_i . (o_i - vbar_i), vbar from sdpa
        o = orc.fwd(*x, scale=0.6, causal=causal)
        t = lambda a: a.transpose(0, 2, 1, 3)
        vbar = t(sdpa_f64(t(x[0]), t(x[1]), t(x[2]), 0.6, causal))
        _close((x[3] * drho).sum(-1), (dout * (o - vbar)).sum(-1), 1e-12,
               "Euler relation in rho")


def pin_bwd_rho_zero_is_sdpa_grad(orc):
    """With rho = 0 the layer is softmax attention: dq, dk, dv equal the
    autograd gradients of torch's attention in fp64 on the CPU."""
    r = _rng(34)
    B, N, H, D = 2, 6, 2, 4
    q, k, v, dout = (r.standard_normal((B, N, H, D)) for _ in range(4))
    rho = np.zeros_like(q)
    for causal in (True, False):
        dq, dk, dv, _ = orc.bwd(q, k, v, rho, dout, scale=0.7, causal=causal)
        tt = [torch.from_numpy(a.transpose(0, 2, 1, 3).copy()).requires_grad_(True)
              for a in (q, k, v)]
        o = torch.nn.functional.scaled_dot_product_attention(
            *tt, is_causal=causal, scale=0.7)
        (o * torch.from_numpy(dout.transpose(0, 2, 1, 3).copy())).sum().backward()
        for name, a, t in zip(("dq", "dk", "dv"), (dq, dk, dv), tt):
            _close(a, t.grad.numpy().transpose(0, 2, 1, 3), 1e-12, f"{name} (rho = 0)")


# ------------------------------------------------- exact local-linear probe

def _ridge_intercept(q, K, V, p, lam):
    """Intercept a of min_a,B sum_j p_j |v_j - a - B (k_j - q)|^2 + lam |B|^2,
    by least squares with the ridge rows appended (numpy)."""
    n, D = K.shape
    w = np.sqrt(p)[:, None]
    X = np.hstack([np.ones((n, 1)), K - q]) * w
    Y = V * w
    if lam > 0:
        X = np.vstack([X, np.hstack([np.zeros((D, 1)), math.sqrt(lam) * np.eye(D)])])
        Y = np.vstack([Y, np.zeros((D, V.shape[1]))])
    coef, *_ = np.linalg.lstsq(X, Y, rcond=None)
    return coef[0]


def pin_lla_probe_ridge_intercept(orc):
    """With the conjugate-gradient probe, the Parallax output is the intercept
    of the softmax-weighted local linear fit with a ridge penalty on the
    slope (numpy least squares), causal and not, with and without ridge."""
    r = _rng(41)
    N, D, scale = 14, 4, 0.7
    q = r.standard_normal((1, N, 1, D))
    k = r.standard_normal((1, N, 1, D)) * 1.3
    v = r.standard_normal((1, N, 1, D))
    for lam, causal in ((0.3, True), (0.3, False), (0.0, False), (2.5, True)):
        rho, its = orc.lla_probe(q, k, scale=scale, causal=causal, lam=lam,
                                 allow_unconverged=True)
        o = orc.fwd(q, k, v, rho, scale=scale, causal=causal)
        for i in range(N):
            n = i + 1 if causal else N
            if lam == 0.0 and n <= D + 1:
                continue                      # singular without ridge
            K, V = k[0, :n, 0], v[0, :n, 0]
            p = scipy.special.softmax(scale * (K @ q[0, i, 0]))
            want = _ridge_intercept(q[0, i, 0], K, V, p, lam)
            _close(o[0, i, 0], want, 1e-8, f"LLA intercept lam={lam} causal={causal} i={i}")


def pin_lla_probe_closed_forms(orc):
    """Identical keys: the covariance vanishes and the probe is (k - q)/lam
    exactly; a query equal to the weighted key mean gets the zero probe."""
    r = _rng(43)
    N, D = 9, 6
    q = r.standard_normal((1, N, 2, D))
    c = r.standard_normal(D)
    k = np.broadcast_to(c, (1, N, 2, D)).copy()
    for lam in (0.5, 3.0):
        rho, _ = orc.lla_probe(q, k, causal=True, lam=lam, allow_unconverged=True)
        _close(rho, (c - q) / lam, 1e-12, f"identical keys lam={lam}")
    # q = kbar: with equal logits for every key (q orthogonal to all keys is
    # not needed: scale 0 makes the weights uniform) kbar is the plain mean
    k = r.standard_normal((1, N, 1, D))
    q = np.broadcast_to(k[0].mean(axis=0), (1, N, 1, D)).copy()
    rho, _ = orc.lla_probe(q, k, scale=0.0, causal=False, lam=0.7,
                           allow_unconverged=True)
    _close(rho, np.zeros_like(rho), 1e-12, "q = kbar")


# ---------------------------------------------------- fused input projection

def pin_project_brute_force(orc=None):
    """The projection equals the element-by-element sum on tiny inputs
    (catches a transposed operand), and zero W_R rows give a zero probe."""
    import oracle
    r = _rng(47)
    M, N, K = 5, 8, 3
    x, w = r.standard_normal((M, K)), r.standard_normal((N, K))
    want = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            for k in range(K):
                want[m, n] += x[m, k] * w[n, k]
    _close(oracle.project(x, w), want, 1e-12, "projection brute force")
    w[6:] = 0.0
    _close(oracle.project(x, w)[:, 6:], np.zeros((M, 2)), 0.0, "zero W_R rows")


ALL_PINS = [
    pin_golden_causal, pin_golden_decode, pin_rho_zero_decode_is_sdpa,
    pin_rho_zero_fwd_is_sdpa, pin_single_key, pin_degenerate_keys_values,
    pin_affine_values, pin_local_linear_intercept, pin_invariances,
    pin_onepass_equals_twopass, pin_split_merge,
    pin_causal_row_is_prefix_decode, pin_lengths,
    pin_bwd_finite_differences, pin_bwd_drho_is_minus_cov_t_g,
    pin_bwd_shift_invariances, pin_bwd_rho_zero_is_sdpa_grad,
    pin_lla_probe_ridge_intercept, pin_lla_probe_closed_forms,
    pin_project_brute_force,
]
