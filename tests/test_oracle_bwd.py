"""Pins for the oracle's backward pass (no GPU needed).

The pages implement only the forward, so the gradients are the plain chain
rule through the forward definition.  They are tied here to things other than
the backward code itself: central finite differences of the (separately
pinned) forward oracle, 40-digit finite differences of a brute-force forward,
the autograd of torch's CPU attention in fp64, and closed forms that follow
from the definition (sums of dV and dK, homogeneity in q/k and in v, the
constant-V and single-key cases, causal structure, and
delta_i = dout_i . o_i).  The last test plants mistakes in copies of the C
source; each must be caught by a pin.
"""
import os
import shutil
import tempfile

import mpmath
import numpy as np
import pytest
import torch

import oracle


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def problem(B, H, Lq, Lk, D, seed):
    q = rnd((B, H, Lq, D), seed)
    k = rnd((B, H, Lk, D), seed + 1)
    v = rnd((B, H, Lk, D), seed + 2)
    g = rnd((B, H, Lq, D), seed + 3)
    return q, k, v, g


def loss(q, k, v, g, causal, scale, lib):
    o, _ = oracle.attention(q, k, v, causal, scale, lib=lib)
    return float(np.sum(o * g))


# --------------------------------------------------------------------------
# Pins
# --------------------------------------------------------------------------

def pin_finite_differences(lib):
    """Every gradient entry against a central difference of
    L = sum(dout * o), with o from the forward oracle."""
    cases = [((1, 2, 5, 7, 4), False, 0.7), ((1, 2, 5, 7, 4), True, 0.7),
             ((1, 1, 6, 3, 3), True, 1.3), ((2, 1, 3, 9, 2), False, -0.4),
             ((1, 1, 1, 1, 2), False, 0.5), ((1, 1, 4, 4, 5), True, 0.45)]
    h = 1e-6
    for n, ((B, H, Lq, Lk, D), causal, scale) in enumerate(cases):
        q, k, v, g = problem(B, H, Lq, Lk, D, 300 + 10 * n)
        grads = oracle.attention_bwd(q, k, v, g, causal, scale, lib=lib)
        for t, (x, gx) in enumerate(zip((q, k, v), grads)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                args = [q.copy(), k.copy(), v.copy()]
                args[t][idx] += h
                lp = loss(*args, g, causal, scale, lib)
                args[t][idx] -= 2 * h
                lm = loss(*args, g, causal, scale, lib)
                num[idx] = (lp - lm) / (2 * h)
            np.testing.assert_allclose(gx, num, rtol=0, atol=2e-8,
                                       err_msg=f"case {n} grad {'qkv'[t]}")


def _mp_loss(q, k, v, g, causal, scale):
    """sum(dout * o) in 40-digit arithmetic from the definition (no max)."""
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    tot = mpmath.mpf(0)
    for b in range(B):
        for hh in range(H):
            for i in range(Lq):
                js = [j for j in range(Lk) if not causal or j <= i]
                e = [mpmath.exp(scale * mpmath.fsum(q[b, hh, i, d] * k[b, hh, j, d]
                                                    for d in range(D))) for j in js]
                z = mpmath.fsum(e)
                for d in range(D):
                    o = mpmath.fsum(e[n] * v[b, hh, j, d] for n, j in enumerate(js)) / z
                    tot += o * g[b, hh, i, d]
    return tot


def pin_mp_finite_differences(lib):
    """A 40-digit brute-force forward, differentiated by a central difference
    with step 1e-15: exact to far below fp64 rounding."""
    mpmath.mp.dps = 40
    for causal, (B, H, Lq, Lk, D), seed in ((False, (1, 1, 3, 4, 2), 400),
                                            (True, (1, 1, 4, 3, 2), 410)):
        q, k, v, g = problem(B, H, Lq, Lk, D, seed)
        scale = 0.8
        grads = oracle.attention_bwd(q, k, v, g, causal, scale, lib=lib)
        mq, mk, mv, mg = ([[[[mpmath.mpf(float(x)) for x in row] for row in hd]
                            for hd in bt] for bt in a] for a in (q, k, v, g))
        hstep = mpmath.mpf("1e-15")
        for t, gx in enumerate(grads):
            for idx in np.ndindex(gx.shape):
                b, hh, r, d = idx
                args = [mq, mk, mv]
                arr = args[t]
                x0 = arr[b][hh][r][d]
                arr[b][hh][r][d] = x0 + hstep
                lp = _mp_loss(np.array(mq, dtype=object), np.array(mk, dtype=object),
                              np.array(mv, dtype=object), np.array(mg, dtype=object),
                              causal, mpmath.mpf(scale))
                arr[b][hh][r][d] = x0 - hstep
                lm = _mp_loss(np.array(mq, dtype=object), np.array(mk, dtype=object),
                              np.array(mv, dtype=object), np.array(mg, dtype=object),
                              causal, mpmath.mpf(scale))
                arr[b][hh][r][d] = x0
                ref = float((lp - lm) / (2 * hstep))
                assert abs(gx[idx] - ref) <= 1e-13 * max(1.0, abs(ref)), \
                    (causal, "qkv"[t], idx, gx[idx], ref)


def pin_torch_autograd(lib):
    """torch's CPU attention routine in fp64 under autograd (its causal mask
    is top-left for Lq != Lk, as here)."""
    F = torch.nn.functional
    for n, ((B, H, Lq, Lk, D), causal, scale) in enumerate(
            [((2, 3, 33, 47, 16), False, 0.25), ((1, 2, 40, 40, 8), True, 0.35),
             ((1, 2, 50, 20, 8), True, 0.6), ((1, 1, 17, 64, 32), True, 0.18)]):
        q, k, v, g = problem(B, H, Lq, Lk, D, 500 + 10 * n)
        qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=causal,
                                           scale=scale)
        o.backward(torch.tensor(g))
        dq, dk, dv = oracle.attention_bwd(q, k, v, g, causal, scale, lib=lib)
        for name, a, b in (("dq", dq, qt.grad), ("dk", dk, kt.grad),
                           ("dv", dv, vt.grad)):
            np.testing.assert_allclose(a, b.numpy(), rtol=0, atol=1e-12,
                                       err_msg=f"case {n} {name}")


def pin_sum_rules(lib):
    """Rows of P sum to one, so sum_j dv_j = sum_i dout_i; rows of the softmax
    Jacobian sum to zero, so sum_j dk_j = 0 (per head, per component)."""
    for causal in (False, True):
        q, k, v, g = problem(2, 2, 19, 23, 8, 600)
        dq, dk, dv = oracle.attention_bwd(q, k, v, g, causal, 0.4, lib=lib)
        np.testing.assert_allclose(dv.sum(2), g.sum(2), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dk.sum(2), 0.0, rtol=0, atol=1e-12)


def pin_homogeneity(lib):
    """o is unchanged by q -> t q, k -> k / t, so sum q*dq = sum k*dk per
    head; o is linear in v, so sum v*dv = sum dout*o per head."""
    for causal in (False, True):
        q, k, v, g = problem(2, 3, 21, 18, 8, 610)
        dq, dk, dv = oracle.attention_bwd(q, k, v, g, causal, 0.5, lib=lib)
        o, _ = oracle.attention(q, k, v, causal, 0.5, lib=lib)
        np.testing.assert_allclose((q * dq).sum((2, 3)), (k * dk).sum((2, 3)),
                                   rtol=0, atol=1e-12)
        np.testing.assert_allclose((v * dv).sum((2, 3)), (g * o).sum((2, 3)),
                                   rtol=0, atol=1e-12)


def pin_constant_v(lib):
    """All value rows equal: o = v_0 whatever q and k are, so dq = dk = 0,
    and dv_j = sum_i p_ij dout_i with p from the forward oracle."""
    for causal in (False, True):
        q, k, _, g = problem(1, 2, 9, 12, 4, 620)
        v = np.broadcast_to(rnd((1, 2, 1, 4), 625), (1, 2, 12, 4)).copy()
        dq, dk, dv = oracle.attention_bwd(q, k, v, g, causal, 0.9, lib=lib)
        assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
        p = oracle.probs(q, k, causal, 0.9, lib=lib)
        np.testing.assert_allclose(dv, np.swapaxes(p, 2, 3) @ g, rtol=0,
                                   atol=1e-13)


def pin_single_key(lib):
    """Lk = 1: p = 1, so dq = dk = 0 and dv_0 = sum_i dout_i."""
    for causal in (False, True):
        q, k, v, g = problem(1, 2, 6, 1, 4, 630)
        dq, dk, dv = oracle.attention_bwd(q, k, v, g, causal, 1.1, lib=lib)
        assert np.abs(dq).max() == 0.0 and np.abs(dk).max() < 1e-15
        np.testing.assert_allclose(dv[:, :, 0], g.sum(2), rtol=0, atol=1e-14)


def pin_causal_structure(lib):
    """Causal, Lq = Lk = L: row 0 sees key 0 alone, so dq_0 = 0; the last key
    is seen by the last row alone, with weight p_{L-1,L-1}, so
    dv_{L-1} = p dout_{L-1} and dk_{L-1} = scale p (dp - delta) q_{L-1}."""
    L, D, scale = 11, 4, 0.7
    q, k, v, g = problem(1, 1, L, L, D, 640)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, True, scale, lib=lib)
    assert np.abs(dq[0, 0, 0]).max() == 0.0
    o, _ = oracle.attention(q, k, v, True, scale, lib=lib)
    p = oracle.probs(q, k, True, scale, lib=lib)[0, 0, L - 1, L - 1]
    gl = g[0, 0, L - 1]
    np.testing.assert_allclose(dv[0, 0, L - 1], p * gl, rtol=0, atol=1e-14)
    dp = gl @ v[0, 0, L - 1]
    delta = gl @ o[0, 0, L - 1]
    np.testing.assert_allclose(dk[0, 0, L - 1], scale * p * (dp - delta) * q[0, 0, L - 1],
                               rtol=0, atol=1e-13)


def pin_delta_identity(lib):
    """delta_i = sum_j p_ij (dout_i . v_j) equals dout_i . o_i, because
    o_i = sum_j p_ij v_j (the backward's per-row statistic)."""
    for causal in (False, True):
        q, k, v, g = problem(2, 2, 13, 17, 8, 650)
        *_, delta = oracle.attention_bwd(q, k, v, g, causal, 0.6, lib=lib,
                                         with_delta=True)
        o, _ = oracle.attention(q, k, v, causal, 0.6, lib=lib)
        np.testing.assert_allclose(delta, (g * o).sum(-1), rtol=0, atol=1e-13)


PINS = [pin_finite_differences, pin_mp_finite_differences, pin_torch_autograd,
        pin_sum_rules, pin_homogeneity, pin_constant_v, pin_single_key,
        pin_causal_structure, pin_delta_identity]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


# --------------------------------------------------------------------------
# Planted mistakes in the backward's C source
# --------------------------------------------------------------------------

MUTANTS = {
    "delta_dropped": ("dsi[jj] = pi[jj] * (dsi[jj] - delta);",
                      "dsi[jj] = pi[jj] * dsi[jj];"),
    "delta_sign": ("dsi[jj] = pi[jj] * (dsi[jj] - delta);",
                   "dsi[jj] = pi[jj] * (dsi[jj] + delta);"),
    "dq_scale_dropped": ("dqh[i * D + d] = scale * acc;", "dqh[i * D + d] = acc;"),
    "dk_scale_dropped": ("dkh[j * D + d] = scale * acck;",
                         "dkh[j * D + d] = acck;"),
    "dv_rows_reversed": ("accv += p[ii * Lk + j] * gh[ii * D + d];",
                         "accv += p[ii * Lk + j] * gh[(Lq - 1 - ii) * D + d];"),
    "dk_uses_dout": ("acck += ds[ii * Lk + j] * qh[ii * D + d];",
                     "acck += ds[ii * Lk + j] * gh[ii * D + d];"),
    "dq_uses_v": ("for (jj = jbeg; jj < jend; ++jj) acc += dsi[jj] * kh[jj * D + d];",
                  "for (jj = jbeg; jj < jend; ++jj) acc += dsi[jj] * vh[jj * D + d];"),
    "dp_uses_k": ("const double *vj = vh + jj * D;",
                  "const double *vj = kh + jj * D;"),
    "dv_uses_ds": ("accv += p[ii * Lk + j] * gh[ii * D + d];",
                   "accv += ds[ii * Lk + j] * gh[ii * D + d];"),
    "delta_unweighted": ("delta += pi[jj] * dp;", "delta += dp / jend;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    src = open(os.path.join(os.path.dirname(oracle.__file__),
                            "fa_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    tmp = tempfile.mkdtemp(prefix="oracle_bwd_mutant_")
    try:
        c = os.path.join(tmp, "m.c")
        open(c, "w").write(src.replace(old, new))
        lib = oracle.load(oracle.build(c, os.path.join(tmp, "libm.so")))
        # the slow 40-digit pin is not needed to catch any of these
        for pin in PINS:
            if pin is pin_mp_finite_differences:
                continue
            try:
                pin(lib)
            except AssertionError:
                return
        raise AssertionError(f"mutant {name} passed every pin")
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
