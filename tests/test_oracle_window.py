"""Pins for the oracle's local (sliding-window) mask (no GPU needed).

Query i keeps key j when i - wl <= j <= i + wr (a negative bound is no bound),
combined with the causal rule j <= i.  The window is tied to things other
than its own code: the plain (pinned) oracle on the sliced key range, a
50-digit brute force, torch's CPU attention with an explicit boolean mask,
and closed forms (wide windows change nothing; wr = 0 is causal; causal with
wl = 0 returns V_i; rows that see no key give O = 0, LSE = -inf).  Planted
off-by-one mistakes in the C source must each fail a pin.
"""
import math
import os
import shutil
import tempfile

import mpmath
import numpy as np
import pytest
import torch

import oracle


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def qkv(B, H, Lq, Lk, D, seed):
    return rnd((B, H, Lq, D), seed), rnd((B, H, Lk, D), seed + 1), rnd((B, H, Lk, D), seed + 2)


def visible(i, Lk, causal, wl, wr):
    return [j for j in range(Lk) if (not causal or j <= i)
            and (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr)]


CASES = [((1, 2, 20, 20, 8), False, (3, 2)), ((1, 2, 20, 20, 8), True, (5, -1)),
         ((2, 1, 17, 29, 4), False, (0, 6)), ((1, 1, 30, 12, 8), False, (4, 4)),
         ((1, 1, 25, 25, 4), True, (0, -1)), ((1, 2, 9, 31, 8), False, (-1, 3))]


def pin_wide_window_is_plain(lib):
    for n, ((B, H, Lq, Lk, D), causal, _) in enumerate(CASES):
        q, k, v = qkv(B, H, Lq, Lk, D, 700 + n)
        o, l = oracle.attention(q, k, v, causal, 0.4, lib=lib)
        w = max(Lq, Lk)
        ow, lw = oracle.attention(q, k, v, causal, 0.4, lib=lib, window=(w, w))
        assert np.array_equal(o, ow) and np.array_equal(l, lw)


def pin_right_zero_is_causal(lib):
    q, k, v = qkv(1, 2, 19, 23, 8, 710)
    o, l = oracle.attention(q, k, v, True, 0.6, lib=lib)
    ow, lw = oracle.attention(q, k, v, False, 0.6, lib=lib, window=(-1, 0))
    assert np.array_equal(o, ow) and np.array_equal(l, lw)


def pin_slice(lib):
    """Row i of windowed attention = plain attention of q_i over the keys in
    its window (sliced out and passed to the plain oracle)."""
    for n, ((B, H, Lq, Lk, D), causal, (wl, wr)) in enumerate(CASES):
        q, k, v = qkv(B, H, Lq, Lk, D, 720 + n)
        o, l = oracle.attention(q, k, v, causal, 0.5, lib=lib, window=(wl, wr))
        for i in range(Lq):
            js = visible(i, Lk, causal, wl, wr)
            if not js:
                continue
            a, b = js[0], js[-1] + 1
            oi, li = oracle.attention(q[:, :, i:i + 1], k[:, :, a:b], v[:, :, a:b], False,
                                      0.5, lib=lib)
            np.testing.assert_allclose(o[:, :, i], oi[:, :, 0], rtol=0, atol=1e-14)
            np.testing.assert_allclose(l[:, :, i], li[:, :, 0], rtol=0, atol=1e-14)


def pin_mp_bruteforce(lib):
    mpmath.mp.dps = 50
    for n, ((B, H, Lq, Lk, D), causal, (wl, wr)) in enumerate(
            [((1, 1, 7, 9, 3), False, (2, 1)), ((1, 1, 8, 8, 2), True, (3, -1)),
             ((1, 1, 9, 4, 2), False, (1, 1))]):
        q, k, v = qkv(B, H, Lq, Lk, D, 730 + n)
        o, l = oracle.attention(q, k, v, causal, 0.7, lib=lib, window=(wl, wr))
        for i in range(Lq):
            js = visible(i, Lk, causal, wl, wr)
            if not js:
                assert np.all(o[0, 0, i] == 0) and l[0, 0, i] == -math.inf
                continue
            e = [mpmath.exp(mpmath.mpf(0.7) * mpmath.fsum(mpmath.mpf(q[0, 0, i, d]) *
                                                          mpmath.mpf(k[0, 0, j, d])
                                                          for d in range(D))) for j in js]
            z = mpmath.fsum(e)
            for d in range(D):
                ref = mpmath.fsum(e[t] * mpmath.mpf(v[0, 0, j, d]) for t, j in enumerate(js)) / z
                assert abs(o[0, 0, i, d] - float(ref)) < 1e-14
            assert abs(l[0, 0, i] - float(mpmath.log(z))) < 1e-14


def pin_torch_mask(lib):
    """torch's CPU attention in fp64 with the window as an explicit boolean
    mask (rows with a visible key only)."""
    F = torch.nn.functional
    for n, ((B, H, Lq, Lk, D), causal, (wl, wr)) in enumerate(CASES):
        q, k, v = qkv(B, H, Lq, Lk, D, 740 + n)
        mask = torch.zeros(Lq, Lk, dtype=torch.bool)
        for i in range(Lq):
            for j in visible(i, Lk, causal, wl, wr):
                mask[i, j] = True
        rows = mask.any(1)
        ref = F.scaled_dot_product_attention(torch.tensor(q), torch.tensor(k),
                                             torch.tensor(v), attn_mask=mask, scale=0.3)
        o, _ = oracle.attention(q, k, v, causal, 0.3, lib=lib, window=(wl, wr))
        np.testing.assert_allclose(o[:, :, rows.numpy()], ref.numpy()[:, :, rows.numpy()],
                                   rtol=0, atol=1e-12)


def pin_causal_w0(lib):
    """Causal with wl = 0: each row sees only its own key."""
    q, k, v = qkv(1, 2, 13, 13, 8, 750)
    o, l = oracle.attention(q, k, v, True, 0.9, lib=lib, window=(0, -1))
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(l, 0.9 * np.einsum("bhid,bhid->bhi", q, k), rtol=0, atol=1e-14)


def pin_empty_rows(lib):
    """Rows whose window lies past the last key see nothing: O = 0,
    LSE = -inf; the other rows are finite."""
    q, k, v = qkv(1, 1, 20, 6, 4, 760)
    o, l = oracle.attention(q, k, v, False, 0.5, lib=lib, window=(2, 1))
    for i in range(20):
        if i - 2 >= 6:
            assert np.all(o[0, 0, i] == 0) and l[0, 0, i] == -math.inf
        else:
            assert np.isfinite(l[0, 0, i])


def pin_rows_entry(lib):
    q, k, v = qkv(2, 2, 15, 21, 8, 770)
    ids = np.array([0, 3, 14, 15, 29, 44, 59])
    for causal, win in ((False, (3, 5)), (True, (4, -1))):
        o, l = oracle.attention(q, k, v, causal, 0.3, lib=lib, window=win)
        ro, rl = oracle.attention_rows(q, k, v, ids, causal, 0.3, lib=lib, window=win)
        assert np.array_equal(ro, o.reshape(-1, 8)[ids])
        assert np.array_equal(rl, l.reshape(-1)[ids])


def _loss(q, k, v, g, causal, scale, win, lib):
    o, _ = oracle.attention(q, k, v, causal, scale, lib=lib, window=win)
    return float(np.sum(o * g))


def pin_bwd_finite_differences(lib):
    """Windowed gradients against central differences of the windowed
    forward (every entry)."""
    h = 1e-6
    for n, ((B, H, Lq, Lk, D), causal, win) in enumerate(
            [((1, 1, 6, 7, 3), False, (1, 2)), ((1, 1, 7, 7, 2), True, (2, -1)),
             ((1, 1, 8, 4, 2), False, (1, 0))]):
        q, k, v = qkv(B, H, Lq, Lk, D, 780 + n)
        g = rnd((B, H, Lq, D), 790 + n)
        grads = oracle.attention_bwd(q, k, v, g, causal, 0.6, lib=lib, window=win)
        for t, (x, gx) in enumerate(zip((q, k, v), grads)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                a = [q.copy(), k.copy(), v.copy()]
                a[t][idx] += h
                lp = _loss(*a, g, causal, 0.6, win, lib)
                a[t][idx] -= 2 * h
                lm = _loss(*a, g, causal, 0.6, win, lib)
                num[idx] = (lp - lm) / (2 * h)
            np.testing.assert_allclose(gx, num, rtol=0, atol=2e-8)


def pin_bwd_torch_mask(lib):
    """torch fp64 autograd of its attention routine with the window as a
    boolean mask (every row keeps a key here)."""
    F = torch.nn.functional
    for n, ((B, H, Lq, Lk, D), causal, (wl, wr)) in enumerate(
            [((1, 2, 20, 20, 8), False, (3, 2)), ((1, 2, 20, 20, 8), True, (5, -1)),
             ((2, 1, 17, 29, 4), False, (0, 6))]):
        q, k, v = qkv(B, H, Lq, Lk, D, 800 + n)
        g = rnd((B, H, Lq, D), 810 + n)
        mask = torch.zeros(Lq, Lk, dtype=torch.bool)
        for i in range(Lq):
            for j in visible(i, Lk, causal, wl, wr):
                mask[i, j] = True
        assert mask.any(1).all()
        qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.3).backward(
            torch.tensor(g))
        grads = oracle.attention_bwd(q, k, v, g, causal, 0.3, lib=lib, window=(wl, wr))
        for a, b in zip(grads, (qt.grad, kt.grad, vt.grad)):
            np.testing.assert_allclose(a, b.numpy(), rtol=0, atol=1e-12)


def pin_bwd_wide_window_is_plain(lib):
    q, k, v = qkv(1, 2, 15, 18, 4, 820)
    g = rnd((1, 2, 15, 4), 821)
    for causal in (False, True):
        a = oracle.attention_bwd(q, k, v, g, causal, 0.5, lib=lib)
        b = oracle.attention_bwd(q, k, v, g, causal, 0.5, lib=lib, window=(40, 40))
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


PINS = [pin_wide_window_is_plain, pin_right_zero_is_causal, pin_slice, pin_mp_bruteforce,
        pin_torch_mask, pin_causal_w0, pin_empty_rows, pin_rows_entry,
        pin_bwd_finite_differences, pin_bwd_torch_mask, pin_bwd_wide_window_is_plain]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


MUTANTS = {
    "left_off_by_one": ("    return i - wl;\n", "    return i - wl + 1;\n"),
    "right_off_by_one": ("if (wr >= 0 && i + wr + 1 < e) e = i + wr + 1;",
                         "if (wr >= 0 && i + wr < e) e = i + wr;"),
    "left_ignored": ("    if (wl < 0 || i - wl <= 0) return 0;", "    return 0;"),
    "right_ignored": ("if (wr >= 0 && i + wr + 1 < e) e = i + wr + 1;", ""),
    "left_is_right": ("    return i - wl;\n", "    return i - wl > i ? i : i - wl / 2;\n"),
    "bwd_window_ignored": ("int64_t jbeg = visible_begin(i, wl), jj, d;",
                           "int64_t jbeg = 0, jj, d;"),
    "bwd_dq_full_range": ("for (jj = jbeg; jj < jend; ++jj) acc += dsi[jj] * kh[jj * D + d];",
                          "for (jj = 0; jj < jend; ++jj) acc += (jj < jbeg ? 1.0 : dsi[jj]) "
                          "* kh[jj * D + d];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "fa_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    tmp = tempfile.mkdtemp(prefix="oracle_win_mutant_")
    try:
        c = os.path.join(tmp, "m.c")
        open(c, "w").write(src.replace(old, new))
        lib = oracle.load(oracle.build(c, os.path.join(tmp, "libm.so")))
        for pin in PINS:
            if pin is pin_mp_bruteforce:
                continue
            try:
                pin(lib)
            except AssertionError:
                return
        raise AssertionError(f"mutant {name} passed every pin")
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
