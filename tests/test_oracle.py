"""Pins for the CPU fp64 oracle (no GPU needed).

The oracle is trusted only because these checks tie it to things other than
itself: hand-derived worked examples, arbitrary-precision brute force, the
library SDPA routine, closed forms, and invariants the pages state (rows of P
sum to one; the online rescan reaches exactly the two-pass result).  The last
test plants mistakes in copies of the oracle's C source and shows that each one
is caught by at least one pin.
"""
import json
import math
import os
import shutil
import tempfile

import mpmath
import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "hand_cases.json")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# --------------------------------------------------------------------------
# Pins.  Each takes a loaded oracle library and raises AssertionError when the
# oracle disagrees with what the pages and mathematics fix.
# --------------------------------------------------------------------------

def pin_hand_cases(lib):
    """Hand-derived worked examples (exact rational softmax weights)."""
    doc = json.load(open(GOLDEN))
    for c in doc["cases"]:
        o, lse = oracle.attention(np.array(c["q"]), np.array(c["k"]),
                                  np.array(c["v"]), c["causal"], c["scale"],
                                  lib=lib)
        np.testing.assert_allclose(o, np.array(c["o"]), rtol=0, atol=1e-13,
                                   err_msg=c["name"])
        np.testing.assert_allclose(lse, np.array(c["lse"]), rtol=0,
                                   atol=1e-13, err_msg=c["name"])


def _mp_reference(q, k, v, causal, scale):
    """50-digit brute force: softmax(s) = exp(s_j) / sum_k exp(s_k), no
    stabilising max (exact arithmetic does not need one)."""
    mpmath.mp.dps = 50
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    o = np.zeros((B, H, Lq, D))
    lse = np.zeros((B, H, Lq))
    for b in range(B):
        for h in range(H):
            for i in range(Lq):
                js = [j for j in range(Lk) if (not causal or j <= i)]
                e = {}
                for j in js:
                    s = mpmath.mpf(scale) * mpmath.fsum(
                        mpmath.mpf(q[b, h, i, d]) * mpmath.mpf(k[b, h, j, d])
                        for d in range(D))
                    e[j] = mpmath.exp(s)
                z = mpmath.fsum(e.values())
                for d in range(D):
                    o[b, h, i, d] = float(mpmath.fsum(
                        e[j] / z * mpmath.mpf(v[b, h, j, d]) for j in js))
                lse[b, h, i] = float(mpmath.log(z))
    return o, lse


def pin_bruteforce(lib):
    """Arbitrary-precision brute force on tiny shapes (Lq != Lk included)."""
    shapes = [(1, 1, 1, 1, 1), (1, 2, 3, 5, 4), (2, 1, 5, 3, 8),
              (1, 1, 16, 16, 4), (1, 1, 2, 16, 8), (1, 1, 16, 2, 1)]
    for n, (B, H, Lq, Lk, D) in enumerate(shapes):
        q = rnd((B, H, Lq, D), 10 + n)
        k = rnd((B, H, Lk, D), 20 + n)
        v = rnd((B, H, Lk, D), 30 + n)
        for causal in (False, True):
            scale = 0.7 if n % 2 else 1.0 / math.sqrt(D)
            o, lse = oracle.attention(q, k, v, causal, scale, lib=lib)
            ro, rlse = _mp_reference(q, k, v, causal, scale)
            np.testing.assert_allclose(o, ro, rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-13)


def pin_torch_sdpa(lib):
    """The library routine (torch CPU fp64 SDPA + logsumexp)."""
    cases = [(2, 3, 37, 53, 16, False), (2, 3, 41, 41, 16, True),
             (1, 2, 29, 45, 8, True), (1, 2, 45, 29, 8, True)]
    for n, (B, H, Lq, Lk, D, causal) in enumerate(cases):
        q, k, v = (rnd((B, H, L, D), 40 + 3 * n + t)
                   for t, L in enumerate((Lq, Lk, Lk)))
        scale = 0.3 + 0.1 * n
        o, lse = oracle.attention(q, k, v, causal, scale, lib=lib)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        if causal:
            mask = torch.ones(Lq, Lk, dtype=torch.bool).tril()
        else:
            mask = None
        ro = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=mask, scale=scale)
        s = torch.matmul(tq, tk.transpose(-1, -2)) * scale
        if mask is not None:
            s = s.masked_fill(~mask, float("-inf"))
        rlse = torch.logsumexp(s, dim=-1)
        np.testing.assert_allclose(o, ro.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, rlse.numpy(), rtol=0, atol=1e-12)


def pin_rows_sum_to_one(lib):
    """Every row of P sums to one, masked entries are zero, and O = P V."""
    for causal in (False, True):
        B, H, Lq, Lk, D = 2, 2, 19, 23, 8
        q, k, v = (rnd((B, H, L, D), 60 + t) for t, L in
                   enumerate((Lq, Lk, Lk)))
        p = oracle.probs(q, k, causal, 0.4, lib=lib)
        np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-13)
        assert (p >= 0).all()
        if causal:
            above = np.triu(np.ones((Lq, Lk), dtype=bool), k=1)
            assert (p[..., above] == 0.0).all()
            assert (p[..., ~above] > 0.0).all()
        o, _ = oracle.attention(q, k, v, causal, 0.4, lib=lib)
        np.testing.assert_allclose(o, np.matmul(p, v), rtol=0, atol=1e-13)


def pin_constant_v(lib):
    """Constant V rows give O equal to that row, causal or not."""
    B, H, Lq, Lk, D = 1, 3, 17, 33, 8
    q, k = rnd((B, H, Lq, D), 70, 3.0), rnd((B, H, Lk, D), 71, 3.0)
    c = rnd((B, H, 1, D), 72)
    v = np.repeat(c, Lk, axis=2)
    for causal in (False, True):
        o, _ = oracle.attention(q, k, v, causal, 0.5, lib=lib)
        np.testing.assert_allclose(o, np.repeat(c, Lq, axis=2), rtol=0,
                                   atol=1e-14)


def pin_causal_row0(lib):
    """Causal row 0 sees only key 0: O_0 = V_0, LSE_0 = scale * q_0 . k_0."""
    B, H, Lq, Lk, D = 2, 2, 9, 11, 16
    q, k, v = (rnd((B, H, L, D), 80 + t) for t, L in enumerate((Lq, Lk, Lk)))
    o, lse = oracle.attention(q, k, v, True, 0.25, lib=lib)
    assert np.array_equal(o[:, :, 0, :], v[:, :, 0, :])
    s00 = np.array([[0.25 * math.fsum(q[b, h, 0] * k[b, h, 0])
                     for h in range(H)] for b in range(B)])
    np.testing.assert_allclose(lse[:, :, 0], s00, rtol=0, atol=1e-13)


def pin_q_zero(lib):
    """Q = 0: every visible score is 0, so O_i is the mean of the visible V
    rows and LSE_i = ln |J_i| (ln Lk, or ln(i+1) when causal)."""
    B, H, Lq, Lk, D = 1, 2, 48, 4000, 8
    q = np.zeros((B, H, Lq, D))
    k, v = rnd((B, H, Lk, D), 90), rnd((B, H, Lk, D), 91)
    o, lse = oracle.attention(q, k, v, False, 0.125, lib=lib)
    np.testing.assert_allclose(lse, math.log(Lk), rtol=0, atol=1e-12)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(2, keepdims=True),
                                                  o.shape), rtol=0, atol=1e-12)
    o, lse = oracle.attention(q, k, v, True, 0.125, lib=lib)
    i = np.arange(Lq)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(i + 1.0), lse.shape),
                               rtol=0, atol=1e-12)
    cum = np.cumsum(v[:, :, :Lq, :], axis=2) / (i + 1.0)[None, None, :, None]
    np.testing.assert_allclose(o, cum, rtol=0, atol=1e-12)


def pin_small_lk(lib):
    """Lk = 1: O = V_0, LSE = s_00.  Lk = 2: O = sig(s0 - s1) V_0 +
    sig(s1 - s0) V_1 with sig the logistic function, LSE = logaddexp."""
    B, H, Lq, D = 1, 2, 5, 8
    q = rnd((B, H, Lq, D), 100)
    k, v = rnd((B, H, 1, D), 101), rnd((B, H, 1, D), 102)
    o, lse = oracle.attention(q, k, v, False, 0.6, lib=lib)
    assert np.array_equal(o, np.broadcast_to(v, o.shape))
    np.testing.assert_allclose(lse, 0.6 * (q @ k.transpose(0, 1, 3, 2))[..., 0],
                               rtol=0, atol=1e-13)
    k, v = rnd((B, H, 2, D), 103), rnd((B, H, 2, D), 104)
    o, lse = oracle.attention(q, k, v, False, 0.6, lib=lib)
    s = 0.6 * (q @ k.transpose(0, 1, 3, 2))
    sig = 1.0 / (1.0 + np.exp(-(s[..., 0] - s[..., 1])))
    want = sig[..., None] * v[:, :, None, 0, :] + \
        (1 - sig)[..., None] * v[:, :, None, 1, :]
    np.testing.assert_allclose(o, want, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, np.logaddexp(s[..., 0], s[..., 1]),
                               rtol=0, atol=1e-13)


def pin_scale_equivariance(lib):
    """f(Q, scale=s) == f(s Q, scale=1), including s = 0 and s < 0."""
    B, H, Lq, Lk, D = 1, 2, 13, 21, 8
    q, k, v = (rnd((B, H, L, D), 110 + t) for t, L in enumerate((Lq, Lk, Lk)))
    for s in (0.0, -0.7, 2.5):
        for causal in (False, True):
            a = oracle.attention(q, k, v, causal, s, lib=lib)
            b = oracle.attention(s * q, k, v, causal, 1.0, lib=lib)
            np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-12)


def pin_key_permutation(lib):
    """Non-causal attention is invariant to a joint permutation of K, V rows."""
    B, H, Lq, Lk, D = 1, 2, 11, 31, 8
    q, k, v = (rnd((B, H, L, D), 120 + t) for t, L in enumerate((Lq, Lk, Lk)))
    perm = np.random.default_rng(123).permutation(Lk)
    a = oracle.attention(q, k, v, False, 0.5, lib=lib)
    b = oracle.attention(q, k[:, :, perm], v[:, :, perm], False, 0.5, lib=lib)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-12)


def online_rescan(q, k, v, causal, scale, tile, l_init=0.0, mask="inf"):
    """fp64 online softmax over key tiles, in the pages' recurrence.

    State per query row: running max m (init -inf), running sum l (init 0 as
    in "Triton Ascend Attention" or 1 as in the FlashAttention-2 article -- the
    first tile's rescale factor exp(-inf) = 0 makes both the same), and the
    unnormalised accumulator.  Per tile: m_new = max(m, tile max); p =
    exp(s - m_new); alpha = exp(m - m_new); l = alpha l + sum p; acc = alpha
    acc + p V; then m = m_new.  Finally O = acc / l and LSE = m + log l.
    Masked keys (beyond Lk, or above the diagonal when causal) get -inf, or
    the article's additive -1e6 when mask == "additive".
    """
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    o = np.zeros((B, H, Lq, D))
    lse = np.zeros((B, H, Lq))
    for b in range(B):
        for h in range(H):
            for i in range(Lq):
                m, l, acc = -np.inf, l_init, np.zeros(D)
                for j0 in range(0, Lk, tile):
                    j = np.arange(j0, j0 + tile)
                    inside = j < Lk
                    kk = np.zeros((tile, D))
                    vv = np.zeros((tile, D))
                    kk[inside] = k[b, h, j[inside]]
                    vv[inside] = v[b, h, j[inside]]
                    s = scale * (kk @ q[b, h, i])
                    keep = inside & ((not causal) | (j <= i))
                    if mask == "inf":
                        s = np.where(keep, s, -np.inf)
                    else:
                        s = s + np.where(keep, 0.0, -1e6)
                    if not keep.any() and mask == "inf":
                        continue
                    m_new = max(m, s.max())
                    p = np.exp(s - m_new)
                    alpha = np.exp(m - m_new)
                    l = alpha * l + p.sum()
                    acc = alpha * acc + p @ vv
                    m = m_new
                o[b, h, i] = acc / l
                lse[b, h, i] = m + np.log(l)
    return o, lse


def pin_online_equals_two_pass(lib):
    """The pages claim the online rescan reaches exactly full softmax."""
    B, H, Lq, Lk, D = 1, 2, 24, 45, 8
    q, k, v = (rnd((B, H, L, D), 130 + t, 1.5) for t, L in
               enumerate((Lq, Lk, Lk)))
    for causal in (False, True):
        want = oracle.attention(q, k, v, causal, 0.5, lib=lib)
        for tile, l_init, mask in ((1, 0.0, "inf"), (7, 1.0, "inf"),
                                   (16, 0.0, "additive"), (64, 1.0, "inf"),
                                   (Lk, 0.0, "inf")):
            got = online_rescan(q, k, v, causal, 0.5, tile, l_init, mask)
            np.testing.assert_allclose(got[0], want[0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(got[1], want[1], rtol=0, atol=1e-12)


def pin_causal_prefix(lib):
    """Causal row i equals non-causal attention of query i over keys 0..i."""
    B, H, L, D = 1, 1, 12, 8
    q, k, v = (rnd((B, H, L, D), 140 + t) for t in range(3))
    o, lse = oracle.attention(q, k, v, True, 0.5, lib=lib)
    for i in range(L):
        oi, li = oracle.attention(q[:, :, i:i + 1], k[:, :, :i + 1],
                                  v[:, :, :i + 1], False, 0.5, lib=lib)
        np.testing.assert_allclose(o[:, :, i], oi[:, :, 0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[:, :, i], li[:, :, 0], rtol=0,
                                   atol=1e-14)


def pin_rows_entry(lib):
    """The selected-rows entry gives exactly the full forward's rows."""
    B, H, Lq, Lk, D = 2, 3, 10, 14, 8
    q, k, v = (rnd((B, H, L, D), 150 + t) for t, L in enumerate((Lq, Lk, Lk)))
    ids = np.array([0, 5, 9, 10, 31, 59, 17])
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, causal, 0.3, lib=lib)
        ro, rl = oracle.attention_rows(q, k, v, ids, causal, 0.3, lib=lib)
        assert np.array_equal(ro, o.reshape(-1, D)[ids])
        assert np.array_equal(rl, lse.reshape(-1)[ids])


PINS = [pin_hand_cases, pin_bruteforce, pin_torch_sdpa, pin_rows_sum_to_one,
        pin_constant_v, pin_causal_row0, pin_q_zero, pin_small_lk,
        pin_scale_equivariance, pin_key_permutation,
        pin_online_equals_two_pass, pin_causal_prefix, pin_rows_entry]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_zero_filled_tail_without_mask_would_leak(oracle_lib):
    """Reading of the tail tile: keys at j >= Lk are excluded.  The article
    loads out-of-range K rows as 0.0 and masks only the causal predicate, so a
    padded key would score 0 and enter the sum.  With Q = 0 the oracle reports
    ln Lk; treating the zero padding as keys would report ln(padded length)."""
    B, H, Lq, Lk, D = 1, 1, 3, 5, 4
    q = np.zeros((B, H, Lq, D))
    k, v = rnd((B, H, Lk, D), 160), rnd((B, H, Lk, D), 161)
    _, lse = oracle.attention(q, k, v, False, 1.0, lib=oracle_lib)
    np.testing.assert_allclose(lse, math.log(Lk), atol=1e-14)
    pad = np.zeros((B, H, 3, D))
    _, leak = oracle.attention(q, np.concatenate([k, pad], 2),
                               np.concatenate([v, pad], 2), False, 1.0,
                               lib=oracle_lib)
    np.testing.assert_allclose(leak, math.log(Lk + 3), atol=1e-14)


# --------------------------------------------------------------------------
# Planted mistakes: each edit below is a plausible bug in the oracle's C
# source.  Every one must be caught by at least one pin.
# --------------------------------------------------------------------------

MUTANTS = {
    "diagonal_excluded": ("if (causal && i + 1 < e) e = i + 1;",
                          "if (causal && i < e) e = i;"),
    "causal_ignored": ("if (causal && i + 1 < e) e = i + 1;", ""),
    "max_not_subtracted": ("p[j] = exp(p[j] - m);", "p[j] = exp(p[j]);"),
    "exp_sign_flipped": ("p[j] = exp(p[j] - m);", "p[j] = exp(m - p[j]);"),
    "not_normalised": ("for (j = jbeg; j < jend; ++j) p[j] /= l;", ""),
    "k_transposed": ("for (d = 0; d < D; ++d) dot += q_row[d] * k_row[d];",
                     "for (d = 0; d < D; ++d) dot += q_row[d] * "
                     "k_head[(d * Lk + j) % (Lk * D)]; (void)k_row;"),
    "v_reversed": ("const double *v_row = v_head + j * D;",
                   "const double *v_row = v_head + (jend - 1 - j) * D;"),
    "lse_log2": ("*lse_out = m + log(l);", "*lse_out = m + log2(l);"),
    "lse_without_max": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "scale_dropped": ("p[j] = scale * dot;", "p[j] = dot;"),
    "k_head_zero": ("const double *k_head = k + bh * Lk * D;",
                    "const double *k_head = k + 0 * bh * Lk * D;"),
    "q_row_off_by_one": ("const double *q_row = q + (bh * Lq + i) * D;",
                         "const double *q_row = q + (bh * Lq + (i > 0 ? i - 1 "
                         ": 0)) * D;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    src = open(os.path.join(os.path.dirname(oracle.__file__),
                            "fa_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mutated = src.replace(old, new)
    tmp = tempfile.mkdtemp(prefix="oracle_mutant_")
    try:
        c = os.path.join(tmp, "m.c")
        open(c, "w").write(mutated)
        so = oracle.build(c, os.path.join(tmp, "libm.so"))
        lib = oracle.load(so)
        caught = []
        for pin in PINS:
            try:
                pin(lib)
            except AssertionError:
                caught.append(pin.__name__)
        assert caught, f"mutant {name} passed every pin"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
