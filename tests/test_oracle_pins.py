"""Pins for the CPU oracle: each checks it against something other than itself --
closed forms, textbook tables, library routines it does not use, brute force on
tiny inputs, invariants and Monte-Carlo against closed forms.  CPU only."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
from scipy import integrate, special, stats

import tq_inputs as TI
from oracle import tq_oracle as O


# ---------------------------------------------------------------------------- rotation
@pytest.mark.parametrize("d", [8, 128, 256])
def test_hadamard_orthogonal_and_matches_library(d):
    H = O.hadamard(d)
    assert np.array_equal(H @ H.T, d * np.eye(d))
    # an independent construction: scipy's natural-order Sylvester routine
    assert np.array_equal(H, scipy.linalg.hadamard(d).astype(np.float64))
    # and the Kronecker power of [[1, 1], [1, -1]]
    K = np.array([[1.0]])
    for _ in range(int(math.log2(d))):
        K = np.kron(K, np.array([[1.0, 1.0], [1.0, -1.0]]))
    assert np.array_equal(H, K)


@pytest.mark.parametrize("d", [8, 128, 256])
def test_rotation_is_orthonormal(d):
    signs, _ = TI.rotation(d, 11)
    x = TI.gen(3).standard_normal((20, d))
    y = O.rotate(x, signs)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    np.testing.assert_allclose(O.unrotate(y, signs), x, atol=1e-12)
    # D precedes H: rotating a unit basis vector e_j gives signs[j] * H[:, j] / sqrt(d)
    j = d // 3
    e = np.zeros(d); e[j] = 1.0
    np.testing.assert_allclose(O.rotate(e[None], signs)[0],
                               signs[j] * scipy.linalg.hadamard(d)[:, j] / math.sqrt(d), atol=1e-15)


# ---------------------------------------------------------------------------- codebook
def _quad_cell(d, lo, hi):
    f = lambda t: O.marginal_pdf(t, d)
    m0 = integrate.quad(f, lo, hi, epsabs=1e-15, epsrel=1e-13, limit=200)[0]
    m1 = integrate.quad(lambda t: t * f(t), lo, hi, epsabs=1e-15, epsrel=1e-13, limit=200)[0]
    return m0, m1


@pytest.mark.parametrize("d,bits", [(8, 2), (128, 1), (128, 2), (128, 3), (128, 4), (256, 3)])
def test_lloyd_conditions_by_independent_quadrature(d, bits):
    c, b, mse = O.lloyd_max(d, bits)
    L = 1 << bits
    assert np.array_equal(c, -c[::-1])                  # exact mirror symmetry
    assert np.all(np.diff(c) > 0)
    np.testing.assert_allclose(b, (c[:-1] + c[1:]) / 2, rtol=0, atol=0)
    edges = np.concatenate([[-1.0], b, [1.0]])
    mse_q = 0.0
    for m in range(L):
        m0, m1 = _quad_cell(d, edges[m], edges[m + 1])
        assert abs(m1 / m0 - c[m]) < 1e-10 * max(1.0, abs(c[m])) + 1e-12
        m2 = integrate.quad(lambda t: (t - c[m]) ** 2 * O.marginal_pdf(t, d), edges[m], edges[m + 1],
                            epsabs=1e-16, epsrel=1e-12, limit=200)[0]
        mse_q += m2
    assert abs(mse - mse_q) < 1e-9 * mse_q + 1e-14   # closed form 1/d - sum c^2 P cancels


def test_marginal_is_a_density_with_variance_one_over_d():
    for d in (8, 128, 256):
        kw = dict(limit=400, epsabs=1e-15, epsrel=1e-14)
        tot = integrate.quad(lambda t: O.marginal_pdf(t, d), -1, 1, **kw)[0]
        var = integrate.quad(lambda t: t * t * O.marginal_pdf(t, d), -1, 1, **kw)[0]
        assert abs(tot - 1) < 1e-10 and abs(var - 1.0 / d) < 1e-12


@pytest.mark.parametrize("d", [8, 128, 256])
def test_one_bit_centroid_closed_form(d):
    # E|z_1| for a coordinate of a uniform unit vector: Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))
    c, _, _ = O.lloyd_max(d, 1)
    closed = math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
    assert abs(c[1] - closed) < 1e-13 and abs(c[0] + closed) < 1e-13


def test_gaussian_limit_matches_max_table():
    # Max (1960) optimum quantizers for N(0,1): positive output levels and MSE
    max_levels = {1: [0.7979], 2: [0.4528, 1.510], 3: [0.2451, 0.7560, 1.344, 2.152],
                  4: [0.1284, 0.3881, 0.6568, 0.9424, 1.256, 1.618, 2.069, 2.733]}
    max_mse = {1: 0.3634, 2: 0.1175, 3: 0.03454, 4: 0.009497}
    d = 1 << 16
    for bits, lv in max_levels.items():
        c, _, mse = O.lloyd_max(d, bits)
        got = c[len(c) // 2:] * math.sqrt(d)
        np.testing.assert_allclose(got, lv, atol=1.5e-3)
        assert abs(mse * d - max_mse[bits]) < 2e-4


def test_mse_decreases_with_bits_and_tables_are_fp32_roundings():
    prev = np.inf
    for bits in (1, 2, 3, 4):
        cb = O.codebook(128, bits)
        c, b, mse = O.lloyd_max(128, bits)
        assert mse < prev
        prev = mse
        assert np.array_equal(cb.centroids, c.astype(np.float32).astype(np.float64))
        assert np.array_equal(cb.bounds, -cb.bounds[::-1])
        assert cb.bounds[len(cb.bounds) // 2] == 0.0


# ---------------------------------------------------------------------------- fp16 rounding
def _fp16_exact(v):
    """Round a positive float to fp16 with exact rational arithmetic, ties to even."""
    f = Fraction(v)
    e = math.floor(math.log2(v))
    if Fraction(2) ** e > f:
        e -= 1
    if Fraction(2) ** (e + 1) <= f:
        e += 1
    e = max(e, -14)
    ulp = Fraction(2) ** (e - 10)
    q, rem = divmod(f, ulp)
    if rem * 2 > ulp or (rem * 2 == ulp and q % 2 == 1):
        q += 1
    return float(q * ulp)


def test_fp16_rounding_is_correct():
    g = TI.gen(5)
    vals = np.concatenate([np.exp(g.uniform(-12, 10, 3000)),
                           [1 + 2 ** -11, 1 + 3 * 2 ** -11, 2049.0, 2051.0, 6.1e-5, 65504.0]])
    got = O.fp16_value(O.fp16_bits(vals))
    ref = np.array([_fp16_exact(float(v)) for v in vals])
    assert np.array_equal(got, ref)


def _fp16_neighbours_exact(bits: int):
    """(value, next value up, next value down) of a positive finite fp16 pattern, exact."""
    val = lambda b: Fraction(float(np.array([b], np.uint16).view(np.float16)[0]))
    return val(bits), val(bits + 1), val(bits - 1)


@pytest.mark.parametrize("rel", [1e-6, 1e-12])
def test_near_fp16_midpoint_against_exact_midpoints(rel):
    """The window that marks norms as ambiguous: a value within rel of a point where fp16
    rounding changes (the exact midpoint between two adjacent fp16 values, found here from
    the bit patterns in rational arithmetic) is flagged, one 3 rel away from every such point
    is not.  Powers of two are included, where the spacing below is half the spacing above."""
    g = TI.gen(17)
    pats = list(g.integers(0x0401, 0x7BFF, 300)) + [0x3C00, 0x4000, 0x0800, 0x7800, 0x5C00]
    near, far, expect_near, expect_far = [], [], [], []
    for b in pats:
        h, up, dn = _fp16_neighbours_exact(int(b))
        for mid in ((h + up) / 2, (h + dn) / 2):
            for f in (0.5, -0.5, 0.0):
                near.append(float(mid * (1 + Fraction(f * rel))))
            for f in (3.0, -3.0):
                v = mid * (1 + Fraction(f * rel))
                # the other midpoints are at least half an fp16 spacing away
                far.append(float(v))
        far.append(float(h))
    assert O._near_fp16_midpoint(np.array(near), rel).all()
    assert not O._near_fp16_midpoint(np.array(far), rel).any()


# ---------------------------------------------------------------------------- 2/pi bias
def test_one_bit_mse_quantizer_has_two_over_pi_bias():
    """163.com explainer, section "第二步：QJL": a 1-bit MSE-optimal quantizer scales inner
    products by 2/pi in high dimension.  Closed form for Gaussian x: d * (E|z_1|)^2."""
    closed = lambda d: d * math.exp(2 * (math.lgamma(d / 2) - math.lgamma((d + 1) / 2))) / math.pi
    assert abs(closed(128) - 0.639111) < 1e-6
    assert abs(closed(1 << 20) - 2 / math.pi) < 1e-6
    d, n = 128, 4000
    fmt = O.Format.uniform(d, 1)
    cb = O.codebook(d, 1)
    ratios = []
    for seed in range(n // 200):
        signs, S = TI.rotation(d, 100 + seed)
        x = TI.gen(7000 + seed).standard_normal((200, d))
        qz = O.quantize(x, fmt, signs, S, cb)
        xh = O.dequantize(qz["idx"], qz["sbit"], qz["n16"], qz["r16"], fmt, signs, S, cb, qjl=False)
        ratios.append(np.sum(x * xh, axis=1) / np.sum(x * x, axis=1))
    ratios = np.concatenate(ratios)
    se = ratios.std(ddof=1) / math.sqrt(len(ratios))
    assert abs(ratios.mean() - closed(d)) < 4 * se + 3e-4   # fp16 norm rounding


# ---------------------------------------------------------------------------- unbiasedness
def test_inner_product_is_unbiased_over_seeds():
    """163.com explainer, section "第二步：QJL": E[<y, Q^-1(Q(x))>] = <y, x>."""
    d, bits, n_seeds = 128, 2, 10000
    fmt = O.Format.uniform(d, bits)
    cb = O.codebook(d, bits)
    g = TI.gen(42)
    x = g.standard_normal(d)
    y = 0.6 * x + g.standard_normal(d)
    vals = np.empty(n_seeds)
    for s in range(n_seeds):
        signs, S = TI.rotation(d, 10_000 + s)
        qz = O.quantize(x[None], fmt, signs, S, cb)
        xt = O.dequantize(qz["idx"], qz["sbit"], qz["n16"], qz["r16"], fmt, signs, S, cb)[0]
        vals[s] = y @ xt
    se = vals.std(ddof=1) / math.sqrt(n_seeds)
    assert abs(vals.mean() - y @ x) < 4 * se


def test_qjl_variance_matches_closed_form():
    """With the rotation fixed and S redrawn, the QJL term's variance is
    (1/d) (pi/2 r16^2 |y'|^2 - r16^2 <y', r^>^2), y' the rotated query."""
    d, bits, n_seeds = 128, 3, 10000
    fmt = O.Format.uniform(d, bits)
    cb = O.codebook(d, bits)
    g = TI.gen(43)
    x = g.standard_normal(d)
    y = g.standard_normal(d)
    signs, _ = TI.rotation(d, 9)
    vals = np.empty(n_seeds)
    for s in range(n_seeds):
        _, S = TI.rotation(d, 20_000 + s)
        qz = O.quantize(x[None], fmt, signs, S, cb)
        xt = O.dequantize(qz["idx"], qz["sbit"], qz["n16"], qz["r16"], fmt, signs, S, cb)[0]
        vals[s] = y @ xt
    qz = O.quantize(x[None], fmt, signs, TI.rotation(d, 0)[1], cb)
    r = qz["r"][0]
    r16 = O.fp16_value(qz["r16"])[0]
    yr = O.rotate(y[None], signs)[0]
    rhat = r / np.linalg.norm(r)
    var_closed = (math.pi / 2 * r16 ** 2 * (yr @ yr) - r16 ** 2 * (yr @ rhat) ** 2) / d
    assert abs(vals.var(ddof=1) / var_closed - 1) < 0.05
    mse_part = y @ O.unrotate((O.fp16_value(qz["n16"])[0] * O.centroid_values(qz["idx"], fmt, cb))[0][None], signs)[0]
    mean_closed = mse_part + r16 * (yr @ rhat)
    assert abs(vals.mean() - mean_closed) < 4 * vals.std(ddof=1) / math.sqrt(n_seeds)


# ---------------------------------------------------------------------------- distortion
def test_distortion_within_constant_of_lower_bound():
    """163.com explainer, section "合起来": MSE distortion within about 2.7x of the
    information-theoretic lower bound (4^-b here), the gap smaller at low widths."""
    d = 128
    ratios = []
    for bits in (1, 2, 3, 4):
        fmt = O.Format.uniform(d, bits)
        cb = O.codebook(d, bits)
        dist = []
        for seed in range(4):
            signs, S = TI.rotation(d, 300 + seed)
            x = TI.gen(400 + seed).standard_normal((500, d))
            qz = O.quantize(x, fmt, signs, S, cb)
            xh = O.dequantize(qz["idx"], qz["sbit"], qz["n16"], qz["r16"], fmt, signs, S, cb, qjl=False)
            dist.append(np.sum((x - xh) ** 2, axis=1) / np.sum(x * x, axis=1))
        dist = np.concatenate(dist)
        closed = d * cb.mse
        assert abs(dist.mean() - closed) < 4 * dist.std(ddof=1) / math.sqrt(len(dist)) + 2e-4 * closed
        ratio = closed / 4.0 ** (-bits)
        assert 1.0 <= ratio <= 2.72
        ratios.append(ratio)
    assert all(a < b for a, b in zip(ratios, ratios[1:]))


# ---------------------------------------------------------------------------- brute force d = 8
def test_encode_is_nearest_codeword_in_product_codebook_d8():
    d, bits = 8, 2
    fmt = O.Format.uniform(d, bits)
    cb = O.codebook(d, bits)
    signs, S = TI.rotation(d, 1)
    x = TI.gen(2).standard_normal((40, d))
    qz = O.quantize(x, fmt, signs, S, cb)
    import itertools
    allcw = np.array(list(itertools.product(range(1 << bits), repeat=d)))
    cvals = cb.centroids[allcw]                                   # [4^8, 8]
    for i in range(len(x)):
        if qz["amb_code"][i].any():
            continue
        dist = np.sum((cvals - qz["z"][i]) ** 2, axis=1)
        assert np.array_equal(allcw[np.argmin(dist)], qz["idx"][i])


def test_fused_estimator_equals_explicit_dequantized_dot():
    for d, bits, split in ((8, 2, 8), (128, 3, 128), (128, 3, 64), (256, 3, 256)):
        fmt = O.Format(d, bits, 2 if split < d else bits, split)
        lo, hi = O.codebook(d, fmt.bits_lo), O.codebook(d, fmt.bits_hi)
        signs, S = TI.rotation(d, 5)
        g = TI.gen(6)
        x = g.standard_normal((30, d)) * 3
        q = g.standard_normal(d)
        qz = O.quantize(x, fmt, signs, S, lo, hi)
        xt = O.dequantize(qz["idx"], qz["sbit"], qz["n16"], qz["r16"], fmt, signs, S, lo, hi)
        est, scale = O.estimator_dot(q, qz["idx"], qz["sbit"], qz["n16"], qz["r16"], fmt, signs, S, lo, hi)
        np.testing.assert_allclose(est, xt @ q, rtol=0, atol=1e-12 * np.max(scale))


def test_search_scores_equal_the_fused_estimator_for_padded_queries():
    """Search scores: queries of d_in < d coordinates are zero-padded and scored against the
    explicit dequantized vectors; they must equal the fused estimator (n16 <q_rot, c> +
    gamma r16 <S q_rot, sigma>) of the padded query to 1e-12."""
    d, d_in = 256, 200
    fmt = O.Format.uniform(d, 3)
    cb = O.codebook(d, 3)
    signs, S = TI.rotation(d, 23)
    g = TI.gen(24)
    x = g.standard_normal((40, d_in))
    qs = g.standard_normal((5, d_in))
    qz = O.quantize(x, fmt, signs, S, cb)
    xt = O.dequantize(qz["idx"], qz["sbit"], qz["n16"], qz["r16"], fmt, signs, S, cb)
    sc = O.search_scores(qs, xt)
    assert sc.shape == (5, 40)
    for i in range(5):
        qp = np.zeros(d)
        qp[:d_in] = qs[i]
        est, scale = O.estimator_dot(qp, qz["idx"], qz["sbit"], qz["n16"], qz["r16"], fmt, signs,
                                     S, cb)
        np.testing.assert_allclose(sc[i], est, rtol=0, atol=1e-12 * np.max(scale))


def test_recall_at_k_hand_cases():
    est = np.array([[1, 2, 3], [4, 5, 6], [9, 8, 7]])
    exact = np.array([[3, 2, 9], [7, 8, 9], [7, 8, 9]])
    assert O.recall_at_k(est, exact) == pytest.approx((2 + 0 + 3) / 9, abs=1e-15)
    assert O.recall_at_k(exact, exact) == 1.0
    assert O.recall_at_k(est[:1, :1], exact[:1, :1]) == 0.0


def test_attention_matches_hand_expanded_softmax():
    d, L = 8, 16
    g = TI.gen(8)
    q = g.standard_normal(d)
    k = g.standard_normal((L, d))
    v = g.standard_normal((L, d))
    scale = 1 / math.sqrt(d)
    out, logits, p, nd, dm = O.attend(q, k, v, scale)
    exps = [math.exp(sum(q[j] * k[t][j] for j in range(d)) * scale) for t in range(L)]
    tot = sum(exps)
    ref = [sum(exps[t] / tot * v[t][j] for t in range(L)) for j in range(d)]
    np.testing.assert_allclose(out, ref, rtol=1e-12)
    assert nd == 0 and dm == 0.0


# ---------------------------------------------------------------------------- special cases
def test_zero_residual_cache_gives_textbook_attention():
    d, L = 128, 50
    fmt = O.Format.uniform(d, 3)
    cb = O.codebook(d, 3)
    signs, S = TI.rotation(d, 3)
    g = TI.gen(9)
    idx = g.integers(0, 8, (L, d))
    sbit = g.integers(0, 2, (L, d)).astype(bool)
    n16 = O.fp16_bits(g.uniform(1, 10, L))
    r16 = np.zeros(L, dtype=np.uint16)                           # r16 = 0
    q = g.standard_normal(d)
    kt = O.dequantize(idx, sbit, n16, r16, fmt, signs, S, cb)
    plain = O.unrotate(O.fp16_value(n16)[:, None] * cb.centroids[idx], signs)
    np.testing.assert_allclose(kt, plain, atol=1e-13)
    out, *_ = O.attend(q, kt, kt, 1 / math.sqrt(d))
    lg = plain @ q / math.sqrt(d)
    w = np.exp(lg - lg.max()); w /= w.sum()
    np.testing.assert_allclose(out, w @ plain, atol=1e-12)


def test_gate_extremes():
    g = TI.gen(10)
    q = g.standard_normal(16)
    k = g.standard_normal((20, 16))
    v = g.standard_normal((20, 16))
    o0, _, p, n0, m0 = O.attend(q, k, v, 0.25, tau=0.0)
    o1, _, _, n1, m1 = O.attend(q, k, v, 0.25, tau=1.0 + 1e-9)
    assert n0 == 0 and np.allclose(o1, 0) and n1 == 20 and abs(m1 - 1) < 1e-12
    tau = np.median(p)
    ot, _, _, nt, mt = O.attend(q, k, v, 0.25, tau=tau)
    np.testing.assert_allclose(ot, (p * (p >= tau)) @ v, atol=1e-14)
    assert nt == int(np.sum(p < tau))


def test_mirror_symmetry():
    d = 128
    for bits in (1, 2, 3):
        fmt = O.Format.uniform(d, bits)
        cb = O.codebook(d, bits)
        signs, S = TI.rotation(d, 12)
        x = TI.gen(13).standard_normal((100, d))
        a = O.quantize(x, fmt, signs, S, cb)
        b = O.quantize(-x, fmt, signs, S, cb)
        ok = ~a["amb_code"]
        assert np.array_equal(b["idx"][ok], ((1 << bits) - 1 - a["idx"])[ok])
        oks = ~(a["amb_sign"] | b["amb_sign"])
        assert np.array_equal(b["sbit"][oks], ~a["sbit"][oks])
        assert np.array_equal(a["n16"], b["n16"]) and np.array_equal(a["r16"], b["r16"])


def test_rotated_coordinates_follow_the_beta_marginal():
    """163.com explainer, section "第一步：PolarQuant": after the random rotation each
    coordinate follows a known, concentrated law.  For isotropic Gaussian inputs the
    rotated direction is exactly uniform on the sphere, so every coordinate has the
    Beta marginal; for the channel-scaled key/value law (std 0.5..8 per channel) the
    marginal stays within KS noise of it.  (The law is over inputs: a one-hot input is
    mapped to +-1/sqrt(d) in every coordinate, so no per-input statement holds.)"""
    d = 128
    cdf = lambda t: O.marginal_cdf(t, d)
    signs, _ = TI.rotation(d, 50_000)
    x = TI.gen(14).standard_normal((4000, d))
    z = O.rotate(x, signs) / np.linalg.norm(x, axis=1, keepdims=True)
    assert stats.kstest(z[:, 5], cdf).pvalue > 1e-3
    assert stats.kstest(z[:, 77], cdf).pvalue > 1e-3
    sig = np.exp(TI.gen(15).uniform(np.log(0.5), np.log(8.0), d))
    xs = TI.gen(16).standard_normal((4000, d)) * sig
    zs = O.rotate(xs, signs) / np.linalg.norm(xs, axis=1, keepdims=True)
    assert stats.kstest(zs[:, 9], cdf).pvalue > 1e-3
    # the unrotated channel-scaled coordinates are far from that law
    assert stats.kstest(xs[:, 0] / np.linalg.norm(xs, axis=1), cdf).pvalue < 1e-6
    e = np.zeros((1, d)); e[0, 3] = 1.0
    assert np.allclose(np.abs(O.rotate(e, signs)), 1 / math.sqrt(d))


# ---------------------------------------------------------------------------- format
def test_bit_accounting_turbo4():
    """zhidx article, section "01 turboquant_plus：介绍与详解": turbo4 is 4.25 bits per value,
    3.8x smaller than fp16.  Here: b = 4 (3-bit codes + 1 QJL bit) at d = 128 plus two
    fp16 norms per vector."""
    fmt = O.Format.uniform(128, 3)
    bits_per_val = (fmt.record_bytes() + 4) * 8 / 128
    assert bits_per_val == 4.25 and abs(16 / bits_per_val - 3.76) < 0.01
    assert O.Format(128, 3, 2, 64).record_bytes() == 56
    assert O.Format.uniform(256, 3).record_bytes() == 128


def test_pack_layout_and_round_trip():
    fmt = O.Format(128, 3, 2, 64)
    g = TI.gen(15)
    n = 37
    idx = np.concatenate([g.integers(0, 8, (n, 64)), g.integers(0, 4, (n, 64))], axis=1)
    sbit = g.integers(0, 2, (n, 128)).astype(bool)
    rec = O.pack(idx, sbit, fmt)
    assert rec.shape == (n, 56)
    i2, s2 = O.unpack(rec, fmt)
    assert np.array_equal(i2, idx) and np.array_equal(s2, sbit)
    # hand-built record: every code = 5 (binary 101) in block 0, signs set only on
    # coordinate 1 of block 0
    idx1 = np.zeros((1, 128), dtype=np.int64); idx1[0, :32] = 5
    sb1 = np.zeros((1, 128), dtype=bool); sb1[0, 1] = True
    w = O.pack(idx1, sb1, fmt).view("<u4")[0]
    assert list(w[:4]) == [0xFFFFFFFF, 0, 0xFFFFFFFF, 2]
    assert not w[4:].any()


# ------------------------------------------------------------------ MSE-only ("PolarQuant alone")
def test_token_sliced_layout_hand_built():
    """The token-sliced layout on a hand-built case: vector 5 of the second group of 32 has
    code 0b101 and sign 1 at coordinate 37 (b = 4: 3 planes + sign per coordinate), every
    other bit 0.  Coordinate 37's words are words 4*37 .. 4*37+3 of group 1 and carry bit 5
    in planes 0 and 2 and in the sign word; nothing else is set."""
    fmt = O.Format.uniform(128, 3)
    idx = np.zeros((64, 128), np.int64)
    sb = np.zeros((64, 128), bool)
    idx[37, 37] = 0b101
    sb[37, 37] = True
    tiles = O.tiles_from_records(O.pack(idx, sb, fmt), fmt)
    assert tiles.shape == (2, 32 * 64)
    w = tiles.view("<u4")
    assert not w[0].any()
    expect = np.zeros(32 * 16, np.uint32)
    expect[4 * 37 + 0] = 1 << 5
    expect[4 * 37 + 2] = 1 << 5
    expect[4 * 37 + 3] = 1 << 5
    assert np.array_equal(w[1], expect)
    # mixed widths: coordinates >= 64 have 2 planes + sign (3 words) after 64 x 4 words
    fm = O.Format(128, 3, 2, 64)
    idx2 = np.zeros((32, 128), np.int64)
    idx2[31, 100] = 0b10
    t2 = O.tiles_from_records(O.pack(idx2, np.zeros((32, 128), bool), fm), fm).view("<u4")[0]
    k = 64 * 4 + (100 - 64) * 3 + 1
    assert t2[k] == 1 << 31 and np.count_nonzero(t2) == 1


def test_mse_only_layout_is_the_qjl_layout_without_sign_words():
    """An MSE-only record holds exactly the code planes of the QJL record, in order: each
    block's sign word removed (4.25 -> 3.25 bit/value at b = 4 with the norms)."""
    g = TI.gen(21)
    for fmt in (O.Format(128, 3, 3, 128), O.Format(128, 3, 2, 64), O.Format(256, 2, 2, 256)):
        mse = O.Format(fmt.d, fmt.bits_lo, fmt.bits_hi, fmt.split, qjl=False)
        idx = np.stack([g.integers(0, 1 << fmt.bits_of_block(j // 32), size=40) for j in range(fmt.d)], 1)
        sbit = g.integers(0, 2, size=(40, fmt.d)).astype(bool)
        full = O.pack(idx, sbit, fmt).view("<u4").reshape(40, -1)
        only = O.pack(idx, sbit, mse).view("<u4").reshape(40, -1)
        keep, k = [], 0
        for blk in range(fmt.d // 32):
            B = fmt.bits_of_block(blk)
            keep += list(range(k, k + B))
            k += B + 1
        assert np.array_equal(only, full[:, keep])
        i2, s2 = O.unpack(O.pack(idx, sbit, mse), mse)
        assert np.array_equal(i2, idx) and not s2.any()
    assert O.Format.uniform(128, 3, qjl=False).record_bytes() == 48


@pytest.mark.parametrize("bits", [2, 3])
def test_mse_only_reconstruction_error_is_d_times_codebook_mse(bits):
    """For unit vectors (n16 = 1 exactly) the MSE-only reconstruction x~ = Pi^T c[idx] has
    E||x - x~||^2 = d * mse, the codebook's expected squared error per coordinate under the
    exact marginal (computed in the oracle by quadrature), by Monte Carlo over random unit
    directions and fresh rotations."""
    d, n = 128, 4000
    fmt = O.Format.uniform(d, bits, qjl=False)
    cb = O.codebook(d, bits)
    errs = []
    for rep in range(5):
        x = TI.gen(300 + rep).standard_normal((n, d))
        x /= np.linalg.norm(x, axis=1, keepdims=True)
        signs, S = TI.rotation(d, 900 + rep)
        q = O.quantize(x, fmt, signs, S, cb)
        assert np.all(q["n16"] == O.fp16_bits(np.array([1.0]))[0])
        idx, sb = O.unpack(O.pack(q["idx"], q["sbit"], fmt), fmt)
        xt = O.dequantize(idx, sb, q["n16"], q["r16"], fmt, signs, S, cb, qjl=False)
        errs.append(np.sum((x - xt) ** 2, axis=1))
    e = np.concatenate(errs)
    se = e.std() / math.sqrt(e.size)
    assert abs(e.mean() - d * cb.mse) < 4 * se + 1e-3 * d * cb.mse, (e.mean(), d * cb.mse, se)


# ---------------------------------------------------------------------------- temporal decay
def _stored(x, fmt, signs, S):
    lo, hi = O.codebook(fmt.d, fmt.bits_lo), O.codebook(fmt.d, fmt.bits_hi)
    q = O.quantize(x, fmt, signs, S, lo, hi)
    return O.pack(q["idx"], q["sbit"], fmt), q["n16"], q["r16"], lo, hi


def test_requantize_is_quantize_of_the_unrotated_reconstruction():
    """Re-encoding a record (b4 -> b3, and b4 -> 2.5 bit) gives the same codes, signs and
    norms as quantizing the un-rotated reconstruction x~ = Pi^T y~ from scratch: the
    re-encode happens in the rotation both formats share."""
    d = 128
    signs, S = TI.rotation(d, 77)
    _, S2 = TI.rotation(d, 78)
    x = TI.gen(79).standard_normal((300, d)) * 3.0
    f_in = O.Format.uniform(d, 3)
    rec, n16, r16, lo, hi = _stored(x, f_in, signs, S)
    for f_out, S_out in ((O.Format.uniform(d, 2), S), (O.Format(d, 2, 1, 64), S2)):
        lo2, hi2 = O.codebook(d, f_out.bits_lo), O.codebook(d, f_out.bits_hi)
        rq = O.requantize(rec, n16, r16, f_in, S, lo, hi, f_out, S_out, lo2, hi2)
        idx, sb = O.unpack(rec, f_in)
        xt = O.dequantize(idx, sb, n16, r16, f_in, signs, S, lo, hi)
        ref = O.quantize(xt, f_out, signs, S_out, lo2, hi2)
        ok_code = ~(rq["amb_code"] | ref["amb_code"])
        assert np.array_equal(rq["idx"][ok_code], ref["idx"][ok_code])
        same_codes = np.all(rq["idx"] == ref["idx"], axis=1)
        ok_sign = ~(rq["amb_sign"] | ref["amb_sign"]) & same_codes[:, None]
        assert np.array_equal(rq["sbit"][ok_sign], ref["sbit"][ok_sign])
        assert np.array_equal(rq["n16"][~rq["amb_n16"]], ref["n16"][~rq["amb_n16"]])


def test_requantize_one_bit_mse_only_is_idempotent_with_closed_form_norm():
    """A 1-bit MSE-only record reconstructs to n16 * c0 * (+-1): re-encoding it at the same
    format keeps every code (z = +-1/sqrt(d), far from the 0 boundary) and stores the norm
    fp16(n16 * c0 * sqrt(d)), c0 = sqrt(2 / (pi d)) to first order, here the codebook's own
    positive centroid."""
    d = 128
    fmt = O.Format.uniform(d, 1, qjl=False)
    cb = O.codebook(d, 1)
    signs, S = TI.rotation(d, 5)
    x = TI.gen(6).standard_normal((200, d))
    rec, n16, r16, _, _ = _stored(x, fmt, signs, S)
    rq = O.requantize(rec, n16, r16, fmt, S, cb, cb, fmt, S, cb, cb)
    idx, _ = O.unpack(rec, fmt)
    assert np.array_equal(rq["idx"], idx)
    c0 = cb.centroids[1]
    assert abs(c0 - math.sqrt(2 / (math.pi * d))) < 0.01 * c0
    want = O.fp16_bits(O.fp16_value(n16) * c0 * math.sqrt(d))
    assert np.array_equal(rq["n16"], want)


def test_requantized_inner_products_stay_unbiased():
    """With a fresh JL matrix for the narrower format, the requantized reconstruction is an
    unbiased estimate of the stored one: E_S <y, x~'> = <y, x~> (163.com explainer, section
    "第二步：QJL", applied to x~ as the input)."""
    d, n_seeds = 128, 6000
    signs, S = TI.rotation(d, 11)
    g = TI.gen(12)
    x = g.standard_normal((1, d))
    y = 0.5 * x[0] + g.standard_normal(d)
    f_in, f_out = O.Format.uniform(d, 3), O.Format(d, 2, 1, 64)
    rec, n16, r16, lo, hi = _stored(x, f_in, signs, S)
    idx, sb = O.unpack(rec, f_in)
    xt = O.dequantize(idx, sb, n16, r16, f_in, signs, S, lo, hi)[0]
    lo2, hi2 = O.codebook(d, 2), O.codebook(d, 1)
    vals = np.empty(n_seeds)
    for s in range(n_seeds):
        _, S2 = TI.rotation(d, 40_000 + s)
        rq = O.requantize(rec, n16, r16, f_in, S, lo, hi, f_out, S2, lo2, hi2)
        x2 = O.dequantize(rq["idx"], rq["sbit"], rq["n16"], rq["r16"], f_out, signs, S2, lo2, hi2)[0]
        vals[s] = y @ x2
    se = vals.std(ddof=1) / math.sqrt(n_seeds)
    assert abs(vals.mean() - y @ xt) < 4 * se



# ---------------------------------------------------------------------------- storage rate
def test_storage_rate_matches_printed_figure():
    """The bytes the oracle stores per vector (packed record + the two fp16 norms), per
    value, against the rate the golden fixture copies from the page."""
    path = os.path.join(os.path.dirname(__file__), "golden", "storage_rate_b4.txt")
    rows = [l.split() for l in open(path, encoding="utf-8") if l.strip() and not l.startswith("#")]
    assert rows
    for d, cbits, qbits, bpv, ratio in rows:
        d, cbits, qbits, bpv, ratio = int(d), int(cbits), int(qbits), float(bpv), float(ratio)
        fmt = O.Format.uniform(d, cbits, qjl=qbits == 1)
        signs, S = TI.rotation(d, 5)
        qz = O.quantize(TI.gen(6).standard_normal((3, d)), fmt, signs, S, O.codebook(d, cbits))
        rec = O.pack(qz["idx"], qz["sbit"], fmt)
        stored = rec.shape[1] + np.asarray(qz["n16"]).itemsize + np.asarray(qz["r16"]).itemsize
        assert rec.shape == (3, fmt.record_bytes())
        assert stored * 8 / d == bpv
        assert round(16 / bpv, 1) == ratio
