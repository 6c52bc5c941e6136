"""The C++ oracle (oracle/tq_oracle.cpp) against the Python oracle (CPU).

Both write out the same definitions; the C++ one exists to time the method on the host
cores.  They must agree: fp16 rounding bit for bit (including midpoints, subnormals and
overflow), packed codes and sign bits bit for bit outside the ambiguity windows the Python
oracle reports, norms bit for bit outside their midpoint windows, dequantized vectors and
attention outputs to ~1e-12, and the thread count must not change a single bit."""
import math

import numpy as np
import pytest

import tq_inputs as TI
from oracle import tq_oracle as O
from oracle import tq_oracle_cpp as C
from parity_utils import oracle_codebooks


@pytest.fixture(scope="module", autouse=True)
def built():
    C.build()
    C.load()


def test_fp16_rounding_bit_for_bit():
    g = TI.gen(4100)
    v = np.concatenate([
        g.standard_normal(20000) * np.exp(g.uniform(-20, 12, 20000)),
        # exact midpoints between adjacent fp16 values (ties) and their neighbours
        ((np.arange(1, 2000, dtype=np.float64) + 0.5) * 2.0 ** -24),
        ((1024 + np.arange(0, 1023, dtype=np.float64) + 0.5) * 2.0 ** -10),
        np.nextafter((1024 + np.arange(0, 1023, dtype=np.float64) + 0.5) * 2.0 ** -10, np.inf),
        [0.0, -0.0, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 65504.0, 65519.99, 65520.0, 1e6, -1e6,
         6.1035156e-05, 6.0975552e-05]])
    assert np.array_equal(C.fp16_bits(v), O.fp16_bits(v))


FORMATS = [(128, 3, 3, 128, True), (128, 2, 2, 128, True), (128, 3, 2, 64, True),
           (128, 3, 3, 128, False), (256, 3, 3, 256, True)]


def _inputs(d, n, seed):
    if d == 128:
        kb, _, _ = TI.kv_layer(1, 1, n, d, seed=seed)
        x = TI.bf16_to_f64(kb.reshape(n, d))
    else:
        x = TI.search_set(n, 200, seed=seed).astype(np.float64)
    return x


@pytest.mark.parametrize("fmt_t", FORMATS)
def test_quantize_matches_python_oracle(fmt_t):
    d = fmt_t[0]
    fmt = O.Format(*fmt_t)
    x = _inputs(d, 384, 4200 + d + fmt_t[1] + fmt_t[2])
    signs, S = O.make_rotation(d, 4300 + d)
    cbs = oracle_codebooks(d, fmt.bits_lo, fmt.bits_hi)
    rec_c, n16_c, r16_c = C.quantize(x, fmt, signs, S, *cbs, threads=3)
    qz = O.quantize(x, fmt, signs, S, *cbs)
    idx_c, sb_c = O.unpack(rec_c, fmt)
    code_ok = (idx_c == qz["idx"]) | qz["amb_code"]
    assert code_ok.all()
    if fmt.qjl:
        sign_ok = (sb_c == qz["sbit"]) | qz["amb_sign"]
        assert sign_ok.all()
    assert np.all((n16_c == qz["n16"]) | qz["amb_n16"])
    assert np.all((r16_c == qz["r16"]) | qz["amb_r16"])
    # most vectors carry no ambiguity at all: their records are identical
    clean = ~(qz["amb_code"].any(axis=1) | qz["amb_sign"].any(axis=1) | qz["amb_n16"] | qz["amb_r16"])
    assert clean.mean() > 0.9
    rec_p = O.pack(qz["idx"], qz["sbit"], fmt)
    assert np.array_equal(rec_c[clean], rec_p[clean])


@pytest.mark.parametrize("fmt_t", FORMATS[:3] + FORMATS[4:])
def test_dequantize_matches_python_oracle(fmt_t):
    d = fmt_t[0]
    fmt = O.Format(*fmt_t)
    x = _inputs(d, 128, 4400 + d)
    signs, S = O.make_rotation(d, 4500 + d)
    cbs = oracle_codebooks(d, fmt.bits_lo, fmt.bits_hi)
    rec, n16, r16 = C.quantize(x, fmt, signs, S, *cbs)
    xc = C.dequantize(rec, n16, r16, fmt, signs, S, *cbs, threads=2)
    idx, sb = O.unpack(rec, fmt)
    xp = O.dequantize(idx, sb, n16, r16, fmt, signs, S, *cbs, qjl=fmt.qjl)
    assert np.max(np.abs(xc - xp)) <= 1e-12 * max(1.0, np.max(np.abs(xp)))


def test_attention_matches_python_oracle_and_threads_do_not_matter():
    d, hq, hkv, cap = 128, 8, 2, 300
    lens = [300, 117]
    fmt = O.Format.uniform(d, 3)
    kb, vb, _ = TI.kv_layer(2, hkv, cap, d, seed=4600)
    qb = TI.decode_queries(2, hq, d, 4600)
    signs, S = O.make_rotation(d, 4601)
    cbs = oracle_codebooks(d, 3, 3)
    kx, vx = TI.bf16_to_f64(kb).reshape(-1, d), TI.bf16_to_f64(vb).reshape(-1, d)
    rk, nk, rrk = C.quantize(kx, fmt, signs, S, *cbs)
    rv, nv, rrv = C.quantize(vx, fmt, signs, S, *cbs)
    kt = C.dequantize(rk, nk, rrk, fmt, signs, S, *cbs).reshape(2, hkv, cap, d)
    vt = C.dequantize(rv, nv, rrv, fmt, signs, S, *cbs).reshape(2, hkv, cap, d)
    q = TI.bf16_to_f64(qb)
    out1, lg1 = C.attend(q, kt, vt, lens, 1 / math.sqrt(d), threads=1)
    out4, lg4 = C.attend(q, kt, vt, lens, 1 / math.sqrt(d), threads=4)
    assert np.array_equal(out1, out4)
    G = hq // hkv
    for b in range(2):
        L = lens[b]
        for h in range(hq):
            o, lg, _, _, _ = O.attend(q[b, h], kt[b, h // G, :L], vt[b, h // G, :L], 1 / math.sqrt(d))
            assert np.max(np.abs(lg1[b, h, :L] - lg)) <= 1e-12 * max(1.0, np.max(np.abs(lg)))
            assert np.max(np.abs(out1[b, h] - o)) <= 1e-12 * max(1.0, np.max(np.abs(o)))
    # quantize: one thread and all threads give the same bytes
    r1 = C.quantize(kx[:64], fmt, signs, S, *cbs, threads=1)
    r8 = C.quantize(kx[:64], fmt, signs, S, *cbs, threads=0)
    for a, b_ in zip(r1, r8):
        assert np.array_equal(a, b_)


def test_gated_attention_matches_python_oracle():
    # Sparse-V gate: rows under tau dropped, no renormalization; one head with a x10 spike so
    # that both kept and dropped rows occur
    d, hq, hkv, cap = 128, 4, 1, 400
    lens = [400]
    fmt = O.Format.uniform(d, 3)
    kb, vb, _ = TI.kv_layer(1, hkv, cap, d, seed=4700, spike_frac=0.02)
    qb = TI.decode_queries(1, hq, d, 4700)
    signs, S = O.make_rotation(d, 4701)
    cbs = oracle_codebooks(d, 3, 3)
    kx, vx = TI.bf16_to_f64(kb).reshape(-1, d), TI.bf16_to_f64(vb).reshape(-1, d)
    rk, nk, rrk = C.quantize(kx, fmt, signs, S, *cbs)
    rv, nv, rrv = C.quantize(vx, fmt, signs, S, *cbs)
    kt = C.dequantize(rk, nk, rrk, fmt, signs, S, *cbs).reshape(1, hkv, cap, d)
    vt = C.dequantize(rv, nv, rrv, fmt, signs, S, *cbs).reshape(1, hkv, cap, d)
    q = TI.bf16_to_f64(qb)
    tau = 1e-3
    out, _, dropped = C.attend(q, kt, vt, lens, 1 / math.sqrt(d), threads=2, tau=tau,
                               return_dropped=True)
    n_total = 0
    for h in range(hq):
        o, _, _, nd, _ = O.attend(q[0, h], kt[0, 0], vt[0, 0], 1 / math.sqrt(d), tau=tau)
        assert dropped[0, h] == nd
        n_total += nd
        assert np.max(np.abs(out[0, h] - o)) <= 1e-12 * max(1.0, np.max(np.abs(o)))
    assert 0 < n_total < hq * cap


def test_topk_matches_python_oracle_scores_with_ties_to_lower_row():
    g = np.random.default_rng(4800)
    n, nq, d, k = 700, 9, 16, 10
    x = g.standard_normal((n, d))
    x[350] = x[20]          # equal scores: the lower row ranks first
    x[600] = x[20]
    q = g.standard_normal((nq, d))
    q[3] = x[20] * 3.0      # row 20 and its copies are the top three of query 3
    ids, sc = C.topk_ip(q, x, k, threads=3)
    ref = O.search_scores(q, x)
    for i in range(nq):
        order = np.lexsort((np.arange(n), -ref[i]))[:k]   # score descending, then row
        assert np.array_equal(ids[i], order)
        assert np.max(np.abs(sc[i] - ref[i, order])) <= 1e-12 * max(1.0, np.max(np.abs(ref[i])))
    assert list(ids[3, :3]) == [20, 350, 600]
    # fewer rows than k: the tail is empty
    ids2, sc2 = C.topk_ip(q[:2], x[:4], 6)
    assert (ids2[:, 4:] == -1).all() and np.isneginf(sc2[:, 4:]).all()
