"""Helpers for GPU-vs-oracle parity tests (imported by test modules; not collected).

The oracle is only ever fed seeded inputs (tq_inputs) or its own outputs.  GPU results
are compared against the oracle's results with plain numpy bit/float operations here.
"""
from __future__ import annotations

import numpy as np

import tq_inputs as TI
from oracle import tq_oracle as O


def rotations(d, seed):
    """Rotation draws for one seed, made by two independent implementations of one
    definition: the oracle's ``make_rotation`` (for the oracle side) and the library's
    ``tq_make_rotation`` (for the tables the GPU path reads).  tests/test_rotation.py pins
    them equal bit for bit.  Returns ((signs, S) oracle, (signs, S) library)."""
    import compressed_attention_rotate_amd as tq
    return O.make_rotation(d, seed), tq.make_rotation(d, seed)


def oracle_codebooks(d, bits_lo, bits_hi):
    return O.codebook(d, bits_lo), O.codebook(d, bits_hi)


KEEP = ("idx", "sbit", "n16", "r16", "amb_code", "amb_sign", "amb_n16", "amb_r16", "z", "r", "u",
        "norm")


def oracle_quantize(x, fmt: O.Format, signs, S, chunk: int = 8192, bf16: bool = False):
    """Oracle quantize + pack, applied to row chunks (each vector is independent; chunks
    only keep temporaries small).  x: float rows, or bf16 bit patterns with bf16=True."""
    lo, hi = oracle_codebooks(fmt.d, fmt.bits_lo, fmt.bits_hi)
    parts = []
    for s in range(0, max(1, x.shape[0]), chunk):
        xc = TI.bf16_to_f64(x[s:s + chunk]) if bf16 else np.asarray(x[s:s + chunk], dtype=np.float64)
        q = O.quantize(xc, fmt, signs, S, lo, hi)
        q["records"] = O.pack(q["idx"], q["sbit"], fmt)
        parts.append({k: q[k] for k in KEEP + ("records",)})
    qz = {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}
    qz["norms"] = np.stack([qz["n16"], qz["r16"]], axis=1).astype(np.uint16)
    return qz


def compare_quantize(gpu_codes: np.ndarray, gpu_norms: np.ndarray, qz: dict, fmt: O.Format,
                     n16_rel: float | None = None, sign_window: float | None = None):
    """Byte-level comparison of packed records and norms.

    Codes and sign bits must be identical except inside the ambiguity windows (a
    coordinate within 1e-6 of a codebook boundary; a projection of the unit residual
    within 1e-6 of zero).  When a vector's code bits differ (only possible inside the
    window) its residual differs, so its sign bits and r16 are not compared.  n16 must be
    identical (window 1e-12 relative); r16 identical except within 1e-6 (relative) of an
    fp16 rounding midpoint, where one ulp is allowed.  Returns a dict of counts.

    n16_rel / sign_window widen the n16 and sign windows for a kernel whose input to the
    encode is itself rounded (re-encoding from an fp32 reconstruction): n16 may then differ
    by one ulp within n16_rel (relative) of an fp16 midpoint, and signs within
    |u| < sign_window."""
    n = qz["idx"].shape[0]
    L = (1 << max(fmt.bits_lo, fmt.bits_hi)) - 1
    ref = qz["records"].view("<u4").reshape(n, -1)
    got = np.ascontiguousarray(gpu_codes, dtype=np.uint8).reshape(n, -1).view("<u4")
    assert got.shape == ref.shape, (got.shape, ref.shape)
    full_idx = np.where(np.arange(fmt.d) < fmt.split, (1 << fmt.bits_lo) - 1, (1 << fmt.bits_hi) - 1)
    code_amb = O.pack(np.where(qz["amb_code"], full_idx[None, :], 0), np.zeros_like(qz["sbit"]),
                      fmt).view("<u4").reshape(n, -1)
    amb_sign = qz["amb_sign"] if sign_window is None else np.abs(qz["u"]) < sign_window
    sign_amb = O.pack(np.zeros_like(qz["idx"]), amb_sign, fmt).view("<u4").reshape(n, -1)
    sign_bits = O.pack(np.zeros_like(qz["idx"]), np.ones_like(qz["sbit"]), fmt).view("<u4").reshape(n, -1)
    code_bits = ~sign_bits
    diff = got ^ ref
    code_diff = diff & code_bits
    assert not np.any(code_diff & ~code_amb), "code bits differ outside the boundary window"
    vec_code_differs = np.any(code_diff != 0, axis=1)
    sdiff = diff & sign_bits & ~sign_amb
    sdiff[vec_code_differs] = 0
    bad = np.nonzero(np.any(sdiff != 0, axis=1))[0]
    assert bad.size == 0, f"sign bits differ outside the zero window, vectors {bad[:10]}"
    gn = np.ascontiguousarray(gpu_norms).view(np.uint16).reshape(n, 2)
    rn = qz["norms"]
    if n16_rel is None:
        bad_n16 = (gn[:, 0] != rn[:, 0]) & ~qz["amb_n16"]
    else:
        near = O._near_fp16_midpoint(qz["norm"], n16_rel)
        ulp1 = np.abs(gn[:, 0].astype(np.int64) - rn[:, 0].astype(np.int64)) <= 1
        bad_n16 = (gn[:, 0] != rn[:, 0]) & ~(near & ulp1)
    assert not bad_n16.any(), f"n16 differs at {np.nonzero(bad_n16)[0][:10]}"
    r16_diff = (gn[:, 1] != rn[:, 1]) & ~vec_code_differs
    one_ulp = np.abs(gn[:, 1].astype(np.int64) - rn[:, 1].astype(np.int64)) <= 1
    assert not np.any(r16_diff & ~(qz["amb_r16"] & one_ulp)), \
        f"r16 differs at {np.nonzero(r16_diff & ~qz['amb_r16'])[0][:10]}"
    return dict(n=n, amb_codes=int(qz["amb_code"].sum()), amb_signs=int(amb_sign.sum()),
                code_diff_vectors=int(vec_code_differs.sum()),
                sign_diffs_in_window=int(np.count_nonzero(diff & sign_bits & sign_amb)),
                r16_midpoint_diffs=int(r16_diff.sum()))


def to_f64(x_np, dtype: str):
    if dtype == "bf16":
        return TI.bf16_to_f64(x_np)
    return np.asarray(x_np, dtype=np.float64)


def oracle_pack_cache(x_bhtd, fmt: O.Format, signs, S, bf16: bool = False):
    """Quantize a cache [batch, hkv, ntok, d] with the oracle; returns records
    [batch, hkv, ntok, rb] uint8, norms [batch, hkv, ntok, 2] uint16 and the quantize dict."""
    b, h, t, d = x_bhtd.shape
    qz = oracle_quantize(x_bhtd.reshape(-1, d), fmt, signs, S, bf16=bf16)
    return (qz["records"].reshape(b, h, t, -1), qz["norms"].reshape(b, h, t, 2), qz)


def oracle_decode(q64, rec_k, nrm_k, rec_v, nrm_v, seq_lens, fmt_k, fmt_v, signs_k, S_k, signs_v,
                  S_v, scale, tau=0.0):
    """Oracle attention for every (batch, q head): explicit dequantization of the packed
    bytes, then textbook softmax attention.  Returns out [b, hq, d], logits list, logit
    scales list, dropped-row counts and masses."""
    batch, hq, d = q64.shape
    hkv = rec_k.shape[1]
    G = hq // hkv
    cbk = oracle_codebooks(d, fmt_k.bits_lo, fmt_k.bits_hi)
    cbv = oracle_codebooks(d, fmt_v.bits_lo, fmt_v.bits_hi)
    out = np.zeros((batch, hq, d))
    logits, scales, drops, masses = {}, {}, {}, {}
    for bi in range(batch):
        L = int(seq_lens[bi])
        for kh in range(hkv):
            ik, sk = O.unpack(rec_k[bi, kh, :L], fmt_k)
            iv, sv = O.unpack(rec_v[bi, kh, :L], fmt_v)
            kt = O.dequantize(ik, sk, nrm_k[bi, kh, :L, 0], nrm_k[bi, kh, :L, 1], fmt_k, signs_k,
                              S_k, *cbk, qjl=fmt_k.qjl)
            vt = O.dequantize(iv, sv, nrm_v[bi, kh, :L, 0], nrm_v[bi, kh, :L, 1], fmt_v, signs_v,
                              S_v, *cbv, qjl=fmt_v.qjl)
            for g in range(G):
                h = kh * G + g
                o, lg, p, nd, dm = O.attend(q64[bi, h], kt, vt, scale, tau)
                out[bi, h] = o
                _, esc = O.estimator_dot(q64[bi, h], ik, sk, nrm_k[bi, kh, :L, 0],
                                         nrm_k[bi, kh, :L, 1], fmt_k, signs_k, S_k, *cbk)
                logits[(bi, h)], scales[(bi, h)] = lg, esc * scale
                drops[(bi, h)], masses[(bi, h)] = nd, dm
    return out, logits, scales, drops, masses


def oracle_search_chunk(args):
    """One chunk of a search database through the oracle, for a process pool: quantize and
    pack the rows, then score them for each query with the oracle's fused estimator.
    args = (rows fp32 [n, d_in], queries fp32 [nq, d_in], d, bits, rotation seed).  Returns
    (records, norms, scores [nq, n], absolute-sum scales [nq, n], ambiguous [n])."""
    from threadpoolctl import threadpool_limits
    x, queries, d, bits, seed = args
    with threadpool_limits(1):
        return _oracle_search_chunk(x, queries, d, bits, seed)


def _oracle_search_chunk(x, queries, d, bits, seed):
    fmt = O.Format.uniform(d, bits)
    signs, S = O.make_rotation(d, seed)
    cb = O.codebook(d, bits)
    qz = O.quantize(np.asarray(x, dtype=np.float64), fmt, signs, S, cb)
    rec = O.pack(qz["idx"], qz["sbit"], fmt)
    scores = np.empty((len(queries), len(x)))
    scales = np.empty((len(queries), len(x)))
    for i, q in enumerate(queries):
        qp = np.zeros(d)
        qp[:len(q)] = q
        scores[i], scales[i] = O.estimator_dot(qp, qz["idx"], qz["sbit"], qz["n16"], qz["r16"],
                                               fmt, signs, S, cb)
    amb = qz["amb_code"].any(axis=1) | qz["amb_sign"].any(axis=1)
    norms = np.stack([qz["n16"], qz["r16"]], axis=1).astype(np.uint16)
    return rec, norms, scores, scales, amb
