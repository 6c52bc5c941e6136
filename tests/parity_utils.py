"""Helpers for GPU-vs-oracle parity tests (imported by test modules; not collected).

The oracle is only ever fed seeded inputs (tq_inputs) or its own outputs.  GPU results
are compared against the oracle's results with plain numpy bit/float operations here.
"""
from __future__ import annotations

import numpy as np

import tq_inputs as TI
from oracle import tq_oracle as O


def oracle_codebooks(d, bits_lo, bits_hi):
    return O.codebook(d, bits_lo), O.codebook(d, bits_hi)


def oracle_quantize(x64, fmt: O.Format, signs, S):
    lo, hi = oracle_codebooks(fmt.d, fmt.bits_lo, fmt.bits_hi)
    qz = O.quantize(x64, fmt, signs, S, lo, hi)
    qz["records"] = O.pack(qz["idx"], qz["sbit"], fmt)
    qz["norms"] = np.stack([qz["n16"], qz["r16"]], axis=1).astype(np.uint16)
    return qz


def compare_quantize(gpu_codes: np.ndarray, gpu_norms: np.ndarray, qz: dict, fmt: O.Format):
    """Byte-level comparison of packed records and norms.

    Codes and sign bits must be identical except inside the ambiguity windows (a
    coordinate within 1e-6 of a codebook boundary; a projection of the unit residual
    within 1e-6 of zero).  When a vector's code bits differ (only possible inside the
    window) its residual differs, so its sign bits and r16 are not compared.  n16 must be
    identical (window 1e-12 relative); r16 identical except within 1e-6 (relative) of an
    fp16 rounding midpoint, where one ulp is allowed.  Returns a dict of counts."""
    n = qz["idx"].shape[0]
    L = (1 << max(fmt.bits_lo, fmt.bits_hi)) - 1
    ref = qz["records"].view("<u4").reshape(n, -1)
    got = np.ascontiguousarray(gpu_codes, dtype=np.uint8).reshape(n, -1).view("<u4")
    assert got.shape == ref.shape, (got.shape, ref.shape)
    full_idx = np.where(np.arange(fmt.d) < fmt.split, (1 << fmt.bits_lo) - 1, (1 << fmt.bits_hi) - 1)
    code_amb = O.pack(np.where(qz["amb_code"], full_idx[None, :], 0), np.zeros_like(qz["sbit"]),
                      fmt).view("<u4").reshape(n, -1)
    sign_amb = O.pack(np.zeros_like(qz["idx"]), qz["amb_sign"], fmt).view("<u4").reshape(n, -1)
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
    bad_n16 = (gn[:, 0] != rn[:, 0]) & ~qz["amb_n16"]
    assert not bad_n16.any(), f"n16 differs at {np.nonzero(bad_n16)[0][:10]}"
    r16_diff = (gn[:, 1] != rn[:, 1]) & ~vec_code_differs
    one_ulp = np.abs(gn[:, 1].astype(np.int64) - rn[:, 1].astype(np.int64)) <= 1
    assert not np.any(r16_diff & ~(qz["amb_r16"] & one_ulp)), \
        f"r16 differs at {np.nonzero(r16_diff & ~qz['amb_r16'])[0][:10]}"
    return dict(n=n, amb_codes=int(qz["amb_code"].sum()), amb_signs=int(qz["amb_sign"].sum()),
                code_diff_vectors=int(vec_code_differs.sum()),
                sign_diffs_in_window=int(np.count_nonzero(diff & sign_bits & sign_amb)),
                r16_midpoint_diffs=int(r16_diff.sum()))


def to_f64(x_np, dtype: str):
    if dtype == "bf16":
        return TI.bf16_to_f64(x_np)
    return np.asarray(x_np, dtype=np.float64)
