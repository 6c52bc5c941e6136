"""ctypes wrapper of the C++ oracle (oracle/tq_oracle.cpp, built as oracle/libtq_oracle.so).

TEST INFRASTRUCTURE ONLY, like oracle/tq_oracle.py: loaded by tests/, smoke() and the
cpu_baseline leg of bench.py, never by the product path.  The codebooks and the rotation's
draws come from the Python oracle; the C++ side quantizes, packs, dequantizes and attends
in fp64 with std::thread workers (threads = 0: every hardware thread)."""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tq_oracle.cpp")
LIB_PATH = os.path.join(HERE, "libtq_oracle.so")
_lib = None


def build() -> str:
    """Compile the C++ oracle (plain -O2, IEEE arithmetic, no fast-math)."""
    cmd = ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", SRC, "-o", LIB_PATH]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"C++ oracle build failed:\n{res.stdout}\n{res.stderr}")
    return LIB_PATH


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, I64, F64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.tqo_hardware_threads.restype = ctypes.c_int
        lib.tqo_fp16_bits.argtypes = [P, I64, P]
        lib.tqo_quantize.argtypes = [P, P, P, P, P, P, P, P, I64, I32, P, P, P, I32]
        lib.tqo_dequantize.argtypes = [P, P, P, P, P, P, P, P, I64, P, I32]
        lib.tqo_attend.argtypes = [P, P, P, P, I32, I32, I32, I64, I32, F64, F64, P, P, P, I32]
        lib.tqo_topk_ip.argtypes = [P, P, I64, I64, I32, I32, P, P, I32]
        _lib = lib
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _fmt5(fmt):
    return np.array([fmt.d, fmt.bits_lo, fmt.bits_hi, fmt.split, 1 if fmt.qjl else 0], np.int32)


def hardware_threads() -> int:
    return int(load().tqo_hardware_threads())


def fp16_bits(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64).ravel()
    out = np.empty(v.size, np.uint16)
    load().tqo_fp16_bits(_p(v), v.size, _p(out))
    return out


def quantize(x, fmt, signs, S, cb_lo, cb_hi=None, threads: int = 0):
    """Rows of x [n, d_in] -> (records uint8 [n, record_bytes], n16 uint16 [n], r16 uint16 [n])."""
    cb_hi = cb_lo if cb_hi is None else cb_hi
    x = np.ascontiguousarray(x, dtype=np.float64)
    n, d_in = x.shape
    words = fmt.words_per_vector()
    rec = np.empty((n, words), np.uint32)
    n16 = np.empty(n, np.uint16)
    r16 = np.empty(n, np.uint16)
    f5 = _fmt5(fmt)
    cl, bl = np.ascontiguousarray(cb_lo.centroids, np.float64), np.ascontiguousarray(cb_lo.bounds, np.float64)
    ch, bh = np.ascontiguousarray(cb_hi.centroids, np.float64), np.ascontiguousarray(cb_hi.bounds, np.float64)
    sg = np.ascontiguousarray(signs, dtype=np.int8)
    Sm = np.ascontiguousarray(S, dtype=np.float64)
    load().tqo_quantize(_p(f5), _p(cl), _p(bl), _p(ch), _p(bh), _p(sg), _p(Sm), _p(x), n, d_in,
                        _p(rec), _p(n16), _p(r16), int(threads))
    return rec.view(np.uint8).reshape(n, 4 * words), n16, r16


def dequantize(records, n16, r16, fmt, signs, S, cb_lo, cb_hi=None, threads: int = 0):
    """Records [n, record_bytes] with their fp16 norms -> x~ [n, d] in the original domain."""
    cb_hi = cb_lo if cb_hi is None else cb_hi
    rec = np.ascontiguousarray(records, dtype=np.uint8)
    n = rec.shape[0]
    x = np.empty((n, fmt.d), np.float64)
    f5 = _fmt5(fmt)
    cl = np.ascontiguousarray(cb_lo.centroids, np.float64)
    ch = np.ascontiguousarray(cb_hi.centroids, np.float64)
    sg = np.ascontiguousarray(signs, dtype=np.int8)
    Sm = np.ascontiguousarray(S, dtype=np.float64)
    a16, b16 = np.ascontiguousarray(n16, np.uint16), np.ascontiguousarray(r16, np.uint16)
    load().tqo_dequantize(_p(f5), _p(cl), _p(ch), _p(sg), _p(Sm), _p(rec), _p(a16), _p(b16), n,
                          _p(x), int(threads))
    return x


def attend(q, kt, vt, lens, scale: float, threads: int = 0, tau: float = 0.0,
           return_dropped: bool = False):
    """q [batch, hq, d] against dequantized caches kt, vt [batch, hkv, cap, d] (fp64), the
    first lens[b] tokens of each sequence -> (out [batch, hq, d], logits [batch, hq, cap]).
    tau > 0: value rows with a final weight below tau are left out (no renormalization);
    with return_dropped the per-(batch, head) counts of those rows come third."""
    q = np.ascontiguousarray(q, np.float64)
    kt = np.ascontiguousarray(kt, np.float64)
    vt = np.ascontiguousarray(vt, np.float64)
    batch, hq, d = q.shape
    hkv, cap = kt.shape[1], kt.shape[2]
    ln = np.ascontiguousarray(lens, np.int32)
    out = np.empty((batch, hq, d), np.float64)
    lg = np.full((batch, hq, cap), np.nan, np.float64)
    dropped = np.zeros((batch, hq), np.int64)
    load().tqo_attend(_p(q), _p(kt), _p(vt), _p(ln), batch, hq, hkv, cap, d, float(scale),
                      float(tau), _p(out), _p(lg), _p(dropped), int(threads))
    return (out, lg, dropped) if return_dropped else (out, lg)


def topk_ip(q, x, k: int, threads: int = 0):
    """Top-k rows of x [n, d] by inner product with each query of q [nq, d] (fp64), ties to
    the lower row -> (ids int64 [nq, k], scores [nq, k])."""
    q = np.ascontiguousarray(q, np.float64)
    x = np.ascontiguousarray(x, np.float64)
    nq, d = q.shape
    n = x.shape[0]
    ids = np.empty((nq, k), np.int64)
    sc = np.empty((nq, k), np.float64)
    load().tqo_topk_ip(_p(q), _p(x), n, nq, d, int(k), _p(ids), _p(sc), int(threads))
    return ids, sc
