"""ctypes binding of libtq.so.  Argument marshalling only: every step of the method runs in
the library's HIP kernels (or, for the codebook, its host C++ code).  PyTorch provides
device memory and the current stream; it does no arithmetic here."""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# TQ_LIB_PATH may name another build of the same library (the host-sanitizer test loads
# one that way); by default the in-tree libtq.so
LIB_PATH = os.environ.get("TQ_LIB_PATH") or os.path.join(_PKG, "libtq.so")

TQ_OK, TQ_ERR_ARG, TQ_ERR_SHAPE, TQ_ERR_ALIGN, TQ_ERR_HIP, TQ_ERR_NOCONV, TQ_ERR_WORKSPACE = \
    0, -1, -2, -3, -4, -5, -6
TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2


class TQError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {_strerror(code)} ({code})")


class c_format(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("bits_lo", ctypes.c_int32),
                ("bits_hi", ctypes.c_int32), ("split", ctypes.c_int32),
                ("qjl", ctypes.c_int32), ("layout", ctypes.c_int32)]


class c_tables(ctypes.Structure):
    _fields_ = [("centroids_lo", ctypes.c_void_p), ("bounds_lo", ctypes.c_void_p),
                ("centroids_hi", ctypes.c_void_p), ("bounds_hi", ctypes.c_void_p),
                ("signs", ctypes.c_void_p), ("S", ctypes.c_void_p)]


class c_cache_segment(ctypes.Structure):
    _fields_ = [("fk", ctypes.c_void_p), ("tk", ctypes.c_void_p), ("fv", ctypes.c_void_p),
                ("tv", ctypes.c_void_p), ("codes_k", ctypes.c_void_p), ("norms_k", ctypes.c_void_p),
                ("codes_v", ctypes.c_void_p), ("norms_v", ctypes.c_void_p),
                ("capacity", ctypes.c_int64), ("seq_lens", ctypes.c_void_p)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libtq.so (built in-tree by build.py); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libtq.so not built: run compressed_attention_rotate_amd/build.py "
                              f"(expected at {LIB_PATH})")
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        sig = {
            "tq_build_codebook": (ctypes.c_int, [I32, I32, P, P, P]),
            "tq_make_rotation": (ctypes.c_int, [I32, ctypes.c_uint64, P, P]),
            "tq_record_bytes": (I64, [P]),
            "tq_check_format": (ctypes.c_int, [P]),
            "tq_quantize_kv": (ctypes.c_int, [P, P, P, I32, I64, I32, I64, P, P, P, P]),
            "tq_attend_workspace_bytes": (I64, [I32, I32, I32, I64, I32]),
            "tq_attend_decode": (ctypes.c_int, [P, P, P, P, P, I32, I32, I32, I32, P, P, P, P, I64,
                                                P, F32, F32, P, P, P, P, I64, P]),
            "tq_attend_decode_noalloc": (ctypes.c_int, [P, P, P, P, P, I32, I32, I32, I32, P, P, P,
                                                        P, I64, P, F32, F32, P, P, P, P]),
            "tq_attend_segments_workspace_bytes": (I64, [I32, I32, I32, I32, P, I32]),
            "tq_attend_decode_segments": (ctypes.c_int, [P, I32, P, I32, I32, I32, I32, F32, F32,
                                                         P, P, P, I64, P]),
            "tq_search_workspace_bytes": (I64, [I64, I32, I64, I32]),
            "tq_ip_search": (ctypes.c_int, [P, P, P, P, I64, P, I32, I64, I32, P, P, P, I64, P]),
            "tq_quantize_kv_paged": (ctypes.c_int, [P, P, P, I32, I64, I32, I32, I64, P, I32, I64,
                                                    P, P, P, P]),
            "tq_attend_decode_paged": (ctypes.c_int, [P, P, P, P, P, I32, I32, I32, I32, P, P, P, P,
                                                      I32, I64, P, I32, P, F32, F32, P, P, P, P, I64,
                                                      P]),
            "tq_prefill_workspace_bytes": (I64, [I32, I32, I32, I64]),
            "tq_prefill_paged": (ctypes.c_int, [P, P, P, P, P, I32, I32, I32, I32, P, P, I32, I64,
                                                I64, P, P, P, P, I32, I64, P, I32, F32, P, P, P, I64,
                                                P]),
            "tq_requantize_workspace_bytes": (I64, [I64, I32]),
            "tq_requantize": (ctypes.c_int, [P, P, P, P, I64, P, P, P, P, P, P, I64, P]),
            "tq_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _strerror(code: int) -> str:
    try:
        return load().tq_strerror(code).decode()
    except Exception:  # pragma: no cover - library missing
        return "error"


def _check(code: int, what: str) -> None:
    if code != TQ_OK:
        raise TQError(code, what)


@dataclass(frozen=True)
class Format:
    """Packed format: codebook bits for coordinates < split and >= split, head dim d; qjl
    False stores the tensor MSE-only (no QJL sign words); layout 1 stores the tensor
    token-sliced (groups of 32 vectors, one word per coordinate and bit-plane; tq.h)."""
    d: int
    bits_lo: int
    bits_hi: int
    split: int
    qjl: bool = True
    layout: int = 0

    @staticmethod
    def uniform(d: int, bits: int, qjl: bool = True, layout: int = 0) -> "Format":
        return Format(d, bits, bits, d, qjl, layout)

    def sliced(self) -> "Format":
        """The same format in the token-sliced layout."""
        return Format(self.d, self.bits_lo, self.bits_hi, self.split, self.qjl, 1)

    def c(self) -> c_format:
        return c_format(self.d, self.bits_lo, self.bits_hi, self.split, 1 if self.qjl else 0,
                        int(self.layout))

    def record_bytes(self) -> int:
        f = self.c()
        n = load().tq_record_bytes(ctypes.byref(f))
        if n < 0:
            raise TQError(TQ_ERR_SHAPE, "tq_record_bytes")
        return int(n)


def build_codebook(d: int, bits: int):
    """Lloyd-Max table for one rotated coordinate: (centroids fp32, bounds fp32, mse)."""
    c = np.zeros(1 << bits, dtype=np.float32)
    b = np.zeros((1 << bits) - 1, dtype=np.float32)
    mse = ctypes.c_double()
    _check(load().tq_build_codebook(d, bits, c.ctypes.data, b.ctypes.data, ctypes.byref(mse)),
           "tq_build_codebook")
    return c, b, mse.value


def make_rotation(d: int, seed: int):
    """Seeded rotation draws from tq_make_rotation: (signs int8 [d], S fp32 [d, d]), host."""
    signs = np.zeros(d, dtype=np.int8)
    S = np.zeros((d, d), dtype=np.float32)
    _check(load().tq_make_rotation(d, ctypes.c_uint64(int(seed) & (2**64 - 1)), signs.ctypes.data,
                                   S.ctypes.data), "tq_make_rotation")
    return signs, S


@dataclass
class Tables:
    """Rotation and codebooks for one format.  signs: host int8 [d]; S: device fp32 [d, d]
    (a torch tensor); codebooks default to tq_build_codebook's.  ``Tables.from_seed`` makes
    the rotation with tq_make_rotation."""
    fmt: Format
    signs: np.ndarray
    S: "object"
    centroids_lo: np.ndarray = None
    bounds_lo: np.ndarray = None
    centroids_hi: np.ndarray = None
    bounds_hi: np.ndarray = None
    _keep: list = field(default_factory=list, repr=False)

    def __post_init__(self):
        self.signs = np.ascontiguousarray(self.signs, dtype=np.int8)
        if self.centroids_lo is None:
            self.centroids_lo, self.bounds_lo, _ = build_codebook(self.fmt.d, self.fmt.bits_lo)
        if self.centroids_hi is None:
            if self.fmt.bits_hi == self.fmt.bits_lo:
                self.centroids_hi, self.bounds_hi = self.centroids_lo, self.bounds_lo
            else:
                self.centroids_hi, self.bounds_hi, _ = build_codebook(self.fmt.d, self.fmt.bits_hi)
        for name in ("centroids_lo", "bounds_lo", "centroids_hi", "bounds_hi"):
            setattr(self, name, np.ascontiguousarray(getattr(self, name), dtype=np.float32))

    @staticmethod
    def from_seed(fmt: Format, seed: int, device="cuda") -> "Tables":
        import torch
        signs, S = make_rotation(fmt.d, seed)
        return Tables(fmt, signs, torch.from_numpy(S).to(device))

    def c(self) -> c_tables:
        S = self.S
        if not (S.is_cuda and S.dtype.is_floating_point and S.is_contiguous()):
            raise ValueError("S must be a contiguous fp32 CUDA tensor")
        return c_tables(self.centroids_lo.ctypes.data, self.bounds_lo.ctypes.data,
                        self.centroids_hi.ctypes.data, self.bounds_hi.ctypes.data,
                        self.signs.ctypes.data, S.data_ptr())
