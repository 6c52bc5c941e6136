"""CPU oracle for the TurboQuant hot path: plain, slow, fp64.

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of bench.py may import this module.  The product path
(the HIP library and its Python binding) never imports, calls or links it, and it
shares no code, table or constant with that path: the only things both sides see
are the seeded inputs from ``tq_inputs`` (data, the +/-1 diagonal and the Gaussian
JL matrix S).

What is computed, and where the pages say so ("163.com explainer" is the page at
m.163.com/dy/article/KOV7P8JI0556C3J2; "juejin post" is juejin.cn/post/7621074045394599990;
"zhidx article" is course.zhidx.com, the turboquant_plus write-up):

* rotation: a random rotation applied before quantizing -- 163.com explainer,
  section "第一步：PolarQuant"; the rotation is a Walsh-Hadamard transform preceded
  by a random sign flip -- zhidx article, intro and section "01 turboquant_plus：介绍与详解".
  Written out as its plain definition: y = H (D x) / sqrt(d), H the natural-order
  Sylvester Hadamard matrix (H_ij = (-1)^popcount(i & j)), built entry by entry.
* codebook: after rotation each coordinate follows a fixed, data-independent
  concentrated Beta law, and each coordinate gets its own scalar Lloyd-Max
  ("Max-Lloyd") quantizer, computed once and stored -- 163.com explainer,
  section "第一步：PolarQuant".  The law used is the exact marginal of one coordinate
  of a uniformly random unit vector in R^d.
* encode: (b-1) bits per coordinate for the direction plus one stored fp16 norm
  (the normalization overhead is a single scalar per vector) -- 163.com explainer,
  sections "TurboQuant 怎么做的" and "合起来".
* QJL: a Johnson-Lindenstrauss transform of the residual keeping only the sign
  (1 bit), with an estimator whose expectation equals the true inner product --
  163.com explainer, section "第二步：QJL"; juejin post, section
  "第二步：QJL —— 用1个比特修正误差".
* decode attention: attention logits computed from the compressed cache, then
  softmax, then the value-weighted sum -- 163.com explainer, section "速度".
  Sparse V (drop value rows with negligible attention weight) and asymmetric K/V
  widths -- zhidx article, section "01 turboquant_plus：介绍与详解".
* search: inner-product nearest neighbours over compressed vectors --
  163.com explainer, section "向量搜索".

Readings taken where the pages are silent: the sign flip D precedes the Hadamard
transform; the codebook law is the exact Beta marginal, not its Gaussian limit; a value
equal to a boundary goes to the lower cell; the residual lives in the rotated domain and
is taken against the stored fp16 norm; a zero projection counts as a 1 bit; decisions
within 1e-6 of a boundary are ambiguous (the windows below); Sparse V drops a value row
whose final weight is below tau without renormalizing; logits use the plain 1/sqrt(d)
scale.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
from scipy import special

# Windows inside which a decision is "ambiguous" (several answers are correct).
CODE_WINDOW = 1e-6      # |z_j - t_m| on the unit-direction coordinate
SIGN_WINDOW = 1e-6      # |u_i| of the projection of the *unit* residual
R16_WINDOW = 1e-6       # relative distance of ||r|| to an fp16 rounding midpoint
N16_WINDOW = 1e-12      # relative distance of ||x|| to an fp16 rounding midpoint


# --------------------------------------------------------------------------------------
# Rotation
# --------------------------------------------------------------------------------------
_H_CACHE: dict = {}


def hadamard(d: int) -> np.ndarray:
    """Natural-order Sylvester Hadamard matrix, H_ij = (-1)^popcount(i & j), float64."""
    if d <= 0 or d & (d - 1):
        raise ValueError("d must be a power of two")
    if d not in _H_CACHE:
        i = np.arange(d, dtype=np.uint64)
        parity = np.bitwise_count(i[:, None] & i[None, :]) & 1
        H = np.where(parity == 0, 1.0, -1.0)
        H.setflags(write=False)
        _H_CACHE[d] = H
    return _H_CACHE[d]


def rotate(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """y = H (D x) / sqrt(d) for each row of x [..., d] (random rotation; see module doc)."""
    d = x.shape[-1]
    H = hadamard(d)
    return (np.asarray(x, dtype=np.float64) * signs.astype(np.float64)) @ H.T / math.sqrt(d)


def unrotate(y: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """x = D H y / sqrt(d): the transpose (= inverse) of ``rotate``."""
    d = y.shape[-1]
    H = hadamard(d)
    return (np.asarray(y, dtype=np.float64) @ H) / math.sqrt(d) * signs.astype(np.float64)


# The seeded draws of a rotation.  The pages fix a random sign flip before the Hadamard
# transform and a Gaussian JL matrix for the residual (163.com explainer, sections
# "第一步：PolarQuant" and "第二步：QJL") but no generator.  Reading: SplitMix64
# (Steele, Lea and Flood, 2014) from the seed for the raw 64-bit draws; u = (x >> 11) 2^-53;
# sign i is -1 exactly when draw i has its top bit set; S in row-major order from
# Box-Muller (1958) pairs in fp64 with u1 = 1 - u (so log never sees 0), each entry rounded
# once to fp32.  Written here with Python integers and the math module, one value at a time.
_SM64_GAMMA = 0x9E3779B97F4A7C15
_SM64_M1 = 0xBF58476D1CE4E5B9
_SM64_M2 = 0x94D049BB133111EB
_U64 = (1 << 64) - 1
_ROT_CACHE: dict = {}


def splitmix64(seed: int, count: int) -> list:
    """The first ``count`` outputs of SplitMix64 started at state ``seed``."""
    state = seed & _U64
    out = []
    for _ in range(count):
        state = (state + _SM64_GAMMA) & _U64
        z = state
        z = ((z ^ (z >> 30)) * _SM64_M1) & _U64
        z = ((z ^ (z >> 27)) * _SM64_M2) & _U64
        out.append(z ^ (z >> 31))
    return out


def make_rotation(d: int, seed: int):
    """(signs int8 [d], S fp32 [d, d]) for one seed, by the reading stated above."""
    key = (d, seed & _U64)
    if key not in _ROT_CACHE:
        draws = splitmix64(seed, d + d * d)
        signs = np.array([-1 if (x >> 63) else 1 for x in draws[:d]], dtype=np.int8)
        vals = []
        for k in range(d, d + d * d, 2):
            u1 = 1.0 - (draws[k] >> 11) * 2.0 ** -53
            u2 = (draws[k + 1] >> 11) * 2.0 ** -53
            r = math.sqrt(-2.0 * math.log(u1))
            a = (2.0 * math.pi) * u2
            vals.append(r * math.cos(a))
            vals.append(r * math.sin(a))
        S = np.array(vals, dtype=np.float64).astype(np.float32).reshape(d, d)
        signs.setflags(write=False)
        S.setflags(write=False)
        _ROT_CACHE[key] = (signs, S)
    return _ROT_CACHE[key]


# --------------------------------------------------------------------------------------
# Codebook: Lloyd-Max for the marginal law of one rotated unit-vector coordinate
# --------------------------------------------------------------------------------------
def marginal_pdf(t, d: int):
    """Density of one coordinate of a uniform unit vector in R^d on [-1, 1]:
    (1 - t^2)^((d-3)/2) / B(1/2, (d-1)/2)."""
    t = np.asarray(t, dtype=np.float64)
    a = (d - 1) / 2.0
    logn = special.betaln(0.5, a)
    return np.exp((a - 1.0) * np.log1p(-t * t) - logn)


def marginal_cdf(t, d: int):
    """P(z <= t): (1 + z)/2 is Beta((d-1)/2, (d-1)/2)."""
    a = (d - 1) / 2.0
    return special.betainc(a, a, (1.0 + np.asarray(t, dtype=np.float64)) / 2.0)


def _cell_mass(lo: float, hi: float, d: int) -> float:
    a = (d - 1) / 2.0
    # use the upper tail where it is the better-conditioned difference
    if lo >= 0.0:
        return float(special.betaincc(a, a, (1.0 + lo) / 2.0) -
                     special.betaincc(a, a, (1.0 + hi) / 2.0))
    return float(special.betainc(a, a, (1.0 + hi) / 2.0) -
                 special.betainc(a, a, (1.0 + lo) / 2.0))


def _cell_first_moment(lo: float, hi: float, d: int) -> float:
    """Integral of t * pdf(t) over [lo, hi] in closed form:
    the primitive of t (1-t^2)^((d-3)/2) is -(1-t^2)^((d-1)/2) / (d-1)."""
    a = (d - 1) / 2.0
    norm = math.exp(special.betaln(0.5, a))
    prim = lambda t: -((1.0 - t * t) ** a) / (d - 1) if abs(t) < 1.0 else 0.0
    return (prim(hi) - prim(lo)) / norm


def lloyd_max(d: int, bits: int, tol: float = 1e-13, max_iter: int = 200000):
    """Lloyd-Max quantizer with 2^bits levels for ``marginal_pdf(., d)``.

    Lloyd's two conditions are iterated: each centroid is the conditional mean of its
    cell, each boundary the midpoint of adjacent centroids.  Only the upper half is
    iterated and mirrored, so c[2^B-1-m] = -c[m] holds exactly.
    Returns (centroids fp64 ascending, boundaries fp64 ascending, mse per coordinate).
    """
    L = 1 << bits
    half = L // 2
    # start from equal-probability cells of the upper half
    probs = (np.arange(half) + 0.5) / half * 0.5 + 0.5
    a = (d - 1) / 2.0
    cpos = 2.0 * special.betaincinv(a, a, probs) - 1.0
    for it in range(max_iter):
        bnd_pos = np.concatenate([[0.0], (cpos[:-1] + cpos[1:]) / 2.0, [1.0]])
        new = np.array([_cell_first_moment(bnd_pos[m], bnd_pos[m + 1], d) /
                        _cell_mass(bnd_pos[m], bnd_pos[m + 1], d) for m in range(half)])
        delta = np.max(np.abs(new - cpos))
        cpos = new
        if delta < tol:
            break
    else:
        raise RuntimeError("Lloyd-Max iteration did not converge")
    cent = np.concatenate([-cpos[::-1], cpos])
    bnd = (cent[:-1] + cent[1:]) / 2.0
    # MSE at the Lloyd point: E[z^2] - sum_m c_m^2 P_m, with E[z^2] = 1/d
    edges = np.concatenate([[-1.0], bnd, [1.0]])
    mass = np.array([_cell_mass(edges[m], edges[m + 1], d) for m in range(L)])
    mse = 1.0 / d - float(np.sum(cent * cent * mass))
    return cent, bnd, mse


@dataclass
class Codebook:
    bits: int
    centroids: np.ndarray   # fp32 values (stored as float64 for arithmetic), ascending
    bounds: np.ndarray      # fp32 values, ascending, 2^bits - 1 of them
    mse: float


_CB_CACHE: dict = {}


def codebook(d: int, bits: int) -> Codebook:
    """The stored table: fp32 round-to-nearest of the Lloyd-Max centroids and of the
    fp64 midpoints between adjacent centroids."""
    key = (d, bits)
    if key not in _CB_CACHE:
        c, b, mse = lloyd_max(d, bits)
        _CB_CACHE[key] = Codebook(bits, c.astype(np.float32).astype(np.float64),
                                  b.astype(np.float32).astype(np.float64), mse)
    return _CB_CACHE[key]


# --------------------------------------------------------------------------------------
# Format
# --------------------------------------------------------------------------------------
@dataclass(frozen=True)
class Format:
    """Per-vector packed format.  Coordinates j < split use bits_lo codebook bits, the
    rest bits_hi (split == d means one width).  With qjl each coordinate also gets one QJL
    bit (one sign word per block); without it the tensor is stored MSE-only ("PolarQuant
    alone": codebook planes and norms, no residual sketch)."""
    d: int
    bits_lo: int
    bits_hi: int
    split: int
    qjl: bool = True

    @staticmethod
    def uniform(d: int, bits: int, qjl: bool = True) -> "Format":
        return Format(d, bits, bits, d, qjl)

    def bits_of_block(self, blk: int) -> int:
        return self.bits_lo if 32 * blk < self.split else self.bits_hi

    def words_per_vector(self) -> int:
        return sum(self.bits_of_block(b) + (1 if self.qjl else 0) for b in range(self.d // 32))

    def record_bytes(self) -> int:
        return 4 * self.words_per_vector()


def fp16_bits(v: np.ndarray) -> np.ndarray:
    """fp64 -> fp16 (round to nearest even), as uint16 bit patterns."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def fp16_value(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _near_fp16_midpoint(v: np.ndarray, rel: float) -> np.ndarray:
    """True where v lies within rel*|v| of a point where fp16 rounding changes."""
    v = np.asarray(v, dtype=np.float64)
    h = v.astype(np.float16)
    up = np.nextafter(h, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(h, np.float16(-np.inf)).astype(np.float64)
    hv = h.astype(np.float64)
    dist = np.minimum(np.abs(v - (hv + up) / 2.0), np.abs(v - (hv + dn) / 2.0))
    return dist <= rel * np.abs(v)


# --------------------------------------------------------------------------------------
# Quantize (rotation -> norm -> per-coordinate codebook -> residual -> QJL sign)
# --------------------------------------------------------------------------------------
def quantize(x: np.ndarray, fmt: Format, signs: np.ndarray, S: np.ndarray,
             cb_lo: Codebook, cb_hi: Codebook | None = None) -> dict:
    """Quantize each row of x [n, d_in] (d_in <= d; missing coordinates are zeros).

    Steps (module doc): y = H D x / sqrt(d); n = ||x||, stored as fp16 n16;
    z = y / n; idx_j = #{m : t_m < z_j} with the coordinate's table; residual
    r = y - n16 * c[idx] in the rotated domain; r16 = fp16(||r||);
    u = S (r / ||r||); sign bit = 1 where u >= 0 (all ones when r = 0).
    Also returns the ambiguity masks used by parity checks.
    """
    x = np.asarray(x, dtype=np.float64)
    n, d_in = x.shape
    xp = np.zeros((n, fmt.d))
    xp[:, :d_in] = x
    y = rotate(xp, signs)
    nrm = np.sqrt(np.sum(xp * xp, axis=1))
    return encode_rotated(y, nrm, fmt, S, cb_lo, cb_hi)


def encode_rotated(y: np.ndarray, nrm: np.ndarray, fmt: Format, S: np.ndarray,
                   cb_lo: Codebook, cb_hi: Codebook | None = None) -> dict:
    """The steps of ``quantize`` after the rotation: y [n, d] rotated rows, nrm [n] their
    norms (||x|| = ||y||, the rotation being orthogonal)."""
    cb_hi = cb_lo if cb_hi is None else cb_hi
    n, d = y.shape
    n16b = fp16_bits(nrm)
    n16 = fp16_value(n16b)
    safe = np.where(nrm > 0.0, nrm, 1.0)
    z = np.where(nrm[:, None] > 0.0, y / safe[:, None], 0.0)

    col_lo = np.arange(d) < fmt.split
    idx = np.zeros((n, d), dtype=np.int64)
    amb_code = np.zeros((n, d), dtype=bool)
    cval = np.zeros((n, d))
    for cb, cols in ((cb_lo, col_lo), (cb_hi, ~col_lo)):
        if not cols.any():
            continue
        zc = z[:, cols]
        # idx = #{m : t_m < z}: searchsorted(side="left") returns exactly that count
        ic = np.searchsorted(cb.bounds, zc, side="left")
        idx[:, cols] = ic
        # the nearest boundary is the last one below z or the first one at/above it
        below = cb.bounds[np.maximum(ic - 1, 0)]
        above = cb.bounds[np.minimum(ic, len(cb.bounds) - 1)]
        amb_code[:, cols] = np.minimum(np.abs(zc - below), np.abs(zc - above)) < CODE_WINDOW
        cval[:, cols] = cb.centroids[ic]

    r = y - n16[:, None] * cval
    rn = np.sqrt(np.sum(r * r, axis=1))
    r16b = fp16_bits(rn)
    rsafe = np.where(rn > 0.0, rn, 1.0)
    rhat = np.where(rn[:, None] > 0.0, r / rsafe[:, None], 0.0)
    u = rhat @ np.asarray(S, dtype=np.float64).T
    sbit = (u >= 0.0)
    return dict(idx=idx, sbit=sbit, n16=n16b, r16=r16b, y=y, z=z, r=r, u=u,
                amb_code=amb_code, amb_sign=np.abs(u) < SIGN_WINDOW,
                amb_n16=_near_fp16_midpoint(nrm, N16_WINDOW),
                amb_r16=_near_fp16_midpoint(rn, R16_WINDOW), norm=nrm, rnorm=rn)


# --------------------------------------------------------------------------------------
# Block-32 bit-sliced packing
# --------------------------------------------------------------------------------------
def pack(idx: np.ndarray, sbit: np.ndarray, fmt: Format) -> np.ndarray:
    """Records [n, record_bytes] uint8.  For each block of 32 coordinates, in order:
    the B code bit-planes (plane p holds bit p of each code) then, with QJL, one word of
    sign bits; bit i of a word belongs to coordinate (or projection) 32*block + i; words
    are little-endian uint32.  Layout idea: the zhidx article's "block-32" layout
    (section "01 turboquant_plus：介绍与详解")."""
    n, d = idx.shape
    chunks = []
    for blk in range(d // 32):
        B = fmt.bits_of_block(blk)
        cols = slice(32 * blk, 32 * blk + 32)
        for p in range(B):
            bitsp = ((idx[:, cols] >> p) & 1).astype(np.uint8)
            # bit i of the word = coordinate 32*blk + i, little-endian bytes
            chunks.append(np.packbits(bitsp, axis=1, bitorder="little"))
        if fmt.qjl:
            chunks.append(np.packbits(sbit[:, cols].astype(np.uint8), axis=1, bitorder="little"))
    return np.ascontiguousarray(np.concatenate(chunks, axis=1)).reshape(n, -1)


def unpack(rec: np.ndarray, fmt: Format):
    """Inverse of ``pack``: (idx [n, d] int64, sbit [n, d] bool; sbit all False when the
    format has no QJL bits)."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    n = rec.shape[0]
    w = rec.view("<u4").reshape(n, fmt.words_per_vector()).astype(np.int64)
    idx = np.zeros((n, fmt.d), dtype=np.int64)
    sbit = np.zeros((n, fmt.d), dtype=bool)
    k = 0
    shifts = np.arange(32)
    for blk in range(fmt.d // 32):
        B = fmt.bits_of_block(blk)
        cols = slice(32 * blk, 32 * blk + 32)
        for p in range(B):
            idx[:, cols] |= ((w[:, k:k + 1] >> shifts) & 1) << p
            k += 1
        if fmt.qjl:
            sbit[:, cols] = ((w[:, k:k + 1] >> shifts) & 1).astype(bool)
            k += 1
    return idx, sbit


def tiles_from_records(rec: np.ndarray, fmt: Format) -> np.ndarray:
    """Token-sliced layout of a tensor's records, for n a multiple of 32: for each group of
    32 consecutive vectors, for each coordinate j = 0 .. d-1 in order, the words of that
    coordinate -- its code bit-planes, then its QJL sign when the format has one -- where
    bit t of a word is that bit of vector 32 * group + t.  It holds the same bits as the
    per-vector records, sliced across tokens instead of across coordinates (the block-32
    idea of the zhidx article, section "01 turboquant_plus：介绍与详解", applied to 32
    tokens), so the bits of one coordinate over 32 tokens are one word.
    Returns uint8 [n // 32, 32 * record_bytes]."""
    idx, sbit = unpack(rec, fmt)
    n, d = idx.shape
    if n % 32:
        raise ValueError("the token-sliced layout holds whole groups of 32 vectors")
    groups = []
    for g0 in range(0, n, 32):
        words = []
        for j in range(d):
            B = fmt.bits_of_block(j // 32)
            for p in range(B):
                words.append(np.packbits(((idx[g0:g0 + 32, j] >> p) & 1).astype(np.uint8),
                                         bitorder="little"))
            if fmt.qjl:
                words.append(np.packbits(sbit[g0:g0 + 32, j].astype(np.uint8), bitorder="little"))
        groups.append(np.concatenate(words))
    return np.stack(groups) if groups else np.zeros((0, 32 * fmt.record_bytes()), np.uint8)


def records_from_tiles(tiles: np.ndarray, fmt: Format) -> np.ndarray:
    """Inverse of ``tiles_from_records``: per-vector records [n, record_bytes]."""
    tiles = np.ascontiguousarray(tiles, dtype=np.uint8)
    ng = tiles.shape[0]
    d = fmt.d
    idx = np.zeros((32 * ng, d), dtype=np.int64)
    sbit = np.zeros((32 * ng, d), dtype=bool)
    t = np.arange(32)
    for g in range(ng):
        w = tiles[g].view("<u4").astype(np.int64)
        k = 0
        for j in range(d):
            B = fmt.bits_of_block(j // 32)
            for p in range(B):
                idx[32 * g:32 * g + 32, j] |= ((w[k] >> t) & 1) << p
                k += 1
            if fmt.qjl:
                sbit[32 * g:32 * g + 32, j] = ((w[k] >> t) & 1).astype(bool)
                k += 1
    return pack(idx, sbit, fmt)


# --------------------------------------------------------------------------------------
# Dequantize and the estimator
# --------------------------------------------------------------------------------------
def gamma(d: int) -> float:
    """QJL scale sqrt(pi/2)/m with m = d projections: E[<s,y> sign<s,r>] = sqrt(2/pi) <y, r/||r||>."""
    return math.sqrt(math.pi / 2.0) / d


def centroid_values(idx: np.ndarray, fmt: Format, cb_lo: Codebook, cb_hi: Codebook | None = None):
    cb_hi = cb_lo if cb_hi is None else cb_hi
    col_lo = np.arange(fmt.d) < fmt.split
    return np.where(col_lo[None, :], cb_lo.centroids[np.minimum(idx, len(cb_lo.centroids) - 1)],
                    cb_hi.centroids[np.minimum(idx, len(cb_hi.centroids) - 1)])


def dequantize_rotated(idx, sbit, n16b, r16b, fmt, S, cb_lo, cb_hi=None, qjl=True):
    """Reconstruction in the rotated domain: n16 * c[idx] + gamma * r16 * S^T (2 sigma - 1)."""
    c = centroid_values(idx, fmt, cb_lo, cb_hi)
    out = fp16_value(n16b)[:, None] * c
    if qjl:
        pm = np.where(sbit, 1.0, -1.0)
        out = out + gamma(fmt.d) * fp16_value(r16b)[:, None] * (pm @ np.asarray(S, dtype=np.float64))
    return out


def dequantize(idx, sbit, n16b, r16b, fmt, signs, S, cb_lo, cb_hi=None, qjl=True):
    """x~ = Pi^T (n16 c[idx] + gamma r16 S^T sigma): the unbiased reconstruction whose inner
    product with any y has expectation <y, x> (163.com explainer, section "第二步：QJL")."""
    return unrotate(dequantize_rotated(idx, sbit, n16b, r16b, fmt, S, cb_lo, cb_hi, qjl), signs)


def requantize(rec, n16b, r16b, fmt_in: Format, S_in, cbi_lo: Codebook, cbi_hi: Codebook | None,
               fmt_out: Format, S_out, cbo_lo: Codebook, cbo_hi: Codebook | None = None) -> dict:
    """Temporal decay: stored tokens move to another (usually narrower) format -- zhidx
    article, section "01 turboquant_plus：介绍与详解" (older tokens drop to lower precision).
    Reading: the record's reconstruction in the rotated domain,
    y~ = n16 c[idx] + gamma r16 S_in^T (2 sigma - 1) (the sign term only when fmt_in has
    QJL), is encoded again as a rotated vector of norm ||y~||, by the same steps as
    ``quantize`` after its rotation (so the rotation D, H is shared by both formats).
    rec [n, record_bytes(fmt_in)] uint8, n16b / r16b [n] fp16 bit patterns."""
    idx, sbit = unpack(rec, fmt_in)
    y = dequantize_rotated(idx, sbit, n16b, r16b, fmt_in, S_in, cbi_lo, cbi_hi, qjl=fmt_in.qjl)
    return encode_rotated(y, np.sqrt(np.sum(y * y, axis=1)), fmt_out, S_out, cbo_lo, cbo_hi)


def estimator_dot(q, idx, sbit, n16b, r16b, fmt, signs, S, cb_lo, cb_hi=None):
    """The fused estimator <q_rot, c[idx]> n16 + gamma r16 <S q_rot, sigma>, with
    q_rot = H D q / sqrt(d); plus the absolute-sum scale of its terms.
    q [d]; returns (values [n], abs_scale [n])."""
    qr = rotate(np.asarray(q, dtype=np.float64)[None, :], signs)[0]
    sq = np.asarray(S, dtype=np.float64) @ qr
    c = centroid_values(idx, fmt, cb_lo, cb_hi)
    pm = np.where(sbit, 1.0, -1.0)
    n16 = fp16_value(n16b)
    r16 = fp16_value(r16b)
    g = gamma(fmt.d)
    val = n16 * (c @ qr) + g * r16 * (pm @ sq)
    scale = n16 * (np.abs(c) @ np.abs(qr)) + g * r16 * np.sum(np.abs(sq))
    return val, scale


# --------------------------------------------------------------------------------------
# Decode attention over a packed cache (plain definition)
# --------------------------------------------------------------------------------------
def attend(q, k_tilde, v_tilde, scale: float, tau: float = 0.0):
    """Textbook softmax attention of one query q [d] over dequantized keys/values [L, d]:
    l = <q, k~> * scale, p = softmax(l), out = sum_t p_t v~_t.
    With tau > 0 value rows whose final weight p_t < tau are dropped from the sum
    (no renormalization).  Returns out, logits, p, n_dropped, dropped_mass."""
    logits = (np.asarray(k_tilde) @ np.asarray(q, dtype=np.float64)) * scale
    if logits.size == 0:
        return np.zeros(k_tilde.shape[1]), logits, logits, 0, 0.0
    m = np.max(logits)
    e = np.exp(logits - m)
    p = e / np.sum(e)
    keep = p >= tau if tau > 0.0 else np.ones_like(p, dtype=bool)
    out = p[keep] @ np.asarray(v_tilde)[keep]
    return out, logits, p, int(np.sum(~keep)), float(np.sum(p[~keep]))


# --------------------------------------------------------------------------------------
# Compressed inner-product search
# --------------------------------------------------------------------------------------
def search_scores(queries, x_tilde):
    """Estimated inner products <q, x~_i> (queries zero-padded to the dequantized width)."""
    qd = np.zeros((queries.shape[0], x_tilde.shape[1]))
    qd[:, :queries.shape[1]] = queries
    return qd @ np.asarray(x_tilde).T


def recall_at_k(est_ids: np.ndarray, exact_ids: np.ndarray) -> float:
    """Mean over queries of |est & exact| / k (recall@k of the estimated top-k against the
    exact top-k; 163.com explainer, section "向量搜索", compares methods by this recall)."""
    k = exact_ids.shape[1]
    hits = [len(set(a.tolist()) & set(b.tolist())) for a, b in zip(est_ids, exact_ids)]
    return float(np.mean(hits)) / k
