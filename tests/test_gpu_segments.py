"""GPU: decode over a cache kept in segments of different formats (temporal decay: older
tokens re-encoded to a narrower format) against the oracle.  Expected values: each
segment's packed bytes dequantized by the oracle with that segment's format, the token
lists concatenated in segment order, then the oracle's textbook softmax attention."""
import math

import numpy as np
import pytest

import tq_inputs as TI
from oracle import tq_oracle as O
from parity_utils import oracle_codebooks, oracle_pack_cache, rotations

pytestmark = pytest.mark.gpu

OUT_ATOL = 2e-3


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import compressed_attention_rotate_amd as tq
    tq.load()
    return torch


def _oracle_segments(q64, segs, scale, signs, S):
    """segs: list of (rec_k, nrm_k, rec_v, nrm_v, seq_lens, fmt_k, fmt_v) packed by the oracle."""
    batch, hq, d = q64.shape
    hkv = segs[0][0].shape[1]
    G = hq // hkv
    out = np.zeros((batch, hq, d))
    for bi in range(batch):
        for kh in range(hkv):
            kts, vts = [], []
            for rk, nk, rv, nv, lens, fk, fv in segs:
                L = int(lens[bi])
                ik, sk = O.unpack(rk[bi, kh, :L], fk)
                iv, sv = O.unpack(rv[bi, kh, :L], fv)
                kts.append(O.dequantize(ik, sk, nk[bi, kh, :L, 0], nk[bi, kh, :L, 1], fk, signs, S,
                                        *oracle_codebooks(d, fk.bits_lo, fk.bits_hi), qjl=fk.qjl))
                vts.append(O.dequantize(iv, sv, nv[bi, kh, :L, 0], nv[bi, kh, :L, 1], fv, signs, S,
                                        *oracle_codebooks(d, fv.bits_lo, fv.bits_hi), qjl=fv.qjl))
            kt, vt = np.concatenate(kts), np.concatenate(vts)
            for g in range(G):
                out[bi, kh * G + g] = O.attend(q64[bi, kh * G + g], kt, vt, scale)[0]
    return out


def _gpu_segments(torch, q_bits, segs, signs, S, tau=0.0):
    import compressed_attention_rotate_amd as tq
    Sd = torch.from_numpy(S).cuda()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    args = []
    for rk, nk, rv, nv, lens, fk, fv in segs:
        tfk, tfv = tq.Format(fk.d, fk.bits_lo, fk.bits_hi, fk.split, fk.qjl), \
            tq.Format(fv.d, fv.bits_lo, fv.bits_hi, fv.split, fv.qjl)
        args.append((dev(rk), dev(nk.view(np.int16)).view(torch.float16), dev(rv),
                     dev(nv.view(np.int16)).view(torch.float16),
                     dev(np.asarray(lens, dtype=np.int32)), tfk, tq.Tables(tfk, signs, Sd), tfv,
                     tq.Tables(tfv, signs, Sd)))
    q = dev(q_bits.view(np.int16)).view(torch.bfloat16)
    sk = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = tq.attend_decode_segments(q, args, tau=tau, skipped=sk)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(sk.item())


def _pack(kb, vb, fk, fv, signs, S):
    rk, nk, _ = oracle_pack_cache(kb, fk, signs, S, bf16=True)
    rv, nv, _ = oracle_pack_cache(vb, fv, signs, S, bf16=True)
    return rk, nk, rv, nv


@pytest.mark.parametrize("old,new", [((128, 2, 2, 128), (128, 3, 3, 128)),
                                     ((128, 2, 1, 64), (128, 3, 2, 64)),
                                     ((128, 1, 1, 128), (128, 3, 3, 128))])
def test_two_segments_against_oracle(torch_gpu, old, new):
    """An old segment (narrower codebook) then a new one, ragged lengths incl. an empty old
    and an empty new segment, GQA group 4."""
    batch, hq, hkv, d = 3, 8, 2, 128
    n_old, n_new = 530, 170
    kb, vb, _ = TI.kv_layer(batch, hkv, n_old + n_new, d, seed=8101)
    q_bits = TI.decode_queries(batch, hq, d, 8101)
    (signs, S), (gsigns, gS) = rotations(d, 8102)
    fo, fn = O.Format(*old), O.Format(*new)
    seg_old = _pack(kb[:, :, :n_old], vb[:, :, :n_old], fo, fo, signs, S) + ([530, 0, 301], fo, fo)
    seg_new = _pack(kb[:, :, n_old:], vb[:, :, n_old:], fn, fn, signs, S) + ([170, 99, 0], fn, fn)
    out_g, _ = _gpu_segments(torch_gpu, q_bits, [seg_old, seg_new], gsigns, gS)
    out_o = _oracle_segments(TI.bf16_to_f64(q_bits), [seg_old, seg_new], 1 / math.sqrt(d), signs, S)
    err = float(np.max(np.abs(out_g - out_o)))
    print(f"\nold {old} new {new}: max|out - oracle| {err:.3g}")
    assert err <= OUT_ATOL


def test_requantized_old_segment(torch_gpu):
    """The temporal-decay flow: 700 tokens packed at b = 4, the oldest 500 re-encoded to
    b = 3 by the oracle's requantize, decoded as two segments (three segments, the old
    part split in two, give the same result)."""
    batch, hq, hkv, d = 2, 8, 2, 128
    n, n_old = 700, 500
    kb, vb, _ = TI.kv_layer(batch, hkv, n, d, seed=8201)
    q_bits = TI.decode_queries(batch, hq, d, 8201)
    (signs, S), (gsigns, gS) = rotations(d, 8202)
    f4, f3 = O.Format.uniform(d, 3), O.Format.uniform(d, 2)
    rk, nk, rv, nv = _pack(kb, vb, f4, f4, signs, S)
    cb4, cb3 = oracle_codebooks(d, 3, 3), oracle_codebooks(d, 2, 2)

    def decay(rec, nrm):
        r = rec[:, :, :n_old].reshape(-1, rec.shape[-1])
        m = nrm[:, :, :n_old].reshape(-1, 2)
        o = O.requantize(r, m[:, 0], m[:, 1], f4, S, *cb4, f3, S, *cb3)
        recs = O.pack(o["idx"], o["sbit"], f3).reshape(batch, hkv, n_old, -1)
        nrms = np.stack([O.fp16_bits(o["n16"]) if o["n16"].dtype != np.uint16 else o["n16"],
                         O.fp16_bits(o["r16"]) if o["r16"].dtype != np.uint16 else o["r16"]],
                        axis=-1).reshape(batch, hkv, n_old, 2)
        return recs, nrms
    ork, onk = decay(rk, nk)
    orv, onv = decay(rv, nv)
    seg_old = (ork, onk, orv, onv, [n_old] * batch, f3, f3)
    seg_new = (rk[:, :, n_old:], nk[:, :, n_old:], rv[:, :, n_old:], nv[:, :, n_old:],
               [n - n_old, 123], f4, f4)
    out_o = _oracle_segments(TI.bf16_to_f64(q_bits), [seg_old, seg_new], 1 / math.sqrt(d), signs, S)
    out_2, _ = _gpu_segments(torch_gpu, q_bits, [seg_old, seg_new], gsigns, gS)
    cut = 256
    seg_a = (ork[:, :, :cut], onk[:, :, :cut], orv[:, :, :cut], onv[:, :, :cut], [cut] * batch, f3, f3)
    seg_b = (ork[:, :, cut:], onk[:, :, cut:], orv[:, :, cut:], onv[:, :, cut:], [n_old - cut] * batch,
             f3, f3)
    out_3, _ = _gpu_segments(torch_gpu, q_bits, [seg_a, seg_b, seg_new], gsigns, gS)
    err = float(np.max(np.abs(out_2 - out_o)))
    print(f"\nrequantized old segment: max|out - oracle| {err:.3g}, "
          f"two vs three segments {float(np.max(np.abs(out_2 - out_3))):.3g}")
    assert err <= OUT_ATOL
    assert float(np.max(np.abs(out_2 - out_3))) <= 1e-5


def test_one_segment_equals_plain_decode(torch_gpu):
    """A single segment is the plain decode: same records, same result up to fp32 rounding
    of the split merge (the split plans are identical, so bit for bit)."""
    import compressed_attention_rotate_amd as tq
    torch = torch_gpu
    batch, hq, hkv, d, n = 2, 8, 2, 128, 900
    kb, vb, _ = TI.kv_layer(batch, hkv, n, d, seed=8301)
    q_bits = TI.decode_queries(batch, hq, d, 8301)
    (signs, S), (gsigns, gS) = rotations(d, 8302)
    f = O.Format.uniform(d, 3)
    rk, nk, rv, nv = _pack(kb, vb, f, f, signs, S)
    out_s, _ = _gpu_segments(torch, q_bits, [(rk, nk, rv, nv, [900, 417], f, f)], gsigns, gS)
    tf = tq.Format.uniform(d, 3)
    tab = tq.Tables(tf, gsigns, torch.from_numpy(gS).cuda())
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out_p = tq.attend_decode(dev(q_bits.view(np.int16)).view(torch.bfloat16), dev(rk),
                             dev(nk.view(np.int16)).view(torch.float16), dev(rv),
                             dev(nv.view(np.int16)).view(torch.float16),
                             dev(np.array([900, 417], dtype=np.int32)), tf, tab).cpu().numpy()
    np.testing.assert_array_equal(out_s, out_p)


def test_value_rotation_mismatch_rejected(torch_gpu):
    """Value tables with different S arrays cannot be merged: the call is rejected before
    any launch."""
    import compressed_attention_rotate_amd as tq
    torch = torch_gpu
    d = 128
    (signs, S), (gsigns, gS) = rotations(d, 8402)
    tf = tq.Format.uniform(d, 3)
    t1 = tq.Tables(tf, gsigns, torch.from_numpy(gS).cuda())
    t2 = tq.Tables(tf, gsigns, torch.from_numpy(gS.copy()).cuda())
    rb = tf.record_bytes()
    ck = torch.zeros((1, 1, 64, rb), dtype=torch.uint8, device="cuda")
    nk = torch.zeros((1, 1, 64, 2), dtype=torch.float16, device="cuda")
    seq = torch.full((1,), 64, dtype=torch.int32, device="cuda")
    q = torch.zeros((1, 1, d), dtype=torch.float32, device="cuda")
    with pytest.raises(tq.TQError):
        tq.attend_decode_segments(q, [(ck, nk, ck, nk, seq, tf, t1, tf, t1),
                                      (ck, nk, ck, nk, seq, tf, t1, tf, t2)])


def _random_cache(g, batch, hkv, L, fmt: O.Format):
    """A packed cache of arbitrary valid contents: every bit pattern is a record, and the
    norms are fp16 values of a plausible range (||x|| in [2, 12), ||r|| in [0.1, 1.5))."""
    rec = g.integers(0, 256, (batch, hkv, L, fmt.record_bytes()), dtype=np.uint8)
    nrm = np.empty((batch, hkv, L, 2), np.uint16)
    nrm[..., 0] = O.fp16_bits(g.uniform(2.0, 12.0, (batch, hkv, L)))
    nrm[..., 1] = O.fp16_bits(g.uniform(0.1, 1.5, (batch, hkv, L)))
    return rec, nrm


def test_many_large_segments_more_partials_than_one_merge_pass(torch_gpu):
    """Five segments of 131072 tokens at batch 1 with one KV head: each segment's scan
    writes 256 split partials, 1280 in all, which the combine must merge in one softmax
    (more than the 1024 a fixed-size merge table held).  Cross-fed: arbitrary packed bytes,
    decoded by the GPU and by the oracle."""
    import compressed_attention_rotate_amd as tq
    batch, hq, hkv, d, L = 1, 4, 1, 128, 131072
    fmts = [(128, 2, 2, 128), (128, 3, 3, 128), (128, 2, 2, 128), (128, 3, 2, 64), (128, 3, 3, 128)]
    assert tq.attend_segments_workspace_bytes(batch, hq, hkv, [L] * 5) == 5 * 256 * hq * 258 * 4
    g = TI.gen(8501)
    segs = []
    for i, f in enumerate(fmts):
        fo = O.Format(*f)
        rk, nk = _random_cache(g, batch, hkv, L, fo)
        rv, nv = _random_cache(g, batch, hkv, L, fo)
        segs.append((rk, nk, rv, nv, [L - 977 * i], fo, fo))
    q_bits = TI.decode_queries(batch, hq, d, 8501)
    (signs, S), (gsigns, gS) = rotations(d, 8502)
    out_g, _ = _gpu_segments(torch_gpu, q_bits, segs, gsigns, gS)
    out_o = _oracle_segments(TI.bf16_to_f64(q_bits), segs, 1 / math.sqrt(d), signs, S)
    err = float(np.max(np.abs(out_g - out_o)))
    print(f"\n5 x 131072-token segments (1280 partials): max|out - oracle| {err:.3g}")
    assert err <= OUT_ATOL


def test_fused_decay_pair_at_layer_size(torch_gpu):
    """The fused two-segment scan as a decayed 32K layer runs it: 24576 old tokens at b = 3
    before 8192 new ones at b = 4, 32 query / 8 KV heads, so the combined split plan gives
    the old segment 24 splits and the new one 8.  Batch 2 with ragged lengths, one of them
    leaving the last splits of the new segment empty.  Sampled (batch, KV head) units
    against the oracle; the whole output against the per-segment path (the old segment cut
    in two, three segments, no fused instance)."""
    import compressed_attention_rotate_amd as tq
    batch, hq, hkv, d, n_old, n_new = 2, 32, 8, 128, 24576, 8192
    f3, f4 = O.Format(128, 2, 2, 128), O.Format(128, 3, 3, 128)
    g = TI.gen(8601)
    rk3, nk3 = _random_cache(g, batch, hkv, n_old, f3)
    rv3, nv3 = _random_cache(g, batch, hkv, n_old, f3)
    rk4, nk4 = _random_cache(g, batch, hkv, n_new, f4)
    rv4, nv4 = _random_cache(g, batch, hkv, n_new, f4)
    lens_old, lens_new = [n_old, 20000], [n_new, 2500]
    q_bits = TI.decode_queries(batch, hq, d, 8601)
    (signs, S), (gsigns, gS) = rotations(d, 8602)
    seg_old = (rk3, nk3, rv3, nv3, lens_old, f3, f3)
    seg_new = (rk4, nk4, rv4, nv4, lens_new, f4, f4)
    out_2, _ = _gpu_segments(torch_gpu, q_bits, [seg_old, seg_new], gsigns, gS)
    cut = 10000
    seg_a = (rk3[:, :, :cut], nk3[:, :, :cut], rv3[:, :, :cut], nv3[:, :, :cut],
             [min(L, cut) for L in lens_old], f3, f3)
    seg_b = (rk3[:, :, cut:], nk3[:, :, cut:], rv3[:, :, cut:], nv3[:, :, cut:],
             [max(L - cut, 0) for L in lens_old], f3, f3)
    out_3, _ = _gpu_segments(torch_gpu, q_bits, [seg_a, seg_b, seg_new], gsigns, gS)
    diff23 = float(np.max(np.abs(out_2 - out_3)))
    q64 = TI.bf16_to_f64(q_bits)
    G = hq // hkv
    worst = 0.0
    for bi, kh in ((0, 0), (0, 5), (1, 3), (1, 7)):
        sub = [(rk[bi:bi + 1, kh:kh + 1], nk[bi:bi + 1, kh:kh + 1], rv[bi:bi + 1, kh:kh + 1],
                nv[bi:bi + 1, kh:kh + 1], [lens[bi]], fk, fv)
               for rk, nk, rv, nv, lens, fk, fv in (seg_old, seg_new)]
        o = _oracle_segments(q64[bi:bi + 1, kh * G:(kh + 1) * G], sub, 1 / math.sqrt(d), signs, S)
        worst = max(worst, float(np.max(np.abs(out_2[bi, kh * G:(kh + 1) * G] - o[0]))))
    print(f"\nfused 24K b3 + 8K b4: max|out - oracle| {worst:.3g} (sampled units), "
          f"fused vs per-segment {diff23:.3g}")
    assert worst <= OUT_ATOL
    assert diff23 <= 1e-4
