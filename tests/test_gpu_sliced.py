"""GPU: the token-sliced value layout and the decode scan that reads it (keys per-vector,
values token-sliced; both dot products on the block-scaled fp6 x fp4 MFMA).

Quantize parity: the GPU's token-sliced bytes, read back into per-vector records by the
oracle's own inverse of the layout, equal the oracle's records outside the ambiguity
windows.  Decode parity is cross-fed: the oracle packs keys and values, lays the values out
token-sliced with its own layout function, and the GPU decodes exactly those bytes; logits
within 1e-4 of the estimator's absolute-sum scale, outputs within 2e-3 (gated outputs
within 5e-3 of the ungated oracle)."""
import math

import numpy as np
import pytest

import tq_inputs as TI
from oracle import tq_oracle as O
from parity_utils import (compare_quantize, oracle_decode, oracle_pack_cache, oracle_quantize,
                          rotations)

pytestmark = pytest.mark.gpu

LOGIT_RTOL = 1e-4
OUT_ATOL = 2e-3
GATED_ATOL = 5e-3


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import compressed_attention_rotate_amd as tq
    tq.load()
    return torch


def _tiles(rec_bhtr, fmt):
    """Oracle token-sliced layout of a [batch, hkv, cap, rb] record array."""
    b, h, t, rb = rec_bhtr.shape
    return O.tiles_from_records(rec_bhtr.reshape(-1, rb), fmt).reshape(b, h, t // 32, 32 * rb)


@pytest.mark.parametrize("fmt_t", [(128, 3, 3, 128), (128, 2, 2, 128), (128, 3, 2, 64)])
def test_sliced_quantize_matches_oracle(torch_gpu, fmt_t):
    import compressed_attention_rotate_amd as tq
    torch = torch_gpu
    n, d = 4096, 128
    kb, _, _ = TI.kv_layer(1, 1, n, d, seed=9100)
    x = kb.reshape(n, d)
    (signs, S), (gsigns, gS) = rotations(d, 9101)
    fmt = tq.Format(*fmt_t, layout=1)
    tab = tq.Tables(fmt, gsigns, torch.from_numpy(gS).cuda())
    codes, norms = tq.quantize_kv(torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16),
                                  fmt, tab)
    torch.cuda.synchronize()
    assert tuple(codes.shape) == (n // 32, 32 * fmt.record_bytes())
    of = O.Format(*fmt_t)
    rec = O.records_from_tiles(codes.cpu().numpy(), of)
    qz = oracle_quantize(x, of, signs, S, bf16=True)
    r = compare_quantize(rec, norms.cpu().view(torch.int16).numpy().view(np.uint16), qz, of)
    print(f"\nsliced quantize {fmt_t}: {r}")


def _sliced_decode(torch, q_bits, q_dtype, rk, nk, rv, nv, seq_lens, fk, fv, gsigns, gS, tau=0.0):
    import compressed_attention_rotate_amd as tq
    fmt_k, fmt_v = tq.Format(*fk), tq.Format(*fv, layout=1)
    Sd = torch.from_numpy(gS).cuda()
    tk, tv = tq.Tables(fmt_k, gsigns, Sd), tq.Tables(fmt_v, gsigns, Sd)
    if q_dtype == "bf16":
        q = torch.from_numpy(q_bits.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        q = torch.from_numpy(np.ascontiguousarray(TI.bf16_to_f32(q_bits))).cuda()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    f16 = lambda a: dev(a.view(np.int16)).view(torch.float16)
    sk = torch.zeros(1, dtype=torch.int64, device="cuda")
    out, lg = tq.attend_decode(q, dev(rk), f16(nk), dev(_tiles(rv, O.Format(*fv))), f16(nv),
                               dev(np.asarray(seq_lens, np.int32)), fmt_k, tk, fmt_v, tv, tau=tau,
                               logits=True, skipped=sk)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lg.cpu().numpy(), int(sk.item())


def _check(out_g, lg_g, out_o, lg_o, sc_o, seq_lens, atol=OUT_ATOL, logits=True):
    worst = 0.0
    if logits:
        for (bi, h), lo in lg_o.items():
            L = int(seq_lens[bi])
            if L == 0:
                continue
            err = np.abs(lg_g[bi, h, :L] - lo)
            bound = LOGIT_RTOL * (np.abs(lo) + sc_o[(bi, h)])
            assert np.all(err <= bound), f"logits differ (b={bi}, h={h}): max ratio {np.max(err / bound)}"
            worst = max(worst, float(np.max(err / bound)))
    dmax = float(np.max(np.abs(out_g - out_o)))
    assert dmax <= atol, f"outputs differ by {dmax}"
    return worst, dmax


@pytest.mark.parametrize("batch,hq,hkv,cap,lens,fk,fv,q_dtype", [
    (1, 32, 8, 4096, [4096], (128, 3, 3, 128), (128, 3, 3, 128), "bf16"),    # b4 / b4, one tile row
    (3, 16, 4, 800, [800, 37, 0], (128, 3, 3, 128), (128, 3, 3, 128), "f32"), # ragged, empty, cap % 128
    (2, 16, 2, 1536, [1536, 700], (128, 3, 3, 128), (128, 2, 2, 128), "bf16"),  # GQA 8, K b4 / V b3
    (1, 8, 2, 2048, [1999], (128, 3, 2, 64), (128, 3, 2, 64), "bf16"),       # 3.5 bit / 3.5 bit
    (2, 4, 1, 640, [640, 129], (128, 2, 2, 128), (128, 2, 2, 128), "bf16"),  # b3 / b3
])
def test_sliced_decode_matches_oracle(torch_gpu, batch, hq, hkv, cap, lens, fk, fv, q_dtype):
    d, seed = 128, 9200 + cap
    kb, vb, _ = TI.kv_layer(batch, hkv, cap, d, seed=seed)
    q_bits = TI.decode_queries(batch, hq, d, seed)
    (signs, S), (gsigns, gS) = rotations(d, seed + 1)
    rk, nk, _ = oracle_pack_cache(kb, O.Format(*fk), signs, S, bf16=True)
    rv, nv, _ = oracle_pack_cache(vb, O.Format(*fv), signs, S, bf16=True)
    out_g, lg_g, _ = _sliced_decode(torch_gpu, q_bits, q_dtype, rk, nk, rv, nv, lens, fk, fv, gsigns, gS)
    q64 = TI.bf16_to_f64(q_bits)
    out_o, lg_o, sc_o, _, _ = oracle_decode(q64, rk, nk, rv, nv, lens, O.Format(*fk), O.Format(*fv),
                                            signs, S, signs, S, 1 / math.sqrt(d))
    worst, dmax = _check(out_g, lg_g, out_o, lg_o, sc_o, lens)
    print(f"\nsliced b={batch} hq={hq} hkv={hkv} cap={cap} {fk}/{fv}: logit err/bound {worst:.3g}, "
          f"out max|diff| {dmax:.3g}")


def test_sliced_decode_gate_with_spikes(torch_gpu):
    """Keys b = 4, values b = 3 token-sliced, 1% of tokens with x10 keys, Sparse-V gate
    tau = 1e-4: gated output within 5e-3 of the ungated oracle; the skip count is at most the
    oracle's number of rows whose final weight is below tau for every head of the group."""
    batch, hq, hkv, cap, d = 2, 16, 4, 8192, 128
    fk, fv = (128, 3, 3, 128), (128, 2, 2, 128)
    seed = 9300
    kb, vb, _ = TI.kv_layer(batch, hkv, cap, d, seed=seed, spike_frac=0.01)
    q_bits = TI.decode_queries(batch, hq, d, seed)
    (signs, S), (gsigns, gS) = rotations(d, seed + 1)
    rk, nk, _ = oracle_pack_cache(kb, O.Format(*fk), signs, S, bf16=True)
    rv, nv, _ = oracle_pack_cache(vb, O.Format(*fv), signs, S, bf16=True)
    lens = [cap, 5000]
    out_g, _, skipped = _sliced_decode(torch_gpu, q_bits, "bf16", rk, nk, rv, nv, lens, fk, fv, gsigns,
                                       gS, tau=1e-4)
    q64 = TI.bf16_to_f64(q_bits)
    out_o, lg_o, sc_o, drops, masses = oracle_decode(q64, rk, nk, rv, nv, lens, O.Format(*fk),
                                                     O.Format(*fv), signs, S, signs, S,
                                                     1 / math.sqrt(d), 0.0)
    _, dmax = _check(out_g, None, out_o, lg_o, sc_o, lens, atol=GATED_ATOL, logits=False)
    # rows below tau for every head of their group, from the ungated oracle weights
    G = hq // hkv
    bound = 0
    for bi in range(batch):
        for kh in range(hkv):
            below = np.ones(lens[bi], bool)
            for gq in range(G):
                lg = lg_o[(bi, kh * G + gq)]
                p = np.exp(lg - lg.max())
                p /= p.sum()
                below &= p < 1e-4
            bound += int(below.sum())
    print(f"\nsliced gated: max|out - ungated oracle| {dmax:.3g}, skipped {skipped} of "
          f"{sum(lens) * hkv} rows (oracle rows under tau for all heads: {bound})")
    assert 0 < skipped <= bound


def test_sliced_full_layer_sampled(torch_gpu):
    """The 32K-token Llama-3.1-8B-shaped layer (32 query / 8 KV heads, b = 4) as the decode
    benchmark runs it: the GPU quantizes keys per-vector and values token-sliced; for sampled
    KV heads the records are replaced by the oracle's packing of the same inputs, so those
    heads decode exactly the bytes the oracle decodes."""
    import compressed_attention_rotate_amd as tq
    torch = torch_gpu
    batch, hq, hkv, ntok, d = 1, 32, 8, 32768, 128
    seed = TI.data_seed(2)
    kb, vb, _ = TI.kv_layer(batch, hkv, ntok, d, seed=seed)
    q_bits = TI.decode_queries(batch, hq, d, seed)
    (signs, S), (gsigns, gS) = rotations(d, TI.rotation_seed(2))
    fk, fv = tq.Format.uniform(d, 3), tq.Format.uniform(d, 3, layout=1)
    Sd = torch.from_numpy(gS).cuda()
    tk, tv = tq.Tables(fk, gsigns, Sd), tq.Tables(fv, gsigns, Sd)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    ck, nk = tq.quantize_kv(bf(kb).view(-1, d), fk, tk)
    cv, nv = tq.quantize_kv(bf(vb).view(-1, d), fv, tv)
    rb = fk.record_bytes()
    ck, nk = ck.view(batch, hkv, ntok, rb), nk.view(batch, hkv, ntok, 2)
    cv, nv = cv.view(batch, hkv, ntok // 32, 32 * rb), nv.view(batch, hkv, ntok, 2)
    of = O.Format.uniform(d, 3)
    units = (0, 3, 7)
    orc = {}
    for kh in units:
        rk, nko, _ = oracle_pack_cache(kb[:, kh:kh + 1], of, signs, S, bf16=True)
        rv, nvo, _ = oracle_pack_cache(vb[:, kh:kh + 1], of, signs, S, bf16=True)
        ck[0, kh] = torch.from_numpy(rk[0, 0]).cuda()
        nk[0, kh] = torch.from_numpy(nko[0, 0].view(np.int16)).cuda().view(torch.float16)
        cv[0, kh] = torch.from_numpy(_tiles(rv, of)[0, 0]).cuda()
        nv[0, kh] = torch.from_numpy(nvo[0, 0].view(np.int16)).cuda().view(torch.float16)
        orc[kh] = (rk, nko, rv, nvo)
    seq = torch.tensor([ntok], dtype=torch.int32, device="cuda")
    out, lg = tq.attend_decode(bf(q_bits), ck, nk, cv, nv, seq, fk, tk, fv, tv, logits=True)
    torch.cuda.synchronize()
    out, lg = out.cpu().numpy(), lg.cpu().numpy()
    q64 = TI.bf16_to_f64(q_bits)
    G = hq // hkv
    worst, dmax = 0.0, 0.0
    for kh in units:
        rk, nko, rv, nvo = orc[kh]
        qs = q64[:, kh * G:(kh + 1) * G]
        out_o, lg_o, sc_o, _, _ = oracle_decode(qs, rk, nko, rv, nvo, [ntok], of, of, signs, S, signs,
                                                S, 1 / math.sqrt(d))
        for gq in range(G):
            lo = lg_o[(0, gq)]
            err = np.abs(lg[0, kh * G + gq] - lo)
            bnd = LOGIT_RTOL * (np.abs(lo) + sc_o[(0, gq)])
            assert np.all(err <= bnd)
            worst = max(worst, float(np.max(err / bnd)))
        dmax = max(dmax, float(np.max(np.abs(out[0, kh * G:(kh + 1) * G] - out_o[0]))))
    print(f"\nsliced 32K layer: logit err/bound {worst:.3g}, out max|diff| {dmax:.3g} (units {units})")
    assert dmax <= OUT_ATOL
