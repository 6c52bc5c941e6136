"""GPU parity of the paged cache: quantize-on-write into slots of a paged cache, and decode
through a block table, against the oracle (records at the same slots; attention over the
gathered tokens) and, exactly, against the contiguous GPU decode of the same data."""
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


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import compressed_attention_rotate_amd as tq
    tq.load()
    return torch


def _paginate(rec, nrm, seq_lens, page_size, seed, holes=()):
    """Scatter a contiguous cache [batch, hkv, cap, ...] into shuffled pages; returns
    (codes_pages [P, hkv, page, rb], norms_pages [P, hkv, page, 2], block_table [batch, mb])."""
    batch, hkv, cap, rb = rec.shape
    mb = (cap + page_size - 1) // page_size
    need = batch * mb
    n_pages = need + 3                                   # spare pages stay unused
    perm = TI.gen(seed).permutation(n_pages)[:need].reshape(batch, mb).astype(np.int32)
    cp = np.full((n_pages, hkv, page_size, rb), 0xA5, np.uint8)
    npg = np.zeros((n_pages, hkv, page_size, 2), np.uint16)
    for b in range(batch):
        for blk in range(mb):
            lo, hi = blk * page_size, min(cap, (blk + 1) * page_size)
            cp[perm[b, blk], :, : hi - lo] = rec[b, :, lo:hi]
            npg[perm[b, blk], :, : hi - lo] = nrm[b, :, lo:hi]
    bt = perm.copy()
    for b, blk in holes:
        bt[b, blk] = -1
    return cp, npg, bt


def _case(torch, fk, fv, page_size, seed, batch=2, hq=32, hkv=8, ntok=1000, seq=(1000, 611),
          holes=()):
    import compressed_attention_rotate_amd as tq
    d = 128
    kb, vb, _ = TI.kv_layer(batch, hkv, ntok, d, seed=seed)
    qb = TI.decode_queries(batch, hq, d, seed)
    (signs, S), (gsigns, gS) = rotations(d, seed + 1)
    rk, nk, _ = oracle_pack_cache(kb, O.Format(*fk), signs, S, bf16=True)
    rv, nv, _ = oracle_pack_cache(vb, O.Format(*fv), signs, S, bf16=True)
    ck, nkp, bt = _paginate(rk, nk, seq, page_size, seed + 2, holes)
    cv, nvp, _ = _paginate(rv, nv, seq, page_size, seed + 2, holes)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    f16 = lambda a: dev(a.view(np.int16)).view(torch.float16)
    fmt_k, fmt_v = tq.Format(*fk), tq.Format(*fv)
    tk = tq.Tables(fmt_k, gsigns, torch.from_numpy(gS).cuda())
    tv = tq.Tables(fmt_v, gsigns, torch.from_numpy(gS).cuda())
    q = dev(qb.view(np.int16)).view(torch.bfloat16)
    sl = dev(np.asarray(seq, np.int32))
    out_p, lg_p = tq.attend_decode_paged(q, dev(ck), f16(nkp), dev(cv), f16(nvp), dev(bt), sl, fmt_k, tk,
                                         fmt_v, tv, logits=True)
    torch.cuda.synchronize()
    out_p, lg_p = out_p.cpu().numpy(), lg_p.cpu().numpy()
    # oracle over the tokens that are present (a hole removes its page's tokens)
    present = np.ones((batch, ntok), bool)
    for b, blk in holes:
        present[b, blk * page_size:(blk + 1) * page_size] = False
    q64 = TI.bf16_to_f64(qb)
    for b in range(batch):
        keep = np.nonzero(present[b, : seq[b]])[0]
        L = len(keep)
        o, lgo, sco, _, _ = oracle_decode(q64[b:b + 1], rk[b:b + 1, :, keep], nk[b:b + 1, :, keep],
                                          rv[b:b + 1, :, keep], nv[b:b + 1, :, keep], [L],
                                          O.Format(*fk), O.Format(*fv), signs, S, signs, S,
                                          1 / math.sqrt(d))
        assert np.max(np.abs(out_p[b] - o[0])) <= OUT_ATOL
        for h in range(hq):
            err = np.abs(lg_p[b, h, keep] - lgo[(0, h)])
            assert np.all(err <= LOGIT_RTOL * (np.abs(lgo[(0, h)]) + sco[(0, h)]))
    if not holes:   # same arithmetic as a contiguous cache of the same capacity: identical bits
        cap = bt.shape[1] * page_size
        pad = lambda a: np.concatenate([a, np.zeros(a.shape[:2] + (cap - a.shape[2],) + a.shape[3:], a.dtype)], 2)
        out_c, lg_c = tq.attend_decode(q, dev(pad(rk)), f16(pad(nk)), dev(pad(rv)), f16(pad(nv)), sl, fmt_k,
                                       tk, fmt_v, tv, logits=True)
        torch.cuda.synchronize()
        out_c, lg_c = out_c.cpu().numpy(), lg_c.cpu().numpy()
        assert np.array_equal(out_p, out_c)
        for b in range(batch):
            assert np.array_equal(lg_p[b, :, : seq[b]], lg_c[b, :, : seq[b]])


@pytest.mark.parametrize("page_size", [64, 128, 256])
def test_paged_decode_b4(torch_gpu, page_size):
    _case(torch_gpu, (128, 3, 3, 128), (128, 3, 3, 128), page_size, 7000 + page_size)


def test_paged_decode_mixed_formats_and_groups(torch_gpu):
    _case(torch_gpu, (128, 3, 2, 64), (128, 2, 1, 64, False), 64, 7100, hq=16, hkv=8, ntok=700, seq=(700, 1))
    _case(torch_gpu, (128, 2, 2, 128), (128, 2, 2, 128), 128, 7101, batch=3, hq=8, hkv=8, ntok=500,
          seq=(500, 0, 257))


def test_paged_decode_page_holes(torch_gpu):
    """A block-table entry of -1 inside a sequence removes that page's tokens."""
    _case(torch_gpu, (128, 3, 3, 128), (128, 2, 2, 128), 64, 7200, holes=((0, 3), (1, 0)))


def test_paged_append_writes_only_its_slots(torch_gpu):
    """Quantize-on-write: records land at their slots, bit-identical to the oracle's records
    of the same vectors; negative slots and every other slot are left untouched."""
    torch = torch_gpu
    import compressed_attention_rotate_amd as tq
    d, hkv, page, n_pages, n_tok = 128, 4, 64, 12, 333
    kb, _, _ = TI.kv_layer(1, hkv, n_tok, d, seed=7300)
    x = np.ascontiguousarray(np.transpose(kb[0], (1, 0, 2)))          # [token][head][d]
    (signs, S), (gsigns, gS) = rotations(d, 7301)
    fmt = tq.Format.uniform(d, 3)
    tab = tq.Tables(fmt, gsigns, torch.from_numpy(gS).cuda())
    g = TI.gen(7302)
    slots = g.permutation(n_pages * page)[:n_tok].astype(np.int64)
    slots[::17] = -1                                                  # padding tokens
    rb = fmt.record_bytes()
    cache = torch.full((n_pages, hkv, page, rb), 0xA5, dtype=torch.uint8, device="cuda")
    norms = torch.full((n_pages, hkv, page, 2), 7.0, dtype=torch.float16, device="cuda")
    xt = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    tq.quantize_kv_paged(xt, fmt, tab, torch.from_numpy(slots).cuda(), cache, norms)
    torch.cuda.synchronize()
    c = cache.cpu().numpy()
    nr = norms.cpu().view(torch.int16).numpy().view(np.uint16)
    qz = oracle_quantize(x.reshape(-1, d), O.Format.uniform(d, 3), signs, S, bf16=True)
    written = np.zeros((n_pages, hkv, page), bool)
    got_c, got_n, rows = [], [], []
    for i, sl in enumerate(slots):
        if sl < 0:
            continue
        pg, off = sl // page, sl % page
        for h in range(hkv):
            written[pg, h, off] = True
            got_c.append(c[pg, h, off]); got_n.append(nr[pg, h, off]); rows.append(i * hkv + h)
    sub = {k: v[rows] for k, v in qz.items()}
    compare_quantize(np.stack(got_c), np.stack(got_n), sub, O.Format.uniform(d, 3))
    assert np.all(c[~written] == 0xA5)
    assert np.all(nr[~written] == np.float16(7.0).view(np.uint16))


def test_paged_full_context_equals_contiguous(torch_gpu):
    """The 32768-token Llama-3.1-8B-shaped layer in 128-token pages in shuffled order: the
    paged decode returns the contiguous decode's output bit for bit."""
    torch = torch_gpu
    import compressed_attention_rotate_amd as tq
    d, hq, hkv, n, page = 128, 32, 8, 32768, 128
    kb, vb, _ = TI.kv_layer(1, hkv, n, d, seed=TI.data_seed(2))
    qb = TI.decode_queries(1, hq, d, TI.data_seed(2))
    (signs, S), (gsigns, gS) = rotations(d, TI.rotation_seed(2))
    fmt = tq.Format.uniform(d, 3)
    tab = tq.Tables(fmt, gsigns, torch.from_numpy(gS).cuda())
    k0 = torch.from_numpy(kb.view(np.int16)).cuda().view(torch.bfloat16)
    v0 = torch.from_numpy(vb.view(np.int16)).cuda().view(torch.bfloat16)
    ck, nk = tq.quantize_kv(k0.view(-1, d), fmt, tab)
    cv, nv = tq.quantize_kv(v0.view(-1, d), fmt, tab)
    rb = fmt.record_bytes()
    ck, nk, cv, nv = ck.view(1, hkv, n, rb), nk.view(1, hkv, n, 2), cv.view(1, hkv, n, rb), nv.view(1, hkv, n, 2)
    mb = n // page
    perm = torch.from_numpy(TI.gen(7400).permutation(mb).astype(np.int64)).cuda()
    def pages(t):   # [1, hkv, n, w] -> [mb, hkv, page, w] with page perm[j] holding block j
        blocks = t[0].view(hkv, mb, page, -1).permute(1, 0, 2, 3)
        out = torch.empty_like(blocks)
        out[perm] = blocks
        return out.contiguous()
    bt = perm.to(torch.int32).view(1, mb)
    q = torch.from_numpy(qb.view(np.int16)).cuda().view(torch.bfloat16)
    sl = torch.full((1,), n, dtype=torch.int32, device="cuda")
    out_c = tq.attend_decode(q, ck, nk, cv, nv, sl, fmt, tab)
    out_p = tq.attend_decode_paged(q, pages(ck), pages(nk), pages(cv), pages(nv), bt, sl, fmt, tab)
    torch.cuda.synchronize()
    assert torch.equal(out_c, out_p)


def _prefill_case(torch, start, n_new, seed, page=64, hq=32, hkv=8, fk=(128, 3, 3, 128),
                  fv=(128, 3, 3, 128)):
    """A sequence with `start` cached tokens and a chunk of n_new new ones, in shuffled pages."""
    import compressed_attention_rotate_amd as tq
    d = 128
    total = start + n_new
    kb, vb, _ = TI.kv_layer(1, hkv, total, d, seed=seed)
    qb = TI.decode_queries(n_new, hq, d, seed)                       # one query row per new token
    (signs, S), (gsigns, gS) = rotations(d, seed + 1)
    rk, nk, _ = oracle_pack_cache(kb, O.Format(*fk), signs, S, bf16=True)
    rv, nv, _ = oracle_pack_cache(vb, O.Format(*fv), signs, S, bf16=True)
    mb = (total + page - 1) // page + 1
    n_pages = mb + 2
    table = TI.gen(seed + 2).permutation(n_pages)[:mb].astype(np.int32)
    fmt_k, fmt_v = tq.Format(*fk), tq.Format(*fv)
    ck = np.full((n_pages, hkv, page, fmt_k.record_bytes()), 0x5A, np.uint8)
    cv = np.full((n_pages, hkv, page, fmt_v.record_bytes()), 0x5A, np.uint8)
    nkc = np.zeros((n_pages, hkv, page, 2), np.uint16)
    nvc = np.zeros((n_pages, hkv, page, 2), np.uint16)
    for t in range(start):                                           # the cached past
        pg, off = table[t // page], t % page
        ck[pg, :, off], cv[pg, :, off] = rk[0, :, t], rv[0, :, t]
        nkc[pg, :, off], nvc[pg, :, off] = nk[0, :, t], nv[0, :, t]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    f16 = lambda a: dev(a.view(np.int16)).view(torch.float16)
    tk = tq.Tables(fmt_k, gsigns, torch.from_numpy(gS).cuda())
    tv = tq.Tables(fmt_v, gsigns, torch.from_numpy(gS).cuda())
    new_k = np.ascontiguousarray(np.transpose(kb[0, :, start:], (1, 0, 2)))   # [n_new][hkv][d]
    new_v = np.ascontiguousarray(np.transpose(vb[0, :, start:], (1, 0, 2)))
    bf = lambda a: dev(a.view(np.int16)).view(torch.bfloat16)
    gck, gnk, gcv, gnv = dev(ck), f16(nkc), dev(cv), f16(nvc)
    out = tq.prefill_paged(bf(qb), bf(new_k), bf(new_v), start, gck, gnk, gcv, gnv, dev(table),
                           fmt_k, tk, fmt_v, tv)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), gck.cpu().numpy(), gnk.cpu().view(torch.int16).numpy().view(np.uint16),
            table, rk, nk, rv, nv, qb, signs, S)


@pytest.mark.parametrize("start,n_new", [(300, 70), (0, 1), (0, 130), (511, 2)])
def test_prefill_writes_the_chunk_and_attends_causally(torch_gpu, start, n_new):
    """The chunk's key records land at their positions, bit-identical to the oracle's; query i
    of the chunk gets the oracle's attention over tokens 0 .. start + i."""
    page, fk = 64, (128, 3, 3, 128)
    out, ck, nk_c, table, rk, nk, rv, nv, qb, signs, S = _prefill_case(torch_gpu, start, n_new, 7500 + start)
    hkv = rk.shape[1]
    got_c, got_n, rows = [], [], []
    for t in range(start, start + n_new):
        pg, off = table[t // page], t % page
        for h in range(hkv):
            got_c.append(ck[pg, h, off]); got_n.append(nk_c[pg, h, off])
    # exact comparison outside the ambiguity windows: the oracle on the chunk's rows
    kb, _, _ = TI.kv_layer(1, hkv, start + n_new, 128, seed=7500 + start)
    rows_x = np.transpose(kb[0, :, start:], (1, 0, 2)).reshape(-1, 128)
    qz = oracle_quantize(rows_x, O.Format(*fk), signs, S, bf16=True)
    compare_quantize(np.stack(got_c), np.stack(got_n), qz, O.Format(*fk))
    q64 = TI.bf16_to_f64(qb)
    for i in range(n_new):
        L = start + i + 1
        o, _, _, _, _ = oracle_decode(q64[i:i + 1], rk[:, :, :L], nk[:, :, :L], rv[:, :, :L], nv[:, :, :L],
                                      [L], O.Format(*fk), O.Format(*fk), signs, S, signs, S, 1 / math.sqrt(128))
        assert np.max(np.abs(out[i] - o[0])) <= OUT_ATOL, (i, np.max(np.abs(out[i] - o[0])))


@pytest.mark.parametrize("fk,fv,hq,hkv,page,start,n_new", [
    ((128, 3, 2, 64), (128, 2, 1, 64), 8, 4, 128, 200, 45),           # 3.5 / 2.5 bit, GQA 2
    ((128, 3, 3, 128), (128, 3, 3, 128, False), 4, 4, 64, 70, 60),   # MSE-only values, MHA
    ((128, 2, 2, 128), (128, 3, 2, 32), 16, 2, 256, 5, 67),          # GQA 8, 3.25-bit values
])
def test_prefill_formats_and_groups(torch_gpu, fk, fv, hq, hkv, page, start, n_new):
    """Prefill over mixed bit widths, MSE-only values and group sizes 1, 2 and 8: query i
    of the chunk gets the oracle's attention over tokens 0 .. start + i."""
    out, _, _, _, rk, nk, rv, nv, qb, signs, S = _prefill_case(torch_gpu, start, n_new, 7700 + start,
                                                               page=page, hq=hq, hkv=hkv, fk=fk, fv=fv)
    q64 = TI.bf16_to_f64(qb)
    for i in range(n_new):
        L = start + i + 1
        o, _, _, _, _ = oracle_decode(q64[i:i + 1], rk[:, :, :L], nk[:, :, :L], rv[:, :, :L], nv[:, :, :L],
                                      [L], O.Format(*fk), O.Format(*fv), signs, S, signs, S, 1 / math.sqrt(128))
        assert np.max(np.abs(out[i] - o[0])) <= OUT_ATOL, (i, np.max(np.abs(out[i] - o[0])))


def test_prefill_rejects_a_chunk_past_the_pages_and_writes_nothing(torch_gpu):
    torch = torch_gpu
    import compressed_attention_rotate_amd as tq
    fmt = tq.Format.uniform(128, 3)
    (signs, S), (gsigns, gS) = rotations(128, 1)
    tab = tq.Tables(fmt, gsigns, torch.from_numpy(gS).cuda())
    ck = torch.full((4, 8, 64, fmt.record_bytes()), 0x5A, dtype=torch.uint8, device="cuda")
    nk = torch.zeros((4, 8, 64, 2), dtype=torch.float16, device="cuda")
    cv, nv = ck.clone(), nk.clone()
    table = torch.arange(2, dtype=torch.int32, device="cuda")         # 2 pages: capacity 128
    q = torch.zeros((10, 32, 128), dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros((10, 8, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tq.TQError):
        tq.prefill_paged(q, kn, kn, 120, ck, nk, cv, nv, table, fmt, tab)
    torch.cuda.synchronize()
    assert bool((ck == 0x5A).all()) and bool((cv == 0x5A).all())


def test_prefill_512_token_chunk_over_32k_context(torch_gpu):
    """The prefill chunk as the layer benchmark runs it: 512 new tokens after 32256 cached
    ones (32 query / 8 KV heads, b = 4, 128-token pages in shuffled order).  The cached past
    is arbitrary packed bytes (cross-fed: the same bytes in the GPU cache and in the
    oracle); the chunk's keys and values are quantized by the GPU inside the call and by the
    oracle from the same inputs.  Sampled query rows of the chunk must get the oracle's causal
    attention over tokens 0 .. start + i within 2e-3."""
    import compressed_attention_rotate_amd as tq
    torch = torch_gpu
    hq, hkv, d, page, start, n_new = 32, 8, 128, 128, 32256, 512
    total = start + n_new
    fk = O.Format(128, 3, 3, 128)
    g = TI.gen(7900)
    rb = fk.record_bytes()
    past_k = g.integers(0, 256, (hkv, start, rb), dtype=np.uint8)
    past_v = g.integers(0, 256, (hkv, start, rb), dtype=np.uint8)
    pnk = np.stack([O.fp16_bits(g.uniform(20.0, 60.0, (hkv, start))),
                    O.fp16_bits(g.uniform(1.0, 8.0, (hkv, start)))], axis=-1)
    pnv = np.stack([O.fp16_bits(g.uniform(20.0, 60.0, (hkv, start))),
                    O.fp16_bits(g.uniform(1.0, 8.0, (hkv, start)))], axis=-1)
    kb, vb, _ = TI.kv_layer(1, hkv, n_new, d, seed=7901)           # the chunk's keys and values
    qb = TI.decode_queries(n_new, hq, d, 7901)
    (signs, S), (gsigns, gS) = rotations(d, 7902)
    mb = total // page
    n_pages = mb + 3
    table = TI.gen(7903).permutation(n_pages)[:mb].astype(np.int32)
    ck = np.full((n_pages, hkv, page, rb), 0x5A, np.uint8)
    cv = np.full((n_pages, hkv, page, rb), 0x5A, np.uint8)
    nkc = np.zeros((n_pages, hkv, page, 2), np.uint16)
    nvc = np.zeros((n_pages, hkv, page, 2), np.uint16)
    for blk in range(start // page):
        sl = slice(blk * page, (blk + 1) * page)
        ck[table[blk]], cv[table[blk]] = past_k[:, sl], past_v[:, sl]
        nkc[table[blk]], nvc[table[blk]] = pnk[:, sl], pnv[:, sl]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    f16 = lambda a: dev(a.view(np.int16)).view(torch.float16)
    bf = lambda a: dev(a.view(np.int16)).view(torch.bfloat16)
    fmt = tq.Format.uniform(d, 3)
    tab = tq.Tables(fmt, gsigns, torch.from_numpy(gS).cuda())
    new_k = np.ascontiguousarray(np.transpose(kb[0], (1, 0, 2)))      # [n_new][hkv][d]
    new_v = np.ascontiguousarray(np.transpose(vb[0], (1, 0, 2)))
    out = tq.prefill_paged(bf(qb), bf(new_k), bf(new_v), start, dev(ck), f16(nkc), dev(cv),
                           f16(nvc), dev(table), fmt, tab, fmt, tab)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    # the oracle's cache: the past bytes, then its own packing of the chunk
    ok = oracle_quantize(kb[0].reshape(-1, d), fk, signs, S, bf16=True)
    ov = oracle_quantize(vb[0].reshape(-1, d), fk, signs, S, bf16=True)
    cbk = O.codebook(d, 3)
    q64 = TI.bf16_to_f64(qb)
    rows = [0, 1, 63, 200, 255, 256, 384, 511]
    G = hq // hkv
    worst = 0.0
    for kh in range(hkv):
        rk = np.concatenate([past_k[kh], ok["records"].reshape(hkv, n_new, rb)[kh]])
        rv = np.concatenate([past_v[kh], ov["records"].reshape(hkv, n_new, rb)[kh]])
        nk = np.concatenate([pnk[kh], ok["norms"].reshape(hkv, n_new, 2)[kh]])
        nv = np.concatenate([pnv[kh], ov["norms"].reshape(hkv, n_new, 2)[kh]])
        ik, sk = O.unpack(rk, fk)
        iv, sv = O.unpack(rv, fk)
        kt = O.dequantize(ik, sk, nk[:, 0], nk[:, 1], fk, signs, S, cbk)
        vt = O.dequantize(iv, sv, nv[:, 0], nv[:, 1], fk, signs, S, cbk)
        for i in rows:
            L = start + i + 1
            for gq in range(G):
                h = kh * G + gq
                o = O.attend(q64[i, h], kt[:L], vt[:L], 1 / math.sqrt(d))[0]
                worst = max(worst, float(np.max(np.abs(out[i, h] - o))))
    print(f"\nprefill 512 over 32K: max|out - oracle| {worst:.3g} on {len(rows)} sampled rows")
    assert worst <= OUT_ATOL
