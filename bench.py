"""Benchmark of the TurboQuant hot path on one MI355X.

One step = the whole path over one batch of synthetic input shaped like a
Llama-3.1-8B decode layer with a 32K-token context (32 query / 8 KV heads, head dim 128,
keys and values bf16 with per-channel std log-uniform in [0.5, 8], b = 4 for K and V):
  1. quantize the layer's 32768 keys and 32768 values of all 8 KV heads
     (rotation, norm, codebook, residual, JL projection on MFMA, packing);
  2. one decode step of attention for the 32 query heads straight from a packed cache.
The timed steps rotate over SLOTS independent inputs/caches; step k quantizes slot k and
decodes slot k+1 (written SLOTS-1 steps earlier), so the decoded cache is not resident in
the 256 MB MALL.  Inputs are resident in HBM before timing starts.

Prints one JSON line (see the README of the repository for the fields).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP32_MFMA_PEAK_TFS = 157.3     # MI355X dense fp32 matrix
FP16_MFMA_PEAK_TFS = 2500.0    # MI355X dense fp16 matrix
SLOTS = 8
BATCH, HQ, HKV, NTOK, D = 1, 32, 8, 32768, 128
BITS = 3                        # codebook bits; b = 4 total with the QJL bit


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the other-format / paged / prefill / re-encode measurements that "
                         "follow the timed steps (profiling runs of the main step)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 4 times (scale reference "
                         "for the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only time the 512-token prefill chunk at 32K context (the "
                         "prefill_chunk variant) and print its JSON (profiling runs)")
    ap.add_argument("--search-only", action="store_true",
                    help="only time the inner-product search on the 10^6 x 200 database "
                         "(the search_1m_x_200 variant) and print its JSON (profiling runs)")
    ap.add_argument("--large-batch", action="store_true",
                    help="only time decode on the two full-size layers larger than the MALL "
                         "(batch 16 x 32K at 3.5 bits; batch 4 x 128K, gated and ungated) "
                         "and print their JSON")
    return ap.parse_args()


def _traffic(kernel_srcs, summary: str):
    """HBM traffic per launch from a committed rocprofv3 --pmc summary, or None when the
    summary is missing or was taken on different kernel sources (SHA-256 over the listed
    files' bytes, concatenated in order)."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for src in kernel_srcs:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    sha = h.hexdigest()
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != sha:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(kb, vb, qb, signs, S):
    """The oracle as it stands, on the host cores, over the same layer (about 15 s of CPU
    work): quantize + pack the keys and values of all 8 KV heads x 32768 tokens, then one
    decode step of attention for the 32 query heads."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from threadpoolctl import threadpool_info
    from oracle import tq_oracle as O
    from parity_utils import oracle_decode, oracle_pack_cache
    import tq_inputs as TI
    nt, nh = NTOK, HKV
    fmt = O.Format.uniform(D, BITS)
    t0 = time.perf_counter()
    rk, nk, _ = oracle_pack_cache(kb[:, :nh, :nt], fmt, signs, S, bf16=True)
    rv, nv, _ = oracle_pack_cache(vb[:, :nh, :nt], fmt, signs, S, bf16=True)
    t1 = time.perf_counter()
    oracle_decode(TI.bf16_to_f64(qb[:, :nh * (HQ // HKV)]), rk, nk, rv, nv, [nt], fmt, fmt,
                  signs, S, signs, S, 1 / math.sqrt(D))
    t2 = time.perf_counter()
    packed = 2 * nh * nt * (fmt.record_bytes() + 4)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": packed / (t2 - t1) / 1e9, "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"whole layer, {nh} KV heads x {nt} tokens: quantize+pack {2 * nh * nt} vectors "
                      f"({t1 - t0:.2f} s, {nt / (t1 - t0) * (nh / HKV):.3g} layer-tokens/s), "
                      f"decode {nh * HQ // HKV} query heads ({t2 - t1:.2f} s); value = packed "
                      f"K+V bytes decoded per second",
            "quantize_tokens_per_s": nt * nh / HKV / (t1 - t0)}


def _variant(tq, torch, dev, ks, vs, q, seq, ws, out, fmt_k, fmt_v, signs, S, steps, nvec):
    """The same layer in other packed formats, timed like the main step: SLOTS caches rotate
    (step i quantizes K and V into slot i and decodes slot i + 1, written SLOTS - 1 steps
    earlier), HIP events on the launch stream around each launch."""
    tab_k = tq.Tables(fmt_k, signs, torch.from_numpy(S).to(dev))
    tab_v = tq.Tables(fmt_v, signs, torch.from_numpy(S).to(dev))
    rk, rv = fmt_k.record_bytes(), fmt_v.record_bytes()
    ck = [torch.empty((BATCH, HKV, NTOK, rk), dtype=torch.uint8, device=dev) for _ in range(SLOTS)]
    cv = [torch.empty((BATCH, HKV, NTOK, rv), dtype=torch.uint8, device=dev) for _ in range(SLOTS)]
    nk = [torch.empty((BATCH, HKV, NTOK, 2), dtype=torch.float16, device=dev) for _ in range(SLOTS)]
    nv = [torch.empty_like(x) for x in nk]
    qk = lambda s: tq.quantize_kv(ks[s].view(-1, D), fmt_k, tab_k, codes=ck[s].view(nvec, rk),
                                  norms=nk[s].view(nvec, 2))
    qv = lambda s: tq.quantize_kv(vs[s].view(-1, D), fmt_v, tab_v, codes=cv[s].view(nvec, rv),
                                  norms=nv[s].view(nvec, 2))
    dc = lambda s: tq.attend_decode(q, ck[s], nk[s], cv[s], nv[s], seq, fmt_k, tab_k, fmt_v, tab_v,
                                    workspace=ws, out=out)
    for s in range(SLOTS):
        qk(s); qv(s)
    for i in range(3):
        qk(i % SLOTS); qv(i % SLOTS); dc((i + 1) % SLOTS)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        e = ev[i]
        e[0].record(); qk(i % SLOTS); e[1].record(); qv(i % SLOTS); e[2].record()
        dc((i + 1) % SLOTS); e[3].record()
    torch.cuda.synchronize()
    t_qk = np.mean([e[0].elapsed_time(e[1]) for e in ev]) * 1e-3
    t_qv = np.mean([e[1].elapsed_time(e[2]) for e in ev]) * 1e-3
    t_dc = np.mean([e[2].elapsed_time(e[3]) for e in ev]) * 1e-3
    nbytes = nvec * (rk + 4) + nvec * (rv + 4)
    desc = lambda f: (f"{f.bits_lo}-bit codebook" if f.bits_lo == f.bits_hi else
                      f"{f.bits_lo}/{f.bits_hi}-bit codebook split at {f.split}") + \
        (" + 1 QJL bit" if f.qjl else ", MSE-only") + f" ({f.record_bytes()} B/vector)"
    return {"format_k": desc(fmt_k), "format_v": desc(fmt_v),
            "quantize_k_us": round(float(t_qk) * 1e6, 3),
            "quantize_v_us": round(float(t_qv) * 1e6, 3),
            "decode_us": round(float(t_dc) * 1e6, 3),
            "decode_gbs": round(nbytes / t_dc / 1e9, 2)}


def _paged_timing(tq, torch, dev, ks, q, codes_k, norms_k, codes_v, norms_v, seq, ws, out, fmt,
                  tab, steps, nvec, page=128):
    """The same layer in a paged cache of 128-token pages in shuffled order: decode through
    the block table (slots rotating as in the main step), and quantize-on-write of the key
    tensor into shuffled slots."""
    mb = NTOK // page
    perm = torch.from_numpy(np.random.default_rng(5).permutation(mb)).to(dev)
    bt = perm.to(torch.int32).view(1, mb).contiguous()

    def pages(t):   # [1, HKV, NTOK, w] -> [mb, HKV, page, w], block j in page perm[j]
        blocks = t[0].view(HKV, mb, page, -1).permute(1, 0, 2, 3)
        o = torch.empty_like(blocks)
        o[perm] = blocks
        return o.contiguous()
    pk = [(pages(codes_k[s]), pages(norms_k[s]), pages(codes_v[s]), pages(norms_v[s])) for s in range(SLOTS)]
    dc = lambda s: tq.attend_decode_paged(q, *pk[s], bt, seq, fmt, tab, workspace=ws, out=out)
    for i in range(3):
        dc(i % SLOTS)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        ev[i].record(); dc((i + 1) % SLOTS)
    ev[steps].record(); torch.cuda.synchronize()
    t_dec = np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]) * 1e-3
    # append: token-major copies of the key tensor, one slot per token
    xs = [ks[s][0].permute(1, 0, 2).contiguous() for s in range(2)]
    slots = torch.from_numpy(np.random.default_rng(6).permutation(NTOK).astype(np.int64)).to(dev)
    rb = fmt.record_bytes()
    cache = torch.empty((mb, HKV, page, rb), dtype=torch.uint8, device=dev)
    cnorm = torch.empty((mb, HKV, page, 2), dtype=torch.float16, device=dev)
    ap = lambda s: tq.quantize_kv_paged(xs[s % 2], fmt, tab, slots, cache, cnorm)
    for i in range(3):
        ap(i)
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i].record(); ap(i)
    ev[steps].record(); torch.cuda.synchronize()
    t_app = np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]) * 1e-3
    nbytes = 2 * nvec * (rb + 4)
    return {"page_tokens": page, "decode_us": round(float(t_dec) * 1e6, 3),
            "decode_gbs": round(nbytes / t_dec / 1e9, 2),
            "append_us_per_tensor": round(float(t_app) * 1e6, 3),
            "append_tokens_per_s": round(NTOK * BATCH / t_app, 1)}


def _prefill_timing(tq, torch, dev, ks, vs, fmt, tab, n_new=512, page=128, reps=3):
    """A 512-token prefill chunk at the end of the 32K-token sequence: its keys and values are
    quantized into the paged cache, then its 512 x 32 queries attend causally to the
    32256..32767-token prefixes of the compressed cache."""
    mb = NTOK // page
    table = torch.from_numpy(np.random.default_rng(7).permutation(mb).astype(np.int32)).to(dev)
    rb = fmt.record_bytes()
    ck = torch.empty((mb, HKV, page, rb), dtype=torch.uint8, device=dev)
    nk = torch.empty((mb, HKV, page, 2), dtype=torch.float16, device=dev)
    cv, nv = torch.empty_like(ck), torch.empty_like(nk)
    kx = ks[0][0].permute(1, 0, 2).contiguous()     # [token][head][d]
    vx = vs[0][0].permute(1, 0, 2).contiguous()
    start = NTOK - n_new
    # the cached past: written once with the paged append
    slots = (table.to(torch.int64)[torch.arange(start, device=dev) // page] * page
             + torch.arange(start, device=dev) % page)
    tq.quantize_kv_paged(kx[:start], fmt, tab, slots, ck, nk)
    tq.quantize_kv_paged(vx[:start], fmt, tab, slots, cv, nv)
    g = torch.Generator(device="cpu").manual_seed(8)
    q = torch.randn((n_new, HQ, D), generator=g).to(torch.bfloat16).to(dev)
    ws = torch.empty(tq.prefill_workspace_bytes(n_new, HQ, HKV, start), dtype=torch.uint8, device=dev)
    out = torch.empty((n_new, HQ, D), dtype=torch.float32, device=dev)
    run = lambda: tq.prefill_paged(q, kx[start:], vx[start:], start, ck, nk, cv, nv, table, fmt, tab,
                                   workspace=ws, out=out)
    run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    for i in range(reps):
        ev[i].record(); run()
    ev[reps].record(); torch.cuda.synchronize()
    t = np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]) * 1e-3
    return {"chunk_tokens": n_new, "context": NTOK, "page_tokens": page,
            "ms_per_chunk": round(float(t) * 1e3, 3), "tokens_per_s": round(n_new / t, 1)}


def _requant_timing(tq, torch, dev, codes_k, norms_k, fmt, tab, signs, S, steps, nvec):
    """Temporal decay on the same layer: re-encode the b=4 key cache of a slot at b=3 (into
    a separate buffer, one workspace of the whole tensor), slots rotating as in the main
    step.  Reports per-call time and the stored bytes read + written per second."""
    fo = tq.Format.uniform(D, BITS - 1)
    to = tq.Tables(fo, signs, torch.from_numpy(S).to(dev))
    out_c = torch.empty((nvec, fo.record_bytes()), dtype=torch.uint8, device=dev)
    out_n = torch.empty((nvec, 2), dtype=torch.float16, device=dev)
    ws = torch.empty(tq.requantize_workspace_bytes(nvec, D), dtype=torch.uint8, device=dev)
    call = lambda s: tq.requantize(codes_k[s].view(nvec, -1), norms_k[s].view(nvec, 2), fmt, tab,
                                   fo, to, codes_out=out_c, norms_out=out_n, workspace=ws)
    for i in range(3):
        call(i % SLOTS)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        ev[i].record(); call(i % SLOTS)
    ev[steps].record(); torch.cuda.synchronize()
    t = np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]) * 1e-3
    stored = nvec * (fmt.record_bytes() + 4 + fo.record_bytes() + 4)
    return {"format_in": "3-bit codebook + 1 QJL bit", "format_out": "2-bit codebook + 1 QJL bit",
            "vectors": nvec, "us_per_call": round(float(t) * 1e6, 3),
            "stored_gbs": round(stored / t / 1e9, 2)}


def _decay_timing(tq, torch, dev, q, codes_k, norms_k, codes_v, norms_v, seq, fmt, tab, signs, S,
                  steps, n_old=24576):
    """Temporal decay as a serving cache holds it: in each cache slot the oldest 24576 tokens
    of every KV head are re-encoded at b=3 (tq_requantize on the GPU) and the newest 8192
    stay at b=4; one decode step reads both segments (slots rotating as in the main step)."""
    fo = tq.Format.uniform(D, BITS - 1)
    to = tq.Tables(fo, signs, tab.S)  # one rotation: the same S array for both segments
    nslot = len(codes_k)
    segs = []
    for s2 in range(nslot):
        old_k = codes_k[s2][:, :, :n_old].contiguous().view(-1, fmt.record_bytes())
        old_nk = norms_k[s2][:, :, :n_old].contiguous().view(-1, 2)
        old_v = codes_v[s2][:, :, :n_old].contiguous().view(-1, fmt.record_bytes())
        old_nv = norms_v[s2][:, :, :n_old].contiguous().view(-1, 2)
        rk, rnk = tq.requantize(old_k, old_nk, fmt, tab, fo, to)
        rv, rnv = tq.requantize(old_v, old_nv, fmt, tab, fo, to)
        shp = (BATCH, HKV, n_old)
        segs.append([(rk.view(*shp, -1), rnk.view(*shp, 2), rv.view(*shp, -1), rnv.view(*shp, 2),
                      torch.full((BATCH,), n_old, dtype=torch.int32, device=dev), fo, to, fo, to),
                     (codes_k[s2][:, :, n_old:].contiguous(), norms_k[s2][:, :, n_old:].contiguous(),
                      codes_v[s2][:, :, n_old:].contiguous(), norms_v[s2][:, :, n_old:].contiguous(),
                      seq - n_old, fmt, tab, fmt, tab)])
    ws = torch.empty(tq.attend_segments_workspace_bytes(BATCH, HQ, HKV, [n_old, NTOK - n_old], D),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((BATCH, HQ, D), dtype=torch.float32, device=dev)
    dec = lambda i: tq.attend_decode_segments(q, segs[i % nslot], workspace=ws, out=out)
    for i in range(3):
        dec(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        ev[i].record(); dec(i)
    ev[steps].record(); torch.cuda.synchronize()
    t = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])) * 1e-3
    # replayed from a HIP graph: the GPU time without the binding's per-call host work
    t_g = _graph_decode_timing(torch, dec)
    packed = 2 * BATCH * HKV * (n_old * (fo.record_bytes() + 4) + (NTOK - n_old) * (fmt.record_bytes() + 4))
    return {"old_tokens": n_old, "old_format": "2-bit codebook + 1 QJL bit (48 B/vector)",
            "new_format": "3-bit codebook + 1 QJL bit (64 B/vector)", "packed_bytes": packed,
            "decode_us": round(t * 1e6, 3), "decode_us_graph_replay": round(t_g * 1e6, 3),
            "decode_gbs_graph_replay": round(packed / t_g / 1e9, 2)}


def _copy_gbs(torch, dev, nbytes=256 << 20, reps=10):
    """Measured HBM bandwidth of a plain device copy (nbytes read + nbytes written per
    copy), the practical ceiling the decode rate is also compared with."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    t = ev[0].elapsed_time(ev[1]) * 1e-3 / reps
    del src, dst
    return 2 * nbytes / t / 1e9


def _graph_decode_timing(torch, decode, reps=5):
    """The decode step of every cache slot captured once into a HIP graph and replayed: the
    per-step time without host launch overhead (the same kernels, caches and order as the
    timed eager steps)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for s in range(SLOTS):
            decode(s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(SLOTS):
            decode(s)
    g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        g.replay()
    ev[1].record()
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) * 1e-3 / (reps * SLOTS)


def _sparse_v_timing(tq, torch, dev, q, codes_k, norms_k, codes_v, norms_v, seq, ws, out, fmt_k,
                     tab_k, fmt_v, tab_v, steps, tau=1e-4):
    """Decode with the Sparse-V gate (tau = 1e-4) against the same decode ungated, on the same
    packed caches: the two run interleaved (cache slots rotating), each launch bracketed by
    HIP events on the launch stream.  skipped_frac = value rows (per KV head and token) the
    gate left unread over all rows, counted by the kernel on one gated pass per slot."""
    nslot = len(codes_k)
    batch, hkv, ntok = codes_k[0].shape[:3]
    dec = lambda s, t, sk=None: tq.attend_decode(q, codes_k[s], norms_k[s], codes_v[s], norms_v[s],
                                                 seq, fmt_k, tab_k, fmt_v, tab_v, tau=t,
                                                 skipped=sk, workspace=ws, out=out)
    sk = torch.zeros(1, dtype=torch.int64, device=dev)
    for s in range(nslot):
        dec(s, 0.0); dec(s, tau, sk)
    torch.cuda.synchronize()
    skipped = int(sk.item())
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        e = ev[i]
        e[0].record(); dec(i % nslot, 0.0); e[1].record(); dec(i % nslot, tau); e[2].record()
    torch.cuda.synchronize()
    t_u = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3
    t_g = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e-3
    rk, rv = fmt_k.record_bytes(), fmt_v.record_bytes()
    rows = batch * hkv * ntok
    return {"tau": tau, "decode_us_ungated": round(t_u * 1e6, 3),
            "decode_us_gated": round(t_g * 1e6, 3),
            "speedup": round(t_u / t_g, 4),
            "skipped_frac": round(skipped / (rows * nslot), 4),
            "packed_gbs_ungated": round(rows * (rk + rv + 8) / t_u / 1e9, 2)}


def _large_layer(tq, torch, dev, TI, cfg, batch, ntok, fk, fv, spikes):
    """One full-size layer of the Llama-3.1-8B law (batch x ntok tokens, 8 KV heads),
    quantized on the GPU; returns the packed caches, queries and decode buffers."""
    seed = TI.data_seed(cfg)
    kb, vb, _ = TI.kv_layer(batch, HKV, ntok, D, seed=seed, spike_frac=spikes)
    qb = TI.decode_queries(batch, HQ, D, seed)
    signs, S = TI.rotation(D, TI.rotation_seed(cfg))
    Sd = torch.from_numpy(S).to(dev)
    tk, tv = tq.Tables(fk, signs, Sd), tq.Tables(fv, signs, Sd)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    k0, v0 = bf(kb).view(-1, D), bf(vb).view(-1, D)
    del kb, vb
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    tq.quantize_kv(k0, fk, tk)                       # warm-up
    ev[0].record()
    ck, nk = tq.quantize_kv(k0, fk, tk)
    ev[1].record()
    cv, nv = tq.quantize_kv(v0, fv, tv)
    ev[2].record()
    torch.cuda.synchronize()
    del k0, v0
    shp = (batch, HKV, ntok)
    caches = (ck.view(*shp, -1), nk.view(*shp, 2), cv.view(*shp, -1), nv.view(*shp, 2))
    q = bf(qb)
    seq = torch.full((batch,), ntok, dtype=torch.int32, device=dev)
    ws = torch.zeros(tq.attend_workspace_bytes(batch, HQ, HKV, ntok, D), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((batch, HQ, D), dtype=torch.float32, device=dev)
    t_q = (ev[0].elapsed_time(ev[1]) + ev[1].elapsed_time(ev[2])) * 1e-3
    return caches, q, seq, ws, out, tk, tv, t_q


def _large_batch(tq, torch, dev, TI, steps):
    """The two full-size layers beside the 32K batch-1 step, each decoded from one packed
    cache larger than the MALL: batch 16 x 32768 tokens at 3.5 bits (3-bit codebook on
    rotated coordinates 0-63, 2-bit on 64-127, + QJL; 60 B per vector with its norms), and
    batch 4 x 131072 tokens with 1% of token positions carrying x10 keys, K b = 4, V b = 3,
    decoded gated (tau = 1e-4) and ungated.  For the gated layer the softmax mass of the
    tokens under tau (from the ungated logits) bounds the mass the gate drops: a dropped
    token's running weight estimate, which is at least its final weight, was under tau."""
    res = {}
    fmt = tq.Format(D, 3, 2, 64)
    (ck, nk, cv, nv), q, seq, ws, out, tk, tv, t_q = _large_layer(
        tq, torch, dev, TI, 3, 16, NTOK, fmt, fmt, 0.0)
    dec = lambda: tq.attend_decode(q, ck, nk, cv, nv, seq, fmt, tk, fmt, tv, workspace=ws, out=out)
    for _ in range(3):
        dec()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        ev[i].record(); dec()
    ev[steps].record()
    torch.cuda.synchronize()
    t = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])) * 1e-3
    nbytes = 2 * ck.shape[0] * HKV * NTOK * (fmt.record_bytes() + 4)
    res["batch16_32k_b3.5"] = {
        "workload": "batch 16 x 32768 tokens, 32 q / 8 kv heads, head_dim 128, K and V at 3.5 "
                    "bits (3/2-bit codebook split at 64 + QJL, 60 B per vector)",
        "packed_bytes": nbytes, "decode_us": round(t * 1e6, 3),
        "decode_gbs": round(nbytes / t / 1e9, 2),
        "decode_pct_hbm_peak": round(100.0 * nbytes / t / 1e9 / HBM_PEAK_GBS, 2),
        "quantize_tokens_per_s": round(16 * NTOK / t_q, 1)}
    del ck, nk, cv, nv, ws
    torch.cuda.empty_cache()

    ntok = 131072
    fk, fv = tq.Format.uniform(D, 3), tq.Format.uniform(D, 2)
    (ck, nk, cv, nv), q, seq, ws, out, tk, tv, t_q = _large_layer(
        tq, torch, dev, TI, 4, 4, ntok, fk, fv, 0.01)
    r = _sparse_v_timing(tq, torch, dev, q, [ck], [nk], [cv], [nv], seq, ws, out, fk, tk, fv, tv,
                         steps)
    _, lg = tq.attend_decode(q, ck, nk, cv, nv, seq, fk, tk, fv, tv, logits=True, workspace=ws)
    p = torch.softmax(lg.double(), dim=-1)
    below = torch.where(p < r["tau"], p, torch.zeros_like(p)).sum(dim=-1)
    r["mass_under_tau_max"] = float(below.max())
    r["quantize_tokens_per_s"] = round(4 * ntok / t_q, 1)
    r["workload"] = ("batch 4 x 131072 tokens, 32 q / 8 kv heads, head_dim 128, 1% of token "
                     "positions with x10 keys; K b=4 (3-bit codebook + QJL), V b=3 (2-bit "
                     "codebook + QJL)")
    res["batch4_128k_sparse_v"] = r
    return res


def _search_timing(tq, torch, dev, TI, reps=2):
    """Inner-product search on the 10^6 x 200 database (unit vectors, std i^-0.3 per
    coordinate), zero-padded to d = 256 and packed at b = 4; 10^4 queries from the same law,
    top-10.  Times the index build (quantize of the database) and the search of all queries.
    Roofline: the estimator's 2 x 256 multiply-adds per (query, vector) pair (two dot
    products of length d) against the dense fp16 MFMA peak the scan runs on; its operands
    are split into fp16 hi + lo halves, so it issues 5 products where the dot products
    count 2."""
    n_db, n_q, d_in, d, k = 10 ** 6, 10 ** 4, 200, 256, 10
    db = torch.from_numpy(TI.search_set(n_db, d_in, seed=TI.data_seed(5))).to(dev)
    qs = torch.from_numpy(TI.search_set(n_q, d_in, seed=TI.data_seed(5) + 1)).to(dev)
    signs, S = TI.rotation(d, TI.rotation_seed(5))
    fmt = tq.Format.uniform(d, BITS)
    tab = tq.Tables(fmt, signs, torch.from_numpy(S).to(dev))
    codes = torch.empty((n_db, fmt.record_bytes()), dtype=torch.uint8, device=dev)
    norms = torch.empty((n_db, 2), dtype=torch.float16, device=dev)
    build = lambda: tq.quantize_kv(db, fmt, tab, codes=codes, norms=norms)
    ws = torch.empty(tq.search_workspace_bytes(n_q, k, n_db, d), dtype=torch.uint8, device=dev)
    search = lambda: tq.ip_search(qs, codes, norms, fmt, tab, k=k, workspace=ws)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        for i in range(reps):
            ev[i].record(); fn()
        ev[reps].record(); torch.cuda.synchronize()
        return float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])) * 1e-3

    tb = timed(build)
    ts = timed(search)
    # unbatched: one query (and one block of 32) streams the whole packed database
    t1 = timed(lambda: tq.ip_search(qs[:1], codes, norms, fmt, tab, k=k, workspace=ws))
    t32 = timed(lambda: tq.ip_search(qs[:32], codes, norms, fmt, tab, k=k, workspace=ws))
    db_bytes = n_db * (fmt.record_bytes() + 4)
    flops = 2.0 * 2 * d * n_db * n_q
    tfs = flops / ts / 1e12
    return {"db_vectors": n_db, "d_in": d_in, "d": d, "queries": n_q, "k": k,
            "format": "3-bit codebook + 1 QJL bit (132 B/vector)",
            "index_build_ms": round(tb * 1e3, 3), "index_vectors_per_s": round(n_db / tb, 1),
            "search_ms": round(ts * 1e3, 3), "queries_per_s": round(n_q / ts, 1),
            "one_query_us": round(t1 * 1e6, 2), "one_query_db_gbs": round(db_bytes / t1 / 1e9, 1),
            "one_query_pct_hbm_peak": round(100.0 * db_bytes / t1 / 1e9 / HBM_PEAK_GBS, 2),
            "queries_32_us": round(t32 * 1e6, 2), "queries_32_per_s": round(32 / t32, 1),
            "roofline": {"bound": "mfma", "kernel": "search_scan", "achieved": round(tfs, 3),
                         "peak": FP16_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": round(tfs / FP16_MFMA_PEAK_TFS, 4), "traffic": None}}


def main():
    args = _parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build measures the single-GPU path "
              "(no collectives); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.calibrate_copy:
        src = torch.ones(args.calibrate_copy // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": args.calibrate_copy}))
        return
    import compressed_attention_rotate_amd as tq
    import tq_inputs as TI
    tq.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.search_only:
        print(json.dumps({"search_1m_x_200": _search_timing(tq, torch, dev, TI)}), flush=True)
        return

    if args.large_batch:
        print(json.dumps(_large_batch(tq, torch, dev, TI, args.steps)), flush=True)
        return

    seed = TI.data_seed(2)
    kb, vb, _ = TI.kv_layer(BATCH, HKV, NTOK, D, seed=seed)
    qb = TI.decode_queries(BATCH, HQ, D, seed)
    signs, S = TI.rotation(D, TI.rotation_seed(2))
    fmt = tq.Format.uniform(D, BITS)
    tab = tq.Tables(fmt, signs, torch.from_numpy(S).to(dev))
    rb = fmt.record_bytes()
    nvec = BATCH * HKV * NTOK

    k0 = torch.from_numpy(kb.view(np.int16)).to(dev).view(torch.bfloat16)
    v0 = torch.from_numpy(vb.view(np.int16)).to(dev).view(torch.bfloat16)
    if args.prefill_only:
        print(json.dumps({"prefill_chunk": _prefill_timing(tq, torch, dev, [k0], [v0], fmt, tab)}),
              flush=True)
        return
    # SLOTS distinct inputs (token order rotated per slot: same law, different bytes)
    ks = [torch.roll(k0, shifts=4099 * i, dims=2).contiguous() for i in range(SLOTS)]
    vs = [torch.roll(v0, shifts=4099 * i, dims=2).contiguous() for i in range(SLOTS)]
    del k0, v0
    codes_k = [torch.empty((BATCH, HKV, NTOK, rb), dtype=torch.uint8, device=dev) for _ in range(SLOTS)]
    codes_v = [torch.empty_like(c) for c in codes_k]
    norms_k = [torch.empty((BATCH, HKV, NTOK, 2), dtype=torch.float16, device=dev) for _ in range(SLOTS)]
    norms_v = [torch.empty_like(n) for n in norms_k]
    q = torch.from_numpy(qb.view(np.int16)).to(dev).view(torch.bfloat16)
    seq = torch.full((BATCH,), NTOK, dtype=torch.int32, device=dev)
    ws = torch.zeros(tq.attend_workspace_bytes(BATCH, HQ, HKV, NTOK, D), dtype=torch.uint8, device=dev)
    out = torch.empty((BATCH, HQ, D), dtype=torch.float32, device=dev)

    def quantize(s):
        tq.quantize_kv(ks[s].view(-1, D), fmt, tab, codes=codes_k[s].view(nvec, rb),
                       norms=norms_k[s].view(nvec, 2))

    def quantize_v(s):
        tq.quantize_kv(vs[s].view(-1, D), fmt, tab, codes=codes_v[s].view(nvec, rb),
                       norms=norms_v[s].view(nvec, 2))

    def decode(s):
        tq.attend_decode(q, codes_k[s], norms_k[s], codes_v[s], norms_v[s], seq, fmt, tab,
                         workspace=ws, out=out)

    for s in range(SLOTS):              # every slot holds a packed cache before timing
        quantize(s)
        quantize_v(s)
    for k in range(args.warmup):
        quantize(k % SLOTS); quantize_v(k % SLOTS); decode((k + 1) % SLOTS)
    torch.cuda.synchronize()

    steps = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        e = ev[k]
        e[0].record()
        quantize(k % SLOTS)
        e[1].record()
        quantize_v(k % SLOTS)
        e[2].record()
        decode((k + 1) % SLOTS)
        e[3].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    qk = np.array([e[0].elapsed_time(e[1]) for e in ev]) * 1e-3
    qv = np.array([e[1].elapsed_time(e[2]) for e in ev]) * 1e-3
    dc = np.array([e[2].elapsed_time(e[3]) for e in ev]) * 1e-3
    packed_bytes = 2 * nvec * (rb + 4)                      # K + V records and norms read
    decode_gbs = packed_bytes * steps / dc.sum() / 1e9
    q_launch = float(np.concatenate([qk, qv]).mean())
    flops_launch = 2.0 * D * D * nvec                         # S r per vector
    q_tfs = flops_launch / q_launch / 1e12
    qtoks = NTOK * BATCH * steps / (qk.sum() + qv.sum())
    copy_gbs = _copy_gbs(torch, dev)
    trafq = _traffic(["compressed_attention_rotate_amd/csrc/tq_quantize_kernel.h"],
                     "quantize_llama8b_32k_traffic.txt")
    trafd = _traffic(["compressed_attention_rotate_amd/csrc/tq_decode_kernel.h",
                      "compressed_attention_rotate_amd/csrc/tq_decode.hip"],
                     "decode_llama8b_32k_traffic.txt")

    line = {
        "metric": "decode-attn packed-KV GB/s & % HBM peak; quantize tokens/s (32K ctx, b=4)",
        "value": round(decode_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B-shaped decode layer: batch 1, 32 q / 8 kv heads, "
                               "head_dim 128, 32768 cached tokens, bf16 K/V (per-channel std "
                               "log-uniform [0.5, 8]), b=4 (3-bit codebook + 1 QJL bit)",
                   "global_batch": BATCH, "seq_len": NTOK, "parallelism": "none (1 GPU)"},
        "decode_pct_hbm_peak": round(100.0 * decode_gbs / HBM_PEAK_GBS, 2),
        "hbm_copy_gbs": round(copy_gbs, 1),
        "decode_pct_copy_bw": round(100.0 * decode_gbs / copy_gbs, 2),
        "decode_us": round(float(dc.mean()) * 1e6, 3),
        "decode_us_graph_replay": round(_graph_decode_timing(torch, decode) * 1e6, 3),
        "quantize_tokens_per_s": round(qtoks, 1),
        "quantize_us_per_launch": round(q_launch * 1e6, 3),
        "roofline": {"bound": "mfma", "kernel": "quantize_kernel<128,3,3>",
                     "achieved": round(q_tfs, 3), "peak": FP32_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": round(q_tfs / FP32_MFMA_PEAK_TFS, 4), "traffic": trafq},
        "roofline_decode": {"bound": "hbm", "kernel": "decode_scan+decode_combine",
                            "achieved": round(decode_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(decode_gbs / HBM_PEAK_GBS, 4), "traffic": trafd},
    }
    # other formats of the same layer (not part of `value`)
    if args.no_variants:
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline(kb, vb, qb, signs, S)
        print(json.dumps(line), flush=True)
        return
    line["variants"] = {
        name: _variant(tq, torch, dev, ks, vs, q, seq, ws, out, fk, fv, signs, S, steps, nvec)
        for name, fk, fv in (
            ("b4_k_mse_only_v", fmt, tq.Format.uniform(D, BITS, qjl=False)),
            ("b3.5_kv", tq.Format(D, 3, 2, 64), tq.Format(D, 3, 2, 64)),
            ("b2.5_kv", tq.Format(D, 2, 1, 64), tq.Format(D, 2, 1, 64)))}
    line["variants"]["paged_b4"] = _paged_timing(tq, torch, dev, ks, q, codes_k, norms_k, codes_v,
                                                 norms_v, seq, ws, out, fmt, tab, steps, nvec)
    line["variants"]["prefill_chunk"] = _prefill_timing(tq, torch, dev, ks, vs, fmt, tab)
    line["variants"]["requantize_b4_to_b3"] = _requant_timing(tq, torch, dev, codes_k, norms_k, fmt,
                                                              tab, signs, S, steps, nvec)
    line["variants"]["decay_24k_b3_8k_b4"] = _decay_timing(
        tq, torch, dev, q, codes_k, norms_k, codes_v, norms_v, seq, fmt, tab, signs, S, steps)
    line["variants"]["sparse_v_32k_b4"] = _sparse_v_timing(
        tq, torch, dev, q, codes_k, norms_k, codes_v, norms_v, seq, ws, out, fmt, tab, fmt, tab,
        steps)
    line["variants"]["search_1m_x_200"] = _search_timing(tq, torch, dev, TI)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(kb, vb, qb, signs, S)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
