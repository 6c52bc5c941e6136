"""Benchmark of the TurboQuant hot path on one MI355X.

One step = the whole path over one batch of synthetic input shaped like a
Llama-3.1-8B decode layer with a 32K-token context (32 query / 8 KV heads, head dim 128,
keys and values bf16 with per-channel std log-uniform in [0.5, 8], b = 4 for K and V):
  1. quantize the layer's 32768 keys and 32768 values of all 8 KV heads
     (rotation, norm, codebook, residual, JL projection on MFMA, packing; the values are
     written token-sliced);
  2. one decode step of attention for the 32 query heads straight from a packed cache.
Beside the timed step the same JSON line reports the other workloads: the single-head
quality setting (C1), 32 full-size layers of batch 16 at 3.5 bits (C3), batch 4 x 131072
tokens with key spikes and the Sparse-V gate (C4), and the 10^6-vector search with
recall@10 (C5).
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
    ap.add_argument("--config", default="all", choices=["all", "C1", "C2", "C3", "C4", "C5"],
                    help="workloads to run: C2 is the timed step (the `value`); C1 quality, "
                         "C3 32 layers of batch 16 x 32K at 3.5 bits, C4 batch 4 x 128K with the "
                         "Sparse-V gate, C5 the 10^6 x 200 search with recall@10")
    ap.add_argument("--seed", type=int, default=0,
                    help="offset added to every data and rotation seed")
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
                    help="only run the two full-size workloads larger than the MALL (C3: 32 "
                         "layers of batch 16 x 32K at 3.5 bits; C4: batch 4 x 128K, gated and "
                         "ungated) and print their JSON")
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


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(kb, vb, qb, rot_seed):
    """The C++ oracle (oracle/tq_oracle.cpp: plain fp64, std::thread over every hardware
    thread) on the host cores, over the same layer: quantize + pack the keys and values of
    all 8 KV heads x 32768 tokens, then one decode step (dequantize the packed cache, softmax
    attention of the 32 query heads).  The single-thread figure runs the same code on one
    thread over a 1/8 sample (KV head 0 and its 4 query heads)."""
    from oracle import tq_oracle as O
    from oracle import tq_oracle_cpp as C
    signs, S = O.make_rotation(D, rot_seed)   # the oracle's own draws of the same rotation
    fmt = O.Format.uniform(D, BITS)
    cb = O.codebook(D, BITS)
    G = HQ // HKV

    def bf(a):
        return a.astype(np.uint32).view(np.uint32) << 16

    def run(nh, threads):
        kx = (bf(kb[:, :nh]).view(np.float32)).reshape(-1, D).astype(np.float64)
        vx = (bf(vb[:, :nh]).view(np.float32)).reshape(-1, D).astype(np.float64)
        q = (bf(qb[:, :nh * G]).view(np.float32)).astype(np.float64)
        t0 = time.perf_counter()
        rk, nk, rrk = C.quantize(kx, fmt, signs, S, cb, threads=threads)
        rv, nv, rrv = C.quantize(vx, fmt, signs, S, cb, threads=threads)
        t1 = time.perf_counter()
        kt = C.dequantize(rk, nk, rrk, fmt, signs, S, cb, threads=threads).reshape(BATCH, nh, NTOK, D)
        vt = C.dequantize(rv, nv, rrv, fmt, signs, S, cb, threads=threads).reshape(BATCH, nh, NTOK, D)
        C.attend(q, kt, vt, [NTOK], 1 / math.sqrt(D), threads=threads)
        t2 = time.perf_counter()
        packed = 2 * BATCH * nh * NTOK * (fmt.record_bytes() + 4)
        return packed / (t2 - t1) / 1e9, BATCH * nh * NTOK / (t1 - t0), t1 - t0, t2 - t1

    threads = C.hardware_threads()
    gbs, qtok, tq_, td = run(HKV, 0)
    gbs1, qtok1, tq1, td1 = run(1, 1)
    return {"value": round(gbs, 5), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"C++ fp64 oracle, {threads} threads, whole layer: quantize+pack "
                      f"{2 * HKV * NTOK} vectors ({tq_:.2f} s), decode of {HQ} query heads "
                      f"(dequantize the packed K and V, softmax attention; {td:.2f} s); value = "
                      f"packed K+V bytes decoded per second",
            "quantize_tokens_per_s": round(qtok, 1),
            "single_thread": {"value": round(gbs1, 5), "unit": "GB/s",
                              "quantize_tokens_per_s": round(qtok1, 1),
                              "sample": f"1 thread, KV head 0 with its {G} query heads (1/8 of "
                                        f"the layer): quantize {tq1:.2f} s, decode {td1:.2f} s"}}


def _bf16_host(t):
    """A bf16 device tensor -> its host bit patterns (uint16 numpy array)."""
    return t.contiguous().view(dtype=__import__("torch").int16).cpu().numpy().view(np.uint16)


def _f64_of_bf16(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def cpu_baseline_configs(samples, seed):
    """The C++ oracle on bounded samples of the other workloads (the same bytes the GPU legs
    used, copied to the host), timed on every hardware thread:
      C1: the whole setting (quantize K and V, decode the 64 queries), with the estimator's
          quality against exact attention computed from the oracle's own reconstruction;
      C3: one sequence of layer 0 (32768 tokens x 8 KV heads at 3.5 bits, 1/16 of the layer),
          with the 32-layer x 16-sequence time extrapolated from it;
      C4: sequence 0 of 4 (131072 tokens x 8 KV heads, K b=4 / V b=3), decoded ungated and
          gated (tau = 1e-4);
      C5: the first 100000 database vectors and the first 100 queries: index build, the
          estimated top-10 (dequantized database) and the exact top-10 within the sample."""
    from oracle import tq_oracle as O
    from oracle import tq_oracle_cpp as C
    threads = C.hardware_threads()
    res = {}
    if "C1" in samples:
        import tq_inputs as TI
        k, v, q, _ = TI.c1_inputs(seed=TI.data_seed(1) + seed)
        n, d = k.shape
        fmt = O.Format.uniform(d, 2)
        signs, S = O.make_rotation(d, TI.rotation_seed(1) + seed)
        cb = O.codebook(d, 2)
        t0 = time.perf_counter()
        rk = C.quantize(k.astype(np.float64), fmt, signs, S, cb)
        rv = C.quantize(v.astype(np.float64), fmt, signs, S, cb)
        t1 = time.perf_counter()
        kt = C.dequantize(*rk, fmt, signs, S, cb).reshape(1, 1, n, d)
        vt = C.dequantize(*rv, fmt, signs, S, cb).reshape(1, 1, n, d)
        oq, lq = C.attend(q.astype(np.float64)[None], kt, vt, [n], 1 / math.sqrt(d))
        t2 = time.perf_counter()
        q64, k64, v64 = q.astype(np.float64), k.astype(np.float64), v.astype(np.float64)
        le = q64 @ k64.T / math.sqrt(d)
        lq = lq[0]
        pe, pq = _softmax_rows(le), _softmax_rows(lq)
        oe = pe @ v64
        kl = np.sum(pe * (np.log(np.maximum(pe, 1e-300)) - np.log(np.maximum(pq, 1e-300))), axis=1)
        rel = np.linalg.norm(oq[0] - oe, axis=1) / np.linalg.norm(oe, axis=1)
        res["C1"] = {"sample": "the whole setting (8192 vectors quantized, 64 queries decoded)",
                     "quantize_s": round(t1 - t0, 4), "decode_s": round(t2 - t1, 4),
                     "oracle_quality": {
                         "logit_rmse_over_sigma": float(np.sqrt(np.mean((lq - le) ** 2)) / np.std(le)),
                         "softmax_max_abs_dp": float(np.max(np.abs(pq - pe))),
                         "kl_mean": float(np.mean(kl)), "out_rel_l2_mean": float(np.mean(rel))}}

    def layer_sample(kbits, vbits, qbits, fk, fv, cbk, cbv, signs, S, taus):
        nh, ntok, d = kbits.shape
        kx, vx = _f64_of_bf16(kbits).reshape(-1, d), _f64_of_bf16(vbits).reshape(-1, d)
        t0 = time.perf_counter()
        rk = C.quantize(kx, fk, signs, S, *cbk)
        rv = C.quantize(vx, fv, signs, S, *cbv)
        t1 = time.perf_counter()
        del kx, vx
        kt = C.dequantize(*rk, fk, signs, S, *cbk).reshape(1, nh, ntok, d)
        vt = C.dequantize(*rv, fv, signs, S, *cbv).reshape(1, nh, ntok, d)
        q = _f64_of_bf16(qbits).reshape(1, -1, d)
        t2 = time.perf_counter()
        out = {}
        for tau in taus:
            ta = time.perf_counter()
            _, _, dropped = C.attend(q, kt, vt, [ntok], 1 / math.sqrt(d), tau=tau, return_dropped=True)
            out[tau] = (time.perf_counter() - ta, int(dropped.sum()))
        packed = nh * ntok * (fk.record_bytes() + fv.record_bytes() + 8)
        return t1 - t0, t2 - t1, out, packed

    if "C3" in samples:
        kbits, vbits, qbits, rseed = samples["C3"]
        signs, S = O.make_rotation(D, rseed)
        f = O.Format(D, 3, 2, 64)
        cbs = (O.codebook(D, 3), O.codebook(D, 2))
        tq_, tdq, att, packed = layer_sample(kbits, vbits, qbits, f, f, cbs, cbs, signs, S, [0.0])
        td = tdq + att[0.0][0]
        ntok = kbits.shape[1]
        res["C3"] = {"sample": "sequence 0 of layer 0: 32768 tokens x 8 KV heads at 3.5 bits "
                               "(1/16 of a layer), its 32 query heads decoded once",
                     "quantize_tokens_per_s": round(ntok / tq_, 1),
                     "decode_gbs": round(packed / td / 1e9, 5),
                     "extrapolated_32_layers_x_16_sequences_s": round(32 * 16 * (tq_ + td), 1)}
    if "C4" in samples:
        kbits, vbits, qbits, rseed, tau = samples["C4"]
        signs, S = O.make_rotation(D, rseed)
        fk, fv = O.Format.uniform(D, 3), O.Format.uniform(D, 2)
        tq_, tdq, att, packed = layer_sample(kbits, vbits, qbits, fk, fv, (O.codebook(D, 3),),
                                             (O.codebook(D, 2),), signs, S, [0.0, tau])
        ntok = kbits.shape[1]
        res["C4"] = {"sample": "sequence 0 of 4: 131072 tokens x 8 KV heads, K b=4 / V b=3, "
                               "its 32 query heads decoded ungated and gated",
                     "quantize_tokens_per_s": round(ntok / tq_, 1),
                     "dequantize_s": round(tdq, 3),
                     "decode_gbs_ungated": round(packed / (tdq + att[0.0][0]) / 1e9, 5),
                     "decode_gbs_gated": round(packed / (tdq + att[tau][0]) / 1e9, 5),
                     "gated_rows_dropped_per_query_head": round(att[tau][1] / HQ, 1),
                     "tau": tau}
    if "C5" in samples:
        db, qs, rseed = samples["C5"]
        d = 256
        signs, S = O.make_rotation(d, rseed)
        fmt = O.Format.uniform(d, BITS)
        cb = O.codebook(d, BITS)
        t0 = time.perf_counter()
        rec = C.quantize(db.astype(np.float64), fmt, signs, S, cb)
        t1 = time.perf_counter()
        xt = C.dequantize(*rec, fmt, signs, S, cb)
        t2 = time.perf_counter()
        qp = np.zeros((qs.shape[0], d))
        qp[:, :qs.shape[1]] = qs
        est, _ = C.topk_ip(qp, xt, 10)
        t3 = time.perf_counter()
        ex, _ = C.topk_ip(qs.astype(np.float64), db.astype(np.float64), 10)
        pairs = qs.shape[0] * db.shape[0]
        res["C5"] = {"sample": f"the first {db.shape[0]} database vectors and the first "
                               f"{qs.shape[0]} queries (d=200 zero-padded to 256, b=4)",
                     "index_vectors_per_s": round(db.shape[0] / (t1 - t0), 1),
                     "dequantize_s": round(t2 - t1, 3),
                     "search_pairs_per_s": round(pairs / (t3 - t2), 1),
                     "queries_per_s_at_1e6_vectors": round(pairs / (t3 - t2) / 1e6, 3),
                     "recall_at_10_in_sample": round(O.recall_at_k(est, ex), 4)}
    return {"cores": int(threads), "configs": res}


def _softmax_rows(x):
    m = x.max(axis=1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=1, keepdims=True)


def _c1_quality(tq, torch, dev, TI, seed):
    """Single head, d = 128: 4096 keys and values N(0, 1) fp32 with 4 of 128 channels scaled
    x20, 64 queries N(0, 1); b = 3 for K and V (2-bit codebook + QJL, values token-sliced),
    quantized and decoded by the library (logits returned), against exact attention over
    the unquantized fp32 inputs (computed here in fp64)."""
    k, v, q, ch = TI.c1_inputs(seed=TI.data_seed(1) + seed)
    n, d = k.shape
    fk = tq.Format.uniform(d, 2)
    fv = fk.sliced()
    signs, S = tq.make_rotation(d, TI.rotation_seed(1) + seed)
    Sd = torch.from_numpy(S).to(dev)
    tk, tv = tq.Tables(fk, signs, Sd), tq.Tables(fv, signs, Sd)
    ck, nk = tq.quantize_kv(torch.from_numpy(k).to(dev), fk, tk)
    cv, nv = tq.quantize_kv(torch.from_numpy(v).to(dev), fv, tv)
    rb = fk.record_bytes()
    qt = torch.from_numpy(q).to(dev).view(1, q.shape[0], d)
    seq = torch.tensor([n], dtype=torch.int32, device=dev)
    out, lg = tq.attend_decode(qt, ck.view(1, 1, n, rb), nk.view(1, 1, n, 2),
                               cv.view(1, 1, n // 32, 32 * rb), nv.view(1, 1, n, 2), seq, fk, tk,
                               fv, tv, logits=True)
    torch.cuda.synchronize()
    lq, oq = lg[0].double().cpu().numpy(), out[0].double().cpu().numpy()
    k64, v64, q64 = k.astype(np.float64), v.astype(np.float64), q.astype(np.float64)
    le = q64 @ k64.T / math.sqrt(d)
    pe, pq = _softmax_rows(le), _softmax_rows(lq)
    oe = pe @ v64
    kl = np.sum(pe * (np.log(np.maximum(pe, 1e-300)) - np.log(np.maximum(pq, 1e-300))), axis=1)
    rel = np.linalg.norm(oq - oe, axis=1) / np.linalg.norm(oe, axis=1)
    return {"workload": "single head, d=128, 4096 keys/values N(0,1) fp32 with 4 of 128 channels "
                        "x20, 64 queries N(0,1); b=3 (2-bit codebook + 1 QJL bit), values "
                        "token-sliced; against exact fp32-input attention",
            "outlier_channels": [int(c) for c in ch],
            "logit_rmse_over_sigma": float(np.sqrt(np.mean((lq - le) ** 2)) / np.std(le)),
            "logit_max_abs_err": float(np.max(np.abs(lq - le))),
            "softmax_max_abs_dp": float(np.max(np.abs(pq - pe))),
            "kl_mean": float(np.mean(kl)), "kl_max": float(np.max(kl)),
            "out_rel_l2_mean": float(np.mean(rel)), "out_rel_l2_max": float(np.max(rel))}


def _decode_roofline(name, nbytes, t):
    gbs = nbytes / t / 1e9
    return {"bound": "hbm", "kernel": name, "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}


def _c3_layers(tq, torch, dev, TI, seed, n_layers=32, batch=16, dec_steps=4, samples=None):
    """32 full-size layers, batch 16 x 32768 tokens each, 32 q / 8 kv heads, distinct seeds
    per layer (data and rotation), K and V at 3.5 bits (3-bit codebook on rotated
    coordinates 0-63, 2-bit on 64-127, + QJL; values token-sliced).  Per layer: the prefill
    quantize of its 32768 new tokens per sequence (K then V, HIP events around each launch),
    then steady-state decode steps over the layer's packed cache."""
    ntok = NTOK
    fk = tq.Format(D, 3, 2, 64)
    fv = fk.sliced()
    rb = fk.record_bytes()
    nvec = batch * HKV * ntok
    ck = torch.empty((nvec, rb), dtype=torch.uint8, device=dev)
    nk = torch.empty((nvec, 2), dtype=torch.float16, device=dev)
    cv = torch.empty((nvec // 32, 32 * rb), dtype=torch.uint8, device=dev)
    nv = torch.empty((nvec, 2), dtype=torch.float16, device=dev)
    ws = torch.empty(tq.attend_workspace_bytes(batch, HQ, HKV, ntok, D), dtype=torch.uint8, device=dev)
    out = torch.empty((batch, HQ, D), dtype=torch.float32, device=dev)
    seq = torch.full((batch,), ntok, dtype=torch.int32, device=dev)
    t_q, t_d = [], []
    for layer in range(n_layers):
        kx, vx = TI.kv_layer_device(batch, HKV, ntok, D, TI.data_seed(3, layer) + seed, dev)
        signs, S = tq.make_rotation(D, TI.rotation_seed(3, layer) + seed)
        Sd = torch.from_numpy(S).to(dev)
        tk, tv = tq.Tables(fk, signs, Sd), tq.Tables(fv, signs, Sd)
        qb = TI.decode_queries(batch, HQ, D, TI.data_seed(3, layer) + seed)
        q = torch.from_numpy(qb.view(np.int16)).to(dev).view(torch.bfloat16)
        if samples is not None and layer == 0:   # for the CPU baseline: sequence 0 of layer 0
            samples["C3"] = (_bf16_host(kx[0]), _bf16_host(vx[0]), qb[0].copy(),
                             TI.rotation_seed(3, layer) + seed)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        torch.cuda.synchronize()
        ev[0].record()
        tq.quantize_kv(kx.view(-1, D), fk, tk, codes=ck, norms=nk)
        tq.quantize_kv(vx.view(-1, D), fv, tv, codes=cv, norms=nv)
        ev[1].record()
        dec = lambda: tq.attend_decode(q, ck.view(batch, HKV, ntok, rb), nk.view(batch, HKV, ntok, 2),
                                       cv.view(batch, HKV, ntok // 32, 32 * rb),
                                       nv.view(batch, HKV, ntok, 2), seq, fk, tk, fv, tv,
                                       workspace=ws, out=out)
        dec()
        ev[2].record()
        for _ in range(dec_steps):
            dec()
        ev[3].record()
        torch.cuda.synchronize()
        t_q.append(ev[0].elapsed_time(ev[1]) * 1e-3)
        t_d.append(ev[2].elapsed_time(ev[3]) * 1e-3 / dec_steps)
        del kx, vx
    packed = 2 * nvec * (rb + 4)
    td = float(np.mean(t_d))
    return {"workload": f"{n_layers} layers x batch {batch} x {ntok} tokens, 32 q / 8 kv heads, "
                        "head_dim 128, distinct seeds per layer; K and V at 3.5 bits (3/2-bit "
                        "codebook split at 64 + QJL, 60 B per vector with norms), values "
                        "token-sliced",
            "layers": n_layers, "packed_bytes_per_layer": packed,
            "prefill_quantize_tokens_per_s": round(n_layers * batch * ntok / float(np.sum(t_q)), 1),
            "prefill_quantize_ms_per_layer": round(float(np.mean(t_q)) * 1e3, 3),
            "decode_us": round(td * 1e6, 3), "decode_us_min_layer": round(float(np.min(t_d)) * 1e6, 3),
            "decode_us_max_layer": round(float(np.max(t_d)) * 1e6, 3),
            "decode_gbs": round(packed / td / 1e9, 2),
            "decode_pct_hbm_peak": round(100.0 * packed / td / 1e9 / HBM_PEAK_GBS, 2),
            "roofline": _decode_roofline("decode_mx_scan+decode_combine", packed, td)}


def _c4_sparse_v(tq, torch, dev, TI, seed, steps, tau=1e-4, samples=None):
    """Batch 4 x 131072 tokens, 32 q / 8 kv heads; keys at b = 4 with 1% of token positions
    per sequence carrying x10 keys, values at b = 3 (token-sliced).  Decode gated
    (tau = 1e-4) and ungated on the same packed cache, interleaved in blocks of 4 launches
    back to back with HIP events around each block.  skipped_rows = value rows (KV head, token) the gate left unread, counted by the
    kernel on one gated pass; the softmax mass of the rows under tau (from the ungated
    logits) bounds the mass the gate dropped, since a dropped row's running weight
    estimate, at least its final weight, was under tau."""
    batch, ntok = 4, 131072
    fk = tq.Format.uniform(D, 3)
    fv = tq.Format.uniform(D, 2).sliced()
    kx, vx = TI.kv_layer_device(batch, HKV, ntok, D, TI.data_seed(4) + seed, dev, spike_frac=0.01)
    signs, S = tq.make_rotation(D, TI.rotation_seed(4) + seed)
    Sd = torch.from_numpy(S).to(dev)
    tk, tv = tq.Tables(fk, signs, Sd), tq.Tables(fv, signs, Sd)
    qb = TI.decode_queries(batch, HQ, D, TI.data_seed(4) + seed)
    q = torch.from_numpy(qb.view(np.int16)).to(dev).view(torch.bfloat16)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    tq.quantize_kv(kx.view(-1, D), fk, tk)   # warm-up
    torch.cuda.synchronize()
    ev[0].record()
    ck, nk = tq.quantize_kv(kx.view(-1, D), fk, tk)
    ev[1].record()
    cv, nv = tq.quantize_kv(vx.view(-1, D), fv, tv)
    ev[2].record()
    torch.cuda.synchronize()
    t_q = (ev[0].elapsed_time(ev[1]) + ev[1].elapsed_time(ev[2])) * 1e-3
    if samples is not None:   # for the CPU baseline: sequence 0
        samples["C4"] = (_bf16_host(kx[0]), _bf16_host(vx[0]), qb[0].copy(),
                         TI.rotation_seed(4) + seed, tau)
    del kx, vx
    rbk, rbv = fk.record_bytes(), fv.record_bytes()
    ck, nk = ck.view(batch, HKV, ntok, rbk), nk.view(batch, HKV, ntok, 2)
    cv, nv = cv.view(batch, HKV, ntok // 32, 32 * rbv), nv.view(batch, HKV, ntok, 2)
    seq = torch.full((batch,), ntok, dtype=torch.int32, device=dev)
    ws = torch.empty(tq.attend_workspace_bytes(batch, HQ, HKV, ntok, D), dtype=torch.uint8, device=dev)
    out_u = torch.empty((batch, HQ, D), dtype=torch.float32, device=dev)
    out_g = torch.empty_like(out_u)
    dec = lambda t, o, sk=None: tq.attend_decode(q, ck, nk, cv, nv, seq, fk, tk, fv, tv, tau=t,
                                                 skipped=sk, workspace=ws, out=o)
    sk = torch.zeros(1, dtype=torch.int64, device=dev)
    dec(0.0, out_u); dec(tau, out_g, sk)
    torch.cuda.synchronize()
    skipped = int(sk.item())
    out_diff = float((out_g - out_u).abs().max())
    for _ in range(100):   # untimed pairs (~25 ms of decode work): clocks up after the set-up
        dec(0.0, out_u); dec(tau, out_g)
    # per step, 4 ungated then 4 gated decodes back to back between events (as in C3), so
    # that a launch's set-up overlaps the previous decode as in a decode loop
    reps = 4
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        e = ev[i]
        e[0].record()
        for _ in range(reps):
            dec(0.0, out_u)
        e[1].record()
        for _ in range(reps):
            dec(tau, out_g)
        e[2].record()
    torch.cuda.synchronize()
    t_u = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3 / reps
    t_g = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e-3 / reps
    _, lg = tq.attend_decode(q, ck, nk, cv, nv, seq, fk, tk, fv, tv, logits=True, workspace=ws)
    p = torch.softmax(lg.double(), dim=-1)
    below = torch.where(p < tau, p, torch.zeros_like(p)).sum(dim=-1)
    del lg, p
    rows = batch * HKV * ntok
    packed = rows * (rbk + rbv + 8)
    return {"workload": "batch 4 x 131072 tokens, 32 q / 8 kv heads, head_dim 128, 1% of token "
                        "positions with x10 keys; K b=4 (3-bit codebook + QJL), V b=3 (2-bit "
                        "codebook + QJL, token-sliced)",
            "tau": tau, "packed_bytes": packed,
            "decode_us_ungated": round(t_u * 1e6, 3), "decode_us_gated": round(t_g * 1e6, 3),
            "decode_gbs_ungated": round(packed / t_u / 1e9, 2),
            "decode_gbs_gated": round(packed / t_g / 1e9, 2),
            "skipped_rows": skipped, "rows": rows, "skipped_frac": round(skipped / rows, 4),
            "dropped_mass_bound_max": float(below.max()),
            "dropped_mass_bound_mean": float(below.mean()),
            "gated_vs_ungated_out_max_abs": out_diff,
            "quantize_tokens_per_s": round(batch * ntok / t_q, 1),
            "roofline": _decode_roofline("decode_mx_scan+decode_combine (ungated)", packed, t_u)}


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


def _search_timing(tq, torch, dev, TI, reps=2, seed=0, samples=None):
    """Inner-product search on the 10^6 x 200 database (unit vectors, std i^-0.3 per
    coordinate), zero-padded to d = 256 and packed at b = 4; 10^4 queries from the same law,
    top-10.  Times the index build (quantize of the database) and the search of all queries.
    Roofline: the estimator's 2 x 256 multiply-adds per (query, vector) pair (two dot
    products of length d) against the dense fp16 MFMA peak the scan runs on; its operands
    are split into fp16 hi + lo halves, so it issues 5 products where the dot products
    count 2."""
    n_db, n_q, d_in, d, k = 10 ** 6, 10 ** 4, 200, 256, 10
    db_h = TI.search_set(n_db, d_in, seed=TI.data_seed(5) + seed)
    qs_h = TI.search_set(n_q, d_in, seed=TI.data_seed(5) + seed + 1)
    if samples is not None:   # for the CPU baseline: a prefix of the database and queries
        samples["C5"] = (db_h[:100000].copy(), qs_h[:100].copy(), TI.rotation_seed(5) + seed)
    db = torch.from_numpy(db_h).to(dev)
    qs = torch.from_numpy(qs_h).to(dev)
    del db_h, qs_h
    signs, S = tq.make_rotation(d, TI.rotation_seed(5) + seed)
    fmt = tq.Format.uniform(d, BITS)
    tab = tq.Tables(fmt, signs, torch.from_numpy(S).to(dev))
    codes = torch.empty((n_db, fmt.record_bytes()), dtype=torch.uint8, device=dev)
    norms = torch.empty((n_db, 2), dtype=torch.float16, device=dev)
    build = lambda: tq.quantize_kv(db, fmt, tab, codes=codes, norms=norms)
    ws = torch.empty(tq.search_workspace_bytes(n_q, k, n_db, d), dtype=torch.uint8, device=dev)
    search = lambda: tq.ip_search(qs, codes, norms, fmt, tab, k=k, workspace=ws)

    def timed(fn, n_rep=reps, lead=2):
        # `lead` untimed calls are queued first, so that the GPU still has work queued when the
        # first event is recorded and no timed call waits on the host's launch work (which
        # would otherwise count in the short calls)
        fn()
        torch.cuda.synchronize()
        for _ in range(lead):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_rep + 1)]
        for i in range(n_rep):
            ev[i].record(); fn()
        ev[n_rep].record(); torch.cuda.synchronize()
        return float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(n_rep)])) * 1e-3

    tb = timed(build)
    ts = timed(search)
    # recall@10 against the exact top-10 of the unquantized fp32 inner products, all queries
    ids, _ = search()
    hit = 0
    for s0 in range(0, n_q, 500):
        sc = qs[s0:s0 + 500] @ db.T
        ex = torch.topk(sc, k, dim=1).indices
        est = ids[s0:s0 + 500]
        hit += int((est.unsqueeze(2) == ex.unsqueeze(1)).any(dim=2).sum())
        del sc
    recall = hit / (n_q * k)
    # unbatched: one query (and one block of 32) streams the whole packed database
    t1 = timed(lambda: tq.ip_search(qs[:1], codes, norms, fmt, tab, k=k, workspace=ws), n_rep=20)
    t4 = timed(lambda: tq.ip_search(qs[:4], codes, norms, fmt, tab, k=k, workspace=ws), n_rep=20)
    t16 = timed(lambda: tq.ip_search(qs[:16], codes, norms, fmt, tab, k=k, workspace=ws), n_rep=10)
    t20 = timed(lambda: tq.ip_search(qs[:20], codes, norms, fmt, tab, k=k, workspace=ws), n_rep=10)
    t32 = timed(lambda: tq.ip_search(qs[:32], codes, norms, fmt, tab, k=k, workspace=ws), n_rep=10)
    db_bytes = n_db * (fmt.record_bytes() + 4)
    flops = 2.0 * 2 * d * n_db * n_q
    tfs = flops / ts / 1e12
    return {"db_vectors": n_db, "d_in": d_in, "d": d, "queries": n_q, "k": k,
            "recall_at_10": round(recall, 4),
            "recall_reference": "exact top-10 of the fp32 inner products over all 10^6 vectors, "
                                "every query",
            "format": "3-bit codebook + 1 QJL bit (132 B/vector)",
            "index_build_ms": round(tb * 1e3, 3), "index_vectors_per_s": round(n_db / tb, 1),
            "search_ms": round(ts * 1e3, 3), "queries_per_s": round(n_q / ts, 1),
            "one_query_us": round(t1 * 1e6, 2), "one_query_db_gbs": round(db_bytes / t1 / 1e9, 1),
            "one_query_pct_hbm_peak": round(100.0 * db_bytes / t1 / 1e9 / HBM_PEAK_GBS, 2),
            "queries_4_us": round(t4 * 1e6, 2), "queries_4_per_s": round(4 / t4, 1),
            "queries_16_us": round(t16 * 1e6, 2), "queries_16_per_s": round(16 / t16, 1),
            "queries_20_us": round(t20 * 1e6, 2), "queries_20_per_s": round(20 / t20, 1),
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
        print(json.dumps({"search_1m_x_200": _search_timing(tq, torch, dev, TI, seed=args.seed)}),
              flush=True)
        return
    if args.large_batch:
        print(json.dumps({"C3": _c3_layers(tq, torch, dev, TI, args.seed),
                          "C4": _c4_sparse_v(tq, torch, dev, TI, args.seed, args.steps)}), flush=True)
        return
    run = {"C1", "C2", "C3", "C4", "C5"} if args.config == "all" else {args.config}

    line = {
        "metric": "decode-attn packed-KV GB/s & % HBM peak; quantize tokens/s (32K ctx, b=4)",
        "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B-shaped decode layer: batch 1, 32 q / 8 kv heads, "
                               "head_dim 128, 32768 cached tokens, bf16 K/V (per-channel std "
                               "log-uniform [0.5, 8]), b=4 (3-bit codebook + 1 QJL bit) for K "
                               "and V, values token-sliced",
                   "global_batch": BATCH, "seq_len": NTOK, "parallelism": "none (1 GPU)",
                   "seed": args.seed},
    }
    kb = vb = qb = None
    if "C2" in run:
        seed = TI.data_seed(2) + args.seed
        kb, vb, _ = TI.kv_layer(BATCH, HKV, NTOK, D, seed=seed)
        qb = TI.decode_queries(BATCH, HQ, D, seed)
        signs, S = tq.make_rotation(D, TI.rotation_seed(2) + args.seed)
        fmt = tq.Format.uniform(D, BITS)
        fsl = fmt.sliced()
        Sd = torch.from_numpy(S).to(dev)
        tab, tsl = tq.Tables(fmt, signs, Sd), tq.Tables(fsl, signs, Sd)
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
        norms_k = [torch.empty((BATCH, HKV, NTOK, 2), dtype=torch.float16, device=dev) for _ in range(SLOTS)]
        codes_vs = [torch.empty((BATCH, HKV, NTOK // 32, 32 * rb), dtype=torch.uint8, device=dev)
                    for _ in range(SLOTS)]
        norms_v = [torch.empty_like(n) for n in norms_k]
        q = torch.from_numpy(qb.view(np.int16)).to(dev).view(torch.bfloat16)
        seq = torch.full((BATCH,), NTOK, dtype=torch.int32, device=dev)
        ws = torch.zeros(tq.attend_workspace_bytes(BATCH, HQ, HKV, NTOK, D), dtype=torch.uint8, device=dev)
        out = torch.empty((BATCH, HQ, D), dtype=torch.float32, device=dev)

        def quantize(s):
            tq.quantize_kv(ks[s].view(-1, D), fmt, tab, codes=codes_k[s].view(nvec, rb),
                           norms=norms_k[s].view(nvec, 2))

        def quantize_v(s):
            tq.quantize_kv(vs[s].view(-1, D), fsl, tsl, codes=codes_vs[s].view(nvec // 32, 32 * rb),
                           norms=norms_v[s].view(nvec, 2))

        def decode(s):
            tq.attend_decode(q, codes_k[s], norms_k[s], codes_vs[s], norms_v[s], seq, fmt, tab, fsl,
                             tsl, workspace=ws, out=out)

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
        q_launch = float(qk.mean())
        flops_launch = 2.0 * D * D * nvec                         # S r per vector
        q_tfs = flops_launch / q_launch / 1e12
        qtoks = NTOK * BATCH * steps / (qk.sum() + qv.sum())
        copy_gbs = _copy_gbs(torch, dev)
        trafq = _traffic(["compressed_attention_rotate_amd/csrc/tq_quantize_kernel.h"],
                         "quantize_llama8b_32k_traffic.txt")
        trafd = _traffic(["compressed_attention_rotate_amd/csrc/tq_decode_mx.hip",
                          "compressed_attention_rotate_amd/csrc/tq_decode.hip"],
                         "decode_sliced_llama8b_32k_traffic.txt")
        line.update({
            "value": round(decode_gbs, 2),
            "ms_per_step": round(wall / steps * 1e3, 4),
            "decode_pct_hbm_peak": round(100.0 * decode_gbs / HBM_PEAK_GBS, 2),
            "hbm_copy_gbs": round(copy_gbs, 1),
            "decode_pct_copy_bw": round(100.0 * decode_gbs / copy_gbs, 2),
            "decode_us": round(float(dc.mean()) * 1e6, 3),
            "decode_us_median": round(float(np.median(dc)) * 1e6, 3),
            "decode_us_graph_replay": round(_graph_decode_timing(torch, decode) * 1e6, 3),
            "quantize_tokens_per_s": round(qtoks, 1),
            "quantize_k_us_per_launch": round(q_launch * 1e6, 3),
            "quantize_k_us_median": round(float(np.median(qk)) * 1e6, 3),
            "quantize_v_sliced_us_per_launch": round(float(qv.mean()) * 1e6, 3),
            "roofline": {"bound": "mfma", "kernel": "quantize_kernel<128,3,3> (key tensor)",
                         "achieved": round(q_tfs, 3), "peak": FP32_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": round(q_tfs / FP32_MFMA_PEAK_TFS, 4), "traffic": trafq},
            # the same launch against the two other ceilings it could meet: the three fp16
            # products it issues (hi.hi + hi.lo + lo.hi) against the fp16 MFMA peak, and its
            # HBM bytes (rocprof traffic, else the algorithmic bytes) against 8 TB/s
            "roofline_quantize_other": {
                "fp16_mfma_issued_tflops": round(3 * flops_launch / q_launch / 1e12, 3),
                "frac_of_fp16_peak": round(3 * flops_launch / q_launch / 1e12 / FP16_MFMA_PEAK_TFS, 4),
                "hbm_gbs": round((trafq or nvec * (2 * D + rb + 4)) / q_launch / 1e9, 1),
                "frac_of_hbm_peak": round((trafq or nvec * (2 * D + rb + 4)) / q_launch / 1e9 / HBM_PEAK_GBS, 4)},
            "roofline_decode": {"bound": "hbm", "kernel": "decode_mx_scan+decode_combine",
                                "achieved": round(decode_gbs, 2), "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": round(decode_gbs / HBM_PEAK_GBS, 4),
                                "traffic": trafd},
        })
        if not args.no_variants:
            # per-vector value caches of the same slots, for the paths that read that layout
            codes_v = [torch.empty((BATCH, HKV, NTOK, rb), dtype=torch.uint8, device=dev)
                       for _ in range(SLOTS)]
            for s2 in range(SLOTS):
                tq.quantize_kv(vs[s2].view(-1, D), fmt, tab, codes=codes_v[s2].view(nvec, rb),
                               norms=norms_v[s2].view(nvec, 2))
            line["variants"] = {
                name: _variant(tq, torch, dev, ks, vs, q, seq, ws, out, fk, fv, signs, S, steps, nvec)
                for name, fk, fv in (
                    ("b4_per_vector_values", fmt, fmt),
                    ("b4_k_mse_only_v", fmt, tq.Format.uniform(D, BITS, qjl=False)),
                    ("b3.5_kv", tq.Format(D, 3, 2, 64), tq.Format(D, 3, 2, 64)),
                    ("b2.5_kv", tq.Format(D, 2, 1, 64), tq.Format(D, 2, 1, 64)))}
            line["variants"]["paged_b4"] = _paged_timing(tq, torch, dev, ks, q, codes_k, norms_k,
                                                         codes_v, norms_v, seq, ws, out, fmt, tab,
                                                         steps, nvec)
            line["variants"]["prefill_chunk"] = _prefill_timing(tq, torch, dev, ks, vs, fmt, tab)
            line["variants"]["requantize_b4_to_b3"] = _requant_timing(tq, torch, dev, codes_k,
                                                                      norms_k, fmt, tab, signs, S,
                                                                      steps, nvec)
            line["variants"]["decay_24k_b3_8k_b4"] = _decay_timing(
                tq, torch, dev, q, codes_k, norms_k, codes_v, norms_v, seq, fmt, tab, signs, S, steps)
            del codes_v
        del ks, vs, codes_k, codes_vs, norms_k, norms_v, ws
        torch.cuda.empty_cache()
    configs = {}
    samples = None if args.no_cpu_baseline else {}
    if "C1" in run:
        configs["C1"] = _c1_quality(tq, torch, dev, TI, args.seed)
        if samples is not None:
            samples["C1"] = True
    if "C3" in run:
        configs["C3"] = _c3_layers(tq, torch, dev, TI, args.seed, samples=samples)
        torch.cuda.empty_cache()
    if "C4" in run:
        configs["C4"] = _c4_sparse_v(tq, torch, dev, TI, args.seed, min(args.steps, 20),
                                     samples=samples)
        torch.cuda.empty_cache()
    if "C5" in run:
        configs["C5"] = _search_timing(tq, torch, dev, TI, seed=args.seed, samples=samples)
    if configs:
        line["configs"] = configs
    if "C2" in run and not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(kb, vb, qb, TI.rotation_seed(2) + args.seed)
    if samples:
        extra = cpu_baseline_configs(samples, args.seed)
        line.setdefault("cpu_baseline", {"kind": "oracle", "cores": extra["cores"]})
        line["cpu_baseline"]["configs"] = extra["configs"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
