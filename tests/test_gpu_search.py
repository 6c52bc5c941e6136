"""GPU parity: tq_ip_search (through the C ABI) against the oracle's estimator.

The returned scores must equal the oracle's estimated inner products of the returned ids
(1e-4 relative to the estimator's absolute-sum scale), the list must be sorted (ties to
the lower id), and no other database vector may beat the k-th returned score by more
than that tolerance (several top-k sets are correct when scores tie within it)."""
import math

import numpy as np
import pytest

import tq_inputs as TI
from oracle import tq_oracle as O
from parity_utils import oracle_quantize, rotations

pytestmark = pytest.mark.gpu
RTOL = 1e-4


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import compressed_attention_rotate_amd as tq
    tq.load()
    return torch


def _oracle_scores(queries, rec, norms, fmt, signs, S):
    """Estimated scores [n_q, n] by explicit dequantization, and the absolute-sum scale of the
    estimator's terms (n16 sum|q_rot c| + gamma r16 sum|S q_rot|) used for the tolerance."""
    cb = O.codebook(fmt.d, fmt.bits_lo)
    idx, sb = O.unpack(rec, fmt)
    xt = O.dequantize(idx, sb, norms[:, 0], norms[:, 1], fmt, signs, S, cb)
    sc = O.search_scores(queries.astype(np.float64), xt)
    qp = np.zeros((len(queries), fmt.d)); qp[:, :queries.shape[1]] = queries
    qr = O.rotate(qp, signs)
    sq = qr @ np.asarray(S, dtype=np.float64).T
    c = O.centroid_values(idx, fmt, cb)
    n16, r16 = O.fp16_value(norms[:, 0]), O.fp16_value(norms[:, 1])
    scale = n16[None, :] * (np.abs(qr) @ np.abs(c).T) + \
        O.gamma(fmt.d) * r16[None, :] * np.abs(sq).sum(axis=1)[:, None]
    return sc, scale


def _check_topk(ids, scores, s_o, tol_o, k):
    for qi in range(ids.shape[0]):
        g, gs = ids[qi], scores[qi]
        assert len(set(g.tolist())) == k
        assert np.all(np.diff(gs) <= 0)
        eq = np.nonzero(np.diff(gs) == 0)[0]
        assert np.all(g[eq] < g[eq + 1]), "equal scores must go to the lower id"
        assert np.all(np.abs(gs - s_o[qi, g]) <= tol_o[qi, g]), "returned scores differ"
        thr = s_o[qi, g[-1]]
        mask = np.ones(s_o.shape[1], dtype=bool); mask[g] = False
        over = s_o[qi, mask] - (thr + tol_o[qi, mask] + tol_o[qi, g[-1]])
        assert np.all(over <= 0), f"query {qi}: a vector outside the list beats the k-th score"


def _gpu_search(torch, queries, rec, norms, fmt_t, gsigns, gS, k):
    import compressed_attention_rotate_amd as tq
    fmt = tq.Format(*fmt_t)
    tab = tq.Tables(fmt, gsigns, torch.from_numpy(gS).cuda())
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ids, sc = tq.ip_search(up(queries.astype(np.float32)), up(rec),
                           up(norms.view(np.int16)).view(torch.float16), fmt, tab, k=k)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), sc.cpu().numpy()


@pytest.mark.parametrize("n_db,n_q,k,bits", [(12000, 37, 10, 3), (6000, 600, 10, 3), (5000, 9, 1, 3),
                                             (5000, 9, 64, 2), (3001, 70, 10, 2)])
def test_search_matches_oracle_estimator(torch_gpu, n_db, n_q, k, bits):
    d_in, d = 200, 256
    db = TI.search_set(n_db, d_in, seed=5001)
    qs = TI.search_set(n_q, d_in, seed=5002)
    (signs, S), (gsigns, gS) = rotations(d, 5500)
    fmt = O.Format.uniform(d, bits)
    qz = oracle_quantize(db, fmt, signs, S)
    ids, sc = _gpu_search(torch_gpu, qs, qz["records"], qz["norms"], (d, bits, bits, d), gsigns, gS, k)
    s_o, scale = _oracle_scores(qs, qz["records"], qz["norms"], fmt, signs, S)
    _check_topk(ids, sc, s_o, RTOL * (np.abs(s_o) + scale), k)
    exact = np.argsort(-(qs.astype(np.float64) @ db.astype(np.float64).T), axis=1, kind="stable")[:, :k]
    print(f"\nn_db={n_db} n_q={n_q} k={k} b={bits + 1}: recall@{k} vs exact {O.recall_at_k(ids, exact):.3f}")


@pytest.fixture(scope="module")
def db_60k():
    """60000 vectors of the search law (200 coordinates, zero-padded to 256), packed at b = 4
    by the oracle."""
    d_in, d = 200, 256
    db = TI.search_set(60000, d_in, seed=5201)
    (signs, S), (gsigns, gS) = rotations(d, 5700)
    fmt = O.Format.uniform(d, 3)
    return db, (signs, S), (gsigns, gS), fmt, oracle_quantize(db, fmt, signs, S)


@pytest.mark.parametrize("n_q,k", [(1, 64), (2, 10), (33, 64)])
def test_search_few_queries_many_splits(torch_gpu, db_60k, n_q, k):
    """Few queries over 60000 vectors: one or two query blocks, so the database is cut into
    58 splits and the merge combines up to 58 x 64 candidates per query."""
    db, (signs, S), (gsigns, gS), fmt, qz = db_60k
    qs = TI.search_set(n_q, db.shape[1], seed=5202)
    ids, sc = _gpu_search(torch_gpu, qs, qz["records"], qz["norms"], (fmt.d, 3, 3, fmt.d), gsigns, gS, k)
    s_o, scale = _oracle_scores(qs, qz["records"], qz["norms"], fmt, signs, S)
    _check_topk(ids, sc, s_o, RTOL * (np.abs(s_o) + scale), k)


@pytest.mark.parametrize("n_db,n_q,k,bits,d,d_in", [(5000, 3, 10, 3, 128, 128), (4000, 4, 16, 2, 128, 100),
                                                    (3000, 1, 5, 1, 128, 128), (6000, 2, 10, 2, 256, 200),
                                                    (2100, 4, 64, 3, 256, 256)])
def test_search_few_queries(torch_gpu, n_db, n_q, k, bits, d, d_in):
    """At most four queries take one block of the few-query matrix-core scan: every supported
    database format against the oracle's estimator."""
    db = TI.search_set(n_db, d_in, seed=5301)
    qs = TI.search_set(n_q, d_in, seed=5302)
    (signs, S), (gsigns, gS) = rotations(d, 5800)
    fmt = O.Format.uniform(d, bits)
    qz = oracle_quantize(db, fmt, signs, S)
    ids, sc = _gpu_search(torch_gpu, qs, qz["records"], qz["norms"], (d, bits, bits, d), gsigns, gS, k)
    s_o, scale = _oracle_scores(qs, qz["records"], qz["norms"], fmt, signs, S)
    _check_topk(ids, sc, s_o, RTOL * (np.abs(s_o) + scale), k)


@pytest.mark.parametrize("n_db,n_q,k,bits,d,d_in", [(900, 13, 7, 3, 256, 200), (1000, 16, 64, 2, 128, 128),
                                                    (9000, 5, 10, 3, 256, 256), (9000, 20, 10, 3, 128, 128),
                                                    (9000, 21, 10, 3, 128, 128)])
def test_search_query_blocks(torch_gpu, n_db, n_q, k, bits, d, d_in):
    """5 to 20 queries take the few-query scan in blocks of four (a ragged last block); a
    database of at most 1024 vectors is one split, so the scan writes the results itself;
    21 queries go to the batched scan."""
    db = TI.search_set(n_db, d_in, seed=5311)
    qs = TI.search_set(n_q, d_in, seed=5312)
    (signs, S), (gsigns, gS) = rotations(d, 5810)
    fmt = O.Format.uniform(d, bits)
    qz = oracle_quantize(db, fmt, signs, S)
    ids, sc = _gpu_search(torch_gpu, qs, qz["records"], qz["norms"], (d, bits, bits, d), gsigns, gS, k)
    s_o, scale = _oracle_scores(qs, qz["records"], qz["norms"], fmt, signs, S)
    _check_topk(ids, sc, s_o, RTOL * (np.abs(s_o) + scale), k)


@pytest.mark.parametrize("n_q", [1, 40])
def test_search_ties_across_splits(torch_gpu, n_q):
    """Exact copies of three vectors at ids spread over a 40000-vector database (so over
    many splits) score identically; the top-k must hold the lowest ids among equal scores,
    on the few-query path (one query) and the batched path (40 queries)."""
    d_in, d, k = 200, 256, 20
    base = TI.search_set(40000, d_in, seed=5401)
    qs = TI.search_set(n_q, d_in, seed=5402)
    # three strong vectors (aligned with the first query) copied to 12 spread ids each
    strong = qs[0][None, :] / np.linalg.norm(qs[0]) * np.array([[1.0], [0.9], [0.8]], dtype=np.float32)
    copies = np.random.default_rng(5403).choice(40000, size=36, replace=False)
    db = base.copy()
    db[copies] = np.repeat(strong, 12, axis=0).astype(np.float32)
    (signs, S), (gsigns, gS) = rotations(d, 5900)
    fmt = O.Format.uniform(d, 3)
    qz = oracle_quantize(db, fmt, signs, S)
    ids, sc = _gpu_search(torch_gpu, qs, qz["records"], qz["norms"], (d, 3, 3, d), gsigns, gS, k)
    s_o, scale = _oracle_scores(qs, qz["records"], qz["norms"], fmt, signs, S)
    _check_topk(ids, sc, s_o, RTOL * (np.abs(s_o) + scale), k)
    # query 0: the 12 copies of the strongest vector first (ascending ids), then the
    # lowest 8 ids of the second one
    groups = [np.sort(copies[12 * j:12 * (j + 1)]) for j in range(3)]
    np.testing.assert_array_equal(ids[0, :12], groups[0])
    np.testing.assert_array_equal(ids[0, 12:20], groups[1][:8])
    assert np.all(sc[0, :12] == sc[0, 0]) and np.all(sc[0, 12:20] == sc[0, 12])


@pytest.mark.parametrize("n_db,n_q,k,bits,d_in", [(4100, 45, 10, 3, 128), (2500, 33, 5, 2, 100),
                                                  (3000, 20, 16, 1, 128)])
def test_search_d128(torch_gpu, n_db, n_q, k, bits, d_in):
    """d = 128 databases (1, 2 and 3 codebook bits), queries of d_in <= 128 coordinates."""
    d = 128
    db = TI.search_set(n_db, d_in, seed=5101)
    qs = TI.search_set(n_q, d_in, seed=5102)
    (signs, S), (gsigns, gS) = rotations(d, 5600)
    fmt = O.Format.uniform(d, bits)
    qz = oracle_quantize(db, fmt, signs, S)
    ids, sc = _gpu_search(torch_gpu, qs, qz["records"], qz["norms"], (d, bits, bits, d), gsigns, gS, k)
    s_o, scale = _oracle_scores(qs, qz["records"], qz["norms"], fmt, signs, S)
    _check_topk(ids, sc, s_o, RTOL * (np.abs(s_o) + scale), k)


def test_full_size_search_complete_for_sampled_queries(torch_gpu):
    """10^6 x 200 database (unit-normalized, std i^-0.3), 10^4 queries, b = 4, top-10.
    The oracle quantizes all 10^6 vectors (in a pool of worker processes that never touch
    the GPU) and scores them for 12 sampled queries; the GPU searches those same packed
    bytes for all 10^4 queries.  For each sampled query: the returned scores equal the
    oracle's within the bar, the list is sorted with ties to the lower id, and no vector of
    the whole database beats the k-th score by more than the bar."""
    import multiprocessing as mp
    import os
    import compressed_attention_rotate_amd as tq
    from parity_utils import oracle_search_chunk
    torch = torch_gpu
    d_in, d, k, n_db, n_q = 200, 256, 10, 10 ** 6, 10 ** 4
    db = TI.search_set(n_db, d_in, seed=TI.data_seed(5))
    qs = TI.search_set(n_q, d_in, seed=TI.data_seed(5) + 1)
    sample_q = np.sort(TI.gen(77).choice(n_q, size=12, replace=False))
    step = 1 << 16
    jobs = [(db[s:s + step], qs[sample_q], d, 3, TI.rotation_seed(5)) for s in range(0, n_db, step)]
    workers = max(1, min(12, (os.cpu_count() or 2) - 1))
    with mp.get_context("spawn").Pool(workers) as pool:
        parts = pool.map(oracle_search_chunk, jobs)
    rec = np.concatenate([p[0] for p in parts])
    nrm = np.concatenate([p[1] for p in parts])
    s_o = np.concatenate([p[2] for p in parts], axis=1)
    tol = RTOL * (np.abs(s_o) + np.concatenate([p[3] for p in parts], axis=1))
    (_, _), (gsigns, gS) = rotations(d, TI.rotation_seed(5))
    fmt = tq.Format.uniform(d, 3)
    tab = tq.Tables(fmt, gsigns, torch.from_numpy(gS).cuda())
    codes = torch.from_numpy(rec).cuda()
    norms = torch.from_numpy(nrm.view(np.int16)).cuda().view(torch.float16)
    ids, sc = tq.ip_search(torch.from_numpy(qs).cuda(), codes, norms, fmt, tab, k=k)
    torch.cuda.synchronize()
    ids, sc = ids.cpu().numpy()[sample_q], sc.cpu().numpy()[sample_q]
    _check_topk(ids, sc, s_o, tol, k)
    print(f"\nfull size: {len(sample_q)} sampled queries checked against all {n_db} vectors")


def test_full_size_search_recall_against_exact(torch_gpu):
    """The product path at full size (GPU index build, then GPU search of 10^4 queries):
    recall@10 of the estimated top-10 against the exact fp32 top-10 (inner products in fp64
    over the 200-d inputs; 163.com explainer, section "向量搜索", rates the method by this
    recall) on 200 sampled queries."""
    import compressed_attention_rotate_amd as tq
    torch = torch_gpu
    d_in, d, k = 200, 256, 10
    db = TI.search_set(10 ** 6, d_in, seed=TI.data_seed(5))
    qs = TI.search_set(10 ** 4, d_in, seed=TI.data_seed(5) + 1)
    fmt = tq.Format.uniform(d, 3)
    tab = tq.Tables.from_seed(fmt, TI.rotation_seed(5))
    codes, norms = tq.quantize_kv(torch.from_numpy(db).cuda(), fmt, tab)
    ids, _ = tq.ip_search(torch.from_numpy(qs).cuda(), codes, norms, fmt, tab, k=k)
    torch.cuda.synchronize()
    ids = ids.cpu().numpy()
    sample_q = np.sort(TI.gen(78).choice(10 ** 4, size=200, replace=False))
    q64 = qs[sample_q].astype(np.float64)
    exact = np.empty((len(sample_q), k), np.int64)
    best = np.full((len(sample_q), 0), 0.0)
    cand_ids = np.zeros((len(sample_q), 0), np.int64)
    for s in range(0, len(db), 1 << 17):
        sc = q64 @ db[s:s + (1 << 17)].astype(np.float64).T
        top = np.argpartition(-sc, k, axis=1)[:, :k]
        cand_ids = np.concatenate([cand_ids, top + s], axis=1)
        best = np.concatenate([best, np.take_along_axis(sc, top, axis=1)], axis=1)
    for i in range(len(sample_q)):
        order = np.lexsort((cand_ids[i], -best[i]))[:k]
        exact[i] = cand_ids[i][order]
    rec = O.recall_at_k(ids[sample_q], exact)
    print(f"\nfull size: recall@10 vs exact fp32 on {len(sample_q)} queries {rec:.3f}")
    assert rec >= 0.5
