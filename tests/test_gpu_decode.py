"""GPU parity: tq_attend_decode (through the C ABI) on packed caches written by the oracle,
against the oracle's explicit dequantization + textbook softmax attention of the same
bytes.  Logits within 1e-4 relative to their absolute-sum scale; outputs (fp32) within
2e-3 max-abs; Sparse-V gated output within 5e-3 of the ungated oracle."""
import math

import numpy as np
import pytest

import tq_inputs as TI
from oracle import tq_oracle as O
from parity_utils import oracle_decode, oracle_pack_cache, rotations

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


def _gpu_decode(torch, q_np, q_dtype, rk, nk, rv, nv, seq_lens, fk, fv, signs_k, S_k, signs_v,
                S_v, tau=0.0, logits=True):
    import compressed_attention_rotate_amd as tq
    fmt_k, fmt_v = tq.Format(*fk), tq.Format(*fv)
    tk = tq.Tables(fmt_k, signs_k, torch.from_numpy(S_k).cuda())
    tv = tq.Tables(fmt_v, signs_v, torch.from_numpy(S_v).cuda())
    if q_dtype == "bf16":
        q = torch.from_numpy(q_np.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        q = torch.from_numpy(np.ascontiguousarray(q_np, dtype=np.float32)).cuda()
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    sk = torch.zeros(1, dtype=torch.int64, device="cuda")
    res = tq.attend_decode(q, to_dev(rk), to_dev(nk.view(np.int16)).view(torch.float16), to_dev(rv),
                           to_dev(nv.view(np.int16)).view(torch.float16),
                           to_dev(np.asarray(seq_lens, dtype=np.int32)), fmt_k, tk, fmt_v, tv,
                           tau=tau, logits=logits, skipped=sk)
    torch.cuda.synchronize()
    out, lg = res if logits else (res, None)
    return out.cpu().numpy(), (lg.cpu().numpy() if logits else None), int(sk.item())


def _compare(out_g, lg_g, out_o, lg_o, sc_o, seq_lens, atol=OUT_ATOL):
    worst = 0.0
    for (bi, h), lo in lg_o.items():
        L = int(seq_lens[bi])
        err = np.abs(lg_g[bi, h, :L] - lo)
        bound = LOGIT_RTOL * (np.abs(lo) + sc_o[(bi, h)])
        assert np.all(err <= bound), f"logits differ (b={bi}, h={h}): max ratio {np.max(err / bound)}"
        worst = max(worst, float(np.max(err / bound)) if L else 0.0)
    dmax = float(np.max(np.abs(out_g - out_o)))
    assert dmax <= atol, f"outputs differ by {dmax}"
    return worst, dmax


def _case(torch, batch, hq, hkv, ntok, seq_lens, fk, fv, seed, q_dtype="bf16", spikes=0.0,
          tau=0.0, atol=OUT_ATOL):
    d = 128
    kb, vb, _ = TI.kv_layer(batch, hkv, ntok, d, seed=seed, spike_frac=spikes)
    q_bits = TI.decode_queries(batch, hq, d, seed)
    (signs, S), (gsigns, gS) = rotations(d, seed + 500000)
    rk, nk, _ = oracle_pack_cache(kb, O.Format(*fk), signs, S, bf16=True)
    rv, nv, _ = oracle_pack_cache(vb, O.Format(*fv), signs, S, bf16=True)
    q64 = TI.bf16_to_f64(q_bits)
    out_g, lg_g, skipped = _gpu_decode(torch, q_bits, q_dtype, rk, nk, rv, nv, seq_lens, fk, fv,
                                       gsigns, gS, gsigns, gS, tau=tau)
    out_o, lg_o, sc_o, dr, dm = oracle_decode(q64, rk, nk, rv, nv, seq_lens, O.Format(*fk),
                                              O.Format(*fv), signs, S, signs, S,
                                              1 / math.sqrt(d), 0.0)
    worst, dmax = _compare(out_g, lg_g, out_o, lg_o, sc_o, seq_lens, atol)
    print(f"\nb={batch} hq={hq} hkv={hkv} L={seq_lens} K{fk} V{fv} tau={tau}: logit err/bound "
          f"{worst:.3g}, out max|diff| {dmax:.3g}, skipped rows {skipped}")
    return out_g, out_o, skipped


def test_llama_layer_shape_b4(torch_gpu):
    _case(torch_gpu, 1, 32, 8, 2048, [2000], (128, 3, 3, 128), (128, 3, 3, 128), 2000)


def test_ragged_batch_and_empty_sequences(torch_gpu):
    _case(torch_gpu, 4, 8, 2, 700, [700, 0, 1, 333], (128, 3, 3, 128), (128, 3, 3, 128), 2100)


def test_mixed_width_b3_5(torch_gpu):
    _case(torch_gpu, 2, 32, 8, 1100, [1100, 1000], (128, 3, 2, 64), (128, 3, 2, 64), 3000)


def test_asymmetric_kv_and_group_sizes(torch_gpu):
    _case(torch_gpu, 1, 8, 8, 900, [900], (128, 3, 3, 128), (128, 2, 2, 128), 4000)     # G = 1
    _case(torch_gpu, 1, 8, 4, 900, [877], (128, 2, 2, 128), (128, 2, 2, 128), 4001)     # G = 2
    _case(torch_gpu, 1, 16, 2, 600, [600], (128, 1, 1, 128), (128, 1, 1, 128), 4002)    # G = 8


def test_mse_only_values(torch_gpu):
    """Values stored without QJL sign words (MSE-only), keys with them: every value width,
    the mixed split, group sizes 1 / 2 / 4 / 8, a ragged batch and the Sparse-V gate."""
    _case(torch_gpu, 2, 32, 8, 1300, [1300, 517], (128, 3, 3, 128), (128, 3, 3, 128, False), 4100)
    _case(torch_gpu, 1, 8, 8, 700, [700], (128, 3, 3, 128), (128, 2, 2, 128, False), 4101)   # G = 1
    _case(torch_gpu, 1, 8, 4, 640, [601], (128, 2, 2, 128), (128, 2, 2, 128, False), 4102)   # G = 2
    _case(torch_gpu, 1, 16, 2, 500, [500], (128, 1, 1, 128), (128, 1, 1, 128, False), 4103)  # G = 8
    _case(torch_gpu, 2, 32, 8, 900, [900, 0], (128, 3, 2, 64), (128, 3, 2, 64, False), 4104)
    _, _, skipped = _case(torch_gpu, 1, 32, 8, 4096, [4096], (128, 3, 3, 128),
                          (128, 3, 3, 128, False), 4105, spikes=0.01, tau=1e-4, atol=5e-3)
    assert skipped > 0


@pytest.mark.parametrize("fk,fv,hq,hkv,seed", [
    ((128, 2, 2, 128), (128, 1, 1, 128), 32, 8, 4200),            # K b3 / V b2
    ((128, 3, 2, 32), (128, 3, 2, 32), 32, 8, 4201),              # 3.25 bit
    ((128, 2, 1, 32), (128, 2, 1, 32), 16, 8, 4202),              # 2.25 bit, G = 2
    ((128, 2, 1, 64), (128, 2, 1, 64), 32, 8, 4203),              # 2.5 bit
    ((128, 2, 1, 64), (128, 2, 1, 64, False), 8, 8, 4204),        # 2.5 bit, MSE-only V, G = 1
    ((128, 2, 1, 96), (128, 2, 1, 96), 32, 4, 4205),              # 2.75 bit, G = 8
    ((128, 3, 3, 128), (128, 2, 1, 64), 32, 8, 4206),             # K b4 / V b2.5
    ((128, 3, 2, 64), (128, 2, 1, 64), 32, 8, 4207),              # K b3.5 / V b2.5
    ((128, 3, 2, 64), (128, 2, 2, 128, False), 32, 8, 4208),      # K b3.5 / V b3 MSE-only
])
def test_channel_group_bit_allocations(torch_gpu, fk, fv, hq, hkv, seed):
    """Two-group bit allocations (codebook widths below / above a split at a 32-coordinate
    block boundary of the rotated vector) for keys and values, incl. the 2.5-bit setting."""
    _case(torch_gpu, 2, hq, hkv, 777, [777, 430], fk, fv, seed)


def test_single_head_64_queries(torch_gpu):
    """One KV head, d = 128, 4096 keys/values N(0,1) fp32 with 4 channels x20, 64 queries,
    b = 3 (2-bit codebook + 1 QJL bit): 64 query heads sharing one KV head."""
    torch = torch_gpu
    k, v, q, _ = TI.c1_inputs(seed=1000)
    d = 128
    (signs, S), (gsigns, gS) = rotations(d, TI.rotation_seed(1))
    fmt = O.Format(128, 2, 2, 128)
    rk, nk, _ = oracle_pack_cache(k.astype(np.float64)[None, None], fmt, signs, S)
    rv, nv, _ = oracle_pack_cache(v.astype(np.float64)[None, None], fmt, signs, S)
    q3 = q[None]                                                       # [1, 64, 128]
    out_g, lg_g, _ = _gpu_decode(torch, q3, "f32", rk, nk, rv, nv, [4096], (128, 2, 2, 128),
                                 (128, 2, 2, 128), gsigns, gS, gsigns, gS)
    out_o, lg_o, sc_o, _, _ = oracle_decode(q3.astype(np.float64), rk, nk, rv, nv, [4096], fmt, fmt,
                                            signs, S, signs, S, 1 / math.sqrt(d))
    worst, dmax = _compare(out_g, lg_g, out_o, lg_o, sc_o, [4096])
    print(f"\nsingle head: logit err/bound {worst:.3g}, out max|diff| {dmax:.3g}")


def test_sparse_v_gate_with_spikes(torch_gpu):
    """Keys with 1% x10 norm spikes, K b = 4 / V b = 3, gate tau = 1e-4: the gated GPU output
    stays within 5e-3 of the ungated oracle and reads fewer value rows."""
    out_g, out_o, skipped = _case(torch_gpu, 2, 32, 8, 4096, [4096, 3000], (128, 3, 3, 128),
                                  (128, 2, 2, 128), 5000, spikes=0.01, tau=1e-4, atol=5e-3)
    assert skipped > 0


def test_full_context_llama_layer(torch_gpu):
    """Full 32768-token cache, 32 query / 8 KV heads, b = 4, launched as bench.py times it;
    every head checked."""
    _case(torch_gpu, 1, 32, 8, 32768, [32768], (128, 3, 3, 128), (128, 3, 3, 128), TI.data_seed(2))


def test_workspace_reuse(torch_gpu):
    """Calls that reuse one workspace (holding whatever the previous call left), with
    different shapes and lengths, must equal calls on fresh workspaces bit for bit."""
    import compressed_attention_rotate_amd as tq
    torch = torch_gpu
    d, seed = 128, TI.data_seed(2) + 31
    fmt = tq.Format.uniform(d, 3)
    (signs, S), (gsigns, gS) = rotations(d, seed + 500000)
    tab = tq.Tables(fmt, gsigns, torch.from_numpy(gS).cuda())
    cases = [(1, 32, 8, 4096, [4096]), (2, 8, 2, 3000, [3000, 17]), (1, 32, 8, 4096, [1000]),
             (3, 16, 4, 700, [0, 700, 333])]
    ws_bytes = max(tq.attend_workspace_bytes(b, hq, hkv, n) for b, hq, hkv, n, _ in cases)
    ws = torch.full((ws_bytes,), 0x7F, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for b, hq, hkv, n, lens in cases:
            kb, vb, _ = TI.kv_layer(b, hkv, n, d, seed=seed + n)
            q = torch.from_numpy(TI.decode_queries(b, hq, d, seed + n).view(np.int16)).cuda() \
                .view(torch.bfloat16)
            ck, nk = tq.quantize_kv(torch.from_numpy(kb.view(np.int16)).cuda()
                                    .view(torch.bfloat16).view(-1, d), fmt, tab)
            cv, nv = tq.quantize_kv(torch.from_numpy(vb.view(np.int16)).cuda()
                                    .view(torch.bfloat16).view(-1, d), fmt, tab)
            rb = fmt.record_bytes()
            args = (q, ck.view(b, hkv, n, rb), nk.view(b, hkv, n, 2), cv.view(b, hkv, n, rb),
                    nv.view(b, hkv, n, 2), torch.tensor(lens, dtype=torch.int32, device="cuda"),
                    fmt, tab)
            shared = tq.attend_decode(*args, workspace=ws).clone()
            fresh = tq.attend_decode(*args)
            torch.cuda.synchronize()
            assert torch.equal(shared, fresh), f"shape {(b, hq, hkv, n, lens)} rep {rep}"


def _full_size_sampled(torch, batch, hq, hkv, ntok, fk, fv, seed, spikes, tau, units, sliced=False):
    """Full-size decode on the GPU with sampled oracle checks.  The GPU quantizes the whole
    cache (product path); for each sampled (batch, KV head) unit the records are replaced by
    the oracle's own packing of the same inputs, so the GPU decodes, for those heads, exactly
    the bytes the oracle decodes.  Logits of the unit's query heads within the logit bar,
    ungated outputs within 2e-3, gated outputs (tau > 0) within 5e-3 of the ungated oracle."""
    import compressed_attention_rotate_amd as tq
    d, G = 128, hq // hkv
    kb, vb, _ = TI.kv_layer(batch, hkv, ntok, d, seed=seed, spike_frac=spikes)
    q_bits = TI.decode_queries(batch, hq, d, seed)
    (signs, S), (gsigns, gS) = rotations(d, seed + 500000)
    fmt_k, fmt_v = tq.Format(*fk), tq.Format(*fv, layout=1 if sliced else 0)
    Sd = torch.from_numpy(gS).cuda()
    tk, tv = tq.Tables(fmt_k, gsigns, Sd), tq.Tables(fmt_v, gsigns, Sd)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    rbk, rbv = fmt_k.record_bytes(), fmt_v.record_bytes()
    ck, nk = tq.quantize_kv(bf(kb).view(-1, d), fmt_k, tk)
    cv, nv = tq.quantize_kv(bf(vb).view(-1, d), fmt_v, tv)
    ck, nk = ck.view(batch, hkv, ntok, rbk), nk.view(batch, hkv, ntok, 2)
    cv = cv.view(batch, hkv, ntok // 32, 32 * rbv) if sliced else cv.view(batch, hkv, ntok, rbv)
    nv = nv.view(batch, hkv, ntok, 2)
    oracle = {}
    for bi, kh in units:
        rk, nko, _ = oracle_pack_cache(kb[bi:bi + 1, kh:kh + 1], O.Format(*fk), signs, S, bf16=True)
        rv, nvo, _ = oracle_pack_cache(vb[bi:bi + 1, kh:kh + 1], O.Format(*fv), signs, S, bf16=True)
        ck[bi, kh] = torch.from_numpy(np.ascontiguousarray(rk[0, 0])).cuda()
        rv_dev = O.tiles_from_records(rv[0, 0], O.Format(*fv)) if sliced else rv[0, 0]
        cv[bi, kh] = torch.from_numpy(np.ascontiguousarray(rv_dev)).cuda()
        nk[bi, kh] = torch.from_numpy(np.ascontiguousarray(nko[0, 0]).view(np.int16)).cuda().view(torch.float16)
        nv[bi, kh] = torch.from_numpy(np.ascontiguousarray(nvo[0, 0]).view(np.int16)).cuda().view(torch.float16)
        oracle[(bi, kh)] = (rk, nko, rv, nvo)
    q = bf(q_bits)
    seq = torch.full((batch,), ntok, dtype=torch.int32, device="cuda")
    out_u, lg = tq.attend_decode(q, ck, nk, cv, nv, seq, fmt_k, tk, fmt_v, tv, logits=True)
    sk = torch.zeros(1, dtype=torch.int64, device="cuda")
    out_g = tq.attend_decode(q, ck, nk, cv, nv, seq, fmt_k, tk, fmt_v, tv, tau=tau, skipped=sk) \
        if tau > 0 else None
    torch.cuda.synchronize()
    q64 = TI.bf16_to_f64(q_bits)
    for (bi, kh), (rk, nko, rv, nvo) in oracle.items():
        hs = slice(kh * G, (kh + 1) * G)
        out_o, lg_o, sc_o, _, _ = oracle_decode(
            q64[bi:bi + 1, hs], rk, nko, rv, nvo, [ntok], O.Format(*fk), O.Format(*fv),
            signs, S, signs, S, 1 / math.sqrt(d), 0.0)
        lg_g = lg[bi:bi + 1, hs].cpu().numpy()
        worst, dmax = _compare(out_u[bi:bi + 1, hs].cpu().numpy(), lg_g, out_o, lg_o, sc_o, [ntok])
        msg = f"\nunit (b={bi}, kv={kh}) of {batch}x{ntok}: logit err/bound {worst:.3g}, out max|diff| {dmax:.3g}"
        if out_g is not None:
            _, _, _, drops, mass = oracle_decode(
                q64[bi:bi + 1, hs], rk, nko, rv, nvo, [ntok], O.Format(*fk), O.Format(*fv),
                signs, S, signs, S, 1 / math.sqrt(d), tau)
            gmax = float(np.max(np.abs(out_g[bi:bi + 1, hs].cpu().numpy() - out_o)))
            assert gmax <= 5e-3, f"gated output differs from the ungated oracle by {gmax}"
            msg += (f", gated vs ungated oracle {gmax:.3g}, rows skipped (whole batch) "
                    f"{int(sk.item())}, oracle drops {sum(drops.values())} mass "
                    f"{max(mass.values()):.3g}")
        print(msg)
    return int(sk.item())


def test_full_size_batch16_mixed_width(torch_gpu):
    """Batch 16 x 32768 tokens of the Llama-3.1-8B layer, b = 3.5 (3-bit codebook on rotated
    coordinates 0-63, 2-bit on 64-127, + QJL) for K and V: the GPU decodes the whole batch;
    two sampled (batch, KV head) units are checked against the oracle."""
    _full_size_sampled(torch_gpu, 16, 32, 8, 32768, (128, 3, 2, 64), (128, 3, 2, 64),
                       TI.data_seed(3), 0.0, 0.0, [(11, 2), (0, 7)])


def test_full_size_long_context_sparse_v(torch_gpu):
    """Batch 4 x 131072 tokens, 1% of token positions with x10 keys, K b = 4, V b = 3,
    Sparse-V gate tau = 1e-4: the GPU decodes the whole batch gated and ungated; one sampled
    (batch, KV head) unit is checked against the oracle, and the gate skips rows."""
    skipped = _full_size_sampled(torch_gpu, 4, 32, 8, 131072, (128, 3, 3, 128), (128, 2, 2, 128),
                                 TI.data_seed(4), 0.01, 1e-4, [(2, 5)])
    assert skipped > 0


def test_full_size_batch16_mixed_width_sliced(torch_gpu):
    """The batch-16 layer of 3.5-bit K and V as the benchmark decodes it: values token-sliced
    (the block-scaled scan); two sampled (batch, KV head) units against the oracle."""
    _full_size_sampled(torch_gpu, 16, 32, 8, 32768, (128, 3, 2, 64), (128, 3, 2, 64),
                       TI.data_seed(3) + 1, 0.0, 0.0, [(5, 1), (15, 6)], sliced=True)


def test_full_size_long_context_sparse_v_sliced(torch_gpu):
    """Batch 4 x 131072 tokens with 1% x10 keys, K b = 4, V b = 3 token-sliced, gated
    (tau = 1e-4) and ungated, as the benchmark decodes it; one sampled unit against the
    oracle, and the gate skips rows."""
    skipped = _full_size_sampled(torch_gpu, 4, 32, 8, 131072, (128, 3, 3, 128), (128, 2, 2, 128),
                                 TI.data_seed(4) + 1, 0.01, 1e-4, [(1, 3)], sliced=True)
    assert skipped > 0
