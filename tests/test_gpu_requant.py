"""GPU parity: tq_requantize (temporal decay re-encode, through the C ABI) on records written
by the oracle, against the oracle's requantize of the same bytes, with the windows of the
quantize path: codes bit-exact outside 1e-6 of a boundary, signs outside |u| < 1e-6, the
fp16 norm exact (1e-12 window) and ||r|| within 1e-6 of a midpoint.  The kernel encodes an
fp32 reconstruction; the decisions that leaves near a boundary are recomputed in fp64 from
the stored record."""

import numpy as np
import pytest

import tq_inputs as TI
from oracle import tq_oracle as O
from parity_utils import compare_quantize, oracle_codebooks, oracle_pack_cache, rotations

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import compressed_attention_rotate_amd as tq
    tq.load()
    return torch


def _oracle_requant(rec, nrm, f_in, S_in, f_out, S_out):
    cin, cout = oracle_codebooks(128, f_in.bits_lo, f_in.bits_hi), oracle_codebooks(128, f_out.bits_lo, f_out.bits_hi)
    q = O.requantize(rec, nrm[:, 0], nrm[:, 1], f_in, S_in, *cin, f_out, S_out, *cout)
    q["records"] = O.pack(q["idx"], q["sbit"], f_out)
    q["norms"] = np.stack([q["n16"], q["r16"]], axis=1).astype(np.uint16)
    return q


def _gpu_requant(torch, rec, nrm, f_in, f_out, signs, S_in, S_out, in_place=False, ws_vectors=None):
    import compressed_attention_rotate_amd as tq
    fi, fo = tq.Format(*f_in), tq.Format(*f_out)
    ti = tq.Tables(fi, signs, torch.from_numpy(S_in).cuda())
    to = tq.Tables(fo, signs, torch.from_numpy(S_out).cuda())
    n = rec.shape[0]
    cin = torch.from_numpy(np.ascontiguousarray(rec)).cuda()
    nin = torch.from_numpy(np.ascontiguousarray(nrm).view(np.int16)).cuda().view(torch.float16)
    ws = None
    if ws_vectors is not None:
        ws = torch.empty(ws_vectors * 580, dtype=torch.uint8, device="cuda")
    cnt = torch.zeros(4, dtype=torch.int64, device="cuda")
    if in_place:
        co, no = tq.requantize(cin, nin, fi, ti, fo, to, codes_out=cin, norms_out=nin, counters=cnt,
                               workspace=ws)
        codes = co.view(-1)[: n * fo.record_bytes()].view(n, -1)
    else:
        codes, no = tq.requantize(cin, nin, fi, ti, fo, to, counters=cnt, workspace=ws)
    torch.cuda.synchronize()
    return (codes.cpu().numpy(), no.cpu().view(torch.int16).numpy().view(np.uint16).reshape(n, 2),
            cnt.cpu().numpy())


def _stored(n, f_in, seed, spikes=0.0):
    kb, vb, _ = TI.kv_layer(1, 2, (n + 3) // 4, 128, seed=seed, spike_frac=spikes)
    x = np.concatenate([kb.reshape(-1, 128), vb.reshape(-1, 128)])[:n]
    (signs, S), (gsigns, gS) = rotations(128, seed + 1)
    rec, nrm, _ = oracle_pack_cache(x[None, None], O.Format(*f_in), signs, S, bf16=True)
    return rec[0, 0], nrm[0, 0], (signs, S), (gsigns, gS)


@pytest.mark.parametrize("f_in,f_out", [
    ((128, 3, 3, 128), (128, 2, 2, 128)),                 # b4 -> b3
    ((128, 3, 3, 128), (128, 2, 1, 64)),                  # b4 -> 2.5 bit
    ((128, 3, 2, 64), (128, 1, 1, 128)),                  # 3.5 bit -> b2
    ((128, 3, 3, 128), (128, 2, 2, 128, False)),          # b4 -> MSE-only 2-bit codebook
    ((128, 3, 3, 128, False), (128, 2, 2, 128)),          # MSE-only source
    ((128, 2, 2, 128), (128, 2, 2, 128)),                 # same width (re-sketch)
])
def test_requantize_matches_oracle(torch_gpu, f_in, f_out):
    rec, nrm, (signs, S), (gsigns, gS) = _stored(2999, f_in, 6100)
    (_, S2), (_, gS2) = rotations(128, 6200)
    codes, norms, cnt = _gpu_requant(torch_gpu, rec, nrm, f_in, f_out, gsigns, gS, gS2)
    q = _oracle_requant(rec, nrm, O.Format(*f_in), S, O.Format(*f_out), S2)
    rep = compare_quantize(codes, norms, q, O.Format(*f_out))
    print(f"\n{f_in} -> {f_out}: {rep} counters={cnt}")


def test_requantize_in_place_in_chunks(torch_gpu):
    """codes_out = codes_in and norms_out = norms_in, with a workspace of 700 vectors so the
    call runs in five chunks (the last one ragged)."""
    f_in, f_out = (128, 3, 3, 128), (128, 2, 1, 64)
    rec, nrm, (signs, S), (gsigns, gS) = _stored(3100, f_in, 6300, spikes=0.01)
    codes, norms, _ = _gpu_requant(torch_gpu, rec, nrm, f_in, f_out, gsigns, gS, gS, in_place=True,
                                   ws_vectors=700)
    q = _oracle_requant(rec, nrm, O.Format(*f_in), S, O.Format(*f_out), S)
    compare_quantize(codes, norms, q, O.Format(*f_out))


def test_requantize_full_layer_sampled(torch_gpu):
    """The 32K-token Llama-3.1-8B-shaped layer tensor (262144 vectors) re-encoded b4 -> b3 in
    one call; a seeded sample of rows and the last rows checked against the oracle."""
    torch = torch_gpu
    import compressed_attention_rotate_amd as tq
    kb, _, _ = TI.kv_layer(1, 8, 32768, 128, seed=TI.data_seed(2))
    x = kb.reshape(-1, 128)
    (signs, S), (gsigns, gS) = rotations(128, TI.rotation_seed(2))
    f_in, f_out = tq.Format.uniform(128, 3), tq.Format.uniform(128, 2)
    ti = tq.Tables(f_in, gsigns, torch.from_numpy(gS).cuda())
    to = tq.Tables(f_out, gsigns, torch.from_numpy(gS).cuda())
    xt = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    c4, n4 = tq.quantize_kv(xt, f_in, ti)
    c3, n3 = tq.requantize(c4, n4, f_in, ti, f_out, to)
    torch.cuda.synchronize()
    rows = np.sort(TI.gen(98).choice(x.shape[0], size=3000, replace=False))
    rows = np.concatenate([rows, np.arange(x.shape[0] - 20, x.shape[0])])
    rec = c4.cpu().numpy()[rows]
    nrm = n4.cpu().view(torch.int16).numpy().view(np.uint16)[rows]
    q = _oracle_requant(rec, nrm, O.Format.uniform(128, 3), S, O.Format.uniform(128, 2), S)
    got_c = c3.cpu().numpy()[rows]
    got_n = n3.cpu().view(torch.int16).numpy().view(np.uint16)[rows]
    print("\nfull layer:", compare_quantize(got_c, got_n, q, O.Format.uniform(128, 2)))


def test_requantize_argument_errors(torch_gpu):
    import compressed_attention_rotate_amd as tq
    torch = torch_gpu
    f4, f3 = tq.Format.uniform(128, 3), tq.Format.uniform(128, 2)
    (signs, S), (gsigns, gS) = rotations(128, 3)
    t4 = tq.Tables(f4, gsigns, torch.from_numpy(gS).cuda())
    t3_other = tq.Tables(f3, -gsigns, torch.from_numpy(gS).cuda())
    c = torch.zeros((64, f4.record_bytes()), dtype=torch.uint8, device="cuda")
    nr = torch.zeros((64, 2), dtype=torch.float16, device="cuda")
    with pytest.raises(tq.TQError):
        tq.requantize(c, nr, f4, t4, f3, t3_other)                 # another rotation
    t3 = tq.Tables(f3, gsigns, torch.from_numpy(gS).cuda())
    buf = torch.zeros((64, f4.record_bytes()), dtype=torch.uint8, device="cuda")
    with pytest.raises(tq.TQError):                                # wider records in place
        tq.requantize(buf, nr, f3, t3, f4, t4, codes_out=buf, norms_out=nr)
