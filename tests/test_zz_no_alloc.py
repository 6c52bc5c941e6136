"""GPU: tq_attend_decode_noalloc (split partials in the library's per-GPU device array, no
allocation) against tq_attend_decode with a caller workspace: the same kernels and plan, so
outputs, logits and skip counts must be identical.  Two calls in a row, the second with a
smaller input, for per-vector and token-sliced values; a shape whose partials exceed the
array is refused."""
import ctypes

import numpy as np
import pytest

import tq_inputs as TI

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tq_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import compressed_attention_rotate_amd as tq
    tq.load()
    return torch, tq


def _cache(torch, tq, batch, hq, hkv, cap, fk, fv, tk, tv, seed):
    kb, vb, _ = TI.kv_layer(batch, hkv, cap, 128, seed=seed)
    qb = TI.decode_queries(batch, hq, 128, seed)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    ck, nk = tq.quantize_kv(bf(kb).view(-1, 128), fk, tk)
    cv, nv = tq.quantize_kv(bf(vb).view(-1, 128), fv, tv)
    rbk, rbv = fk.record_bytes(), fv.record_bytes()
    cv_shape = (batch, hkv, cap // 32, 32 * rbv) if fv.layout == 1 else (batch, hkv, cap, rbv)
    return (bf(qb), ck.view(batch, hkv, cap, rbk), nk.view(batch, hkv, cap, 2), cv.view(*cv_shape),
            nv.view(batch, hkv, cap, 2))


@pytest.mark.parametrize("sliced", [False, True])
def test_noalloc_matches_workspace_entry_point(tq_gpu, sliced):
    torch, tq = tq_gpu
    fk = tq.Format.uniform(128, 3)
    fv = fk.sliced() if sliced else fk
    tk = tq.Tables.from_seed(fk, 4711)
    tv = tq.Tables(fv, tk.signs, tk.S)
    tau = 1e-4 if sliced else 0.0
    for (batch, hq, hkv, cap, lens, seed) in ((2, 32, 8, 4096, [4096, 2917], 31), (1, 8, 2, 512, [300], 32)):
        print(f"noalloc sliced={sliced} batch={batch} hq={hq} hkv={hkv} cap={cap} lens={lens}", flush=True)
        q, ck, nk, cv, nv = _cache(torch, tq, batch, hq, hkv, cap, fk, fv, tk, tv, seed)
        seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
        sk_ref = torch.zeros(1, dtype=torch.int64, device="cuda")
        out_ref, lg_ref = tq.attend_decode(q, ck, nk, cv, nv, seq, fk, tk, fv, tv, tau=tau, logits=True,
                                           skipped=sk_ref)
        out = torch.full((batch, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
        lg = torch.zeros((batch, hq, cap), dtype=torch.float32, device="cuda")
        sk = torch.zeros(1, dtype=torch.int64, device="cuda")
        tq.attend_decode_noalloc(q, ck, nk, cv, nv, seq, fk, tk, out, fv, tv, tau=tau, logits=lg, skipped=sk)
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref)
        for b, L in enumerate(lens):
            assert torch.equal(lg[b, :, :L], lg_ref[b, :, :L])
        assert int(sk.item()) == int(sk_ref.item())


def test_noalloc_refuses_partials_beyond_its_array(tq_gpu):
    torch, tq = tq_gpu
    batch, hq, hkv, cap = 128, 64, 16, 32
    assert tq.attend_workspace_bytes(batch, hq, hkv, cap) > 8 << 20
    fk = tq.Format.uniform(128, 3)
    tk = tq.Tables.from_seed(fk, 4712)
    rb = fk.record_bytes()
    q = torch.zeros((batch, hq, 128), dtype=torch.bfloat16, device="cuda")
    ck = torch.zeros((batch, hkv, cap, rb), dtype=torch.uint8, device="cuda")
    nk = torch.zeros((batch, hkv, cap, 2), dtype=torch.float16, device="cuda")
    seq = torch.zeros(batch, dtype=torch.int32, device="cuda")
    out = torch.zeros((batch, hq, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(tq.TQError) as err:
        tq.attend_decode_noalloc(q, ck, nk, ck, nk, seq, fk, tk, out)
    assert err.value.code == -6   # TQ_ERR_WORKSPACE
    assert torch.count_nonzero(out).item() == 0
