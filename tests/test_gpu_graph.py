"""GPU: the quantize and decode entry points capture into a HIP graph (they allocate, set
memory and synchronize nothing), and every replay gives the eager results bit for bit.
Replays are separated by eager work on the same buffers, as a serving loop would."""
import numpy as np
import pytest

import tq_inputs as TI
from parity_utils import rotations

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import compressed_attention_rotate_amd as tq
    tq.load()
    return torch


def test_quantize_and_decode_replay_in_a_graph(torch_gpu):
    import compressed_attention_rotate_amd as tq
    torch = torch_gpu
    dev = torch.device("cuda:0")
    d, hq, hkv, n = 128, 8, 2, 1000
    kb, vb, _ = TI.kv_layer(1, hkv, n, d, seed=4401)
    qb = TI.decode_queries(1, hq, d, 4401)
    (signs, S), (gsigns, gS) = rotations(d, 4402)
    fmt = tq.Format.uniform(d, 3)
    tab = tq.Tables(fmt, gsigns, torch.from_numpy(gS).to(dev))
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    xk, xv, q = bf(kb).view(-1, d), bf(vb).view(-1, d), bf(qb)
    rb = fmt.record_bytes()
    ck = torch.empty((hkv * n, rb), dtype=torch.uint8, device=dev)
    cv = torch.empty_like(ck)
    nk = torch.empty((hkv * n, 2), dtype=torch.float16, device=dev)
    nv = torch.empty_like(nk)
    seq = torch.full((1,), n, dtype=torch.int32, device=dev)
    ws = torch.empty(tq.attend_workspace_bytes(1, hq, hkv, n, d), dtype=torch.uint8, device=dev)
    out = torch.empty((1, hq, d), dtype=torch.float32, device=dev)

    def step():
        tq.quantize_kv(xk, fmt, tab, codes=ck, norms=nk)
        tq.quantize_kv(xv, fmt, tab, codes=cv, norms=nv)
        tq.attend_decode(q, ck.view(1, hkv, n, rb), nk.view(1, hkv, n, 2), cv.view(1, hkv, n, rb),
                         nv.view(1, hkv, n, 2), seq, fmt, tab, workspace=ws, out=out)

    step()
    torch.cuda.synchronize()
    ref_out, ref_ck, ref_nk = out.clone(), ck.clone(), nk.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        out.fill_(float("nan"))
        ck.zero_()
        nk.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ck, ref_ck), f"replay {r}: codes differ"
        assert torch.equal(nk.view(torch.int16), ref_nk.view(torch.int16)), f"replay {r}: norms differ"
        assert torch.equal(out, ref_out), f"replay {r}: decode output differs"
        step()                              # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)
