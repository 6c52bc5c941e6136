"""GPU parity: tq_quantize_kv (through the C ABI) against the CPU oracle on the same
seeded inputs.  Bit-exact packed codes and signs outside the ambiguity windows."""
import numpy as np
import pytest

import tq_inputs as TI
from oracle import tq_oracle as O
from parity_utils import compare_quantize, oracle_quantize, rotations, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import compressed_attention_rotate_amd as tq
    tq.load()
    return torch


def _run(torch, x_np, dtype, fmt_t, seed, counters=True):
    import compressed_attention_rotate_amd as tq
    d = fmt_t[0]
    fmt = tq.Format(*fmt_t)
    (signs, S), (gsigns, gS) = rotations(d, seed)
    tab = tq.Tables(fmt, gsigns, torch.from_numpy(gS).cuda())
    if dtype == "bf16":
        xt = torch.from_numpy(x_np.view(np.int16)).cuda().view(torch.bfloat16)
    elif dtype == "f16":
        xt = torch.from_numpy(x_np.astype(np.float16)).cuda()
    else:
        xt = torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32)).cuda()
    cnt = torch.zeros(4, dtype=torch.int64, device="cuda") if counters else None
    codes, norms = tq.quantize_kv(xt, fmt, tab, counters=cnt)
    torch.cuda.synchronize()
    return (codes.cpu().numpy(), norms.cpu().view(torch.int16).numpy().view(np.uint16),
            None if cnt is None else cnt.cpu().numpy(), signs, S)


def _check(torch, x_np, dtype, fmt_t, seed):
    codes, norms, cnt, signs, S = _run(torch, x_np, dtype, fmt_t, seed)
    x64 = to_f64(x_np, dtype) if dtype != "f16" else x_np.astype(np.float16).astype(np.float64)
    qz = oracle_quantize(x64, O.Format(*fmt_t), signs, S)
    rep = compare_quantize(codes, norms, qz, O.Format(*fmt_t))
    print(f"\n{fmt_t} {dtype} n={x_np.shape[0]}: {rep} counters={cnt}")
    return rep, cnt


def test_single_head_fp32_b3_with_outliers(torch_gpu):
    k, v, _, _ = TI.c1_inputs(seed=1000)
    x = np.concatenate([k, v])
    _check(torch_gpu, x, "f32", (128, 2, 2, 128), TI.rotation_seed(1))


@pytest.mark.parametrize("fmt_t", [(128, 3, 3, 128), (128, 1, 1, 128), (128, 2, 2, 128),
                                   (128, 3, 2, 64), (128, 2, 1, 96), (128, 3, 2, 32)])
def test_bf16_channel_scaled(torch_gpu, fmt_t):
    kb, vb, _ = TI.kv_layer(1, 2, 1500, 128, seed=77)
    x = np.concatenate([kb.reshape(-1, 128), vb.reshape(-1, 128)])
    _check(torch_gpu, x, "bf16", fmt_t, 5)


@pytest.mark.parametrize("fmt_t", [(128, 3, 3, 128, False), (128, 1, 1, 128, False),
                                   (128, 3, 2, 64, False), (128, 2, 1, 96, False)])
def test_mse_only_formats(torch_gpu, fmt_t):
    """Records without QJL sign words: same codes and norms as the QJL format, no signs."""
    kb, vb, _ = TI.kv_layer(1, 2, 700, 128, seed=78)
    x = np.concatenate([kb.reshape(-1, 128), vb.reshape(-1, 128)])
    x = x[:1391]                                                   # ragged last tile
    _check(torch_gpu, x, "bf16", fmt_t, 6)


def test_mse_only_d256_padded(torch_gpu):
    x = TI.search_set(1000, 200, seed=5006)
    _check(torch_gpu, x, "f32", (256, 3, 3, 256, False), 5501)


def test_ragged_and_tiny_sizes(torch_gpu):
    g = TI.gen(3)
    for n in (1, 31, 33, 127, 129, 1000):
        x = (g.standard_normal((n, 128)) * 3).astype(np.float32)
        _check(torch_gpu, x, "f32", (128, 3, 3, 128), 9 + n)


def test_zero_vectors_and_fp16_input(torch_gpu):
    g = TI.gen(4)
    x = (g.standard_normal((300, 128))).astype(np.float32)
    x[::7] = 0.0
    _check(torch_gpu, x, "f32", (128, 3, 3, 128), 21)
    _check(torch_gpu, x, "f16", (128, 2, 2, 128), 22)


@pytest.mark.parametrize("bits", [2, 3])
def test_search_width_d256_padded(torch_gpu, bits):
    x = TI.search_set(3000, 200, seed=5005)
    _check(torch_gpu, x, "f32", (256, bits, bits, 256), 5500)


def test_full_layer_sampled(torch_gpu):
    """Full Llama-3.1-8B decode layer (8 KV heads x 32768 tokens, K and V, b = 4) quantized
    in one launch; a seeded sample of rows is checked against the oracle."""
    kb, vb, _ = TI.kv_layer(1, 8, 32768, 128, seed=TI.data_seed(2))
    x = np.concatenate([kb.reshape(-1, 128), vb.reshape(-1, 128)])
    codes, norms, cnt, signs, S = _run(torch_gpu, x, "bf16", (128, 3, 3, 128), TI.rotation_seed(2))
    rows = np.sort(TI.gen(99).choice(x.shape[0], size=6000, replace=False))
    rows = np.concatenate([rows, np.arange(x.shape[0] - 40, x.shape[0])])
    qz = oracle_quantize(x[rows], O.Format(128, 3, 3, 128), signs, S, bf16=True)
    rep = compare_quantize(codes[rows], norms[rows], qz, O.Format(128, 3, 3, 128))
    print(f"\nfull layer: {rep} counters={cnt}")
    assert cnt[3] == 0


def test_argument_errors_launch_nothing(torch_gpu):
    import compressed_attention_rotate_amd as tq
    torch = torch_gpu
    fmt = tq.Format(128, 3, 3, 128)
    (signs, S), (gsigns, gS) = rotations(128, 1)
    tab = tq.Tables(fmt, gsigns, torch.from_numpy(gS).cuda())
    x = torch.zeros((4, 129), device="cuda")
    with pytest.raises(tq.TQError):
        tq.quantize_kv(x, fmt, tab)            # d_in > d
    with pytest.raises(tq.TQError):
        tq.quantize_kv(torch.zeros((4, 128), device="cuda"), tq.Format(128, 4, 4, 128), tab)
