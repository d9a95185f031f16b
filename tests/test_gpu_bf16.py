"""GPU parity of the bf16 paths (through the C ABI) against the oracle: the
solve on bf16 weights (hqq_quantize_batch_ex) and dequantization into bf16
(hqq_dequantize_ex).  The kernels widen bf16 exactly and form the group sum
in the oracle's order, so codes, scale and zero are required bit for bit, as
for fp16; dequantized values too."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hq():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import weight_quantization_group_amd as w

    w.load_library()
    return w


def random_bf16(rng, shape, std=0.02, outlier_frac=0.002, wide=False):
    w = rng.randn(*shape) * std
    if outlier_frac:
        m = rng.rand(*shape) < outlier_frac
        w = np.where(m, w * 20.0, w)
    if wide:
        # a few rows far outside fp16's range, and some tiny values
        w[:4] *= 1e6
        w[4:8] *= 1e-9
    f = w.astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _gpu_bf16(hq, WB, nbits, gs, axis, iters=20):
    import torch

    Wd = torch.from_numpy(WB.view(np.int16)).cuda().view(torch.bfloat16)
    packed, scale, zero = hq.hqq_quantize(Wd, nbits, gs, axis, iters=iters)
    torch.cuda.synchronize()
    return packed.cpu().numpy().view(np.uint32), scale.cpu().numpy(), zero.cpu().numpy()


CASES = [(4, 64, 1, (256, 512)), (4, 64, 0, (256, 192)), (3, 64, 0, (320, 128)),
         (2, 16, 1, (64, 512)), (2, 16, 0, (128, 160)), (8, 128, 1, (96, 512)),
         (1, 32, 1, (64, 256)), (4, 128, 1, (48, 1024)), (4, 8, 1, (40, 64)), (3, 256, 1, (16, 2560))]


@pytest.mark.parametrize("nbits,gs,axis,shape", CASES)
def test_bf16_solve_parity(hq, oracle_mod, nbits, gs, axis, shape):
    rng = np.random.RandomState(nbits * 31 + gs + axis * 7 + shape[0])
    WB = random_bf16(rng, shape)
    g = _gpu_bf16(hq, WB, nbits, gs, axis)
    o = oracle_mod.quantize(WB, nbits, gs, axis, iters=20, dtype="bf16")
    assert np.array_equal(g[1].view(np.uint32), o[1].view(np.uint32)), "scale"
    assert np.array_equal(g[2].view(np.uint32), o[2].view(np.uint32)), "zero"
    assert np.array_equal(g[0], o[0]), "packed codes"


@pytest.mark.parametrize("nbits,gs,axis", [(4, 64, 1), (2, 16, 0), (8, 32, 1)])
def test_bf16_solve_wide_range_rows(hq, oracle_mod, nbits, gs, axis):
    """Rows scaled by 1e6 and 1e-9: outside fp16's range, and sums of mixed
    magnitudes that fp64 rounds (the order then matters)."""
    rng = np.random.RandomState(77 + nbits + gs)
    WB = random_bf16(rng, (64, 256), wide=True)
    g = _gpu_bf16(hq, WB, nbits, gs, axis)
    o = oracle_mod.quantize(WB, nbits, gs, axis, iters=20, dtype="bf16")
    for a, b in zip(g, o):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("iters", [0, 1, 5])
def test_bf16_iteration_counts(hq, oracle_mod, iters):
    rng = np.random.RandomState(400 + iters)
    WB = random_bf16(rng, (128, 256))
    g = _gpu_bf16(hq, WB, 4, 64, 1, iters=iters)
    o = oracle_mod.quantize(WB, 4, 64, 1, iters=iters, dtype="bf16")
    for a, b in zip(g, o):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("nbits,gs,axis", [(4, 64, 1), (3, 64, 0), (2, 16, 1), (8, 128, 0), (1, 32, 1)])
def test_bf16_dequantize_parity(hq, oracle_mod, nbits, gs, axis):
    import torch

    rng = np.random.RandomState(900 + nbits + gs + axis)
    rows, cols = (640, 96) if axis == 0 else (48, 512)
    qmax = (1 << nbits) - 1
    codes = rng.randint(0, qmax + 1, size=(rows, cols)).astype(np.uint8)
    ms = (rows, cols // gs) if axis == 1 else (rows // gs, cols)
    scale = (rng.uniform(1, 2, ms) * 2.0 ** rng.randint(-8, 30, ms)).astype(np.float32)
    zero = rng.uniform(-20, 20, ms).astype(np.float32)
    packed = oracle_mod.pack(codes, nbits, axis)
    out = hq.hqq_dequantize(torch.from_numpy(packed.view(np.int32)).cuda(), torch.from_numpy(scale).cuda(),
                            torch.from_numpy(zero).cuda(), rows, cols, nbits, gs, axis,
                            dtype=torch.bfloat16)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle_mod.dequantize(packed, scale, zero, rows, cols, nbits, gs, axis, dtype="bf16")
    assert np.array_equal(got, ref)


def test_bf16_roundtrip_through_gpu(hq):
    """quantize(bf16) -> dequantize(bf16) on the GPU lands within half a step
    of each weight except where the clamp engaged."""
    import torch

    rng = np.random.RandomState(12)
    WB = random_bf16(rng, (64, 512), outlier_frac=0.0)
    Wd = torch.from_numpy(WB.view(np.int16)).cuda().view(torch.bfloat16)
    p, s, z = hq.hqq_quantize(Wd, 4, 64, 1, iters=20)
    Wh = hq.hqq_dequantize(p, s, z, 64, 512, 4, 64, 1, dtype=torch.bfloat16)
    w = Wd.float().cpu().numpy()
    wh = Wh.float().cpu().numpy()
    step = 1.0 / np.repeat(s.cpu().numpy(), 64, axis=1)
    assert np.mean(np.abs(w - wh) <= 0.51 * step + 1e-6) > 0.95
