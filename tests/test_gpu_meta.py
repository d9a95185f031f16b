"""GPU parity of the metadata quantization (hqq_quantize_meta,
hqq_dequantize_meta and their batched forms, through the C ABI) against the
oracle, and the path W codes + quantized meta -> dequantize end to end."""
import numpy as np
import pytest

from helpers import random_f16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hq():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import weight_quantization_group_amd as w

    w.load_library()
    return w


def same_value(a, b):
    """Equal as fp32 values (a zero's sign may differ: -0 == +0)."""
    return np.array_equal(np.asarray(a, np.float32), np.asarray(b, np.float32))


def _check(hq, oracle_mod, meta, gs):
    import torch

    m = torch.from_numpy(np.ascontiguousarray(meta, np.float32).ravel()).cuda()
    codes, ms, mz = hq.hqq_quantize_meta(m, gs)
    back = hq.hqq_dequantize_meta(codes, ms, mz, gs)
    torch.cuda.synchronize()
    oc, os_, oz = oracle_mod.quantize_meta(meta, gs)
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert same_value(ms.cpu().numpy(), os_) and same_value(mz.cpu().numpy(), oz)
    assert same_value(back.cpu().numpy(), oracle_mod.dequantize_meta(oc, os_, oz, gs))


@pytest.mark.parametrize("n,gs", [(1000, 128), (4096, 128), (77, 16), (5, 1), (3000, 1024), (129, 64),
                                  (100003, 128)])
def test_meta_parity_random(hq, oracle_mod, n, gs):
    rng = np.random.RandomState(n + gs)
    meta = rng.uniform(-400, 400, n).astype(np.float32)
    meta[: min(n, 3 * gs): 2] = 0.0          # zeros, and a constant stretch
    _check(hq, oracle_mod, meta, gs)


def test_meta_batch_parity(hq, oracle_mod):
    """140 arrays of ragged sizes in one call (three launches of up to 64
    arrays), each checked against the oracle, quantize and dequantize."""
    import torch

    rng = np.random.RandomState(31)
    sizes = [int(x) for x in rng.randint(1, 3000, size=135)] + [1, 127, 128, 129, 65536 + 5]
    metas = [rng.uniform(-50, 50, n).astype(np.float32) for n in sizes]
    metas[3][:] = 7.0                                 # a constant array
    for gs in (128, 64):
        dev = [torch.from_numpy(m).cuda() for m in metas]
        q = hq.hqq_quantize_meta_batch(dev, gs)
        back = hq.hqq_dequantize_meta_batch(q, gs)
        torch.cuda.synchronize()
        for m, (c, ms, mz), b in zip(metas, q, back):
            oc, os_, oz = oracle_mod.quantize_meta(m, gs)
            assert np.array_equal(c.cpu().numpy(), oc), (m.size, gs)
            assert same_value(ms.cpu().numpy(), os_) and same_value(mz.cpu().numpy(), oz), (m.size, gs)
            assert same_value(b.cpu().numpy(), oracle_mod.dequantize_meta(oc, os_, oz, gs)), (m.size, gs)


@pytest.mark.parametrize("gs", [16, 32, 64, 256, 512, 1024, 100, 3])
def test_meta_batch_group_sizes_and_alignment(hq, oracle_mod, gs):
    """Every group size of the vector path and two others; arrays that start
    4 bytes past a 16-byte boundary, codes at odd addresses (both take the
    value-by-value path), sizes below one group and ragged last groups."""
    import torch

    rng = np.random.RandomState(40 + gs)
    sizes = [1, gs - 1 if gs > 1 else 1, gs, gs + 1, 5 * gs + 7, 20000 + 3]
    items, refs = [], []
    for k, n in enumerate(sizes):
        m = rng.uniform(-3, 3, n).astype(np.float32)
        shift_m, shift_c = (k % 2, (k // 2) % 2)      # misaligned meta / codes
        mbuf = torch.empty(n + 4, dtype=torch.float32, device="cuda")
        md = mbuf[shift_m:shift_m + n]
        md.copy_(torch.from_numpy(m))
        cbuf = torch.empty(n + 4, dtype=torch.uint8, device="cuda")
        ng = -(-n // gs)
        items.append((md, cbuf[shift_c:shift_c + n], torch.empty(ng, dtype=torch.float32, device="cuda"),
                      torch.empty(ng, dtype=torch.float32, device="cuda")))
        refs.append(m)
    mb = hq.MetaBatch(items, gs)
    mb.quantize()
    torch.cuda.synchronize()
    for (md, c, ms, mz), m in zip(items, refs):
        oc, os_, oz = oracle_mod.quantize_meta(m, gs)
        assert np.array_equal(c.cpu().numpy(), oc), (m.size, gs)
        assert same_value(ms.cpu().numpy(), os_) and same_value(mz.cpu().numpy(), oz), (m.size, gs)
        md.fill_(float("nan"))
    mb.dequantize()
    torch.cuda.synchronize()
    for (md, c, ms, mz), m in zip(items, refs):
        oc, os_, oz = oracle_mod.quantize_meta(m, gs)
        assert same_value(md.cpu().numpy(), oracle_mod.dequantize_meta(oc, os_, oz, gs)), (m.size, gs)


def test_meta_batch_equals_single_calls(hq):
    """The batch and the single-array entry points agree bit for bit."""
    import torch

    rng = np.random.RandomState(32)
    dev = [torch.from_numpy(rng.uniform(-1, 1, n).astype(np.float32)).cuda() for n in (5000, 17, 40000, 1)]
    batch = hq.hqq_quantize_meta_batch(dev, 128)
    for m, (c, ms, mz) in zip(dev, batch):
        c1, ms1, mz1 = hq.hqq_quantize_meta(m, 128)
        assert torch.equal(c, c1) and torch.equal(ms.view(torch.int32), ms1.view(torch.int32))
        assert torch.equal(mz.view(torch.int32), mz1.view(torch.int32))


def test_meta_parity_solver_outputs(hq, oracle_mod):
    rng = np.random.RandomState(9)
    W16 = random_f16(rng, (128, 2048), std=0.02, outlier_frac=0.002)
    _, scale, zero = oracle_mod.quantize(W16, 4, 64, 1, iters=5)
    _check(hq, oracle_mod, scale, 128)
    _check(hq, oracle_mod, zero, 128)


def test_meta_constant_and_extreme_groups(hq, oracle_mod):
    meta = np.concatenate([np.full(128, 2.5, np.float32), np.full(128, -0.0, np.float32),
                           np.array([1e30, -1e30] * 64, np.float32), np.linspace(-1, 1, 77).astype(np.float32)])
    _check(hq, oracle_mod, meta, 128)


def test_weights_with_quantized_meta_end_to_end(hq, oracle_mod):
    """Solved codes and meta (from the oracle), meta through 8 bits and back,
    then dequantize: the GPU path and the oracle agree bit for bit."""
    import torch

    rng = np.random.RandomState(10)
    rows, cols, nbits, gs = 64, 1024, 4, 64
    W16 = random_f16(rng, (rows, cols), std=0.02, outlier_frac=0.002)
    p, s, z = oracle_mod.quantize(W16, nbits, gs, 1, iters=5)
    ds, dz = torch.from_numpy(s).cuda(), torch.from_numpy(z).cuda()
    s_back = hq.hqq_dequantize_meta(*hq.hqq_quantize_meta(ds, 128), 128).view(ds.shape)
    z_back = hq.hqq_dequantize_meta(*hq.hqq_quantize_meta(dz, 128), 128).view(dz.shape)
    Wh = hq.hqq_dequantize(torch.from_numpy(p.view(np.int32)).cuda(), s_back, z_back, rows, cols, nbits,
                           gs, 1)
    torch.cuda.synchronize()
    os_ = oracle_mod.dequantize_meta(*oracle_mod.quantize_meta(s, 128), 128).reshape(s.shape)
    oz = oracle_mod.dequantize_meta(*oracle_mod.quantize_meta(z, 128), 128).reshape(z.shape)
    ref = oracle_mod.dequantize(p, os_, oz, rows, cols, nbits, gs, 1)
    assert np.array_equal(Wh.view(torch.int16).cpu().numpy().view(np.uint16), ref)
