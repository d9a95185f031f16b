"""GPU: hqq_quantize_streamed (weights in pinned host memory, copied in
double-buffered chunks while the solve runs) gives exactly the resident
hqq_quantize results, with small staging buffers that force row-block
splits, several tensors per chunk, and both axes.  The resident path is
itself checked against the oracle (test_gpu_parity.py); here the two HIP
paths must agree bit for bit."""
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


def _outputs(hq, rows, cols, nbits, gs, axis):
    import torch

    ms = hq.meta_shape(rows, cols, gs, axis)
    return (torch.zeros(hq.packed_shape(rows, cols, nbits, axis), dtype=torch.int32, device="cuda"),
            torch.zeros(ms, dtype=torch.float32, device="cuda"),
            torch.zeros(ms, dtype=torch.float32, device="cuda"))


def _check(hq, shapes, nbits, gs, axis, staging_bytes, seed, separate_streams=True):
    import torch

    rng = np.random.RandomState(seed)
    Ws = [random_f16(rng, s, std=0.02, outlier_frac=0.002) for s in shapes]
    host = [torch.from_numpy(W.view(np.int16)).pin_memory() for W in Ws]
    outs = [_outputs(hq, *s, nbits, gs, axis) for s in shapes]
    staging = torch.empty(staging_bytes, dtype=torch.uint8, device="cuda")
    cs = torch.cuda.Stream() if separate_streams else torch.cuda.current_stream()
    ks = torch.cuda.Stream() if separate_streams else torch.cuda.current_stream()
    hq.hqq_quantize_streamed([(h, *o) for h, o in zip(host, outs)], nbits, gs, axis, staging,
                             copy_stream=cs, compute_stream=ks)
    ks.synchronize()
    for W, h, (pk, sc, ze) in zip(Ws, host, outs):
        rp, rs, rz = hq.hqq_quantize(h.cuda(), nbits, gs, axis)
        torch.cuda.synchronize()
        assert torch.equal(pk, rp), (W.shape, "packed")
        assert torch.equal(sc.view(torch.int32), rs.view(torch.int32)), (W.shape, "scale")
        assert torch.equal(ze.view(torch.int32), rz.view(torch.int32)), (W.shape, "zero")


def test_streamed_axis1_splits_and_packs_chunks(hq):
    # halves of 96 KiB: the 512-row tensors split, the small ones share chunks
    _check(hq, [(512, 256), (40, 256), (24, 256), (300, 512), (7, 128)], 4, 64, 1, 2 * 96 * 1024, 1)


def test_streamed_axis1_same_stream(hq):
    _check(hq, [(200, 1024), (64, 1024)], 4, 64, 1, 2 * 64 * 1024, 2, separate_streams=False)


def test_streamed_axis0_3bit(hq):
    # axis 0, 3-bit g64: row blocks of lcm(64, 10) = 320 rows
    _check(hq, [(1280, 96), (640, 200)], 3, 64, 0, 2 * 330 * 400, 3)


def test_streamed_axis0_2bit_g16_and_8bit(hq):
    _check(hq, [(256, 136), (48, 64)], 2, 16, 0, 2 * 40 * 1024, 4)
    _check(hq, [(96, 320), (33, 64)], 8, 32, 1, 2 * 16 * 1024, 5)


def test_streamed_one_chunk_covers_all(hq):
    _check(hq, [(64, 256), (64, 256)], 4, 64, 1, 8 << 20, 6)


def test_streamed_many_small_tensors_over_batch_limit(hq):
    # more than 24 row blocks fit a half: chunks close at 24 pieces
    _check(hq, [(8, 64)] * 30, 4, 64, 1, 2 << 20, 7)
