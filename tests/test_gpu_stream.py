"""GPU: hqq_quantize_streamed (weights in pinned host memory, copied in
double-buffered chunks while the solve runs) against the oracle, and bit for
bit against the resident hqq_quantize, with small staging buffers that force
row-block splits, several tensors per chunk, and both axes; and two calls in
a row that share one staging buffer with nothing between them."""
import numpy as np
import pytest

from helpers import oracle_codes_parallel, random_f16

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


def _against_oracle(oracle_mod, W, nbits, gs, axis, pk, sc, ze):
    rows, cols = W.shape
    o_codes, o_scale, o_zero = oracle_codes_parallel(oracle_mod, W, nbits, gs, axis)
    assert np.array_equal(pk.cpu().numpy().view(np.uint32), oracle_mod.pack(o_codes, nbits, axis)), \
        (W.shape, "codes differ from the oracle")
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), o_scale.view(np.uint32)), (W.shape, "scale")
    assert np.array_equal(ze.cpu().numpy(), o_zero), (W.shape, "zero")


def _check(hq, oracle_mod, shapes, nbits, gs, axis, staging_bytes, seed, separate_streams=True):
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
        _against_oracle(oracle_mod, W, nbits, gs, axis, pk, sc, ze)
        rp, rs, rz = hq.hqq_quantize(h.cuda(), nbits, gs, axis)
        torch.cuda.synchronize()
        assert torch.equal(pk, rp), (W.shape, "packed")
        assert torch.equal(sc.view(torch.int32), rs.view(torch.int32)), (W.shape, "scale")
        assert torch.equal(ze.view(torch.int32), rz.view(torch.int32)), (W.shape, "zero")


def test_streamed_axis1_splits_and_packs_chunks(hq, oracle_mod):
    # halves of 96 KiB: the 512-row tensors split, the small ones share chunks
    _check(hq, oracle_mod, [(512, 256), (40, 256), (24, 256), (300, 512), (7, 128)], 4, 64, 1, 2 * 96 * 1024, 1)


def test_streamed_axis1_same_stream(hq, oracle_mod):
    _check(hq, oracle_mod, [(200, 1024), (64, 1024)], 4, 64, 1, 2 * 64 * 1024, 2, separate_streams=False)


def test_streamed_axis0_3bit(hq, oracle_mod):
    # axis 0, 3-bit g64: row blocks of lcm(64, 10) = 320 rows
    _check(hq, oracle_mod, [(1280, 96), (640, 200)], 3, 64, 0, 2 * 330 * 400, 3)


def test_streamed_axis0_2bit_g16_and_8bit(hq, oracle_mod):
    _check(hq, oracle_mod, [(256, 136), (48, 64)], 2, 16, 0, 2 * 40 * 1024, 4)
    _check(hq, oracle_mod, [(96, 320), (33, 64)], 8, 32, 1, 2 * 16 * 1024, 5)


def test_streamed_one_chunk_covers_all(hq, oracle_mod):
    _check(hq, oracle_mod, [(64, 256), (64, 256)], 4, 64, 1, 8 << 20, 6)


def test_streamed_many_small_tensors_over_batch_limit(hq, oracle_mod):
    # more than 48 row blocks fit a half: chunks close at 48 pieces
    _check(hq, oracle_mod, [(8, 64)] * 60, 4, 64, 1, 2 << 20, 7)


def test_streamed_back_to_back_calls_share_staging(hq, oracle_mod):
    """Two calls in a row on one staging buffer, separate copy and compute
    streams, no synchronisation between them: the second call's copies must
    not overwrite halves the first call's solves still read."""
    import torch

    rng = np.random.RandomState(11)
    shapes = [[(512, 1024), (96, 1024)], [(384, 1024), (200, 1024)]]
    staging = torch.empty(2 * 128 * 1024, dtype=torch.uint8, device="cuda")
    cs, ks = torch.cuda.Stream(), torch.cuda.Stream()
    calls = []
    for sh in shapes:
        Ws = [random_f16(rng, s, std=0.03, outlier_frac=0.002) for s in sh]
        host = [torch.from_numpy(W.view(np.int16)).pin_memory() for W in Ws]
        outs = [_outputs(hq, *s, 4, 64, 1) for s in sh]
        calls.append((Ws, outs, host))   # the pinned weights stay alive until the sync
        hq.hqq_quantize_streamed([(h, *o) for h, o in zip(host, outs)], 4, 64, 1, staging,
                                 copy_stream=cs, compute_stream=ks)
    ks.synchronize()
    for Ws, outs, _ in calls:
        for W, (pk, sc, ze) in zip(Ws, outs):
            _against_oracle(oracle_mod, W, 4, 64, 1, pk, sc, ze)
