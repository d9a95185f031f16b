"""GPU: hqq_quantize_streamed_static (the streamed solve through the library's
static staging array, no device allocation in the call) against
hqq_quantize_streamed (the same solve through a caller's staging buffer), bit
for bit, on two calls in a row: the first large enough to need several
chunks of the 64 MiB array, the second smaller and of another format."""
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


def test_static_staging_matches_caller_staging(hq):
    import torch

    cases = [
        # 3 x 32 MiB of fp16 weights: four 32 MiB halves' worth of chunks
        ("4b g64 axis 1, three 4096x4096", [(4096, 4096)] * 3, 4, 64, 1, 11),
        # smaller, another format, after the first with nothing in between
        ("2b g16 axis 0, 1024x4096 and 512x1000", [(1024, 4096), (512, 1000)], 2, 16, 0, 12),
    ]
    cs, ks = torch.cuda.Stream(), torch.cuda.Stream()
    for name, shapes, nbits, gs, axis, seed in cases:
        print("case", name, flush=True)
        rng = np.random.RandomState(seed)
        host = [torch.from_numpy(random_f16(rng, s, std=0.02, outlier_frac=0.002).view(np.int16)).pin_memory()
                for s in shapes]
        got = [_outputs(hq, *s, nbits, gs, axis) for s in shapes]
        ref = [_outputs(hq, *s, nbits, gs, axis) for s in shapes]
        hq.hqq_quantize_streamed_static([(h, *o) for h, o in zip(host, got)], nbits, gs, axis,
                                        copy_stream=cs, compute_stream=ks)
        staging = torch.empty(8 << 20, dtype=torch.uint8, device="cuda")
        hq.hqq_quantize_streamed([(h, *o) for h, o in zip(host, ref)], nbits, gs, axis, staging,
                                 copy_stream=cs, compute_stream=ks)
        ks.synchronize()
        for s, g, r in zip(shapes, got, ref):
            assert torch.equal(g[0], r[0]), (name, s, "packed")
            assert torch.equal(g[1].view(torch.int32), r[1].view(torch.int32)), (name, s, "scale")
            assert torch.equal(g[2].view(torch.int32), r[2].view(torch.int32)), (name, s, "zero")
        del host


def test_static_staging_rejects_oversized_blocks(hq):
    import torch

    # a 3-bit axis-0 block unit is 320 rows: at 65536 columns, 40 MiB, more
    # than half the array; refused before anything is enqueued
    h = torch.zeros((320, 65536), dtype=torch.int16).pin_memory()
    out = _outputs(hq, 320, 65536, 3, 64, 0)
    with pytest.raises(hq.HQQError) as e:
        hq.hqq_quantize_streamed_static([(h, *out)], 3, 64, 0)
    assert "(status -9)" in str(e.value)
    torch.cuda.synchronize()
    assert int(out[0].abs().sum()) == 0
