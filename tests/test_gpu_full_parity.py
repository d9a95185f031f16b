"""GPU parity at full size: the five workloads, in the benchmark's launch
configuration, against the oracle element by element.

  single Linear [4096, 1024] 4b g64          every element (test_gpu_parity.py)
  7B decoder layer, 4b g64 axis 1            every element of the 7 tensors
  7B decoder layer, 3b g64 / 2b g16 axis 0   every element of the 7 tensors
  7B stack, 32 layers, 4b g64                layers 0 and 31 in full, 1% of the
                                             rows of every other tensor
  70B stack, 80 layers, mixed 4/2/1 bits     quantized layer by layer (one
                                             layer's fp16 weights resident at a
                                             time); layers 0 and 79 in full, 1%
                                             of the rows of every other tensor

The sampled rows come from a generator seeded with (seed, layer, tensor): a
deterministic sample.  A group's solve reads only its own weights, so a row
of the oracle's output needs only that row of W.

Bar (the method's tolerances): codes identical on >= 99.99% of the elements
and the rest within +-1; scale and zero within 1e-4 relative; per-tensor
reconstruction MSE within 0.1%; packed words exactly the packing of the
codes.  The kernels reproduce the oracle's fp32 arithmetic, so the tests also
require identical codes, scale bit for bit and zero equal in value (+0 and -0
are the same zero), and print the tolerance statistics beside.

The oracle runs as independent row slices on worker threads (the host's
cores, at most 16); each slice is the single-threaded oracle unchanged.
"""
import time

import numpy as np
import pytest

import synth
from helpers import oracle_codes_parallel, recon_mse_chunked

pytestmark = pytest.mark.gpu

QMAX = {1: 1, 2: 3, 3: 7, 4: 15, 8: 255}


@pytest.fixture(scope="module")
def hq():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import weight_quantization_group_amd as w

    w.load_library()
    return w


def _launch_chunks(tensors, max_batch):
    """The benchmark's launches: runs of consecutive tensors of one format,
    each cut into as even pieces of at most max_batch as it allows (one
    hqq_quantize_batch call each)."""
    runs = []
    for i, t in enumerate(tensors):
        fmt = (t["nbits"], t["group_size"], t["axis"])
        if runs and runs[-1][0] == fmt:
            runs[-1][1].append(i)
        else:
            runs.append((fmt, [i]))
    chunks = []
    for fmt, idx in runs:
        per = -(-len(idx) // -(-len(idx) // max_batch))
        chunks += [(fmt, idx[k:k + per]) for k in range(0, len(idx), per)]
    return chunks


def _generate_and_quantize(hq, tensors):
    """Generate the tensors on the GPU and quantize them with the benchmark's
    launches.  Returns [(W, packed, scale, zero)] on the device."""
    import torch

    items = []
    for t in tensors:
        W = torch.empty((t["rows"], t["cols"]), dtype=torch.float16, device="cuda")
        synth.generate_gpu(W, t["seed"], t["layer"], t["tensor_id"])
        ms = hq.meta_shape(t["rows"], t["cols"], t["group_size"], t["axis"])
        items.append((W, torch.empty(hq.packed_shape(t["rows"], t["cols"], t["nbits"], t["axis"]),
                                     dtype=torch.int32, device="cuda"),
                      torch.empty(ms, dtype=torch.float32, device="cuda"),
                      torch.empty(ms, dtype=torch.float32, device="cuda")))
    for fmt, idx in _launch_chunks(tensors, hq.MAX_BATCH):
        hq.QuantizeBatch([items[i] for i in idx], *fmt).run()
    torch.cuda.synchronize()
    return items


def _host(t):
    return t.cpu().numpy()


def compare(oracle_mod, W16, nb, gs, axis, g_packed, g_scale, g_zero, tag):
    """Every element of (W16 -> GPU outputs) against the oracle; returns the
    statistics and asserts the bar."""
    rows, cols = W16.shape
    t0 = time.perf_counter()
    o_codes, o_scale, o_zero = oracle_codes_parallel(oracle_mod, W16, nb, gs, axis)
    t_oracle = time.perf_counter() - t0
    g_codes = oracle_mod.unpack(g_packed, rows, cols, nb, axis)
    assert np.array_equal(g_packed, oracle_mod.pack(g_codes, nb, axis)), f"{tag}: packing"
    diff = g_codes.astype(np.int16) - o_codes.astype(np.int16)
    mism = int(np.count_nonzero(diff))
    maxd = int(np.abs(diff).max(initial=0))
    o_zero64 = o_zero.astype(np.float64)
    zrel = np.abs(g_zero.astype(np.float64) - o_zero64) / np.maximum(np.abs(o_zero64), 1e-30)
    srel = np.abs(g_scale.astype(np.float64) - o_scale) / np.abs(o_scale.astype(np.float64))
    mg = recon_mse_chunked(W16, g_codes, g_scale, g_zero, gs, axis)
    mo = recon_mse_chunked(W16, o_codes, o_scale, o_zero, gs, axis)
    st = dict(tag=tag, elements=int(diff.size), groups=int(o_scale.size),
              code_identical=1.0 - mism / diff.size, code_max_diff=maxd,
              scale_max_rel=float(srel.max()), zero_max_rel=float(zrel.max()),
              zero_equal=float(np.mean(g_zero == o_zero)), mse_gpu=mg, mse_oracle=mo,
              mse_rel=abs(mg - mo) / mo, oracle_s=round(t_oracle, 2))
    print(st, flush=True)
    # the method's tolerances
    assert maxd <= 1 and mism <= 1e-4 * diff.size, f"{tag}: {mism} codes differ (max {maxd})"
    assert g_codes.max() <= QMAX[nb]
    assert srel.max() <= 1e-4 and zrel.max() <= 1e-4, f"{tag}: scale/zero beyond 1e-4"
    assert st["mse_rel"] <= 1e-3, f"{tag}: MSE {mg} vs {mo}"
    # the kernels' exactness
    assert mism == 0, f"{tag}: {mism} codes differ"
    assert np.array_equal(g_scale.view(np.uint32), o_scale.view(np.uint32)), f"{tag}: scale bits"
    assert np.array_equal(g_zero, o_zero), f"{tag}: {np.sum(g_zero != o_zero)} zeros differ"
    return st


def _full(oracle_mod, t, item, tag):
    W, pk, sc, ze = item
    return compare(oracle_mod, _host(W).view(np.uint16), t["nbits"], t["group_size"], t["axis"],
                   _host(pk).view(np.uint32), _host(sc), _host(ze), tag)


def sample_rows(t, frac=0.01):
    """A deterministic 1% of the rows of an axis-1 tensor (at least 8)."""
    rng = np.random.default_rng([t["seed"], t["layer"], t["tensor_id"]])
    n = max(8, int(np.ceil(frac * t["rows"])))
    return np.sort(rng.choice(t["rows"], n, replace=False))


def _sampled(oracle_mod, t, item, tag):
    import torch

    assert t["axis"] == 1
    W, pk, sc, ze = item
    rows = sample_rows(t)
    it = torch.from_numpy(rows).cuda()
    return compare(oracle_mod, _host(W.index_select(0, it)).view(np.uint16), t["nbits"],
                   t["group_size"], 1, _host(pk.index_select(0, it)).view(np.uint32),
                   _host(sc.index_select(0, it)), _host(ze.index_select(0, it)),
                   tag + f" ({rows.size} sampled rows)")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wl", ["llama7b_layer_4b_g64", "llama7b_layer_3b2b_axis0"])
def test_7b_layer_every_element(hq, oracle_mod, wl):
    """One 7B-shaped decoder layer (both formats), every element of the seven
    tensors, after the benchmark's launches of that workload."""
    tensors = synth.workload(wl)
    items = _generate_and_quantize(hq, tensors)
    for t, item in zip(tensors, items):
        _full(oracle_mod, t, item, f"{wl} {t['name']} {t['nbits']}b g{t['group_size']} ax{t['axis']}")


@pytest.mark.timeout(900)
def test_7b_stack_layers_0_31_full_others_sampled(hq, oracle_mod):
    """The 32-layer 7B stack quantized with the benchmark's ten launches
    (all 224 tensors resident): layers 0 and 31 every element, 1% of the rows
    of every tensor of layers 1-30."""
    import torch

    tensors = synth.workload("llama7b_stack32_4b_g64")
    items = _generate_and_quantize(hq, tensors)
    n_sampled = 0
    for t, item in zip(tensors, items):
        tag = f"7B stack L{t['layer']} {t['name']}"
        if t["layer"] in (0, 31):
            _full(oracle_mod, t, item, tag)
        else:
            n_sampled += _sampled(oracle_mod, t, item, tag)["elements"]
    print("7B stack: sampled elements", n_sampled)
    del items
    torch.cuda.empty_cache()


def _70b_layer(hq, oracle_mod, layer, full):
    import torch

    tensors = [t for t in synth.workload("llama70b_stack80_mixed") if t["layer"] == layer]
    items = _generate_and_quantize(hq, tensors)
    for t, item in zip(tensors, items):
        tag = f"70B L{layer} {t['name']} {t['nbits']}b g{t['group_size']}"
        (_full if full else _sampled)(oracle_mod, t, item, tag)
    del items
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("layer", [0, 79])
def test_70b_first_and_last_layer_every_element(hq, oracle_mod, layer):
    """70B-shaped layers 0 (with the 1-bit down projection) and 79, every
    element, one layer's weights resident at a time (the layer's launches are
    the benchmark's)."""
    _70b_layer(hq, oracle_mod, layer, full=True)


@pytest.mark.timeout(900)
def test_70b_layers_1_to_78_sampled(hq, oracle_mod):
    """Layers 1-78 of the 70B-shaped stack, layer by layer, 1% of the rows of
    every tensor against the oracle."""
    for layer in range(1, 79):
        _70b_layer(hq, oracle_mod, layer, full=False)
