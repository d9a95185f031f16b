"""GPU parity of the fused dequantize + matmul (hqq_linear, through the C ABI)
against the oracle's linear layer (fp64 sums of X . W_hat^T, W_hat exactly
dequantized).

Bar.  W_hat inside the kernel is bit-exact (the identity-input tests see it
directly).  Each product X[m][k] * W_hat[n][k] of two fp16 values is exact
in fp32, so the kernel's fp32 result differs from the fp64 sum Yref only by
fp32 accumulation, at most K * 2^-24 * A with A = sum_k |X[m][k] W_hat[n][k]|
(the standard bound for any summation order), and the final rounding to fp16
adds at most half an ulp of fp16, 2^-11 relative (2^-25 absolute in the
subnormal range).  The test requires, per output,
    |Y - Yref| <= 2^-11 |Yref| + 1.01 K 2^-24 A + 2^-24 .
Inputs: seeded synthetic fp16 activations and weights; the weights are
quantized by the oracle (or, for the large cases, given random codes and
oracle-style min/max meta), so no input comes from the HIP path.
"""
import numpy as np
import pytest

from helpers import f16_bits_to_f32, random_f16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hq():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import weight_quantization_group_amd as w

    w.load_library()
    return w


def _cuda(a: np.ndarray):
    import torch

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).cuda()


def gpu_linear(hq, X16, packed, scale, zero, N, nbits, gs):
    import torch

    Y = hq.hqq_linear(_cuda(X16), _cuda(packed), _cuda(scale), _cuda(zero), N, nbits, gs)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def random_quantized(oracle_mod, rng, N, K, nbits, gs, solve=True):
    """(packed, scale, zero) of an axis = 1 weight [N, K]: the oracle's solve
    on a synthetic weight, or (solve=False) random codes with min/max meta of a
    synthetic weight (cheap at large sizes)."""
    if solve:
        W16 = random_f16(rng, (N, K), std=0.02, outlier_frac=0.002)
        return oracle_mod.quantize(W16, nbits, gs, 1, iters=4)
    qmax = (1 << nbits) - 1
    codes = rng.randint(0, qmax + 1, size=(N, K)).astype(np.uint8)
    lo = -np.abs(rng.normal(0.03, 0.01, (N, K // gs)))
    hi = np.abs(rng.normal(0.03, 0.01, (N, K // gs))) + 1e-3
    scale = (qmax / (hi - lo)).astype(np.float32)
    zero = (-lo * scale).astype(np.float32)
    return oracle_mod.pack(codes, nbits, 1), scale, zero


def check(Y16, Yref, A, K, tag=""):
    Y = Y16.astype(np.float64)
    assert Y.shape == Yref.shape, tag
    assert np.all(np.isfinite(Y)), tag
    err = np.abs(Y - Yref)
    bound = 2.0 ** -11 * np.abs(Yref) + 1.01 * K * 2.0 ** -24 * A + 2.0 ** -24
    worst = np.max(err / bound)
    assert worst <= 1.0, f"{tag}: worst error / bound = {worst:.3g}"
    return worst


# (M, N, K, nbits, gs): one and several m tiles, ragged M and N, K not a
# multiple of the 128-wide wave step, every supported width, small groups
# (several groups per 32-k lane chunk), the smallest K
CASES = [
    (1, 64, 128, 4, 64),
    (1, 40, 96, 4, 32),
    (7, 100, 256, 4, 64),
    (16, 48, 512, 4, 128),
    (17, 33, 256, 4, 64),
    (32, 64, 512, 4, 256),
    (45, 70, 320, 4, 64),
    (3, 50, 256, 2, 16),
    (9, 24, 160, 2, 32),
    (2, 36, 256, 1, 64),
    (5, 20, 64, 1, 8),
    (4, 30, 256, 8, 128),
    (11, 18, 192, 8, 8),
    (1, 16, 32, 4, 8),
    (1, 1, 32, 4, 16),
    # M >= 384 and K % 64 == 0: the tiled kernel (256 x 128 tiles, table and
    # direct dequantization, ragged M and N); below: the row blocks
    (64, 128, 256, 4, 64),
    (100, 70, 320, 4, 64),
    (130, 200, 192, 2, 16),
    (77, 96, 128, 8, 32),
    (64, 64, 64, 4, 8),
    (96, 130, 512, 4, 32),
    (200, 260, 256, 4, 128),
    (65, 33, 128, 2, 64),
    (128, 128, 512, 8, 256),
    (300, 140, 256, 4, 64),
    (257, 129, 128, 2, 32),
    (512, 256, 320, 8, 64),
    (384, 64, 192, 4, 16),
    (400, 300, 256, 4, 64),
    (513, 130, 128, 2, 32),
    (640, 256, 320, 8, 64),
    (448, 96, 384, 4, 32),      # tiled, 4-bit: two groups per 64-k step
    (390, 140, 512, 4, 128),    # tiled, 4-bit: a group spans two steps
    (400, 70, 64, 4, 64),       # tiled, a single k step
    (390, 40, 64, 8, 32),       # tiled, a single k step, 8-bit
]


@pytest.mark.parametrize("M,N,K,nbits,gs", CASES)
def test_linear_parity(hq, oracle_mod, M, N, K, nbits, gs):
    rng = np.random.RandomState(1000 + M * 7 + N + K + nbits * 13 + gs)
    packed, scale, zero = random_quantized(oracle_mod, rng, N, K, nbits, gs)
    X16 = random_f16(rng, (M, K), std=1.0)
    Y = gpu_linear(hq, X16, packed, scale, zero, N, nbits, gs)
    Yref, A = oracle_mod.linear(X16, packed, scale, zero, N, nbits, gs, with_abs=True)
    check(f16_bits_to_f32(Y.view(np.uint16)), Yref, A, K, f"{M}x{N}x{K} b{nbits} g{gs}")


@pytest.mark.parametrize("nbits,gs", [(4, 64), (2, 16), (1, 32), (8, 128), (4, 8)])
def test_identity_input_gives_dequantized_weights_exactly(hq, oracle_mod, nbits, gs):
    """X = I: Y[m][n] = W_hat[n][m], bit-exact against the oracle's dequantize
    (one nonzero product per output, so the kernel's W_hat is seen directly)."""
    rng = np.random.RandomState(7 + nbits + gs)
    K, N = 256, 40
    packed, scale, zero = random_quantized(oracle_mod, rng, N, K, nbits, gs)
    X = np.zeros((K, K), np.float16)
    np.fill_diagonal(X, 1.0)
    Y = gpu_linear(hq, X.view(np.uint16), packed, scale, zero, N, nbits, gs)
    W_hat = oracle_mod.dequantize(packed, scale, zero, N, K, nbits, gs, 1)
    assert_same_weights(Y.view(np.uint16), W_hat.T)


def test_identity_extreme_meta_exact(hq, oracle_mod):
    """Scales over many binades and zeros far outside the code range: the
    in-kernel quotient (one fp64 product) still matches the fp32 division,
    down to fp16 subnormals.  (Scales stay >= 2^-7 so that no |W_hat| exceeds
    the fp16 range: an infinite weight makes its whole output row NaN through
    0 * inf, in any matmul.)"""
    rng = np.random.RandomState(99)
    K, N, gs, nbits = 128, 64, 32, 4
    codes = rng.randint(0, 16, size=(N, K)).astype(np.uint8)
    scale = (rng.uniform(1, 2, (N, K // gs)) * 2.0 ** rng.randint(-7, 31, (N, K // gs))).astype(np.float32)
    zero = rng.uniform(-300, 300, (N, K // gs)).astype(np.float32)
    packed = oracle_mod.pack(codes, nbits, 1)
    X = np.zeros((K, K), np.float16)
    np.fill_diagonal(X, 1.0)
    Y = gpu_linear(hq, X.view(np.uint16), packed, scale, zero, N, nbits, gs)
    W_hat = oracle_mod.dequantize(packed, scale, zero, N, K, nbits, gs, 1)
    assert_same_weights(Y.view(np.uint16), W_hat.T)


def assert_same_weights(Y_bits, W_bits):
    """Bit-equal, except that a weight of -0 comes out as +0: the output adds
    the +0 products of the zero inputs to it (IEEE: -0 + +0 = +0)."""
    Yf, Wf = f16_bits_to_f32(Y_bits), f16_bits_to_f32(W_bits)
    nz = Wf != 0
    bad = np.argwhere((Y_bits != W_bits) & (nz | (Yf != 0)))
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0]}: {Y_bits[tuple(bad[0])]:#06x} vs {W_bits[tuple(bad[0])]:#06x}"


def test_matches_gpu_dequantize_then_matmul_operand(hq, oracle_mod):
    """The kernel's W_hat equals hqq_dequantize's output: X = e_k picks columns."""
    import torch

    rng = np.random.RandomState(5)
    N, K, nbits, gs = 96, 512, 4, 64
    packed, scale, zero = random_quantized(oracle_mod, rng, N, K, nbits, gs, solve=False)
    Wd = hq.hqq_dequantize(_cuda(packed), _cuda(scale), _cuda(zero), N, K, nbits, gs, 1)
    sel = rng.choice(K, 24, replace=False)
    X = np.zeros((24, K), np.float16)
    X[np.arange(24), sel] = 1.0
    Y = gpu_linear(hq, X.view(np.uint16), packed, scale, zero, N, nbits, gs)
    torch.cuda.synchronize()
    W = Wd.cpu().numpy().view(np.uint16)
    assert_same_weights(Y.view(np.uint16), W[:, sel].T)


# the 7B decoder's linear shapes at one token (decode): q/k/v/o, gate/up, down;
# and batches of rows: M = 96 and 200 take the tiled kernel by its time
# estimate, M = 64 at N = 4096 the row blocks; the tiled kernel runs 128-row
# tiles where they fit the CUs in as few rounds (M = 96 ... 512 here) and
# 256-row tiles at M = 768, N = 11008
@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (1, 11008, 4096), (1, 4096, 11008),
                                   (8, 11008, 4096), (32, 4096, 4096), (512, 4096, 4096),
                                   (256, 11008, 4096), (96, 11008, 4096), (200, 4096, 4096),
                                   (64, 4096, 4096), (768, 11008, 4096)])
def test_linear_full_size(hq, oracle_mod, M, N, K):
    rng = np.random.RandomState(M + N // 7 + K // 5)
    nbits, gs = 4, 64
    packed, scale, zero = random_quantized(oracle_mod, rng, N, K, nbits, gs, solve=False)
    X16 = random_f16(rng, (M, K), std=1.0)
    Y = gpu_linear(hq, X16, packed, scale, zero, N, nbits, gs)
    # the oracle on a sample of output columns (rows of W are independent)
    cols = np.sort(rng.choice(N, min(N, 768 if M <= 32 else 80), replace=False))
    cols[0], cols[-1] = 0, N - 1
    Yref, A = oracle_mod.linear(X16, packed[cols], scale[cols], zero[cols], len(cols), nbits, gs,
                                with_abs=True)
    check(f16_bits_to_f32(Y.view(np.uint16))[:, cols], Yref, A, K, f"{M}x{N}x{K}")


def test_linear_repeat_and_out_buffer(hq, oracle_mod):
    """Two calls into one preallocated output give identical bits, and rows of
    a previous larger result do not leak into a smaller call."""
    import torch

    rng = np.random.RandomState(11)
    N, K, nbits, gs = 64, 256, 4, 64
    packed, scale, zero = random_quantized(oracle_mod, rng, N, K, nbits, gs)
    X16 = random_f16(rng, (20, K), std=1.0)
    args = (_cuda(packed), _cuda(scale), _cuda(zero), N, nbits, gs)
    out = torch.empty((20, N), dtype=torch.float16, device="cuda")
    y1 = hq.hqq_linear(_cuda(X16), *args, out=out).cpu().numpy().copy()
    y2 = hq.hqq_linear(_cuda(X16), *args, out=out).cpu().numpy()
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
    small = hq.hqq_linear(_cuda(X16[:3]), *args).cpu().numpy()
    assert np.array_equal(small.view(np.uint16), y1[:3].view(np.uint16))
    Yref, A = oracle_mod.linear(X16[:3], packed, scale, zero, N, nbits, gs, with_abs=True)
    check(f16_bits_to_f32(small.view(np.uint16)), Yref, A, K, "small after large")


BATCH_CASES = [  # (M, K, nbits, gs, [N of each weight])
    (1, 256, 4, 64, [64, 40, 300]),
    (5, 512, 2, 32, [16, 17, 48, 100]),
    (16, 256, 8, 64, [32, 96]),
    (33, 128, 1, 32, [50, 16, 70]),
    (400, 256, 4, 64, [130, 256, 60]),          # tiled kernel: 128-column tiles
    (1, 256, 4, 16, [16] * 5 + [48] * 6),       # 11 weights: two launches
]


@pytest.mark.parametrize("M,K,nbits,gs,Ns", BATCH_CASES)
def test_linear_batch_equals_single_calls(hq, oracle_mod, M, K, nbits, gs, Ns):
    """hqq_linear_batch gives each weight exactly what hqq_linear gives it
    (bit for bit), and the first weight's output meets the oracle bound."""
    import torch

    rng = np.random.RandomState(M * 31 + K + nbits + len(Ns))
    X16 = random_f16(rng, (M, K), std=1.0, outlier_frac=0.0)
    Xd = _cuda(X16)
    ws = [random_quantized(oracle_mod, rng, N, K, nbits, gs, solve=False) for N in Ns]
    dev = [(_cuda(p), _cuda(s), _cuda(z), N) for (p, s, z), N in zip(ws, Ns)]
    outs = hq.hqq_linear_batch(Xd, dev, nbits, gs)
    torch.cuda.synchronize()
    for (pk, sc, ze, N), Y in zip(dev, outs):
        Y1 = hq.hqq_linear(Xd, pk, sc, ze, N, nbits, gs)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), Y1.view(torch.int16)), (M, N)
    p0, s0, z0 = ws[0]
    Yref, A = oracle_mod.linear(X16, p0, s0, z0, Ns[0], nbits, gs, with_abs=True)
    check(outs[0].cpu().numpy(), Yref, A, K, "batch weight 0")


# ---------------------------------------------------------------------------
# compute dtype bf16 (hqq_linear_ex): X and Y in bf16, W_hat the bf16
# rounding of the same fp32 quotient.  Products of bf16 values are exact in
# fp32; the output rounds once to bf16 (half an ulp: 2^-8 relative), so the
# bound is |Y - Yref| <= 2^-8 |Yref| + 1.01 K 2^-24 A + 2^-133.


def bf16_bits_to_f32(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32)


def random_bf16(rng, shape, std=1.0):
    """bf16 bits of seeded normal values (truncated to bf16: exact inputs)."""
    f = (rng.randn(*shape) * std).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def gpu_linear_bf16(hq, Xb, packed, scale, zero, N, nbits, gs):
    import torch

    X = torch.from_numpy(Xb.view(np.int16)).cuda().view(torch.bfloat16)
    Y = hq.hqq_linear(X, _cuda(packed), _cuda(scale), _cuda(zero), N, nbits, gs)
    torch.cuda.synchronize()
    assert Y.dtype == torch.bfloat16
    return Y.view(torch.int16).cpu().numpy().view(np.uint16)


def check_bf16(Yb, Yref, A, K, tag=""):
    Y = bf16_bits_to_f32(Yb).astype(np.float64)
    assert np.all(np.isfinite(Y)), tag
    err = np.abs(Y - Yref)
    bound = 2.0 ** -8 * np.abs(Yref) + 1.01 * K * 2.0 ** -24 * A + 2.0 ** -133
    worst = np.max(err / bound)
    assert worst <= 1.0, f"{tag}: worst error / bound = {worst:.3g}"


@pytest.mark.parametrize("M,N,K", [(768, 11008, 4096), (300, 4096, 4096)])
def test_linear_bf16_full_size(hq, oracle_mod, M, N, K):
    """bf16 at full size, 256-row tiles (M = 768, N = 11008) and 128-row tiles
    (M = 300), against the oracle on a sample of output columns."""
    rng = np.random.RandomState(7000 + M + N // 7)
    nbits, gs = 4, 64
    packed, scale, zero = random_quantized(oracle_mod, rng, N, K, nbits, gs, solve=False)
    Xb = random_bf16(rng, (M, K))
    Y = gpu_linear_bf16(hq, Xb, packed, scale, zero, N, nbits, gs)
    cols = np.sort(rng.choice(N, 64, replace=False))
    cols[0], cols[-1] = 0, N - 1
    Yref, A = oracle_mod.linear(Xb, packed[cols], scale[cols], zero[cols], len(cols), nbits, gs,
                                with_abs=True, dtype="bf16")
    check_bf16(Y[:, cols], Yref, A, K, f"bf16 {M}x{N}x{K}")


BF16_CASES = list(dict.fromkeys([c for i, c in enumerate(CASES) if i % 3 == 0]
                                + [(400, 300, 256, 4, 64), (640, 256, 320, 8, 64), (390, 140, 512, 4, 128)]))


@pytest.mark.parametrize("M,N,K,nbits,gs", BF16_CASES)
def test_linear_bf16_parity(hq, oracle_mod, M, N, K, nbits, gs):
    rng = np.random.RandomState(5000 + M * 7 + N + K + nbits * 13 + gs)
    packed, scale, zero = random_quantized(oracle_mod, rng, N, K, nbits, gs)
    Xb = random_bf16(rng, (M, K))
    Y = gpu_linear_bf16(hq, Xb, packed, scale, zero, N, nbits, gs)
    Yref, A = oracle_mod.linear(Xb, packed, scale, zero, N, nbits, gs, with_abs=True, dtype="bf16")
    check_bf16(Y, Yref, A, K, f"bf16 {M}x{N}x{K} b{nbits} g{gs}")


@pytest.mark.parametrize("nbits,gs,K", [(4, 64, 256), (2, 16, 256), (8, 128, 256), (4, 32, 384), (1, 32, 256)])
def test_linear_bf16_identity_gives_bf16_w_hat_exactly(hq, oracle_mod, nbits, gs, K):
    """X = I in bf16: Y = the oracle's bf16 dequantization, bit for bit (one
    nonzero product per output; -0 weights come out +0).  K = 384 runs the
    tiled kernel."""
    rng = np.random.RandomState(70 + nbits + gs)
    N = 40
    codes = rng.randint(0, (1 << nbits), size=(N, K)).astype(np.uint8)
    scale = (rng.uniform(1, 2, (N, K // gs)) * 2.0 ** rng.randint(-20, 60, (N, K // gs))).astype(np.float32)
    zero = rng.uniform(-300, 300, (N, K // gs)).astype(np.float32)
    packed = oracle_mod.pack(codes, nbits, 1)
    X = (np.eye(K, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    Y = gpu_linear_bf16(hq, X, packed, scale, zero, N, nbits, gs)
    W = oracle_mod.dequantize(packed, scale, zero, N, K, nbits, gs, 1, dtype="bf16").T
    Yf, Wf = bf16_bits_to_f32(Y), bf16_bits_to_f32(W)
    bad = np.argwhere((Y != W) & ((Wf != 0) | (Yf != 0)))
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0]}"


def test_linear_bf16_batch_equals_single_calls(hq, oracle_mod):
    import torch

    rng = np.random.RandomState(77)
    M, K, nbits, gs, Ns = 3, 256, 4, 64, [64, 100, 32]
    X = torch.from_numpy(random_bf16(rng, (M, K)).view(np.int16)).cuda().view(torch.bfloat16)
    dev = []
    for N in Ns:
        p, s, z = random_quantized(oracle_mod, rng, N, K, nbits, gs, solve=False)
        dev.append((_cuda(p), _cuda(s), _cuda(z), N))
    outs = hq.hqq_linear_batch(X, dev, nbits, gs)
    torch.cuda.synchronize()
    for (pk, sc, ze, N), Y in zip(dev, outs):
        assert Y.dtype == torch.bfloat16
        Y1 = hq.hqq_linear(X, pk, sc, ze, N, nbits, gs)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), Y1.view(torch.int16))


# ---------------------------------------------------------------------------
# split K (hqq_linear_batch_ws): the tiled kernel's K steps divided over 2, 4
# or 8 workgroups per output tile, fp32 partials in the caller's workspace,
# added in split order by a second launch.  The same bound holds (fp32 sums
# in some order); HQQ_LINEAR_SPLITS forces each split count.

SPLIT_CASES = [
    # M, K, nbits, gs, Ns
    (400, 512, 4, 64, [256]),              # 8 steps: 2, 4, 8 splits
    (512, 640, 2, 32, [130]),              # 10 steps: 2 and 4 splits (8 would leave one empty)
    (384, 128, 8, 64, [64]),               # 2 steps: 2 splits
    (400, 512, 4, 32, [130, 256, 60]),     # three weights: per-weight partial slices
    (448, 1024, 4, 128, [96]),             # a group spans two steps
]


@pytest.mark.parametrize("splits", [1, 2, 4, 8])
@pytest.mark.parametrize("M,K,nbits,gs,Ns", SPLIT_CASES)
def test_linear_split_k(hq, oracle_mod, monkeypatch, M, K, nbits, gs, Ns, splits):
    import torch

    steps = K // 64
    per = -(-steps // splits)
    if splits > 1 and (splits - 1) * per >= steps:
        pytest.skip("a split would be empty: the launcher does not use this count")
    monkeypatch.setenv("HQQ_LINEAR_SPLITS", str(splits))
    monkeypatch.setenv("HQQ_LINEAR_PATH", "fused")   # the split-K kernels, not the GEMM route
    rng = np.random.RandomState(M + K * 3 + nbits + gs + len(Ns) * 101)
    X16 = random_f16(rng, (M, K), std=1.0, outlier_frac=0.0)
    Xd = _cuda(X16)
    ws = [random_quantized(oracle_mod, rng, N, K, nbits, gs, solve=False) for N in Ns]
    dev = [(_cuda(p), _cuda(s), _cuda(z), N) for (p, s, z), N in zip(ws, Ns)]
    work = torch.empty(hq.linear_workspace_bytes(M, Ns) // 4, dtype=torch.float32, device="cuda")
    outs = hq.hqq_linear_batch(Xd, dev, nbits, gs, workspace=work)
    torch.cuda.synchronize()
    for (p, s, z), N, Y in zip(ws, Ns, outs):
        Yref, A = oracle_mod.linear(X16, p, s, z, N, nbits, gs, with_abs=True)
        check(Y.cpu().numpy(), Yref, A, K, f"{M}x{N}x{K} b{nbits} g{gs} splits {splits}")
    if splits == 1:
        # no split: exactly the workspace-free call
        ref = hq.hqq_linear_batch(Xd, dev, nbits, gs)
        torch.cuda.synchronize()
        for Y, R in zip(outs, ref):
            assert torch.equal(Y.view(torch.int16), R.view(torch.int16))


@pytest.mark.parametrize("M", [128, 256, 512, 1024])
def test_linear_workspace_auto_mid_rows(hq, oracle_mod, monkeypatch, M):
    """With a workspace and the library's own choice (up to 512 rows the
    fused kernels, which split K over few output tiles; at 1024 rows one
    weight with K <= 4096 takes dequantize + GEMM), the outputs meet the
    bound."""
    import torch

    K, N, nbits, gs = 1024, 512, 4, 64
    rng = np.random.RandomState(M + 7)
    X16 = random_f16(rng, (M, K), std=1.0, outlier_frac=0.0)
    p, s, z = random_quantized(oracle_mod, rng, N, K, nbits, gs, solve=False)
    monkeypatch.delenv("HQQ_LINEAR_PATH", raising=False)
    wb = hq.linear_workspace_bytes(M, [N], K)
    assert hq.hqq_linear_route(M, K, 1, N, wb) == (hq.ROUTE_GEMM if M >= 1024 else hq.ROUTE_FUSED)
    work = torch.empty(wb // 4, dtype=torch.float32, device="cuda")
    (Y,) = hq.hqq_linear_batch(_cuda(X16), [(_cuda(p), _cuda(s), _cuda(z), N)], nbits, gs, workspace=work)
    torch.cuda.synchronize()
    Yref, A = oracle_mod.linear(X16, p, s, z, N, nbits, gs, with_abs=True)
    check(Y.cpu().numpy(), Yref, A, K, f"auto {M}x{N}x{K}")


# The dequantize-then-GEMM route of hqq_linear_batch_ws: each weight's W_hat
# (bit-exact, as hqq_dequantize writes it) goes to the workspace and a
# hipBLASLt GEMM with fp32 accumulation forms X . W_hat^T, so each output is
# an fp32 sum of the exact products in some order, rounded once: the same
# bound as the fused kernels.

GEMM_CASES = [
    # M, K, nbits, gs, Ns
    (1, 256, 4, 64, [128]),
    (33, 128, 1, 32, [96]),
    (64, 1024, 2, 32, [300, 64]),            # two weights, N not a multiple of 8
    (300, 512, 8, 128, [256]),
    (256, 4096, 4, 64, [1024, 512]),
]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("M,K,nbits,gs,Ns", GEMM_CASES)
def test_linear_gemm_route(hq, oracle_mod, monkeypatch, M, K, nbits, gs, Ns, dtype):
    import torch

    monkeypatch.setenv("HQQ_LINEAR_PATH", "gemm")
    rng = np.random.RandomState(M * 7 + K + nbits * 3 + gs + len(Ns))
    if dtype == "bf16":
        Xh = random_bf16(rng, (M, K))
        Xd = torch.from_numpy(Xh.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        Xh = random_f16(rng, (M, K), std=1.0, outlier_frac=0.0)
        Xd = _cuda(Xh)
    ws = [random_quantized(oracle_mod, rng, N, K, nbits, gs, solve=False) for N in Ns]
    dev = [(_cuda(p), _cuda(s), _cuda(z), N) for (p, s, z), N in zip(ws, Ns)]
    work = torch.empty(hq.linear_workspace_bytes(M, Ns, K) // 4, dtype=torch.float32, device="cuda")
    work.fill_(float("nan"))   # stale contents must not leak into the outputs
    outs = hq.hqq_linear_batch(Xd, dev, nbits, gs, workspace=work)
    torch.cuda.synchronize()
    for (p, s, z), N, Y in zip(ws, Ns, outs):
        tag = f"gemm {dtype} {M}x{N}x{K} b{nbits} g{gs}"
        if dtype == "bf16":
            Yref, A = oracle_mod.linear(Xh, p, s, z, N, nbits, gs, with_abs=True, dtype="bf16")
            check_bf16(Y.view(torch.int16).cpu().numpy().view(np.uint16), Yref, A, K, tag)
        else:
            Yref, A = oracle_mod.linear(Xh, p, s, z, N, nbits, gs, with_abs=True)
            check(Y.cpu().numpy(), Yref, A, K, tag)


def test_linear_gemm_route_identity_gives_w_hat(hq, oracle_mod, monkeypatch):
    """X = I through the GEMM route: Y = W_hat^T, bit for bit (one nonzero
    product per output)."""
    import torch

    monkeypatch.setenv("HQQ_LINEAR_PATH", "gemm")
    rng = np.random.RandomState(3)
    K, N, nbits, gs = 256, 192, 4, 64
    packed, scale, zero = random_quantized(oracle_mod, rng, N, K, nbits, gs)
    X = np.eye(K, dtype=np.float16).view(np.uint16)
    work = torch.empty(hq.linear_workspace_bytes(K, [N], K) // 4, dtype=torch.float32, device="cuda")
    (Y,) = hq.hqq_linear_batch(_cuda(X), [(_cuda(packed), _cuda(scale), _cuda(zero), N)], nbits, gs,
                               workspace=work)
    torch.cuda.synchronize()
    W = oracle_mod.dequantize(packed, scale, zero, N, K, nbits, gs, 1)
    assert np.array_equal(Y.cpu().numpy().view(np.uint16), np.ascontiguousarray(W.T))


def test_linear_gemm_route_without_room_is_fused(hq, oracle_mod, monkeypatch):
    """A workspace too small for W_hat: the fused kernels run (bit-identical to
    the workspace-free call), whatever HQQ_LINEAR_PATH asks."""
    import torch

    monkeypatch.setenv("HQQ_LINEAR_PATH", "gemm")
    rng = np.random.RandomState(4)
    M, K, N, nbits, gs = 64, 512, 256, 4, 64
    X16 = random_f16(rng, (M, K), std=1.0, outlier_frac=0.0)
    p, s, z = random_quantized(oracle_mod, rng, N, K, nbits, gs, solve=False)
    dev = [(_cuda(p), _cuda(s), _cuda(z), N)]
    small = torch.empty((N * K * 2 - 256) // 4, dtype=torch.float32, device="cuda")
    (Y,) = hq.hqq_linear_batch(_cuda(X16), dev, nbits, gs, workspace=small)
    (R,) = hq.hqq_linear_batch(_cuda(X16), dev, nbits, gs)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), R.view(torch.int16))


def test_linear_gemm_route_many_row_counts(hq, oracle_mod, monkeypatch):
    """300 distinct row counts through the GEMM route: more shapes than the
    library keeps plans for, so its plan cache starts over on the way; the
    outputs before and after meet the bound."""
    import torch

    monkeypatch.setenv("HQQ_LINEAR_PATH", "gemm")
    rng = np.random.RandomState(12)
    K, N, nbits, gs = 128, 64, 4, 64
    p, s, z = random_quantized(oracle_mod, rng, N, K, nbits, gs, solve=False)
    dev = [(_cuda(p), _cuda(s), _cuda(z), N)]
    X16 = random_f16(rng, (300, K), std=1.0, outlier_frac=0.0)
    Xd = _cuda(X16)
    work = torch.empty(hq.linear_workspace_bytes(300, [N], K) // 4, dtype=torch.float32, device="cuda")
    checked = 0
    for M in range(1, 301):
        (Y,) = hq.hqq_linear_batch(Xd[:M], dev, nbits, gs, workspace=work)
        if M in (1, 7, 255, 256, 257, 300):
            torch.cuda.synchronize()
            Yref, A = oracle_mod.linear(X16[:M], p, s, z, N, nbits, gs, with_abs=True)
            check(Y.cpu().numpy(), Yref, A, K, f"gemm route M={M}")
            checked += 1
    torch.cuda.synchronize()
    assert checked == 6


@pytest.mark.parametrize("path", ["gemm", "fused"])
def test_linear_routes_in_a_replayed_graph(hq, oracle_mod, monkeypatch, path):
    """Both routes captured in a HIP graph (after an eager call, which creates
    the GEMM plan outside capture), replayed three times with eager work and
    synchronizations between the replays: every replay's outputs meet the
    bound and equal the eager call's."""
    import torch

    monkeypatch.setenv("HQQ_LINEAR_PATH", path)
    rng = np.random.RandomState(21)
    M, K, nbits, gs, Ns = 320, 1024, 4, 64, [512, 256]
    X16 = random_f16(rng, (M, K), std=1.0, outlier_frac=0.0)
    Xd = _cuda(X16)
    ws = [random_quantized(oracle_mod, rng, N, K, nbits, gs, solve=False) for N in Ns]
    items = [(_cuda(p), _cuda(s), _cuda(z), N, torch.empty((M, N), dtype=torch.float16, device="cuda"))
             for (p, s, z), N in zip(ws, Ns)]
    work = torch.empty(hq.linear_workspace_bytes(M, Ns, K) // 4, dtype=torch.float32, device="cuda")
    b = hq.LinearBatch(items, nbits, gs, workspace=work)
    eager = [Y.clone() for Y in b.run(Xd)]
    torch.cuda.synchronize()
    refs = [oracle_mod.linear(X16, p, s, z, N, nbits, gs, with_abs=True) for (p, s, z), N in zip(ws, Ns)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            b.run(Xd)
    torch.cuda.synchronize()
    other = torch.randn(512, 512, device="cuda")
    for rep in range(3):
        for it in items:
            it[4].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for it, E, (Yref, A), N in zip(items, eager, refs, Ns):
            Y = it[4]
            check(Y.cpu().numpy(), Yref, A, K, f"{path} replay {rep} N={N}")
            assert torch.equal(Y.view(torch.int16), E.view(torch.int16)), f"{path} replay {rep} differs from eager"
        other = (other @ other).clamp_(-1, 1)   # eager work between replays
        torch.cuda.synchronize()
