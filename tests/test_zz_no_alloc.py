"""sq_w8a8_linear_noalloc (the layer without a workspace, for callers that cannot
allocate) against sq_w8a8_linear on the same inputs: per-token scales and outputs
bit-identical, on consecutive calls whose second input is smaller than the first
(the library's scratch keeps the previous call's contents), on every path: the
MFMA tile GEMM, the decode kernel, the fused one-kernel decode layer, per-token
scales kept in the scratch or returned to the caller, and the largest input the
scratch takes."""
import numpy as np
import pytest
import torch

from gpu_helpers import Guarded, assert_bits_equal, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import int8_quantization_amd as sq
    return sq


def _inputs(seed, M, K, N, dt, smooth, gran, use_bias):
    r = np.random.default_rng(seed)
    X = (r.standard_normal((M, K)) * r.uniform(0.5, 4.0, (M, 1))).astype(dt)
    X[:, r.choice(K, max(1, K // 300), replace=False)] *= 40.0
    s = r.uniform(0.1, 10.0, K).astype(np.float32) if smooth else None
    Wq = r.integers(-127, 128, (N, K), dtype=np.int8)
    ws = (r.uniform(1e-4, 1e-2, N if gran == 0 else 1)).astype(np.float32)
    bias = r.standard_normal(N).astype(np.float32) if use_bias else None
    return X, s, Wq, ws, bias


def _both(sq, case, give_xs):
    seed, M, K, N, dt, smooth, gran, use_bias, out_dt = case
    X, s, Wq, ws, bias = _inputs(seed, M, K, N, dt, smooth, gran, use_bias)
    print(f"no-alloc layer: M={M} K={K} N={N} x={np.dtype(dt).name} smooth={smooth} gran={gran} "
          f"x_scale={'caller' if give_xs else 'scratch'}", flush=True)
    d = [dev(X), None if s is None else dev(s), dev(Wq), dev(ws), None if bias is None else dev(bias)]
    ydt = torch.float16 if out_dt == np.float16 else torch.float32
    # the existing entry point, with its workspace
    Y_ref = Guarded((M, N), ydt)
    xs_ref = Guarded((M,), torch.float32, fill=-1.0)
    wsp = torch.empty(sq.sq_workspace_size(sq.SQ_OP_LINEAR, M, N, K), dtype=torch.uint8, device="cuda")
    sq.sq_w8a8_linear(d[0], d[1], d[2], d[3], gran, d[4], Y_ref.t, wsp, xs_ref.t)
    # the no-allocation entry point
    Y = Guarded((M, N), ydt, fill=7.0)
    xs = Guarded((M,), torch.float32, fill=-1.0) if give_xs else None
    sq.sq_w8a8_linear_noalloc(d[0], d[1], d[2], d[3], gran, d[4], Y.t, None if xs is None else xs.t)
    torch.cuda.synchronize()
    assert_bits_equal(Y.np(), Y_ref.np(), "Y (no-alloc vs workspace)")
    if give_xs:
        assert_bits_equal(xs.np(), xs_ref.np(), "x_scale (no-alloc vs workspace)")


# (seed, M, K, N, x dtype, smoothing, granularity, bias, out dtype): first a larger call,
# then a smaller one on the same path
PAIRS = [
    # MFMA tile GEMM (M > 16)
    ((1, 300, 4096, 1000, np.float16, True, 0, False, np.float16),
     (2, 40, 1040, 520, np.float16, True, 0, True, np.float32)),
    # decode kernel (M <= 16, beyond the fused case)
    ((3, 16, 8192, 4100, np.float16, True, 0, False, np.float16),
     (4, 5, 4096, 777, np.float32, False, 1, True, np.float16)),
    # fused one-kernel decode layer (fp16, M <= 2, K <= 8192), twice
    ((5, 2, 8192, 3000, np.float16, True, 1, False, np.float16),
     (6, 1, 512, 300, np.float16, True, 0, True, np.float32)),
    # the largest input the scratch takes (M * K = 16 MiB), then a small one
    ((7, 2048, 8192, 512, np.float16, True, 0, False, np.float16),
     (8, 3, 64, 48, np.float32, True, 0, False, np.float32)),
]


@pytest.mark.parametrize("give_xs", [False, True])
@pytest.mark.parametrize("pair", range(len(PAIRS)))
def test_noalloc_matches_workspace_layer(sq, pair, give_xs):
    first, second = PAIRS[pair]
    _both(sq, first, give_xs)
    _both(sq, second, give_xs)


def test_noalloc_refuses_beyond_its_scratch(sq):
    """An input beyond the fixed scratch is refused on the host (nothing is enqueued)."""
    M, K, N = 1025, 16384, 16
    X = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    Wq = torch.zeros((N, K), dtype=torch.int8, device="cuda")
    ws = torch.ones(N, dtype=torch.float32, device="cuda")
    Y = torch.zeros((M, N), dtype=torch.float16, device="cuda")
    with pytest.raises(sq.SqError) as e:
        sq.sq_w8a8_linear_noalloc(X, None, Wq, ws, 0, None, Y)
    assert e.value.code == 6          # SQ_ERR_WORKSPACE
