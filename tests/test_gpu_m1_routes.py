"""GPU probes of every one-row-of-x (M = 1) table route, binary and affine, and the cross-kernel
check of the prefill tiles against the one-row kernels.

Each route is first confirmed with the library's launch plan (bonsai_plan), so that a change of
routing cannot silently leave a kernel untested.  On each route:
- poison and guard band: y sits inside NaN padding; nothing outside y is written, every element
  of y is, and y matches the oracle;
- bitwise metamorphic identities: y(-x) = -y(x) and y(x; 2s) = 2 y(x; s) hold bit for bit (every
  step of the table kernels is sign-symmetric and commutes with scaling by 2), flipping every sign
  bit negates y within the acceptance bound;
- one-hot x = e_k for every bit position of the four words of the first, last and slice-boundary
  groups: y[n] = W[n][k] exactly (the oracle's dequantized weight).
"""

import numpy as np
import pytest

import synth
from gpu_util import assert_close, call, note, ref, to_dev, torch_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    pytest.importorskip("torch")
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ternary_weight_quantized_bonsai_amd  # noqa: F401  (fails loudly if not built)


def _plan(op, M, N, K):
    import ternary_weight_quantized_bonsai_amd as bonsai
    return bonsai.plan(op, M, N, K)


# (launcher of the route, N, K): 32-row tiles (one round of the CUs), 64-row tiles, the
# persistent nibble-table kernel, the byte-table kernel (a ragged N, a short last slice, odd G)
BINARY_ROUTES = [
    ("launch_lut4[ROWS = 32", 5000, 5120),
    ("launch_lut4[ROWS = 64", 20000, 640),
    ("launch_lutp", 100003, 5120),
    ("launch_lut8", 160001, 5120),
    ("launch_lut8", 160003, 4224),
]
AFFINE_ROUTES = [
    ("launch_lut4[ROWS = 32", 5000, 5120),
    ("launch_lut4[ROWS = 64", 20000, 640),
    ("launch_lutp", 100003, 4992),
    ("launch_lut8", 160001, 5120),
    ("launch_lut8", 160003, 6272),
]


def _rows(N, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(min(N, 48)), np.arange(max(0, N - 48), N),
                                     rng.integers(0, N, 160)]))


def _affine(w, a, b, x, out=None):
    import ternary_weight_quantized_bonsai_amd as bonsai
    torch, _ = torch_dev()
    note(f"q1a_matmul M={x.shape[0]} N={w.shape[0]} K={x.shape[1]}")
    y = bonsai.q1a_matmul(to_dev(w), to_dev(a), to_dev(b), to_dev(x), out=out)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _affine_magnitude(orc, w, a, b, x, n_idx):
    K = x.shape[1]
    zero = np.zeros_like(a)
    _, mq = orc.q1a_matmul(w, a, zero, x, K, None, n_idx)
    _, mb = orc.q1a_matmul(w, zero, b, x, K, None, n_idx)
    return mq + mb


def _poisoned(fn, M, N):
    """Run fn(y_ptr) with y inside NaN padding; returns y, after checking the padding."""
    torch, dev = torch_dev()
    pad = 64
    buf = torch.full((M * N + 2 * pad,), float("nan"), dtype=torch.float32, device=dev)
    assert fn(buf.data_ptr() + 4 * pad) == 0
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(np.isnan(host[:pad])) and np.all(np.isnan(host[-pad:])), "write outside y"
    y = host[pad:-pad].reshape(M, N)
    assert not np.isnan(y).any(), "element of y left unwritten"
    return y


@pytest.mark.parametrize("route,N,K", BINARY_ROUTES)
def test_binary_m1_route_poison_guard_band(route, N, K, orc):
    assert _plan("q1_gemv", 1, N, K).startswith(route)
    import ternary_weight_quantized_bonsai_amd as bonsai
    torch, _ = torch_dev()
    w, s, x = synth.make_q1(1, N, K, 51, f"route/{N}x{K}")
    wd, sd, xd = to_dev(w), to_dev(s), to_dev(x)
    note(f"poison q1_gemv route {route} N={N} K={K}")
    y = _poisoned(lambda yp: bonsai.raw().bonsai_q1_gemv(wd.data_ptr(), sd.data_ptr(), xd.data_ptr(), yp, 1, N, K,
                                                         torch.cuda.current_stream().cuda_stream), 1, N)
    rows = _rows(N, 52)
    yref, a = ref("q1_gemv", orc, w, s, x, n_idx=rows)
    assert_close(y[:, rows], yref, a, f"{route} poisoned run")


@pytest.mark.parametrize("route,N,K", BINARY_ROUTES)
def test_binary_m1_route_metamorphic_bitwise(route, N, K, orc):
    assert _plan("q1_gemv", 1, N, K).startswith(route)
    w, s, x = synth.make_q1(1, N, K, 53, f"route/{N}x{K}")
    y = call("q1_gemv", w, s, x)
    assert np.array_equal(call("q1_gemv", w, s, x ^ np.uint16(0x8000)), -y)                     # y(-x) = -y(x)
    s2 = (2.0 * s.view(np.float16).astype(np.float32)).astype(np.float16).view(np.uint16)
    assert np.array_equal(call("q1_gemv", w, s2, x), 2.0 * y)                                    # y(2s) = 2 y(s)
    rows = _rows(N, 54)
    yflip = call("q1_gemv", ~w, s, x)                                                            # flipped signs
    yref, a = ref("q1_gemv", orc, w, s, x, n_idx=rows)
    assert_close(-yflip[:, rows], yref, a, f"{route} flipped signs")


def _onehot_positions(K):
    """Every bit of the four words of the first and last groups; bits 0, 7, 8, 15, 16, 23, 24, 31
    (the ends of every byte) of the four words of the groups on either side of each 1024-k slice
    boundary the byte-table kernel crosses (the first three)."""
    G = K // 128
    ends = [128 * g + 32 * j + b for g in (0, G - 1) for j in range(4) for b in range(32)]
    inner = sorted({g for b in (8, 16, 24) for g in (b - 1, b) if 0 < g < G - 1})
    return ends + [128 * g + 32 * j + b for g in inner for j in range(4) for b in (0, 7, 8, 15, 16, 23, 24, 31)]


def _onehot_rows(op, weights, N, K, positions, rows):
    """y[rows] for x = e_k, k in positions, with the weights uploaded once; op is 'q1_gemv' (weights
    = (wbits, scales)) or 'q1a_matmul' (wbits, scales, biases)."""
    import ternary_weight_quantized_bonsai_amd as bonsai
    torch, dev = torch_dev()
    wd = [to_dev(a) for a in weights]
    ridx = torch.from_numpy(rows.astype(np.int64)).to(dev)
    x = torch.zeros((1, K), dtype=torch.int16, device=dev)
    y = torch.empty((1, N), dtype=torch.float32, device=dev)
    out = []
    note(f"one-hot {op} N={N} K={K} ({len(positions)} positions)")
    for k in positions:
        x.zero_()
        x[0, k] = 0x3C00
        if op == "q1_gemv":
            bonsai.q1_gemv(wd[0], wd[1], x, out=y)
        else:
            bonsai.q1a_matmul(wd[0], wd[1], wd[2], x, out=y)
        out.append(y[0].index_select(0, ridx))
    torch.cuda.synchronize()
    return torch.stack(out).cpu().numpy()          # [positions, rows]


@pytest.mark.parametrize("route,N,K", BINARY_ROUTES)
def test_binary_m1_route_onehot(route, N, K, orc):
    assert _plan("q1_gemv", 1, N, K).startswith(route)
    w, s, _ = synth.make_q1(1, N, K, 55, f"route/{N}x{K}")
    # the oracle's dequantized rows: the first and last 64 and a run in the middle
    spans = [(0, min(N, 64)), (N // 2, N // 2 + 64), (max(0, N - 64), N)]
    W = np.concatenate([orc.q1_dequant(w, s, K, a, b) for a, b in spans]).astype(np.float32)
    rows = np.concatenate([np.arange(a, b) for a, b in spans])
    pos = _onehot_positions(K)
    y = _onehot_rows("q1_gemv", (w, s), N, K, pos, rows)
    for i, k in enumerate(pos):
        assert np.array_equal(y[i], W[:, k]), (route, k)


@pytest.mark.parametrize("route,N,K", AFFINE_ROUTES)
def test_affine_m1_route_poison_metamorphic_onehot(route, N, K, orc):
    assert _plan("q1a_matmul", 1, N, K).startswith(route)
    import ternary_weight_quantized_bonsai_amd as bonsai
    torch, _ = torch_dev()
    w, a, b, x = synth.make_q1a(1, N, K, 57, f"aroute/{N}x{K}")
    wd, ad, bd, xd = to_dev(w), to_dev(a), to_dev(b), to_dev(x)
    note(f"poison q1a_matmul route {route} N={N} K={K}")
    y = _poisoned(lambda yp: bonsai.raw().bonsai_q1a_matmul(wd.data_ptr(), ad.data_ptr(), bd.data_ptr(),
                                                            xd.data_ptr(), yp, 1, N, K,
                                                            torch.cuda.current_stream().cuda_stream), 1, N)
    rows = _rows(N, 58)
    yref, _ = orc.q1a_matmul(w, a, b, x, K, None, rows)
    assert_close(y[:, rows], yref, _affine_magnitude(orc, w, a, b, x, rows), f"{route} poisoned run")
    # y(-x) = -y(x) and y(2a, 2b) = 2 y(a, b), bit for bit
    assert np.array_equal(_affine(w, a, b, x ^ np.uint16(0x8000)), -y)
    dbl = lambda v: (2.0 * v.view(np.float16).astype(np.float32)).astype(np.float16).view(np.uint16)  # noqa: E731
    assert np.array_equal(_affine(w, dbl(a), dbl(b), x), 2.0 * y)
    # one-hot x: y[n] = a q + b of weight k, exactly, with power-of-two scales and biases on a
    # grid of 1/8 (every sum the kernel forms is then exact in float32)
    rng = np.random.default_rng(59)
    a1 = (2.0 ** rng.integers(-2, 3, a.shape)).astype(np.float16).view(np.uint16)
    b1 = (rng.integers(-8, 9, b.shape) / 8.0).astype(np.float16).view(np.uint16)
    spans = [(0, min(N, 48)), (max(0, N - 48), N)]
    Wd = np.concatenate([orc.q1a_dequant(w, a1, b1, K, s0, s1) for s0, s1 in spans]).astype(np.float32)
    rws = np.concatenate([np.arange(s0, s1) for s0, s1 in spans])
    G = K // 128
    pos = [128 * g + 32 * j + bit for g in (0, G // 2, G - 1) for j in range(4) for bit in range(32)]
    y1 = _onehot_rows("q1a_matmul", (w, a1, b1), N, K, pos, rws)
    for i, k in enumerate(pos):
        assert np.array_equal(y1[i], Wd[:, k]), (route, k)


# ---- the prefill tiles against the one-row kernels on the same weights and x ------------------
@pytest.mark.parametrize("M,N,K,gemm", [(96, 1000, 2048, "launch_skinny_t"), (512, 1000, 2048, "q1_gemm_kernel"),
                                        (130, 1000, 1152, "q1_gemm_kernel"), (200, 9000, 5120, "q1_gemm_kernel"),
                                        (33, 9000, 5120, "launch_skinny_t")])
def test_prefill_tiles_match_one_row_kernels(M, N, K, gemm, orc):
    """q1_gemm on the matrix cores (the 128 x 256 tiles past 128 rows of x, the skinny GEMM from 17
    to 128) against q1_gemv at M = 1 (the table kernels) on rows of the same x, each against the
    oracle and both against each other."""
    gemm_plan, gemv_plan = _plan("q1_gemm", M, N, K), _plan("q1_gemv", 1, N, K)
    assert gemm_plan.startswith(gemm) and gemv_plan.startswith("launch_lut"), (gemm_plan, gemv_plan)
    w, s, x = synth.make_q1(M, N, K, 61, f"cross/{N}x{K}")
    yg = call("q1_gemm", w, s, x)
    ms = [0, 1, M // 2, M - 1]
    rows = _rows(N, 62)
    yref, a = ref("q1_gemm", orc, w, s, x, m_idx=np.array(ms), n_idx=rows)
    assert_close(yg[np.ix_(ms, rows)], yref, a, "tiles")
    for i, m in enumerate(ms):
        yv = call("q1_gemv", w, s, x[m:m + 1])
        assert_close(yv[:, rows], yref[i:i + 1], a[i:i + 1], f"one-row kernel, row {m} of x")
        assert_close(yg[m:m + 1], yv.astype(np.float64), 2 * orc.q1_matmul(w, s, x[m:m + 1], K)[1],
                     f"tiles vs one-row kernel, row {m}")


def test_prefill_and_decode_configs_share_weights_and_agree(orc):
    """The pp512 workload's weights are the MLP decode projection's (the same seeded stream), and
    the prefill tiles agree with the decode kernel on its rows of X."""
    c4, c2 = synth.CONFIGS["C4"], synth.CONFIGS["C2a"]
    w4, s4, x4 = synth.make_q1(c4.M, c4.N, c4.K)
    w2, s2, _ = synth.make_q1(c2.M, c2.N, c2.K)
    assert np.array_equal(w4, w2) and np.array_equal(s4, s2)
    assert _plan("q1_gemm", c4.M, c4.N, c4.K).startswith("q1_gemm_kernel")
    yg = call("q1_gemm", w4, s4, x4)
    for m in (0, 255, 511):
        yv = call("q1_gemv", w2, s2, x4[m:m + 1])
        _, a = orc.q1_matmul(w2, s2, x4[m:m + 1], c4.K, None, np.arange(0, c4.N, 97))
        assert_close(yg[m:m + 1, ::97], yv[:, ::97].astype(np.float64), 2 * a, f"pp512 row {m} vs decode")
