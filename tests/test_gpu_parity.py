"""GPU parity: every entry point against the oracle, through the C ABI, on seeded inputs.

Float results must satisfy |y - y_ref| <= 1e-3 * sum_k |w x| + 1e-6 elementwise.  Exact probes
(one-hot x, integer-valued x with power-of-two scales) must match bit for bit, since every
partial sum is then exactly representable in float32 whatever the summation order.
"""

import numpy as np
import pytest

import synth
from gpu_util import assert_close, call, exact, note, ref, to_dev, torch_dev

pytestmark = pytest.mark.gpu

KINDS = ["q1_gemv", "q1_gemm", "q2t_gemv", "q2t_gemm"]


def make(kind, M, N, K, seed=0, tag=None):
    if kind.startswith("q1"):
        return synth.make_q1(M, N, K, seed, tag)
    return synth.make_q2t(M, N, K, seed, tag)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    pytest.importorskip("torch")
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ternary_weight_quantized_bonsai_amd  # noqa: F401  (fails loudly if not built)


# ---- the workload configurations --------------------------------------------------------
@pytest.mark.parametrize("name", ["C1", "C2a", "C2b", "C5", "C5m8"])
def test_config_full(name, orc):
    c = synth.CONFIGS[name]
    w, s, x = make(c.kind, c.M, c.N, c.K)
    y = call(c.kind, w, s, x)
    yref, a = ref(c.kind, orc, w, s, x)
    assert_close(y, yref, a, name)


def test_config_c3_lm_head_sampled(orc):
    c = synth.CONFIGS["C3"]
    w, s, x = make(c.kind, c.M, c.N, c.K)
    y = call(c.kind, w, s, x)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(c.N - 64, c.N),
                                     rng.choice(c.N, 384, replace=False)]))
    yref, a = ref(c.kind, orc, w, s, x, n_idx=rows)
    assert_close(y[:, rows], yref, a, "C3 sampled rows")


def test_config_c3_popcount_all_rows():
    """x = 1, s = 1 at the LM-head shape: y[n] = 2 popcount(row n) - K, checked on every row."""
    c = synth.CONFIGS["C3"]
    w = synth.sign_words(c.N, c.K // 32, 0, f"{c.N}x{c.K}")
    s = np.full((c.N, c.K // 128), 0x3C00, np.uint16)
    x = np.full((1, c.K), 0x3C00, np.uint16)
    y = call("q1_gemv", w, s, x)
    v = w - ((w >> 1) & np.uint32(0x55555555))
    v = (v & np.uint32(0x33333333)) + ((v >> 2) & np.uint32(0x33333333))
    v = (((v + (v >> 4)) & np.uint32(0x0F0F0F0F)) * np.uint32(0x01010101)) >> 24
    pop = v.astype(np.int64).sum(axis=1)
    assert np.array_equal(y[0], (2 * pop - c.K).astype(np.float32))


# Every row of x (all four 128-row tiles) against about 512 weight rows: the first and the last
# 64 (in the first and last column tiles), one whole 256-column tile in the middle and 128 drawn
# at random, about 4 % of the outputs; the oracle's naive double sums take seconds for them.
@pytest.mark.parametrize("name", ["C4", "C6"])
def test_config_prefill_sampled(name, orc):
    c = synth.CONFIGS[name]
    w, s, x = make(c.kind, c.M, c.N, c.K)
    y = call(c.kind, w, s, x)
    rng = np.random.default_rng(1)
    ms = np.arange(c.M)
    mid = (c.N // 512) * 256
    ns = np.unique(np.concatenate([np.arange(64), np.arange(c.N - 64, c.N), np.arange(mid, mid + 256),
                                   rng.choice(c.N, 128, replace=False)]))
    yref, a = ref(c.kind, orc, w, s, x, m_idx=ms, n_idx=ns)
    assert_close(y[np.ix_(ms, ns)], yref, a, f"{name} sampled")


# ---- integer-valued inputs at full shapes: bit-exact -------------------------------------
def integer_inputs(kind, M, N, K, seed):
    rng = np.random.default_rng(seed)
    w, _, _ = make(kind, 1, N, K, seed, f"int/{N}x{K}")
    s = (2.0 ** rng.integers(-2, 3, (N, K // 128))).astype(np.float16).view(np.uint16)
    x = rng.integers(-8, 9, (M, K)).astype(np.float16).view(np.uint16)
    return w, s, x


@pytest.mark.parametrize("name", ["C2a", "C2b", "C5", "C5m8"])
def test_integer_inputs_bit_exact_full(name, orc):
    c = synth.CONFIGS[name]
    w, s, x = integer_inputs(c.kind, c.M, c.N, c.K, 7)
    y = call(c.kind, w, s, x)
    ye = exact(c.kind, orc, w, s, x).astype(np.float32)
    assert np.array_equal(y, ye)


@pytest.mark.parametrize("name", ["C3", "C4", "C6"])
def test_integer_inputs_bit_exact_sampled(name, orc):
    c = synth.CONFIGS[name]
    w, s, x = integer_inputs(c.kind, c.M, c.N, c.K, 8)
    y = call(c.kind, w, s, x)
    rng = np.random.default_rng(2)
    ns = np.unique(np.concatenate([np.arange(32), np.arange(c.N - 32, c.N), rng.choice(c.N, 96, replace=False)]))
    ms = np.arange(c.M)                                  # every row of x: all row tiles of C4 / C6
    ye = exact(c.kind, orc, w, s, x, m_idx=ms, n_idx=ns).astype(np.float32)
    assert np.array_equal(y[np.ix_(ms, ns)], ye)


# ---- one-hot probes: every bit / field position, bit-exact --------------------------------
def test_q1_gemv_onehot_every_bit(orc):
    N, K = 300, 512
    w, s, _ = make("q1_gemv", 1, N, K, 3, "onehot")
    W = orc.q1_dequant(w, s, K).astype(np.float32)          # +-s, exact in float32
    for k0 in range(0, K, 8):
        x = np.zeros((8, K), np.uint16)
        x[np.arange(8), k0 + np.arange(8)] = 0x3C00
        y = call("q1_gemv", w, s, x)
        assert np.array_equal(y, W[:, k0:k0 + 8].T), k0


def test_q2t_gemv_onehot_every_field(orc):
    N, K = 200, 256
    w, s, _ = make("q2t_gemv", 1, N, K, 4, "onehot")
    W = orc.q2t_dequant(w, s, K).astype(np.float32)
    for k0 in range(0, K, 8):
        x = np.zeros((8, K), np.uint16)
        x[np.arange(8), k0 + np.arange(8)] = 0x3C00
        y = call("q2t_gemv", w, s, x)
        assert np.array_equal(y, W[:, k0:k0 + 8].T), k0


@pytest.mark.parametrize("kind,M", [("q1_gemm", 512), ("q2t_gemm", 512), ("q1_gemm", 70), ("q2t_gemm", 70)])
def test_gemm_identity_gives_dequantized_weights(kind, M, orc):
    """x = the first M rows of the identity: y = the first M columns of the dequantized W^T (the
    128 x 256 tiles at M = 512; the small-M kernel, five 16-row blocks, at M = 70)."""
    N, K = 300, 512
    w, s, _ = make(kind, 1, N, K, 5, f"identity/{kind}")
    x = np.where(np.eye(K, dtype=bool), 0x3C00, 0).astype(np.uint16)[:M]
    y = call(kind, w, s, x)
    deq = orc.q1_dequant if kind.startswith("q1") else orc.q2t_dequant
    assert np.array_equal(y, deq(w, s, K).astype(np.float32).T[:M])


# ---- ragged and edge shapes ---------------------------------------------------------------
EDGE = {
    "q1_gemv": [(1, 1, 128), (1, 63, 256), (1, 65, 384), (3, 1000, 1152), (8, 777, 2048), (5, 64, 128),
                (2, 130, 131072), (1, 4097, 640),
                # M = 1 around the kernel boundaries: 32-row tiles up to N = 8192, 64-row tiles up
                # to six rounds of 256 CUs (N = 98304, and the most groups whose tables fit), then
                # the persistent kernel (odd G, ragged N), and K too long for the tables on the
                # matrix-core kernel (G even and odd)
                (1, 8192, 640), (1, 8193, 640), (1, 16384, 384), (1, 16385, 1152), (1, 20000, 640),
                (1, 40000, 256), (1, 17000, 6144), (1, 98304, 384), (1, 98305, 384), (1, 100003, 640),
                (1, 16500, 8192), (1, 5000, 7808),
                # the persistent kernel past six rounds for long K, past 14 rounds for middling K,
                # and where K is past the 64-row tiles' tables
                (1, 100003, 3712), (1, 230001, 2176), (1, 9000, 6784),
                # 32-row tiles at two groups per lane, up to their 60 groups (G even and odd)
                (1, 3000, 7680), (1, 2999, 7552)],
    "q2t_gemv": [(1, 1, 128), (1, 63, 256), (2, 65, 384), (8, 1000, 1152), (7, 777, 2048),
                 (1, 130, 131072), (4, 4097, 640)],
    # M <= 16 runs the small-M kernel (one 16-row block of x), 17 .. 128 the skinny GEMM (ragged
    # blocks of 32 rows of x), above it the tiles
    "q1_gemm": [(1, 1, 128), (17, 100, 256), (130, 257, 384), (128, 128, 512), (256, 384, 1024),
                (5, 3000, 640), (300, 70, 2048), (16, 40, 131072), (64, 300, 1152), (200, 520, 3200),
                (33, 2000, 1024), (80, 777, 640), (81, 777, 640)],
    # ternary prefill: 512-k chunks, odd G (2-byte scale copies), K not a multiple of 512
    "q2t_gemm": [(1, 1, 128), (17, 100, 256), (130, 257, 384), (128, 128, 512), (256, 384, 1024),
                 (5, 3000, 640), (300, 70, 2048), (16, 40, 131072), (64, 300, 1152), (200, 520, 3200),
                 (33, 2000, 1024), (80, 777, 640), (81, 777, 640)],
}


@pytest.mark.parametrize("kind,M,N,K", [(k, *shape) for k in KINDS for shape in EDGE[k]])
def test_edge_shapes(kind, M, N, K, orc):
    w, s, x = make(kind, M, N, K, 11, f"edge/{kind}/{N}x{K}")
    y = call(kind, w, s, x)
    yref, a = ref(kind, orc, w, s, x)
    assert_close(y, yref, a, f"{kind} {M}x{N}x{K}")


# The small-M matrix-core kernel picks, per call, a slice width (four or two groups of K), a row
# tile (16, 32 or 64 rows) and, from the parity of K / 128, paired or single scale copies; a slice
# width that does not divide K / 128 leaves a partial last slice.  These shapes were chosen so that
# the launcher's choices, as they stand, reach every such combination of each weight form (no
# 64-row tile for the affine form).  Whatever the launcher picks, each case is checked against the
# oracle on sampled rows.  (From 17 rows of x the binary and ternary GEMM entry points take the
# skinny GEMM instead, tested below; the affine form keeps the small-M kernel there.)
SMALL_M_VARIANTS = sorted({(2, 33, 128), (2, 33, 256), (2, 5000, 128), (2, 5000, 256), (2, 13824, 128),
                           (2, 13824, 256), (2, 33, 1152), (16, 33, 5120), (2, 33, 1280), (2, 5000, 1152),
                           (2, 5000, 1280), (2, 13824, 1152), (2, 13824, 1280), (33, 1500, 5120),
                           (33, 3000, 5120), (12, 5000, 5120), (12, 9000, 5120), (3, 9000, 5120)})


def _sampled_rows(N, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(min(N, 40)), np.arange(max(0, N - 40), N),
                                     rng.integers(0, N, 200)]))


@pytest.mark.parametrize("form", ["binary", "ternary", "affine"])
@pytest.mark.parametrize("M,N,K", SMALL_M_VARIANTS)
def test_small_m_kernel_variants(form, M, N, K, orc):
    rows = _sampled_rows(N, 91)
    if form == "affine":
        w, a, b, x = synth.make_q1a(M, N, K, 91, f"smv{N}x{K}")
        y = _affine(w, a, b, x)
        yref, _ = orc.q1a_matmul(w, a, b, x, K, None, rows)
        assert_close(y[:, rows], yref, _affine_magnitude(orc, w, a, b, x, None, rows),
                     f"q1a M={M} N={N} K={K}")
        return
    kind = ("q1" if form == "binary" else "q2t") + ("_gemv" if M <= 8 else "_gemm")
    w, s, x = make(kind, M, N, K, 91, f"smv{N}x{K}")
    y = call(kind, w, s, x)
    yref, a = ref(kind, orc, w, s, x, n_idx=rows)
    assert_close(y[:, rows], yref, a, f"{kind} M={M} N={N} K={K}")


# The skinny GEMM (17 to 128 rows of x through the GEMM entry points): one, two and four blocks of
# 32 rows of x, ragged M and N, and K split over its four waves unevenly (K / 128 = 11: 2, 3, 3, 3
# groups, which leave one or two groups after whole triples), with waves left idle (K / 128 = 1
# and 3) and with a long K.  Random inputs against the oracle's tolerance, integer-valued inputs
# bit for bit (every partial sum is exact in float32).
SKINNY_SHAPES = [(17, 100, 128), (32, 64, 384), (33, 1000, 1408), (48, 777, 1152), (64, 2000, 5120),
                 (65, 300, 640), (96, 129, 2560), (128, 128, 16384), (100, 65, 1280)]


@pytest.mark.parametrize("kind", ["q1_gemm", "q2t_gemm"])
@pytest.mark.parametrize("M,N,K", SKINNY_SHAPES)
def test_skinny_gemm_shapes(kind, M, N, K, orc):
    import ternary_weight_quantized_bonsai_amd as bonsai
    assert bonsai.plan(kind, M, N, K).startswith("launch_skinny_t")
    note(f"skinny {kind} M={M} N={N} K={K}")
    rows = _sampled_rows(N, 94)
    w, s, x = make(kind, M, N, K, 93, f"sk/{N}x{K}")
    y = call(kind, w, s, x)
    yref, a = ref(kind, orc, w, s, x, n_idx=rows)
    assert_close(y[:, rows], yref, a, f"skinny {kind} {M}x{N}x{K}")
    wi, si, xi = integer_inputs(kind, M, N, K, 95)
    yi = call(kind, wi, si, xi)
    ye = exact(kind, orc, wi, si, xi, n_idx=rows).astype(np.float32)
    assert np.array_equal(yi[:, rows], ye), f"skinny {kind} {M}x{N}x{K} integer inputs"


@pytest.mark.parametrize("kind", KINDS)
def test_every_m_from_1_to_8(kind, orc):
    for M in range(1, 9):
        w, s, x = make(kind, M, 193, 640, 12 + M, f"m/{kind}/{M}")
        y = call(kind, w, s, x)
        yref, a = ref(kind, orc, w, s, x)
        assert_close(y, yref, a, f"{kind} M={M}")


# ---- poison, canaries, empty products, K = 0 ----------------------------------------------
def raw_call(kind, w_t, s_t, x_t, y_ptr, M, N, K):
    import ternary_weight_quantized_bonsai_amd as bonsai
    torch, _ = torch_dev()
    f = getattr(bonsai.raw(), "bonsai_" + kind)
    st = f(w_t.data_ptr() if w_t is not None else None, s_t.data_ptr() if s_t is not None else None,
           x_t.data_ptr() if x_t is not None else None, y_ptr, M, N, K,
           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return st


@pytest.mark.parametrize("kind,M,N,K", [("q1_gemv", 3, 1001, 640), ("q2t_gemv", 8, 333, 384),
                                        ("q1_gemm", 131, 259, 512), ("q2t_gemm", 131, 259, 640)])
def test_poison_and_guard_band(kind, M, N, K, orc):
    torch, dev = torch_dev()
    w, s, x = make(kind, M, N, K, 21, f"poison/{kind}")
    pad = 64                                                   # floats on each side (256 B)
    buf = torch.full((M * N + 2 * pad,), float("nan"), dtype=torch.float32, device=dev)
    note(f"poison {kind} M={M} N={N} K={K}")
    st = raw_call(kind, to_dev(w), to_dev(s), to_dev(x), buf.data_ptr() + 4 * pad, M, N, K)
    assert st == 0
    host = buf.cpu().numpy()
    assert np.all(np.isnan(host[:pad])) and np.all(np.isnan(host[-pad:])), "write outside y"
    y = host[pad:-pad].reshape(M, N)
    assert not np.isnan(y).any(), "element of y left unwritten"
    yref, a = ref(kind, orc, w, s, x)
    assert_close(y, yref, a, "poisoned run")


@pytest.mark.parametrize("kind", KINDS)
def test_empty_products_and_k0(kind):
    torch, dev = torch_dev()
    buf = torch.full((64,), float("nan"), dtype=torch.float32, device=dev)
    note(f"empty {kind}")
    assert raw_call(kind, None, None, None, buf.data_ptr(), 0, 16, 128) == 0
    assert raw_call(kind, None, None, None, buf.data_ptr(), 4, 0, 128) == 0
    assert torch.isnan(buf).all()
    assert raw_call(kind, None, None, None, buf.data_ptr(), 4, 8, 0) == 0
    host = buf.cpu().numpy()
    assert np.all(host[:32] == 0) and np.all(np.isnan(host[32:]))


# ---- determinism, symmetry, cross-kernel consistency --------------------------------------
@pytest.mark.parametrize("name", ["C2a", "C4", "C5m8", "C6"])
def test_bitwise_deterministic(name):
    c = synth.CONFIGS[name]
    w, s, x = make(c.kind, c.M, c.N, c.K)
    assert np.array_equal(call(c.kind, w, s, x), call(c.kind, w, s, x))


@pytest.mark.parametrize("kind,M,N,K", [("q1_gemv", 2, 2000, 5120), ("q1_gemm", 96, 700, 1024),
                                        ("q2t_gemv", 8, 1500, 2048), ("q2t_gemm", 96, 700, 1024)])
def test_metamorphic(kind, M, N, K, orc):
    w, s, x = make(kind, M, N, K, 31, f"meta/{kind}")
    y = call(kind, w, s, x)
    yneg = call(kind, w, s, x ^ np.uint16(0x8000))                                # y(-x) = -y(x)
    if kind.endswith("gemm"):
        # The matrix cores' float32 accumulation is not sign-symmetric bit for bit: -y(-x) and
        # y(x) differ in some elements, by an amount that scales with the sum's magnitude
        # A = sum_k |w x| (measured bound below, in units of 2^-24 A), and both meet the
        # acceptance bound against the oracle.
        yref, a = ref(kind, orc, w, s, x)
        assert_close(-yneg, yref, a, "negated x")
        d = np.abs(-yneg.astype(np.float64) - y.astype(np.float64)) / (2.0 ** -24 * a)
        note(f"{kind} y(-x) vs -y(x): {int((d > 0).sum())} of {d.size} differ, max {d.max():.2f} x 2^-24 A, "
             f"max {int(ulp_distance(-yneg, y).max())} ulp of y")
        assert d.max() <= GEMM_SIGN_BOUND
    else:
        assert np.array_equal(yneg, -y)
    s2 = (2.0 * s.view(np.float16).astype(np.float32)).astype(np.float16).view(np.uint16)
    assert np.array_equal(call(kind, w, s2, x), 2.0 * y)                          # y(2s) = 2 y(s)
    if kind.startswith("q1"):
        yflip = call(kind, ~w, s, x)                                              # flipped signs
        yref, a = ref(kind, orc, w, s, x)
        assert_close(-yflip, yref, a, "flipped signs")


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Units in the last place between float32 arrays (the distance of their ordered bit patterns)."""
    def ordered(v):
        i = np.ascontiguousarray(v, dtype=np.float32).view(np.int32).astype(np.int64)
        return np.where(i < 0, -(i & 0x7FFFFFFF), i)
    return np.abs(ordered(a) - ordered(b))


# The largest |-y(-x) - y(x)| the matrix-core GEMMs are allowed, in units of 2^-24 sum_k |w x|.
GEMM_SIGN_BOUND = 2.0


def test_gemm_matches_gemv_on_the_same_rows(orc):
    M, N, K = 8, 1000, 2048
    w, s, x = make("q1_gemm", M, N, K, 41, "cross")
    yg = call("q1_gemm", w, s, x)
    yv = call("q1_gemv", w, s, x)
    yref, a = ref("q1_gemm", orc, w, s, x)
    assert_close(yg, yref, a, "gemm")
    assert_close(yv, yref, a, "gemv")
    assert_close(yg, yv.astype(np.float64), 2 * a, "gemm vs gemv")


# ---- base-3 ternary (five trits per byte) ------------------------------------------------------
def _t5(codes, s, x):
    import ternary_weight_quantized_bonsai_amd as bonsai
    torch, dev = torch_dev()
    note(f"t5_matmul M={x.shape[0]} N={codes.shape[0]} K={x.shape[1]}")
    y = bonsai.t5_matmul(torch.from_numpy(codes).to(dev), to_dev(s), to_dev(x))
    torch.cuda.synchronize()
    return y.cpu().numpy()


T5_SHAPES = [(1, 256, 640), (1, 300, 384), (2, 1000, 1152), (8, 2000, 1024), (16, 777, 768),
             (17, 500, 1280), (3, 130, 13824), (1, 5, 128), (40, 96, 896),
             # the largest K the library accepts (820 superblocks, several slices per wave), and
             # many 16-row blocks of x
             (1, 40, 131072), (5, 33, 131072), (200, 70, 640)]


@pytest.mark.parametrize("M,N,K", T5_SHAPES)
def test_t5_matmul_vs_oracle(M, N, K, orc):
    codes, s, x = synth.make_t5(M, N, K, 71, f"t5{N}x{K}")
    y = _t5(codes, s, x)
    yref, a = orc.t5_matmul(codes, s, x, K)
    assert_close(y, yref, a, f"t5 M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(1, 5120, 5120), (8, 5120, 5120), (1, 5120, 13824)])
def test_t5_matmul_decode_shapes_sampled(M, N, K, orc):
    codes, s, x = synth.make_t5(M, N, K, 0, f"t5{N}x{K}")
    y = _t5(codes, s, x)
    rng = np.random.default_rng(72)
    n_idx = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 200)]))
    yref, a = orc.t5_matmul(codes, s, x, K, None, n_idx)
    assert_close(y[:, n_idx], yref, a, "t5 sampled")


@pytest.mark.parametrize("M,N,K", [(1, 300, 640), (5, 260, 1152), (20, 129, 384)])
def test_t5_integer_inputs_bit_exact(M, N, K, orc):
    """Small integer x and power-of-two scales: exact partial sums, so bit for bit."""
    rng = np.random.default_rng(73 + M)
    codes = synth.t5_bytes(N, K, 73, f"t5int{N}x{K}")
    s = (2.0 ** rng.integers(-3, 4, (N, K // 128))).astype(np.float16).view(np.uint16)
    x = rng.integers(-8, 9, (M, K)).astype(np.float16).view(np.uint16)
    y = _t5(codes, s, x)
    yref, _ = orc.t5_matmul(codes, s, x, K)
    assert np.array_equal(y.astype(np.float64), yref)


def test_t5_onehot_every_digit(orc):
    """x = e_k for every k of two superblocks and a ragged third: y = W[:, k] exactly."""
    N, K = 40, 384
    codes, s, _ = synth.make_t5(1, N, K, 74, "t5onehot")
    x = np.eye(K, dtype=np.float16).view(np.uint16)
    y = _t5(codes, s, x)
    assert np.array_equal(y.astype(np.float64), orc.t5_dequant(codes, s, K).T)


def test_t5_matches_two_bit_ternary_on_the_same_trits(orc):
    """The same trits in both ternary layouts give the same products (integer data: bit for bit)."""
    import ternary_weight_quantized_bonsai_amd as bonsai
    M, N, K = 4, 700, 1280
    rng = np.random.default_rng(75)
    t = synth.trits_i8(N, K, 75, "t5vsq2t")
    s = (2.0 ** rng.integers(-2, 3, (N, K // 128))).astype(np.float16).view(np.uint16)
    x = rng.integers(-8, 9, (M, K)).astype(np.float16).view(np.uint16)
    y5 = _t5(bonsai.t5_pack(t), s, x)
    y2 = call("q2t_gemv", bonsai.q2t_pack(t), s, x)
    assert np.array_equal(y5, y2)


def test_t5_poison_guard_and_empty(orc):
    import ternary_weight_quantized_bonsai_amd as bonsai
    torch, dev = torch_dev()
    M, N, K = 9, 131, 768
    codes, s, x = synth.make_t5(M, N, K, 76, "t5poison")
    buf = torch.full((M * N + 64,), float("nan"), dtype=torch.float32, device=dev)
    cd, sd, xd = torch.from_numpy(codes).to(dev), to_dev(s), to_dev(x)
    note(f"t5_matmul poison M={M} N={N} K={K}")
    st = bonsai.raw().bonsai_t5_matmul(cd.data_ptr(), sd.data_ptr(), xd.data_ptr(), buf.data_ptr(), M, N, K,
                                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == bonsai.OK
    host = buf.cpu().numpy()
    yref, a = orc.t5_matmul(codes, s, x, K)
    assert_close(host[:M * N].reshape(M, N), yref, a, "t5 poison")
    assert np.isnan(host[M * N:]).all()
    out = torch.full((3, 5), 7.0, dtype=torch.float32, device=dev)
    assert bonsai.raw().bonsai_t5_matmul(0, 0, 0, out.data_ptr(), 3, 5, 0, None) == bonsai.OK
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == 0).all()


# ---- affine 1-bit (MLX's scale-and-bias form) ------------------------------------------------
def _affine(w, a, b, x):
    import ternary_weight_quantized_bonsai_amd as bonsai
    torch, _ = torch_dev()
    note(f"q1a_matmul M={x.shape[0]} N={w.shape[0]} K={x.shape[1]}")
    y = bonsai.q1a_matmul(to_dev(w), to_dev(a), to_dev(b), to_dev(x))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _affine_magnitude(orc, w, a, b, x, m_idx=None, n_idx=None):
    """sum_k |a q x| + |b x|: the size of the two terms the kernel sums separately (oracle)."""
    K = x.shape[1]
    zero = np.zeros_like(a)
    _, mq = orc.q1a_matmul(w, a, zero, x, K, m_idx, n_idx)
    _, mb = orc.q1a_matmul(w, zero, b, x, K, m_idx, n_idx)
    return mq + mb


AFFINE_SHAPES = [(1, 256, 512), (1, 300, 640), (2, 1000, 1152), (8, 2000, 1024), (16, 777, 640),
                 (17, 500, 1152), (33, 130, 384), (80, 300, 896), (1, 5, 128),
                 (1, 40, 131072), (6, 33, 131072), (200, 70, 640),
                 # one row of x on the table kernels: 64-row tiles (N > 8192), G even and odd
                 (1, 9000, 1024), (1, 9000, 1152), (1, 20000, 640)]


@pytest.mark.parametrize("M,N,K", AFFINE_SHAPES)
def test_affine_matmul_vs_oracle(M, N, K, orc):
    w, a, b, x = synth.make_q1a(M, N, K, 61, f"aff{N}x{K}")
    y = _affine(w, a, b, x)
    yref, _ = orc.q1a_matmul(w, a, b, x, K)
    assert_close(y, yref, _affine_magnitude(orc, w, a, b, x), f"q1a M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(1, 5120, 5120), (8, 13824, 5120),
                                   # one row of x past six rounds of 64-row tiles (ragged N, odd G)
                                   (1, 100003, 1152),
                                   # the persistent table kernel: paired and single scale copies,
                                   # and K past the 64-row tiles' tables at small N
                                   (1, 248320, 5120), (1, 110001, 4224), (1, 9000, 6528),
                                   # short K: the persistent kernel only past 12 rounds of tiles
                                   (1, 200003, 1152)])
def test_affine_matmul_decode_shapes_sampled(M, N, K, orc):
    w, a, b, x = synth.make_q1a(M, N, K, 0, f"aff{N}x{K}")
    y = _affine(w, a, b, x)
    rng = np.random.default_rng(62)
    n_idx = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 300)]))
    yref, _ = orc.q1a_matmul(w, a, b, x, K, None, n_idx)
    assert_close(y[:, n_idx], yref, _affine_magnitude(orc, w, a, b, x, None, n_idx), "q1a sampled")


@pytest.mark.parametrize("M,N,K", [(1, 5120, 5120), (5, 700, 896), (24, 300, 640)])
def test_affine_bonsai_packing_matches_binary(M, N, K, orc):
    """The binary weights carried as (2 s, -s) give the binary product (model card, 'MLX packaging')."""
    import ternary_weight_quantized_bonsai_amd as bonsai
    w, s, x = synth.make_q1(M, N, K, 63, f"affpk{N}x{K}")
    a, b = bonsai.q1_to_affine(s)
    y = _affine(w, a, b, x)
    yref, mag = orc.q1_matmul(w, s, x, K)
    assert_close(y, yref, 3 * mag, "q1a as binary")


@pytest.mark.parametrize("M,N,K", [(1, 300, 640), (1, 9000, 1024), (7, 260, 1024), (20, 129, 384),
                                   (1, 110000, 4352)])
def test_affine_integer_inputs_bit_exact(M, N, K, orc):
    """Small integer x, scales and biases: every partial sum is exact in float32, so the kernel
    must equal the exact result bit for bit."""
    rng = np.random.default_rng(64 + M)
    w = synth.sign_words(N, K // 32, 64, f"affint{N}x{K}")
    f16 = lambda v: v.astype(np.float16).view(np.uint16)
    a = f16(rng.integers(-4, 5, (N, K // 128)))
    b = f16(rng.integers(-4, 5, (N, K // 128)))
    x = f16(rng.integers(-8, 9, (M, K)))
    y = _affine(w, a, b, x)
    yref, _ = orc.q1a_matmul(w, a, b, x, K)
    assert np.array_equal(y.astype(np.float64), yref)


def test_affine_poison_guard_and_empty(orc):
    """Only y[:M, :N] is written; M = 0 / N = 0 are no-ops; K = 0 writes zeros."""
    import ternary_weight_quantized_bonsai_amd as bonsai
    torch, dev = torch_dev()
    M, N, K = 9, 131, 640
    w, a, b, x = synth.make_q1a(M, N, K, 65, "affpoison")
    buf = torch.full((M * N + 64,), float("nan"), dtype=torch.float32, device=dev)
    wd, ad, bd, xd = to_dev(w), to_dev(a), to_dev(b), to_dev(x)
    note(f"q1a_matmul poison M={M} N={N} K={K}")
    st = bonsai.raw().bonsai_q1a_matmul(wd.data_ptr(), ad.data_ptr(), bd.data_ptr(), xd.data_ptr(),
                                        buf.data_ptr(), M, N, K, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == bonsai.OK
    host = buf.cpu().numpy()
    yref, _ = orc.q1a_matmul(w, a, b, x, K)
    assert_close(host[:M * N].reshape(M, N), yref, _affine_magnitude(orc, w, a, b, x), "q1a poison")
    assert np.isnan(host[M * N:]).all()
    out = torch.full((3, 5), 7.0, dtype=torch.float32, device=dev)
    assert bonsai.raw().bonsai_q1a_matmul(0, 0, 0, 0, out.data_ptr(), 3, 5, 0, None) == bonsai.OK
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == 0).all()


# ---- embedding gather ---------------------------------------------------------------------
def _embed(w, s, ids):
    import ternary_weight_quantized_bonsai_amd as bonsai
    torch, dev = torch_dev()
    note(f"q1_embed n={ids.size} V={w.shape[0]} K={w.shape[1] * 32}")
    out = bonsai.q1_embed(to_dev(w), to_dev(s), torch.from_numpy(ids).to(dev))
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


def _embed_ref(orc, w, s, ids, K):
    V = w.shape[0]
    ref = np.zeros((ids.size, K), np.uint16)
    for i, r in enumerate(ids):
        if 0 <= r < V:
            ref[i] = orc.q1_dequant(w, s, K, int(r), int(r) + 1)[0].astype(np.float16).view(np.uint16)
    return ref


def test_embed_gather_bit_exact(orc):
    """Rows of +-s exactly (binary16), odd G, ids out of range give zero rows."""
    V, K = 1000, 640
    w, s, _ = make("q1_gemv", 1, V, K, 51, "embed")
    rng = np.random.default_rng(5)
    ids = np.concatenate([[0, V - 1, -1, V, 1 << 40], rng.integers(0, V, 300)]).astype(np.int64)
    assert np.array_equal(_embed(w, s, ids), _embed_ref(orc, w, s, ids, K))


def test_embed_gather_vocab_shape(orc):
    """The LM-head table shape (V = 248320, K = 5120), 512 sampled ids."""
    V, K = 248320, 5120
    w, s, _ = make("q1_gemv", 1, V, K, 0, f"{V}x{K}")
    ids = np.random.default_rng(6).integers(0, V, 512).astype(np.int64)
    assert np.array_equal(_embed(w, s, ids), _embed_ref(orc, w, s, ids, K))


# ---- HIP graph capture ------------------------------------------------------------------------
def test_graph_capture_and_replay_of_every_entry_point(orc):
    """Each matmul entry point captured in one HIP graph (on torch's capture stream), replayed
    several times with eager work and synchronisations between the replays; every replay must
    equal the eager result bit for bit, and the eager result must meet the oracle."""
    import ternary_weight_quantized_bonsai_amd as bonsai
    torch, dev = torch_dev()
    calls = []
    w, s, x = synth.make_q1(1, 700, 1024, 81, "graph/q1")
    calls.append(("q1_gemv M=1", bonsai.q1_gemv, (to_dev(w), to_dev(s), to_dev(x)), orc.q1_matmul(w, s, x, 1024)))
    w, s, x = synth.make_q1(5, 700, 1024, 82, "graph/q1m")
    calls.append(("q1_gemv M=5", bonsai.q1_gemv, (to_dev(w), to_dev(s), to_dev(x)), orc.q1_matmul(w, s, x, 1024)))
    w, s, x = synth.make_q1(130, 300, 768, 83, "graph/gemm")
    calls.append(("q1_gemm M=130", bonsai.q1_gemm, (to_dev(w), to_dev(s), to_dev(x)), orc.q1_matmul(w, s, x, 768)))
    w, s, x = synth.make_q1(40, 700, 1408, 88, "graph/skinny")             # the skinny GEMM
    calls.append(("q1_gemm M=40", bonsai.q1_gemm, (to_dev(w), to_dev(s), to_dev(x)), orc.q1_matmul(w, s, x, 1408)))
    w, s, x = synth.make_q1(1, 160001, 2048, 89, "graph/lut8")             # the byte tables
    calls.append(("q1_gemv M=1 N=160001", bonsai.q1_gemv, (to_dev(w), to_dev(s), to_dev(x)),
                  orc.q1_matmul(w, s, x, 2048)))
    w, s, x = synth.make_q2t(3, 500, 640, 84, "graph/q2t")
    calls.append(("q2t_gemv M=3", bonsai.q2t_gemv, (to_dev(w), to_dev(s), to_dev(x)), orc.q2t_matmul(w, s, x, 640)))
    w, s, x = synth.make_q2t(100, 300, 640, 85, "graph/q2tg")
    calls.append(("q2t_gemm M=100", bonsai.q2t_gemm, (to_dev(w), to_dev(s), to_dev(x)), orc.q2t_matmul(w, s, x, 640)))
    c, s, x = synth.make_t5(2, 400, 1152, 86, "graph/t5")
    calls.append(("t5_matmul M=2", bonsai.t5_matmul, (torch.from_numpy(c).to(dev), to_dev(s), to_dev(x)),
                  orc.t5_matmul(c, s, x, 1152)))
    w, a, b, x = synth.make_q1a(4, 300, 640, 87, "graph/q1a")
    calls.append(("q1a_matmul M=4", bonsai.q1a_matmul, (to_dev(w), to_dev(a), to_dev(b), to_dev(x)),
                  (orc.q1a_matmul(w, a, b, x, 640)[0], _affine_magnitude(orc, w, a, b, x))))
    w, a, b, x = synth.make_q1a(1, 160001, 2048, 90, "graph/lut8a")       # the affine byte tables
    calls.append(("q1a_matmul M=1 N=160001", bonsai.q1a_matmul, (to_dev(w), to_dev(a), to_dev(b), to_dev(x)),
                  (orc.q1a_matmul(w, a, b, x, 2048)[0], _affine_magnitude(orc, w, a, b, x))))
    outs = [torch.empty((args[-1].shape[0], args[0].shape[0]), dtype=torch.float32, device=dev)
            for _, _, args, _ in calls]
    note("graph: eager reference run")
    eager = []
    for (name, fn, args, (yref, mag)), out in zip(calls, outs):
        fn(*args, out=out)
        torch.cuda.synchronize()
        eager.append(out.clone())
        assert_close(out.cpu().numpy(), yref, mag, f"eager {name}")
    note("graph: capture")
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for out in outs:
            out.fill_(float("nan"))
        with torch.cuda.graph(g, stream=stream):
            for (name, fn, args, _), out in zip(calls, outs):
                fn(*args, out=out)
    torch.cuda.synchronize()
    for rep in range(4):
        note(f"graph: replay {rep}")
        for out in outs:
            out.fill_(float("nan"))               # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (name, _, _, _), out, ref in zip(calls, outs, eager):
            assert torch.equal(out, ref), f"replay {rep}: {name} differs from the eager result"


# ---- seeded random shapes over every entry point ----------------------------------------
# Beside the hand-picked boundary shapes: shapes drawn from a fixed generator, so that routing
# combinations nobody listed (table kernels, slice widths, tiles, passes over 16-row blocks of x,
# ragged tails) get exercised.  Sizes are capped so the whole set runs in seconds; each case is
# checked against the oracle on sampled rows.
def _random_shapes(kind, count, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        # one row of x half of the time where it has kernels of its own (the table GEMVs)
        if kind in ("q1_gemv", "q2t_gemv"):
            M = 1 if rng.random() < 0.5 else int(rng.integers(2, 9))
        elif kind in ("q1_gemm", "q2t_gemm"):
            M = int(rng.choice([rng.integers(1, 97), rng.integers(97, 600)]))
        elif kind == "q1a_matmul":
            M = 1 if rng.random() < 0.5 else int(rng.integers(2, 41))
        else:
            M = int(rng.integers(1, 41))
        N = int(np.exp(rng.uniform(0.0, np.log(30000.0)))) + 1
        K = 128 * int(rng.integers(1, 71))
        if N * K <= 40_000_000 and M * N <= 2_000_000 and M * K <= 2_000_000:
            out.append((M, N, K))
    return out


RANDOM_CASES = [(kind, *shape) for i, kind in enumerate(KINDS + ["t5_matmul", "q1a_matmul"])
                for shape in _random_shapes(kind, 10, 1000 + i)]


@pytest.mark.parametrize("kind,M,N,K", RANDOM_CASES)
def test_random_shapes(kind, M, N, K, orc):
    rows = _sampled_rows(N, 7)
    tag = f"rnd{N}x{K}"
    if kind == "t5_matmul":
        codes, s, x = synth.make_t5(M, N, K, 7, tag)
        y = _t5(codes, s, x)
        yref, a = orc.t5_matmul(codes, s, x, K, None, rows)
    elif kind == "q1a_matmul":
        w, sa, b, x = synth.make_q1a(M, N, K, 7, tag)
        y = _affine(w, sa, b, x)
        yref, _ = orc.q1a_matmul(w, sa, b, x, K, None, rows)
        a = _affine_magnitude(orc, w, sa, b, x, None, rows)
    else:
        w, s, x = make(kind, M, N, K, 7, tag)
        y = call(kind, w, s, x)
        yref, a = ref(kind, orc, w, s, x, n_idx=rows)
    assert_close(y[:, rows], yref, a, f"{kind} M={M} N={N} K={K}")


# ---- concurrency: several host threads, each on its own stream ---------------------------
def test_concurrent_calls_from_threads_on_their_own_streams():
    """The C ABI is reentrant and asynchronous on the caller's stream: host threads that call
    different entry points at once, each on a stream of its own, get exactly the results of
    one-thread calls (every kernel is deterministic, so the comparison is bitwise)."""
    import threading

    import ternary_weight_quantized_bonsai_amd as bonsai
    torch, dev = torch_dev()

    def d(a):
        return to_dev(a)

    cases = []
    w, s, x = synth.make_q1(1, 13824, 5120, 3, "thr1")
    cases.append(("q1_gemv M=1", lambda o, w=d(w), s=d(s), x=d(x): bonsai.q1_gemv(w, s, x, out=o), (1, 13824)))
    w, s, x = synth.make_q1(4, 5000, 2048, 3, "thr2")
    cases.append(("q1_gemv M=4", lambda o, w=d(w), s=d(s), x=d(x): bonsai.q1_gemv(w, s, x, out=o), (4, 5000)))
    w, s, x = synth.make_q1(300, 2048, 1024, 3, "thr3")
    cases.append(("q1_gemm M=300", lambda o, w=d(w), s=d(s), x=d(x): bonsai.q1_gemm(w, s, x, out=o), (300, 2048)))
    w, s, x = synth.make_q2t(1, 5120, 5120, 3, "thr4")
    cases.append(("q2t_gemv M=1", lambda o, w=d(w), s=d(s), x=d(x): bonsai.q2t_gemv(w, s, x, out=o), (1, 5120)))
    c5, s, x = synth.make_t5(2, 3000, 1152, 3, "thr5")
    cases.append(("t5_matmul M=2", lambda o, c=torch.from_numpy(c5).to(dev), s=d(s), x=d(x):
                  bonsai.t5_matmul(c, s, x, out=o), (2, 3000)))
    w, a, b, x = synth.make_q1a(1, 9000, 1024, 3, "thr6")
    cases.append(("q1a_matmul M=1", lambda o, w=d(w), a=d(a), b=d(b), x=d(x):
                  bonsai.q1a_matmul(w, a, b, x, out=o), (1, 9000)))
    w, s, x = synth.make_q2t(48, 3000, 2048, 3, "thr7")                    # the skinny GEMM
    cases.append(("q2t_gemm M=48", lambda o, w=d(w), s=d(s), x=d(x): bonsai.q2t_gemm(w, s, x, out=o), (48, 3000)))
    w, s, x = synth.make_q1(1, 160001, 2048, 3, "thr8")                     # the byte tables
    cases.append(("q1_gemv M=1 N=160001", lambda o, w=d(w), s=d(s), x=d(x): bonsai.q1_gemv(w, s, x, out=o),
                  (1, 160001)))
    torch.cuda.synchronize()

    expected = []
    for name, fn, shape in cases:
        note(f"concurrency reference {name}")
        o = torch.empty(shape, dtype=torch.float32, device=dev)
        fn(o)
        torch.cuda.synchronize()
        expected.append(o.cpu().numpy())

    threads, reps = 4, 3
    outs = [[torch.full(shape, float("nan"), dtype=torch.float32, device=dev) for _, _, shape in cases]
            for _ in range(threads)]
    torch.cuda.synchronize()
    errors = []

    def worker(t):
        try:
            stream = torch.cuda.Stream(device=dev)
            order = list(range(len(cases)))
            np.random.default_rng(t).shuffle(order)
            with torch.cuda.stream(stream):
                for _ in range(reps):
                    for i in order:
                        cases[i][1](outs[t][i])
            stream.synchronize()
        except Exception as e:      # reported by the main thread
            errors.append(f"thread {t}: {e!r}")

    note(f"concurrency: {threads} threads x {reps} passes over {len(cases)} entry points")
    pool = [threading.Thread(target=worker, args=(t,)) for t in range(threads)]
    for th in pool:
        th.start()
    for th in pool:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in pool), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for t in range(threads):
        for i, (name, _, _) in enumerate(cases):
            got = outs[t][i].cpu().numpy()
            assert np.array_equal(got.view(np.uint32), expected[i].view(np.uint32)), f"thread {t}: {name}"


# ---- the C ABI from plain C ---------------------------------------------------------------
def test_c_abi_from_plain_c():
    """tests/c_abi/abi_from_c.c (built by __graft_entry__.build()): host pack, HIP device buffers
    and a stream, then the binary, affine, ternary and base-3 entry points from C alone, checked
    bit for bit on exactly representable inputs, and the refused calls' statuses."""
    import subprocess
    from pathlib import Path

    exe = Path(__file__).resolve().parent / "c_abi" / "_build" / "abi_from_c"
    assert exe.exists(), f"{exe} is missing: run `python -c 'import __graft_entry__ as g; g.build()'`"
    note("C ABI program")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"exit {r.returncode}:\n{r.stdout}{r.stderr}"
    assert "all checks passed" in r.stdout
