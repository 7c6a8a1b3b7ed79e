"""Pins that tie the oracle to facts fixed outside it.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with the fact it checks.  None of them recomputes the
oracle's own formula: they use library fp16 decoding, closed forms, exhaustive
bit probes read through the little-endian byte view of the words, exact
integer arithmetic in Python, the MLX affine re-encoding from the model card,
hand-worked fixtures and the pages' printed storage figures.

``tests/test_oracle_pins.py`` runs every pin on the real oracle and on planted
mutants of it (a pin set that a plausible mistake slips through is a gap).
"""
from __future__ import annotations

import json
import math
from pathlib import Path

import numpy as np

import oracle as oracle_mod
import synth

GOLDEN = Path(__file__).resolve().parent / "golden"
F16_ONE = 0x3C00


def _f16(values) -> np.ndarray:
    return np.asarray(values, dtype=np.float64).astype(np.float16).view(np.uint16)


def _lib_f16(bits: np.ndarray) -> np.ndarray:
    """binary16 bit patterns -> float64 through numpy's own conversion."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _sign_bit(words: np.ndarray, n: int, k: int) -> int:
    """Bit of weight (n, k) read through the little-endian byte view: byte k//8, bit k%8."""
    return int((np.ascontiguousarray(words[n]).view(np.uint8)[k // 8] >> (k % 8)) & 1)


def _trit(words: np.ndarray, n: int, k: int) -> int:
    """Code of weight (n, k) through the byte view: byte k//4, bits 2(k%4)..2(k%4)+1."""
    code = int((np.ascontiguousarray(words[n]).view(np.uint8)[k // 4] >> (2 * (k % 4))) & 3)
    return {0: 0, 1: 1, 3: -1}[code]


# --------------------------------------------------------------------------------------------
def pin_f16_decoder(o):
    """Every one of the 65536 binary16 patterns decodes as numpy decodes it."""
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = _lib_f16(bits)
    got = np.array([o.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "NaN patterns differ"
    assert np.array_equal(got[~nan], ref[~nan]), "finite/inf patterns differ"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), "signed zeros differ"


def pin_all_ones_all_zero(o):
    """All-one signs give sum_g s_g * sum_{k in g} x_k; all-zero signs give exactly its negation."""
    N, K, M = 3, 384, 2
    rng = np.random.default_rng(1)
    s = _f16(np.abs(rng.normal(0, 0.5, (N, K // 128))) + 0.01)
    x = _f16(rng.normal(0, 1, (M, K)))
    ones = np.full((N, K // 32), 0xFFFFFFFF, dtype=np.uint32)
    zeros = np.zeros_like(ones)
    y1, a1 = o.q1_matmul(ones, s, x, K)
    y0, a0 = o.q1_matmul(zeros, s, x, K)
    xs = _lib_f16(x).reshape(M, K // 128, 128).sum(axis=2)          # group sums of x
    closed = xs @ _lib_f16(s).T                                       # sum_g s_g * X_g
    assert np.allclose(y1, closed, rtol=1e-12, atol=1e-12), (y1, closed)
    assert np.array_equal(y0, -y1), "all-zero signs are not the exact negation"
    assert np.array_equal(a0, a1)


def pin_popcount(o):
    """x = 1, s = 1: y[n] = 2 * popcount(row n) - K exactly (binary)."""
    N, K = 17, 1024
    w = synth.sign_words(N, K // 32, 3, "pin/popcount")
    s = np.full((N, K // 128), F16_ONE, dtype=np.uint16)
    x = np.full((1, K), F16_ONE, dtype=np.uint16)
    y, a = o.q1_matmul(w, s, x, K)
    pop = np.unpackbits(w.view(np.uint8), axis=1).sum(axis=1)
    assert np.array_equal(y[0], 2.0 * pop - K)
    assert np.array_equal(a[0], np.full(N, float(K)))


def pin_onehot(o):
    """x = e_k (all k at once): y[k][n] = +s or -s by the bit read through the byte view."""
    N, K = 5, 256
    w = synth.sign_words(N, K // 32, 4, "pin/onehot")
    s = synth.scales_f16(N, K // 128, 4, "pin/onehot")
    x = np.where(np.eye(K, dtype=bool), F16_ONE, 0).astype(np.uint16)
    y, _ = o.q1_matmul(w, s, x, K)
    sv = _lib_f16(s)
    for n in range(N):
        for k in range(K):
            want = sv[n, k // 128] if _sign_bit(w, n, k) else -sv[n, k // 128]
            assert y[k, n] == want, (n, k, y[k, n], want)


def pin_byte_patterns(o):
    """All 256 byte patterns in each byte lane q of a word: x_k = 2^(k-8q) on that byte, s = 1,
    gives y = 2 * byte - 255 exactly (little-endian byte q holds k = 8q..8q+7, LSB first)."""
    K = 128
    pats = np.arange(256, dtype=np.uint32)
    for q in range(4):
        w = np.zeros((256, K // 32), dtype=np.uint32)
        w[:, 1] = pats << (8 * q)                   # word 1 of every row holds the pattern
        w[:, 0] = 0x5A5A5A5A                        # words that x ignores
        s = np.full((256, 1), F16_ONE, dtype=np.uint16)
        xv = np.zeros(K)
        xv[32 + 8 * q: 32 + 8 * q + 8] = 2.0 ** np.arange(8)
        y, _ = o.q1_matmul(w, s, _f16(xv[None, :]), K)
        want = 2.0 * pats - 255.0 - np.zeros(256)   # bits outside the byte see x = 0
        assert np.array_equal(y[0], want), q


def pin_exact_vs_double(o):
    """4 x 256 brute force (and other small shapes): the double sum sits within K 2^-53 a
    of the exact 128-bit result; the exact path matches Python integers on integer data."""
    for (N, K, M, seed) in [(4, 256, 1, 5), (7, 640, 3, 6), (1, 128, 8, 7), (13, 1152, 2, 8)]:
        w, s, x = synth.make_q1(M, N, K, seed, f"pin/exact{seed}")
        y, a = o.q1_matmul(w, s, x, K)
        ye = o.q1_exact(w, s, x, K)
        assert np.all(np.abs(y - ye) <= K * 2.0 ** -53 * a + 1e-300), (N, K)
        t, s2, x2 = synth.make_q2t(M, N, K, seed, f"pin/exactt{seed}")
        y, a = o.q2t_matmul(t, s2, x2, K)
        ye = o.q2t_exact(t, s2, x2, K)
        assert np.all(np.abs(y - ye) <= K * 2.0 ** -53 * a + 1e-300), (N, K)
    # integer-valued data: exact results from Python integers through the byte view
    N, K = 3, 256
    rng = np.random.default_rng(9)
    w = synth.sign_words(N, K // 32, 9, "pin/exactint")
    sv = rng.integers(1, 5, (N, K // 128))
    xv = rng.integers(-8, 9, (2, K))
    ye = o.q1_exact(w, _f16(sv), _f16(xv), K)
    for m in range(2):
        for n in range(N):
            want = sum((1 if _sign_bit(w, n, k) else -1) * int(sv[n, k // 128]) * int(xv[m, k])
                       for k in range(K))
            assert ye[m, n] == want, (m, n)


def pin_mlx_identity(o):
    """MLX affine re-encoding (model card, 'MLX packaging'): scale 2 s_g, bias -s_g, q = bit
    gives exactly the same weights as the native sign form."""
    N, K = 6, 512
    w = synth.sign_words(N, K // 32, 10, "pin/mlx")
    s = synth.scales_f16(N, K // 128, 10, "pin/mlx")
    bits = np.unpackbits(w.view(np.uint8), axis=1, bitorder="little").astype(np.float64)
    sg = np.repeat(_lib_f16(s), 128, axis=1)
    mlx = (2.0 * sg) * bits + (-sg)
    assert np.array_equal(o.q1_dequant(w, s, K), mlx)


def pin_affine_forms(o):
    """Affine 1-bit weights (model card, 'MLX packaging': a scale and a bias per group of 128,
    weight = scale * bit + bias).  Fixed outside the oracle by: the native sign form re-encoded
    as (2 s, -s), which must reproduce the binary oracle exactly; one-hot bit probes read through
    the byte view with distinct scales and biases per group; a zero scale, where y reduces to
    the bias times the group sums of x; and Python integer brute force on integer data."""
    # (2 s, -s): same weights, same sums, same magnitudes as the native binary form
    M, N, K = 3, 5, 640
    w, s, x = synth.make_q1(M, N, K, 21, "pin/affine")
    a2 = _f16(2.0 * _lib_f16(s))
    bneg = s ^ np.uint16(0x8000)
    assert np.array_equal(o.q1a_dequant(w, a2, bneg, K), o.q1_dequant(w, s, K))
    y1, m1 = o.q1_matmul(w, s, x, K)
    ya, ma = o.q1a_matmul(w, a2, bneg, x, K)
    assert np.array_equal(ya, y1) and np.array_equal(ma, m1)

    # one-hot bits: only weight (n, k) takes scale + bias, every other weight its group's bias
    N, K = 2, 384
    sc = _f16([[3.0, 5.0, 7.0], [11.0, 13.0, 17.0]])
    bi = _f16([[-0.5, -0.25, -2.0], [-4.0, 0.75, 1.5]])
    for (n, k) in [(0, 0), (0, 31), (0, 32), (0, 200), (1, 127), (1, 128), (1, 383)]:
        words = np.zeros((N, K // 32), dtype=np.uint32)
        words[n].view(np.uint8)[k // 8] = np.uint8(1 << (k % 8))
        assert _sign_bit(words, n, k) == 1
        W = o.q1a_dequant(words, sc, bi, K)
        want = np.repeat(_lib_f16(bi), 128, axis=1)
        want[n, k] += _lib_f16(sc)[n, k // 128]
        assert np.array_equal(W, want), (n, k)

    # zero scale: y[m][n] = sum over groups of bias(n, g) * (sum of x over the group)
    M, N, K = 2, 3, 512
    w, s, x = synth.make_q1(M, N, K, 22, "pin/affine0")
    b = synth.scales_f16(N, K // 128, 23, "pin/affine0b")
    y, _ = o.q1a_matmul(w, np.zeros_like(s), b, x, K)
    gx = _lib_f16(x).reshape(M, K // 128, 128).sum(axis=2)            # [M, G]
    want = gx @ _lib_f16(b).T                                           # [M, N]
    assert np.allclose(y, want, rtol=1e-12, atol=1e-12)

    # integer data: exact from Python integers through the byte view
    N, K = 3, 256
    rng = np.random.default_rng(24)
    w = synth.sign_words(N, K // 32, 24, "pin/affineint")
    av = rng.integers(-6, 7, (N, K // 128))
    bv = rng.integers(-6, 7, (N, K // 128))
    xv = rng.integers(-8, 9, (2, K))
    y, _ = o.q1a_matmul(w, _f16(av), _f16(bv), _f16(xv), K)
    for m in range(2):
        for n in range(N):
            want = sum((int(av[n, k // 128]) * _sign_bit(w, n, k) + int(bv[n, k // 128])) * int(xv[m, k])
                       for k in range(K))
            assert y[m, n] == want, (m, n)


def _t5_pack(trits: np.ndarray) -> np.ndarray:
    """Base-3 layout from its definition: byte c of superblock b is sum_i (w mod 3) 3^i over
    the weights k = 160 b + c + 32 i (zero past K)."""
    N, K = trits.shape
    SB = -(-K // 160)
    out = np.zeros((N, 32 * SB), dtype=np.uint8)
    for n in range(N):
        for b in range(SB):
            for c in range(32):
                v = 0
                for i in range(5):
                    k = 160 * b + c + 32 * i
                    v += (int(trits[n, k]) % 3 if k < K else 0) * 3 ** i
                out[n, 32 * b + c] = v
    return out


def pin_t5_forms(o):
    """Base-3 ternary (five trits per byte).  Fixed outside the oracle by: the same trits read
    from 2-bit words through the byte view, packed from the layout's definition, must give
    exactly the 2-bit oracle's weights and products; one-hot digits at every byte and digit of
    two superblocks and a ragged third; reserved bytes; the density bound of the pages."""
    for (N, K, seed) in [(3, 640, 31), (2, 1152, 32), (4, 384, 33)]:
        words = synth.trit_words(N, K // 16, seed, f"pin/t5/{K}")
        trits = np.array([[_trit(words, n, k) for k in range(K)] for n in range(N)])
        codes = _t5_pack(trits)
        s = synth.scales_f16(N, K // 128, seed, f"pin/t5/{K}")
        assert np.array_equal(o.t5_dequant(codes, s, K), o.q2t_dequant(words, s, K)), K
        x = synth.activations_f16(2, K, seed, f"pin/t5/{K}")
        yt, at = o.t5_matmul(codes, s, x, K)
        yq, aq = o.q2t_matmul(words, s, x, K)
        assert np.array_equal(yt, yq) and np.array_equal(at, aq), K

    # one-hot digits: byte c of superblock b = 3^i (digit 1, +1) or 2 3^i (digit 2, -1)
    N, K = 1, 384                                  # superblocks 0, 1 whole, 2 holds k 320..383
    s = _f16([[3.0, 5.0, 7.0]])
    sv = _lib_f16(s)[0]
    for b in range(3):
        for c in range(32):
            for i in range(5):
                k = 160 * b + c + 32 * i
                for digit, sign in ((1, 1.0), (2, -1.0)):
                    codes = np.zeros((N, 96), dtype=np.uint8)
                    codes[0, 32 * b + c] = digit * 3 ** i
                    want = np.zeros((N, K))
                    if k < K:
                        want[0, k] = sign * sv[k // 128]
                    assert np.array_equal(o.t5_dequant(codes, s, K), want), (b, c, i, digit)

    # reserved bytes 243..255 are refused; every byte below them decodes
    for v in (243, 250, 255):
        codes = np.zeros((1, 32), dtype=np.uint8)
        codes[0, 5] = v
        try:
            o.t5_dequant(codes, _f16([[1.0]]), 128)
        except oracle_mod.OracleError as e:
            assert e.rc == oracle_mod.ERR_CODE
        else:
            raise AssertionError(f"reserved byte {v} accepted")
    o.t5_dequant(np.full((1, 32), 242, np.uint8), _f16([[1.0]]), 128)

    # density: at or above the pages' log2(3) + 16/128 bound, within 1 % of it
    ideal = math.log2(3) + 16 / 128
    bpw = oracle_mod.bits_per_weight("t5")
    assert ideal <= bpw <= 1.01 * ideal
    assert oracle_mod.packed_bytes("t5", 5120, 5120) * 8 / (5120 * 5120) == bpw


def pin_metamorphic(o):
    """y(-x) = -y(x), y(2s) = 2 y(s) and y(~signs) = -y(signs), all exactly."""
    M, N, K = 3, 9, 768
    w, s, x = synth.make_q1(M, N, K, 11, "pin/meta")
    y, _ = o.q1_matmul(w, s, x, K)
    yneg, _ = o.q1_matmul(w, s, x ^ np.uint16(0x8000), K)
    assert np.array_equal(yneg, -y)
    y2, _ = o.q1_matmul(w, _f16(2.0 * _lib_f16(s)), x, K)
    assert np.array_equal(y2, 2.0 * y)
    yflip, _ = o.q1_matmul(~w, s, x, K)
    assert np.array_equal(yflip, -y)


def pin_ternary_zero_and_mask(o):
    """Ternary: all-00 codes give y = 0 exactly; a random zero mask gives exactly the binary
    result on x with the masked entries set to 0."""
    M, N, K = 2, 7, 512
    w, s, x = synth.make_q1(M, N, K, 12, "pin/tmask")
    yz, az = o.q2t_matmul(np.zeros((N, K // 16), np.uint32), s, x, K)
    assert np.array_equal(yz, np.zeros((M, N))) and np.array_equal(az, np.zeros((M, N)))
    rng = np.random.default_rng(12)
    mask = rng.random((N, K)) < 0.6
    bits = np.unpackbits(w.view(np.uint8), axis=1, bitorder="little").astype(bool)
    codes = np.where(mask, np.where(bits, 1, 3), 0).astype(np.uint32)      # 01 = +1, 11 = -1
    words = np.bitwise_or.reduce(codes.reshape(N, K // 16, 16) << (2 * np.arange(16, dtype=np.uint32)),
                                 axis=2).astype(np.uint32)
    for n in range(N):
        xm = np.where(mask[n][None, :], x, 0).astype(np.uint16)
        yb, _ = o.q1_matmul(w[n:n + 1], s[n:n + 1], xm, K)
        yt, _ = o.q2t_matmul(words[n:n + 1], s[n:n + 1], x, K)
        assert np.array_equal(yt, yb), n


def pin_ternary_counts_and_onehot(o):
    """Ternary with x = 1, s = 1: y = #(+1) - #(-1); with x = e_k: y = t(n,k) s exactly."""
    N, K = 9, 512
    t = synth.trit_words(N, K // 16, 13, "pin/tcount")
    s1 = np.full((N, K // 128), F16_ONE, dtype=np.uint16)
    y, _ = o.q2t_matmul(t, s1, np.full((1, K), F16_ONE, np.uint16), K)
    fields = (t[..., None] >> (2 * np.arange(16, dtype=np.uint32))) & 3
    want = (fields == 1).sum(axis=(1, 2)) - (fields == 3).sum(axis=(1, 2))
    assert np.array_equal(y[0], want.astype(np.float64))
    K2, N2 = 256, 3
    t2 = synth.trit_words(N2, K2 // 16, 14, "pin/tonehot")
    s2 = synth.scales_f16(N2, K2 // 128, 14, "pin/tonehot")
    x = np.where(np.eye(K2, dtype=bool), F16_ONE, 0).astype(np.uint16)
    y2, _ = o.q2t_matmul(t2, s2, x, K2)
    sv = _lib_f16(s2)
    for n in range(N2):
        for k in range(K2):
            assert y2[k, n] == _trit(t2, n, k) * sv[n, k // 128], (n, k)


def pin_reserved_and_shapes(o):
    """The reserved ternary code 10 and K not a multiple of 128 are rejected."""
    K = 128
    words = np.zeros((1, K // 16), np.uint32)
    words[0, 3] = 0b10 << 6
    try:
        o.q2t_matmul(words, np.full((1, 1), F16_ONE, np.uint16), np.zeros((1, K), np.uint16), K)
        raise AssertionError("reserved code accepted")
    except oracle_mod.OracleError as e:
        assert e.rc == oracle_mod.ERR_CODE
    try:
        o.q1_matmul(np.zeros((1, 3), np.uint32), np.zeros((1, 1), np.uint16),
                    np.zeros((1, 96), np.uint16), 96)
        raise AssertionError("K % 128 != 0 accepted")
    except oracle_mod.OracleError as e:
        assert e.rc == oracle_mod.ERR_SHAPE


def _golden_x(spec, M_hint, K):
    if spec == "k+1":
        return _f16(np.arange(1, K + 1)[None, :])
    if spec == "ones":
        return _f16(np.ones((1, K)))
    if isinstance(spec, dict) and "onehot" in spec:
        rows = np.zeros((len(spec["onehot"]), K))
        for i, (k, v) in enumerate(spec["onehot"]):
            rows[i, k] = v
        return _f16(rows)
    if isinstance(spec, dict) and "rows" in spec:
        vals = {"ones": 1.0, "twos": 2.0}
        return _f16(np.array([[vals[r[0]]] * K for r in spec["rows"]]))
    raise ValueError(spec)


def pin_golden_hand_cases(o):
    """The hand-worked fixtures in tests/golden/hand_cases.json."""
    cases = json.loads((GOLDEN / "hand_cases.json").read_text())["cases"]
    for c in cases:
        K = c["K"]
        words = np.array([[int(v, 16) for v in row] for row in c["words"]], dtype=np.uint32)
        scales = np.array([[int(v, 16) for v in row] for row in c["scales"]], dtype=np.uint16)
        x = _golden_x(c["x"], None, K)
        fn = o.q1_matmul if c["kind"] == "q1" else o.q2t_matmul
        y, a = fn(words, scales, x, K)
        assert np.array_equal(y, np.array(c["y"])), (c["name"], y, c["y"])
        assert np.array_equal(a, np.array(c["a"])), (c["name"], a, c["a"])


def pin_storage_figures(o):
    """Byte accounting against the storage figures the pages print."""
    fig = {e["name"]: e for e in json.loads((GOLDEN / "pages_figures.json").read_text())["entries"]}

    def near(name, v):
        assert abs(v - fig[name]["value"]) <= fig[name]["tol"] + 1e-12, (name, v, fig[name]["value"])

    bpw = oracle_mod.bits_per_weight
    near("binary_bits_per_weight", bpw("q1"))
    near("binary_bits_per_weight", 8 * oracle_mod.packed_bytes("q1", 4096, 5120) / (4096 * 5120))
    near("binary_reduction_vs_fp16", bpw("fp16") / bpw("q1"))
    P = fig["binary_params"]["value"]
    near("binary_deployed_gb", P * bpw("q1") / 8 / 1e9)
    near("fp16_gb", P * bpw("fp16") / 8 / 1e9)
    near("ternary_deployed_gb_2bit", P * bpw("q2t") / 8 / 1e9)
    near("ternary_deployed_gb_2bit", P * 8 * oracle_mod.packed_bytes("q2t", 5120, 5120)
         / (5120 * 5120) / 8 / 1e9)
    near("ternary_ideal_bpw", math.log2(3) + 16 / 128)
    near("ternary_ideal_gb", P * (math.log2(3) + 16 / 128) / 8 / 1e9)
    near("mlx_affine_bits_per_weight", bpw("mlx_affine_1bit"))


ALL_PINS = [
    pin_f16_decoder, pin_all_ones_all_zero, pin_popcount, pin_onehot, pin_byte_patterns,
    pin_exact_vs_double, pin_mlx_identity, pin_affine_forms, pin_t5_forms, pin_metamorphic, pin_ternary_zero_and_mask,
    pin_ternary_counts_and_onehot, pin_reserved_and_shapes, pin_golden_hand_cases,
    pin_storage_figures,
]


def run_all(o) -> list[str]:
    """Names of the pins that fail on oracle ``o`` (an exception counts as a failure)."""
    failed = []
    for pin in ALL_PINS:
        try:
            pin(o)
        except Exception:  # noqa: BLE001 - any error means the pin caught the mutant
            failed.append(pin.__name__)
    return failed


if __name__ == "__main__":  # used by the mutation test: python tests/oracle_pins.py <lib.so>
    import sys
    print(json.dumps(run_all(oracle_mod.Oracle(sys.argv[1]))))
