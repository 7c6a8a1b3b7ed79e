"""The C ABI on the host: exported symbols, the executable layout spec (pack/unpack) and
argument validation.  None of these touch a GPU: validation returns before any launch."""
import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

ROOT = Path(__file__).resolve().parents[1]
bonsai = pytest.importorskip("ternary_weight_quantized_bonsai_amd")


def declared_functions():
    text = (ROOT / "include" / "bonsai.h").read_text()
    return sorted(set(re.findall(r"^\s*(?:bonsai_status|const char \*)\s*(bonsai_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("bonsai_q1_gemv", "bonsai_q1_gemm", "bonsai_q2t_gemv", "bonsai_q2t_gemm", "bonsai_q1_pack",
                 "bonsai_q1_unpack", "bonsai_q2t_pack", "bonsai_q2t_unpack", "bonsai_status_str",
                 "bonsai_last_device_error", "bonsai_time_next_launch"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(str(bonsai.LIB_PATH))
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for s in range(7):
        assert bonsai.status_str(s)
    assert bonsai.status_str(99) == "unknown status"


# ---- layout spec -----------------------------------------------------------------------
def test_q1_pack_unpack_roundtrip_random():
    rng = np.random.default_rng(0)
    signs = np.where(rng.random((37, 1024)) < 0.5, 1, -1).astype(np.int8)
    words = bonsai.q1_pack(signs)
    assert words.shape == (37, 32) and words.nbytes == 37 * 1024 // 8
    assert np.array_equal(bonsai.q1_unpack(words, 1024), signs)
    # pack . unpack is the identity on arbitrary words (binary storage is a bijection)
    w = rng.integers(0, 1 << 32, (5, 64), dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(bonsai.q1_pack(bonsai.q1_unpack(w, 2048)), w)


def test_q1_pack_matches_little_endian_bit_order():
    # bit j of word w <-> k = 32 w + j, i.e. numpy's little-endian bit order over the bytes
    rng = np.random.default_rng(1)
    signs = np.where(rng.random((3, 256)) < 0.5, 1, -1).astype(np.int8)
    words = bonsai.q1_pack(signs)
    bits = np.unpackbits(words.view(np.uint8), axis=1, bitorder="little")
    assert np.array_equal(bits.astype(np.int8) * 2 - 1, signs)


def test_q1_pack_exhaustive_halfword_patterns():
    pats = np.arange(1 << 16, dtype=np.uint32)
    words = np.stack([pats, pats << 16], axis=1).reshape(-1, 1)     # low half, then high half
    signs = bonsai.q1_unpack(words, 32)
    assert np.array_equal(bonsai.q1_pack(signs), words)
    j = np.arange(16)
    want_low = np.where((pats[:, None] >> j) & 1, 1, -1)
    assert np.array_equal(signs[0::2, :16], want_low)
    assert np.all(signs[0::2, 16:] == -1)
    assert np.array_equal(signs[1::2, 16:], want_low)


def test_q2t_pack_unpack_roundtrip_and_codes():
    rng = np.random.default_rng(2)
    trits = rng.choice(np.array([-1, 0, 1], dtype=np.int8), size=(29, 512), p=[0.3, 0.4, 0.3])
    words = bonsai.q2t_pack(trits)
    assert words.shape == (29, 32) and words.nbytes == 29 * 512 // 4
    assert np.array_equal(bonsai.q2t_unpack(words, 512), trits)
    fields = (words[..., None] >> (2 * np.arange(16, dtype=np.uint32))) & 3
    assert np.array_equal(fields.reshape(29, 512), np.choose(trits + 1, [3, 0, 1]))


def test_q2t_exhaustive_halfword_patterns_without_reserved_code():
    pats = np.arange(1 << 16, dtype=np.uint32)
    f = (pats[:, None] >> (2 * np.arange(8, dtype=np.uint32))) & 3
    valid = pats[~(f == 2).any(axis=1)]
    assert valid.size == 3 ** 8
    words = np.stack([valid, valid << 16], axis=1).reshape(-1, 1)
    trits = bonsai.q2t_unpack(words, 16)
    assert np.array_equal(bonsai.q2t_pack(trits), words)


def test_q2t_unpack_rejects_reserved_code():
    w = np.zeros((1, 4), np.uint32)
    w[0, 2] = 0b10 << 10
    with pytest.raises(bonsai.BonsaiError) as e:
        bonsai.q2t_unpack(w, 64)
    assert e.value.status == bonsai.ERR_CODE


def test_pack_rejects_values_and_shapes():
    with pytest.raises(bonsai.BonsaiError) as e:
        bonsai.q1_pack(np.zeros((1, 32), np.int8))
    assert e.value.status == bonsai.ERR_VALUE
    with pytest.raises(bonsai.BonsaiError) as e:
        bonsai.q2t_pack(np.full((1, 16), 2, np.int8))
    assert e.value.status == bonsai.ERR_VALUE
    with pytest.raises(bonsai.BonsaiError) as e:
        bonsai.q1_pack(np.ones((1, 33), np.int8))
    assert e.value.status == bonsai.ERR_SHAPE


# ---- GPU entry points: host-side validation only (nothing is launched) ------------------
GPU_FNS = ["bonsai_q1_gemv", "bonsai_q1_gemm", "bonsai_q2t_gemv", "bonsai_q2t_gemm"]
FAKE = 0x7F0000000000          # aligned, never dereferenced: every case below fails validation


@pytest.mark.parametrize("fn", GPU_FNS)
def test_gpu_entry_validation(fn):
    f = getattr(bonsai.raw(), fn)
    p = FAKE
    assert f(None, p, p, p, 1, 64, 128, None) == bonsai.ERR_NULL
    assert f(p, None, p, p, 1, 64, 128, None) == bonsai.ERR_NULL
    assert f(p, p, None, p, 1, 64, 128, None) == bonsai.ERR_NULL
    assert f(p, p, p, None, 1, 64, 128, None) == bonsai.ERR_NULL
    assert f(p, p, p, p, 1, 64, 100, None) == bonsai.ERR_SHAPE
    assert f(p, p, p, p, -1, 64, 128, None) == bonsai.ERR_SHAPE
    assert f(p, p, p, p, 1, -5, 128, None) == bonsai.ERR_SHAPE
    assert f(p, p, p, p, 1, 64, 131072 + 128, None) == bonsai.ERR_SHAPE
    assert f(p + 4, p, p, p, 1, 64, 128, None) == bonsai.ERR_ALIGN
    assert f(p, p + 2, p, p, 1, 64, 128, None) == bonsai.ERR_ALIGN
    assert f(p, p, p + 8, p, 1, 64, 128, None) == bonsai.ERR_ALIGN
    assert f(p, p, p, p + 4, 1, 64, 128, None) == bonsai.ERR_ALIGN
    # empty products are no-ops that never look at the pointers
    assert f(None, None, None, None, 0, 64, 128, None) == bonsai.OK
    assert f(None, None, None, None, 3, 0, 128, None) == bonsai.OK


@pytest.mark.parametrize("fn", ["bonsai_q1_gemv", "bonsai_q2t_gemv"])
def test_gemv_rejects_m_above_8(fn):
    f = getattr(bonsai.raw(), fn)
    assert f(FAKE, FAKE, FAKE, FAKE, 9, 64, 128, None) == bonsai.ERR_SHAPE


@pytest.mark.parametrize("fn", ["bonsai_q1_gemm", "bonsai_q2t_gemm"])
def test_gemm_accepts_large_m_in_validation_only(fn):
    # M = 2^30 + 1 is rejected; nothing is launched for it
    f = getattr(bonsai.raw(), fn)
    assert f(FAKE, FAKE, FAKE, FAKE, (1 << 30) + 1, 64, 128, None) == bonsai.ERR_SHAPE


def test_t5_pack_unpack_roundtrip_and_layout(orc):
    """Round trip, and packed bytes dequantize (oracle, whose decoder is pinned to the layout's
    definition) to trit x scale."""
    import synth
    for N, K in ((3, 640), (2, 1152), (5, 384), (1, 128), (2, 13824)):
        t = synth.trits_i8(N, K, 7, f"abi/t5/{K}")
        c = bonsai.t5_pack(t)
        assert c.shape == (N, 32 * -(-K // 160))
        assert c.max() < 243
        assert np.array_equal(bonsai.t5_unpack(c, K), t)
        s = synth.scales_f16(N, K // 128, 7, f"abi/t5/{K}")
        want = t.astype(np.float64) * np.repeat(s.view(np.float16).astype(np.float64), 128, axis=1)
        assert np.array_equal(orc.t5_dequant(c, s, K), want)


def test_t5_unpack_rejects_reserved_and_padding():
    c = bonsai.t5_pack(np.zeros((1, 384), np.int8))
    bad = c.copy()
    bad[0, 7] = 243
    with pytest.raises(bonsai.BonsaiError) as e:
        bonsai.t5_unpack(bad, 384)
    assert e.value.status == bonsai.ERR_CODE
    bad = c.copy()
    bad[0, 64 + 3] = 3 ** 2          # superblock 2, digit 2: k = 320 + 3 + 64 = 387 >= K
    with pytest.raises(bonsai.BonsaiError):
        bonsai.t5_unpack(bad, 384)
    ok = c.copy()
    ok[0, 64 + 3] = 3 ** 1           # k = 320 + 3 + 32 = 355 < K: a real weight
    assert bonsai.t5_unpack(ok, 384)[0, 355] == 1
    with pytest.raises(bonsai.BonsaiError) as e:
        bonsai.t5_pack(np.full((1, 160), 2, np.int8))
    assert e.value.status == bonsai.ERR_VALUE


def test_q2t_t5_direct_conversions():
    """The direct conversions agree with unpack-then-pack both ways, and refuse what the
    packers and unpackers refuse."""
    import synth
    for N, K in ((3, 640), (2, 1152), (5, 384), (1, 16), (2, 13824)):
        t = synth.trits_i8(N, K, 9, f"abi/conv/{K}")
        w2 = bonsai.q2t_pack(t)
        c5 = bonsai.t5_pack(t)
        assert np.array_equal(bonsai.q2t_to_t5(w2, K), c5)
        assert np.array_equal(bonsai.t5_to_q2t(c5, K), w2)
    bad = bonsai.q2t_pack(np.zeros((1, 160), np.int8))
    bad[0, 3] |= np.uint32(2 << 6)                  # field value 2
    with pytest.raises(bonsai.BonsaiError):
        bonsai.q2t_to_t5(bad, 160)
    c = bonsai.t5_pack(np.zeros((1, 176), np.int8))  # K = 176: superblock 1 holds k 160..175
    c[0, 32 + 20] = 3                                # digit 1 of byte 20: k = 160 + 20 + 32 >= K
    with pytest.raises(bonsai.BonsaiError):
        bonsai.t5_to_q2t(c, 176)
    c[0, 32 + 20] = 250
    with pytest.raises(bonsai.BonsaiError):
        bonsai.t5_to_q2t(c, 176)


def test_t5_matmul_validation():
    f = bonsai.raw().bonsai_t5_matmul
    p = FAKE
    assert f(None, p, p, p, 1, 64, 128, None) == bonsai.ERR_NULL
    assert f(p, p, p, None, 1, 64, 128, None) == bonsai.ERR_NULL
    assert f(p, p, p, p, 1, 64, 100, None) == bonsai.ERR_SHAPE
    assert f(p + 8, p, p, p, 1, 64, 128, None) == bonsai.ERR_ALIGN
    assert f(None, None, None, None, 0, 64, 128, None) == bonsai.OK


def test_affine_matmul_validation():
    f = bonsai.raw().bonsai_q1a_matmul
    p = FAKE
    assert f(p, p, None, p, p, 1, 64, 128, None) == bonsai.ERR_NULL
    assert f(p, p, p + 2, p, p, 1, 64, 128, None) == bonsai.ERR_ALIGN
    assert f(None, p, p, p, p, 1, 64, 128, None) == bonsai.ERR_NULL
    assert f(p, p, p, p, None, 1, 64, 128, None) == bonsai.ERR_NULL
    assert f(p, p, p, p, p, 1, 64, 100, None) == bonsai.ERR_SHAPE
    assert f(p, p, p, p, p, -1, 64, 128, None) == bonsai.ERR_SHAPE
    assert f(p, p, p, p + 8, p, 1, 64, 128, None) == bonsai.ERR_ALIGN
    assert f(None, None, None, None, None, 0, 64, 128, None) == bonsai.OK
    assert f(None, None, None, None, None, 3, 0, 128, None) == bonsai.OK


def test_affine_conversion_every_f16_pattern():
    """to_affine gives (2 s, -s) exactly for every binary16 s whose double is finite, rejects
    the rest, and from_affine takes each pair back to the same bits."""
    s = np.arange(1 << 16, dtype=np.uint16)
    sv = s.view(np.float16).astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        ok = np.isfinite(sv) & np.isfinite((2.0 * sv).astype(np.float16).astype(np.float64))
    good = s[ok]
    a, b = bonsai.q1_to_affine(good)
    gv = good.view(np.float16).astype(np.float64)
    assert np.array_equal(a.view(np.float16).astype(np.float64), 2.0 * gv)       # exact doubling
    assert np.array_equal(np.signbit(a.view(np.float16)), np.signbit(good.view(np.float16)))
    assert np.array_equal(b, good ^ np.uint16(0x8000))
    assert np.array_equal(bonsai.q1_from_affine(a, b), good)
    for bad in s[~ok]:                    # |s| >= 32768, inf, NaN
        with pytest.raises(bonsai.BonsaiError):
            bonsai.q1_to_affine(np.array([bad], np.uint16))


def test_affine_from_rejects_non_binary_pairs():
    s = np.array([0x3C00, 0x2E66, 0x0001, 0x8400], np.uint16)
    a, b = bonsai.q1_to_affine(s)
    for i in range(s.size):
        for bad_a, bad_b in ((a[i] ^ np.uint16(1), b[i]), (a[i], b[i] ^ np.uint16(1)), (a[i], b[i] ^ np.uint16(0x8000))):
            aa, bb = a.copy(), b.copy()
            aa[i], bb[i] = bad_a, bad_b
            with pytest.raises(bonsai.BonsaiError):
                bonsai.q1_from_affine(aa, bb)
    assert bonsai.q1_from_affine(a[:0], b[:0]).size == 0


def test_affine_conversion_gives_the_binary_weights(orc):
    """The converted pairs dequantize (oracle, affine form) to the native binary weights."""
    import synth
    N, K = 7, 640
    w, s, _ = synth.make_q1(1, N, K, 3, "abi/affine")
    a, b = bonsai.q1_to_affine(s)
    assert np.array_equal(orc.q1a_dequant(w, a, b, K), orc.q1_dequant(w, s, K))


def test_embed_validation():
    f = bonsai.raw().bonsai_q1_embed
    p = FAKE
    assert f(p, p, p, p, 0, 10, 128, None) == bonsai.OK              # no ids: no-op
    assert f(None, None, None, None, 4, 10, 0, None) == bonsai.OK    # K = 0: no-op
    assert f(p, p, None, p, 4, 10, 128, None) == bonsai.ERR_NULL
    assert f(p, p, p, None, 4, 10, 128, None) == bonsai.ERR_NULL
    assert f(None, p, p, p, 4, 10, 128, None) == bonsai.ERR_NULL
    assert f(p, p, p, p, 4, 10, 100, None) == bonsai.ERR_SHAPE
    assert f(p, p, p, p, -1, 10, 128, None) == bonsai.ERR_SHAPE
    assert f(p, p, p, p, 4, -1, 128, None) == bonsai.ERR_SHAPE
    assert f(p, p, p + 8, p, 4, 10, 128, None) == bonsai.ERR_ALIGN
    assert f(p, p, p, p + 2, 4, 10, 128, None) == bonsai.ERR_ALIGN


# ---- launch plans: the routing, on any compute-unit count, with no GPU ------------------
def _plan_kernel(op, M, N, K, cus):
    return bonsai.plan(op, M, N, K, cus).split(" grid=")[0]


def _plan_grid(op, M, N, K, cus):
    return int(bonsai.plan(op, M, N, K, cus).split(" grid=")[1].split(",")[0])


def test_plan_names_each_route_of_the_decode_gemv():
    # one row of x: 32-row table tiles while one round of the CUs holds them, 64-row tiles up
    # to six rounds, then the persistent kernel; more rows of x go to the matrix cores
    assert _plan_kernel("q1_gemv", 1, 5120, 5120, 256) == "launch_lut4[ROWS = 32, AFF = false, GPL = 2]"
    assert _plan_kernel("q1_gemv", 1, 13824, 5120, 256) == "launch_lut4[ROWS = 64, AFF = false, GPL = 4]"
    assert _plan_kernel("q1_gemv", 1, 248320, 5120, 256).startswith("launch_lut8")
    assert _plan_kernel("q1_gemv", 1, 100003, 5120, 256) == "launch_lutp[AFF = false]"
    # the affine form follows the same routes, on its own instances
    assert _plan_kernel("q1a_matmul", 1, 248320, 5120, 256).startswith("launch_lut8_t")
    assert "AFF = true" in _plan_kernel("q1a_matmul", 1, 248320, 5120, 256)
    assert "AFF = false" in _plan_kernel("q1_gemv", 1, 248320, 5120, 256)
    assert _plan_kernel("q1a_matmul", 1, 100003, 4992, 256) == "launch_lutp[AFF = true]"
    assert _plan_kernel("q1_gemv", 8, 5120, 5120, 256).startswith("launch_rt[TERN = false")
    assert _plan_kernel("q1_gemm", 512, 13824, 5120, 256) == "q1_gemm_kernel<false, 16>"
    assert _plan_kernel("q1_gemm", 512, 13824, 5248, 256) == "q1_gemm_kernel<false, 2>"
    assert _plan_kernel("q2t_gemm", 512, 13824, 5120, 256) == "q1_gemm_kernel<true, 4>"
    assert _plan_kernel("q2t_gemv", 1, 5120, 5120, 256).startswith("launch_rt[TERN = true")
    assert _plan_kernel("t5_matmul", 1, 5120, 5120, 256).startswith("t5_launch_rt")
    assert _plan_kernel("q1_embed", 512, 248320, 5120, 256) == "q1_embed_kernel"
    assert bonsai.plan("q1_gemv", 0, 64, 128, 256) == "none"
    assert bonsai.plan("q1_gemv", 1, 64, 0, 256).startswith("fill_zero_kernel")


def test_plan_routing_follows_the_compute_unit_count():
    # 32-row tiles run while one round of the device's CUs holds them: 5120 rows make 160 tiles
    # of 32, so a device of 128 CUs takes 64-row tiles instead
    assert _plan_kernel("q1_gemv", 1, 5120, 5120, 256).startswith("launch_lut4[ROWS = 32")
    assert _plan_kernel("q1_gemv", 1, 5120, 5120, 160).startswith("launch_lut4[ROWS = 32")
    assert _plan_kernel("q1_gemv", 1, 5120, 5120, 128).startswith("launch_lut4[ROWS = 64")
    # the persistent LM-head kernels take one workgroup per CU (the byte-table kernel more when a
    # CU's share of rows would exceed what its waves hold); the byte tables take over at 600 rows
    # per CU
    for cus in (80, 256, 304):
        plan = bonsai.plan("q1_gemv", 1, 248320, 5120, cus)
        assert plan.startswith("launch_lut8") or plan.startswith("launch_lutp"), plan
        grid = _plan_grid("q1_gemv", 1, 248320, 5120, cus)
        assert grid == cus or (plan.startswith("launch_lut8") and grid > cus and grid * 16 * 8 * 8 >= 248320)
    assert _plan_kernel("q1_gemv", 1, 600 * 200, 5120, 200).startswith("launch_lut8")
    assert not _plan_kernel("q1_gemv", 1, 600 * 200 - 1, 5120, 200).startswith("launch_lut8")
    # the small-M kernel's tiles always cover every row, whatever tile the CU count selects
    for cus in (32, 64, 256, 304):
        plan = bonsai.plan("q2t_gemv", 8, 5120, 5120, cus)
        rows = int(plan.split("RT = ")[1].split(",")[0]) * 16
        assert _plan_grid("q2t_gemv", 8, 5120, 5120, cus) * rows >= 5120


def test_plan_runs_the_entry_points_argument_checks():
    with pytest.raises(bonsai.BonsaiError) as e:
        bonsai.plan("q1_gemv", 9, 64, 128, 256)
    assert e.value.status == bonsai.ERR_SHAPE
    with pytest.raises(bonsai.BonsaiError) as e:
        bonsai.plan("q1_gemm", 4, 64, 100, 256)
    assert e.value.status == bonsai.ERR_SHAPE
    assert bonsai.raw().bonsai_plan(99, 1, 64, 128, 256, None, 0) == bonsai.ERR_VALUE


def test_timing_hook_is_consumed_by_a_call_that_fails_or_enqueues_nothing():
    lib = bonsai.raw()
    ev = 0x7F0000001000            # stand-in event handles: planned launches never touch them
    # armed: the next planned launch would be timed, and consumes the hook
    assert lib.bonsai_time_next_launch(ev, ev) == bonsai.OK
    assert bonsai.plan("q1_gemv", 1, 256, 512, 256).endswith(" timed")
    assert not bonsai.plan("q1_gemv", 1, 256, 512, 256).endswith(" timed")
    # a call that fails its argument checks consumes it too
    for call, status in ((lambda: lib.bonsai_q1_gemv(FAKE, FAKE, FAKE, FAKE, 1, 64, 100, None), bonsai.ERR_SHAPE),
                         (lambda: lib.bonsai_q1_gemm(None, FAKE, FAKE, FAKE, 1, 64, 128, None), bonsai.ERR_NULL),
                         (lambda: lib.bonsai_q1_gemv(FAKE, FAKE, FAKE, FAKE, 0, 64, 128, None), bonsai.OK),
                         (lambda: lib.bonsai_q1a_matmul(FAKE, FAKE, None, FAKE, FAKE, 1, 64, 128, None),
                          bonsai.ERR_NULL),
                         (lambda: lib.bonsai_q1_embed(FAKE, FAKE, FAKE, FAKE, 0, 10, 128, None), bonsai.OK),
                         (lambda: lib.bonsai_probe_stream(FAKE, 1000, 0, FAKE, None), bonsai.ERR_SHAPE),
                         (lambda: lib.bonsai_probe_clock(None, 10, None), bonsai.ERR_NULL)):
        assert lib.bonsai_time_next_launch(ev, ev) == bonsai.OK
        assert call() == status
        assert not bonsai.plan("q1_gemv", 1, 256, 512, 256).endswith(" timed")


def test_probe_validation():
    lib = bonsai.raw()
    assert lib.bonsai_probe_stream(FAKE, 1000, 0, FAKE, None) == bonsai.ERR_SHAPE     # not a multiple of 1 KiB
    assert lib.bonsai_probe_stream(FAKE, 0, 0, FAKE, None) == bonsai.ERR_SHAPE
    assert lib.bonsai_probe_stream(FAKE, 1024, 3, FAKE, None) == bonsai.ERR_SHAPE
    assert lib.bonsai_probe_stream(None, 1024, 0, FAKE, None) == bonsai.ERR_NULL
    assert lib.bonsai_probe_stream(FAKE, 1024, 0, None, None) == bonsai.ERR_NULL
    assert lib.bonsai_probe_stream(FAKE + 4, 1024, 1, FAKE, None) == bonsai.ERR_ALIGN
    assert lib.bonsai_probe_clock(None, 10, None) == bonsai.ERR_NULL
    assert lib.bonsai_probe_clock(FAKE, -1, None) == bonsai.ERR_SHAPE
    assert lib.bonsai_probe_clock(FAKE, 2_000_000_000, None) == bonsai.ERR_SHAPE
