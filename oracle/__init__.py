"""CPU oracle for the binary / ternary g128 weight-only matmul (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never touches it,
and it imports nothing from the product package.

The arithmetic lives in ``bonsai_oracle.c`` (plain C, double precision, natural
k order); this module compiles it with gcc and wraps it with ctypes and numpy.
Every function follows the definition on the "1-bit Bonsai 27B" model card
(section "Weight representation: Binary g128": sign bit 0 -> -scale,
1 -> +scale, 128 consecutive weights per FP16 scale), for MLX's affine 1-bit form
(section "MLX packaging": scale * bit + bias per group), and, for ternary weights,
the "Ternary Bonsai 27B" article ({-1, 0, +1} x FP16 group scale on 2-bit
storage; the 2-bit code 00 -> 0, 01 -> +1, 11 -> -1 is this library's reading).

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, exhaustive bit-order probes, exact 128-bit brute force, the MLX
affine identity, library fp16 decoding, hand-worked fixtures under
``tests/golden/``).  No function is left "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SRC = HERE / "bonsai_oracle.c"
LIB = HERE / "_build" / "libbonsai_oracle.so"

OK, ERR_SHAPE, ERR_CODE, ERR_NONFINITE, ERR_NOMEM = 0, 2, 5, 7, 8

# Plain IEEE evaluation: no fast-math, no FMA contraction, so the double sum is
# the left-to-right sum of exactly rounded additions.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off"]


def build(src: Path = SRC, out: Path = LIB) -> Path:
    """Compile the oracle with gcc (always recompiles)."""
    out.parent.mkdir(parents=True, exist_ok=True)
    tmp = out.with_suffix(f".so.tmp{os.getpid()}")
    subprocess.run(["gcc", *CFLAGS, str(src), "-o", str(tmp), "-lm"], check=True)
    os.replace(tmp, out)
    return out


_i64p = ctypes.POINTER(ctypes.c_int64)
_dp = ctypes.POINTER(ctypes.c_double)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_MM_ARGS = [_u32p, _u16p, _u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            _i64p, ctypes.c_int64, _i64p, ctypes.c_int64, _dp]


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(t)


class OracleError(RuntimeError):
    def __init__(self, fn: str, rc: int):
        super().__init__(f"{fn} returned status {rc}")
        self.rc = rc


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: Path | str):
        self.path = Path(path)
        lib = ctypes.CDLL(str(self.path))
        lib.bo_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.bo_f16_to_f64.restype = ctypes.c_double
        for fn in ("bo_q1_dequant", "bo_q2t_dequant"):
            f = getattr(lib, fn)
            f.argtypes = [_u32p, _u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                          ctypes.c_int64, _dp]
            f.restype = ctypes.c_int
        for fn in ("bo_q1_matmul", "bo_q2t_matmul"):
            f = getattr(lib, fn)
            f.argtypes = _MM_ARGS + [_dp]
            f.restype = ctypes.c_int
        lib.bo_q1a_dequant.argtypes = [_u32p, _u16p, _u16p, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int64, _dp]
        lib.bo_q1a_dequant.restype = ctypes.c_int
        lib.bo_q1a_matmul.argtypes = [_u32p, _u16p, _u16p] + _MM_ARGS[2:] + [_dp]
        lib.bo_q1a_matmul.restype = ctypes.c_int
        _u8p = ctypes.POINTER(ctypes.c_uint8)
        lib.bo_t5_dequant.argtypes = [_u8p, _u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int64, _dp]
        lib.bo_t5_dequant.restype = ctypes.c_int
        lib.bo_t5_matmul.argtypes = [_u8p] + _MM_ARGS[1:] + [_dp]
        lib.bo_t5_matmul.restype = ctypes.c_int
        for fn in ("bo_q1_exact", "bo_q2t_exact"):
            f = getattr(lib, fn)
            f.argtypes = _MM_ARGS
            f.restype = ctypes.c_int
        self._lib = lib

    # -- scalars ---------------------------------------------------------------------------
    def f16_to_f64(self, bits: int) -> float:
        return self._lib.bo_f16_to_f64(int(bits) & 0xFFFF)

    # -- dense dequantisation --------------------------------------------------------------
    def _dequant(self, fn, words, scales, K, n0, n1, wtype=np.uint32, wptr=_u32p):
        words = np.ascontiguousarray(words, dtype=wtype)
        scales = np.ascontiguousarray(scales, dtype=np.uint16)
        N = words.shape[0]
        W = np.empty((n1 - n0, K), dtype=np.float64)
        rc = getattr(self._lib, fn)(_ptr(words, wptr), _ptr(scales, _u16p), N, K, n0, n1,
                                    _ptr(W, _dp))
        if rc:
            raise OracleError(fn, rc)
        return W

    def q1_dequant(self, wbits, scales, K, n0=0, n1=None):
        """Dense double rows [n0, n1) of the binary weight matrix."""
        return self._dequant("bo_q1_dequant", wbits, scales, K, n0,
                             wbits.shape[0] if n1 is None else n1)

    def q2t_dequant(self, wcodes, scales, K, n0=0, n1=None):
        return self._dequant("bo_q2t_dequant", wcodes, scales, K, n0,
                             wcodes.shape[0] if n1 is None else n1)

    def t5_dequant(self, codes, scales, K, n0=0, n1=None):
        """Dense double rows of the base-3 ternary matrix (five trits per byte)."""
        return self._dequant("bo_t5_dequant", codes, scales, K, n0,
                             codes.shape[0] if n1 is None else n1, np.uint8, ctypes.POINTER(ctypes.c_uint8))

    def q1a_dequant(self, wbits, scales, biases, K, n0=0, n1=None):
        """Dense double rows of the affine 1-bit matrix: w = scale * bit + bias per group."""
        wbits = np.ascontiguousarray(wbits, dtype=np.uint32)
        scales = np.ascontiguousarray(scales, dtype=np.uint16)
        biases = np.ascontiguousarray(biases, dtype=np.uint16)
        N = wbits.shape[0]
        n1 = N if n1 is None else n1
        W = np.empty((n1 - n0, K), dtype=np.float64)
        rc = self._lib.bo_q1a_dequant(_ptr(wbits, _u32p), _ptr(scales, _u16p), _ptr(biases, _u16p),
                                      N, K, n0, n1, _ptr(W, _dp))
        if rc:
            raise OracleError("bo_q1a_dequant", rc)
        return W

    # -- matmul ------------------------------------------------------------------------------
    def _mm(self, fn, words, scales, x, K, m_idx, n_idx, with_abs, biases=None, wtype=np.uint32,
            wptr=_u32p):
        words = np.ascontiguousarray(words, dtype=wtype)
        scales = np.ascontiguousarray(scales, dtype=np.uint16)
        x = np.ascontiguousarray(x, dtype=np.uint16)
        M, N = x.shape[0], words.shape[0]
        mi = None if m_idx is None else np.ascontiguousarray(m_idx, dtype=np.int64)
        ni = None if n_idx is None else np.ascontiguousarray(n_idx, dtype=np.int64)
        mc = M if mi is None else mi.size
        nc = N if ni is None else ni.size
        y = np.empty((mc, nc), dtype=np.float64)
        args = [_ptr(words, wptr), _ptr(scales, _u16p), _ptr(x, _u16p), M, N, K,
                None if mi is None else _ptr(mi, _i64p), mc,
                None if ni is None else _ptr(ni, _i64p), nc, _ptr(y, _dp)]
        if biases is not None:
            biases = np.ascontiguousarray(biases, dtype=np.uint16)
            args.insert(2, _ptr(biases, _u16p))
        a = None
        if with_abs is not None:
            a = np.empty_like(y)
            args.append(_ptr(a, _dp))
        rc = getattr(self._lib, fn)(*args)
        if rc:
            raise OracleError(fn, rc)
        return (y, a) if with_abs is not None else y

    def q1_matmul(self, wbits, scales, x, K, m_idx=None, n_idx=None):
        """(y, a): y = x W^T and a = |x| |W|^T in double, [len(m_idx), len(n_idx)]."""
        return self._mm("bo_q1_matmul", wbits, scales, x, K, m_idx, n_idx, True)

    def q2t_matmul(self, wcodes, scales, x, K, m_idx=None, n_idx=None):
        return self._mm("bo_q2t_matmul", wcodes, scales, x, K, m_idx, n_idx, True)

    def t5_matmul(self, codes, scales, x, K, m_idx=None, n_idx=None):
        """(y, a) for base-3 ternary weights (five trits per byte)."""
        return self._mm("bo_t5_matmul", codes, scales, x, K, m_idx, n_idx, True, wtype=np.uint8,
                        wptr=ctypes.POINTER(ctypes.c_uint8))

    def q1a_matmul(self, wbits, scales, biases, x, K, m_idx=None, n_idx=None):
        """(y, a) for affine 1-bit weights (MLX's scale-and-bias form, model card 'MLX packaging')."""
        return self._mm("bo_q1a_matmul", wbits, scales, x, K, m_idx, n_idx, True, biases=biases)

    def q1_exact(self, wbits, scales, x, K, m_idx=None, n_idx=None):
        """y computed exactly (128-bit fixed point), rounded once to double."""
        return self._mm("bo_q1_exact", wbits, scales, x, K, m_idx, n_idx, None)

    def q2t_exact(self, wcodes, scales, x, K, m_idx=None, n_idx=None):
        return self._mm("bo_q2t_exact", wcodes, scales, x, K, m_idx, n_idx, None)


_default: Oracle | None = None


def load() -> Oracle:
    """The oracle built from this directory (compiled on first use if absent)."""
    global _default
    if _default is None:
        if not LIB.exists() or LIB.stat().st_mtime < SRC.stat().st_mtime:
            build()
        _default = Oracle(LIB)
    return _default


def tolerance(a: np.ndarray) -> np.ndarray:
    """Acceptance bound for a float result against the oracle: 1e-3 * sum|w x| + 1e-6."""
    return 1e-3 * a + 1e-6


# -- storage accounting ------------------------------------------------------------------------
# Bits per weight of each storage form, from the pages: one sign bit plus a 16-bit
# scale shared by 128 weights (model card, "Weight representation" and "Memory
# requirement"); 2-bit ternary codes plus the same scale (ternary article, limitations);
# MLX's scale-plus-bias packing of the binary weights (model card, "MLX packaging");
# this library's base-3 ternary layout, five trits per byte plus the same scale (its own
# layout: the ternary article gives only the log2(3) + 16/128 bound it approaches).
def bits_per_weight(form: str) -> float:
    return {"q1": 1 + 16 / 128, "q2t": 2 + 16 / 128, "mlx_affine_1bit": 1 + 32 / 128,
            "t5": 8 / 5 + 16 / 128, "fp16": 16.0}[form]


def packed_bytes(form: str, N: int, K: int) -> int:
    """Bytes the packed weights of an N x K matrix occupy (words + scales)."""
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    if form == "q1":
        return N * K // 8 + 2 * N * (K // 128)
    if form == "q2t":
        return N * K // 4 + 2 * N * (K // 128)
    if form == "t5":
        return N * 32 * ((K + 159) // 160) + 2 * N * (K // 128)
    raise ValueError(form)
