"""Python binding of libbonsai (binary / ternary g128 weight-only matmul on MI355X).

Argument marshalling only: every step of the computation runs in the gfx950 kernels of
``_lib/libbonsai.so``, reached through its C ABI (``include/bonsai.h``).  PyTorch supplies
device memory and the current HIP stream; nothing here computes a result on the host.
If the shared library has not been built, importing this package raises ImportError.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import numpy as np

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "_lib" / "libbonsai.so"

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_VALUE, ERR_CODE, ERR_DEVICE = range(7)
MAX_K = 131072
GEMV_MAX_M = 8

# PyTorch ships its own HIP runtime, loaded under the name libamdhip64.so.  Importing torch
# first makes libbonsai's libamdhip64.so.7 dependency resolve to that same runtime (same
# SONAME), so the process holds one HIP runtime and torch's streams and memory are valid here.
import torch  # noqa: E402,F401

if not LIB_PATH.exists():
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python -c 'import __graft_entry__ as g; g.build()'` (hipcc, gfx950)")

_lib = ctypes.CDLL(str(LIB_PATH))
_c_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
for _name in ("bonsai_q1_gemv", "bonsai_q1_gemm", "bonsai_q2t_gemv", "bonsai_q2t_gemm"):
    _f = getattr(_lib, _name)
    _f.argtypes = [_vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _vp]
    _f.restype = ctypes.c_int
for _name in ("bonsai_q1_pack", "bonsai_q1_unpack", "bonsai_q2t_pack", "bonsai_q2t_unpack"):
    _f = getattr(_lib, _name)
    _f.argtypes = [_vp, _c_i64, _c_i64, _vp]
    _f.restype = ctypes.c_int
_lib.bonsai_t5_matmul.argtypes = [_vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _vp]
_lib.bonsai_t5_matmul.restype = ctypes.c_int
for _name in ("bonsai_t5_pack", "bonsai_t5_unpack", "bonsai_q2t_to_t5", "bonsai_t5_to_q2t"):
    _f = getattr(_lib, _name)
    _f.argtypes = [_vp, _c_i64, _c_i64, _vp]
    _f.restype = ctypes.c_int
_lib.bonsai_q1a_matmul.argtypes = [_vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _vp]
_lib.bonsai_q1a_matmul.restype = ctypes.c_int
_lib.bonsai_q1_to_affine.argtypes = [_vp, _c_i64, _vp, _vp]
_lib.bonsai_q1_to_affine.restype = ctypes.c_int
_lib.bonsai_q1_from_affine.argtypes = [_vp, _vp, _c_i64, _vp]
_lib.bonsai_q1_from_affine.restype = ctypes.c_int
_lib.bonsai_q1_embed.argtypes = [_vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _vp]
_lib.bonsai_q1_embed.restype = ctypes.c_int
_lib.bonsai_plan.argtypes = [ctypes.c_int, _c_i64, _c_i64, _c_i64, ctypes.c_int, ctypes.c_char_p, _c_i64]
_lib.bonsai_plan.restype = ctypes.c_int
_lib.bonsai_probe_stream.argtypes = [_vp, _c_i64, ctypes.c_int, _vp, _vp]
_lib.bonsai_probe_stream.restype = ctypes.c_int
_lib.bonsai_probe_clock.argtypes = [_vp, _c_i64, _vp]
_lib.bonsai_probe_clock.restype = ctypes.c_int
_lib.bonsai_time_next_launch.argtypes = [_vp, _vp]
_lib.bonsai_time_next_launch.restype = ctypes.c_int
_lib.bonsai_last_device_error.argtypes = []
_lib.bonsai_last_device_error.restype = ctypes.c_char_p
_lib.bonsai_status_str.argtypes = [ctypes.c_int]
_lib.bonsai_status_str.restype = ctypes.c_char_p


class BonsaiError(RuntimeError):
    def __init__(self, fn: str, status: int):
        detail = f" [{_lib.bonsai_last_device_error().decode()}]" if status == ERR_DEVICE else ""
        super().__init__(f"{fn}: {status_str(status)} (status {status}){detail}")
        self.status = status


def status_str(status: int) -> str:
    return _lib.bonsai_status_str(int(status)).decode()


def raw():
    """The ctypes handle of libbonsai.so (argtypes set), for callers passing raw pointers."""
    return _lib


def time_next_launch(start_event: int, stop_event: int) -> None:
    """Arm the measurement hook: the next GPU call on this thread records the two hipEvent_t
    handles around its kernel's execution (bonsai_time_next_launch)."""
    _check("bonsai_time_next_launch", _lib.bonsai_time_next_launch(start_event, stop_event))


PLAN_OPS = {"q1_gemv": 0, "q1_gemm": 1, "q2t_gemv": 2, "q2t_gemm": 3, "t5_matmul": 4, "q1a_matmul": 5,
            "q1_embed": 6}


def plan(op: str, M: int, N: int, K: int, cus: int = 0) -> str:
    """The kernel launch the entry point `op` would enqueue for these sizes (bonsai_plan):
    "<kernel> grid=x,y block=b lds=l", or "none".  cus > 0 plans for a device with that many
    compute units without touching any GPU; cus = 0 plans for the current device."""
    buf = ctypes.create_string_buffer(512)
    _check("bonsai_plan", _lib.bonsai_plan(PLAN_OPS[op], M, N, K, cus, buf, len(buf)))
    return buf.value.decode()


def probe_stream(buf, nbytes: int, mode: int, sink) -> None:
    """Stream nbytes of the device tensor buf once (mode 0: vector loads, 1: direct global->LDS
    copies, 2: write zeros); sink: a device tensor of at least 64 KiB (bonsai_probe_stream)."""
    import torch

    if buf.numel() * buf.element_size() < nbytes or sink.numel() * sink.element_size() < 65536:
        raise ValueError("buffer shorter than nbytes, or sink under 64 KiB")
    stream = torch.cuda.current_stream(buf.device).cuda_stream
    _check("bonsai_probe_stream", _lib.bonsai_probe_stream(buf.data_ptr(), nbytes, mode, sink.data_ptr(), stream))


def probe_clock(stamps, spin_ns: int, stream: int | None = None) -> None:
    """One wave stamps the shader and real-time clocks, waits spin_ns, stamps again into the
    int64 device tensor stamps[4] (bonsai_probe_clock); on `stream` (a hipStream_t) if given."""
    import torch

    if stamps.dtype != torch.int64 or stamps.numel() < 4 or not stamps.is_cuda:
        raise ValueError("stamps must be an int64 device tensor of 4 elements")
    if stream is None:
        stream = torch.cuda.current_stream(stamps.device).cuda_stream
    _check("bonsai_probe_clock", _lib.bonsai_probe_clock(stamps.data_ptr(), spin_ns, stream))


def _check(fn: str, status: int):
    if status != OK:
        raise BonsaiError(fn, status)


# ---------------------------------------------------------------------------------------
# GPU entry points (torch tensors in device memory)
# ---------------------------------------------------------------------------------------
def _dev_args(words, scales, x, out, n_word_div: int):
    import torch

    for name, t, ok in (("words", words, (torch.int32, torch.uint32)),
                        ("scales", scales, (torch.float16, torch.int16, torch.uint16)),
                        ("x", x, (torch.float16, torch.int16, torch.uint16))):
        if t.dtype not in ok:
            raise TypeError(f"{name}: dtype {t.dtype} not in {ok}")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if words.dim() != 2 or scales.dim() != 2 or x.dim() != 2:
        raise ValueError("words [N, K/w], scales [N, K/128] and x [M, K] must be 2-D")
    M, K = x.shape
    N = words.shape[0]
    if words.shape[1] * n_word_div != K or tuple(scales.shape) != (N, K // 128):
        raise ValueError(f"inconsistent shapes words {tuple(words.shape)}, scales "
                         f"{tuple(scales.shape)}, x {tuple(x.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [M, N] tensor")
    stream = torch.cuda.current_stream(x.device).cuda_stream
    return M, N, K, out, stream


def _call(fn: str, words, scales, x, out, div):
    M, N, K, out, stream = _dev_args(words, scales, x, out, div)
    _check(fn, getattr(_lib, fn)(words.data_ptr(), scales.data_ptr(), x.data_ptr(), out.data_ptr(),
                                 M, N, K, stream))
    return out


def q1_gemv(wbits, scales, x, out=None):
    """y[M, N] = x[M, K] W^T for binary g128 weights, 1 <= M <= 8 (bonsai_q1_gemv)."""
    return _call("bonsai_q1_gemv", wbits, scales, x, out, 32)


def q1_gemm(wbits, scales, x, out=None):
    """y[M, N] = x[M, K] W^T for binary g128 weights, any M (bonsai_q1_gemm)."""
    return _call("bonsai_q1_gemm", wbits, scales, x, out, 32)


def q2t_gemv(wcodes, scales, x, out=None):
    """y[M, N] = x[M, K] W^T for ternary g128 weights on 2-bit codes, 1 <= M <= 8."""
    return _call("bonsai_q2t_gemv", wcodes, scales, x, out, 16)


def q2t_gemm(wcodes, scales, x, out=None):
    """y[M, N] = x[M, K] W^T for ternary g128 weights on 2-bit codes, any M (bonsai_q2t_gemm)."""
    return _call("bonsai_q2t_gemm", wcodes, scales, x, out, 16)


def t5_row_bytes(K: int) -> int:
    """Bytes per row of the base-3 ternary layout: 32-byte superblocks of 160 weights."""
    return 32 * ((K + 159) // 160)


def t5_matmul(codes, scales, x, out=None):
    """y[M, N] = x[M, K] W^T for base-3 ternary weights (five trits per byte; bonsai_t5_matmul),
    any M.  codes: uint8 [N, 32 ceil(K/160)]."""
    import torch

    if codes.dtype not in (torch.uint8, torch.int8) or codes.dim() != 2:
        raise TypeError("codes must be a 2-D uint8 tensor")
    if scales.dtype not in (torch.float16, torch.int16, torch.uint16) or x.dtype not in (torch.float16, torch.int16, torch.uint16):
        raise TypeError("scales and x must be binary16 tensors")
    for name, t in (("codes", codes), ("scales", scales), ("x", x)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    M, K = x.shape
    N = codes.shape[0]
    if codes.shape[1] != t5_row_bytes(K) or tuple(scales.shape) != (N, K // 128):
        raise ValueError(f"inconsistent shapes codes {tuple(codes.shape)}, scales {tuple(scales.shape)}, "
                         f"x {tuple(x.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [M, N] tensor")
    stream = torch.cuda.current_stream(x.device).cuda_stream
    _check("bonsai_t5_matmul", _lib.bonsai_t5_matmul(codes.data_ptr(), scales.data_ptr(), x.data_ptr(),
                                                     out.data_ptr(), M, N, K, stream))
    return out


def q1a_matmul(wbits, mlx_scales, biases, x, out=None):
    """y[M, N] = x[M, K] W^T for affine 1-bit weights W = a q + b per group of 128 (MLX's 1-bit
    form of the binary words; bonsai_q1a_matmul), any M."""
    import torch

    M, N, K, out, stream = _dev_args(wbits, mlx_scales, x, out, 32)
    if biases.dtype not in (torch.float16, torch.int16, torch.uint16) or not biases.is_cuda \
            or not biases.is_contiguous() or tuple(biases.shape) != tuple(mlx_scales.shape):
        raise ValueError("biases must be a contiguous binary16 device tensor shaped like the scales")
    _check("bonsai_q1a_matmul", _lib.bonsai_q1a_matmul(wbits.data_ptr(), mlx_scales.data_ptr(), biases.data_ptr(),
                                                       x.data_ptr(), out.data_ptr(), M, N, K, stream))
    return out


def q1_embed(wbits, scales, ids, out=None):
    """out[i, :] = dequantized row ids[i] of a binary g128 table (binary16, exact); ids outside
    [0, V) give zero rows (bonsai_q1_embed)."""
    import torch

    if wbits.dtype not in (torch.int32, torch.uint32) or scales.dtype not in (torch.float16, torch.int16, torch.uint16):
        raise TypeError("wbits must be int32/uint32 and scales float16/int16/uint16")
    if ids.dtype != torch.int64:
        raise TypeError("ids must be int64")
    for name, t in (("wbits", wbits), ("scales", scales), ("ids", ids)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    V, K = wbits.shape[0], wbits.shape[1] * 32
    if tuple(scales.shape) != (V, K // 128):
        raise ValueError(f"inconsistent shapes wbits {tuple(wbits.shape)}, scales {tuple(scales.shape)}")
    n = ids.numel()
    if out is None:
        out = torch.empty((n, K), dtype=torch.float16, device=ids.device)
    elif out.dtype not in (torch.float16, torch.int16) or tuple(out.shape) != (n, K) or not out.is_contiguous():
        raise ValueError("out must be a contiguous float16 [n_ids, K] tensor")
    stream = torch.cuda.current_stream(ids.device).cuda_stream
    _check("bonsai_q1_embed", _lib.bonsai_q1_embed(wbits.data_ptr(), scales.data_ptr(), ids.data_ptr(),
                                                   out.data_ptr(), n, V, K, stream))
    return out


# ---------------------------------------------------------------------------------------
# Host layout functions (numpy arrays in host memory)
# ---------------------------------------------------------------------------------------
def _host(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def q1_to_affine(scales: np.ndarray):
    """Binary scales (binary16 bits) -> MLX (scale, bias) = (2 s, -s), bit-exact (bonsai_q1_to_affine)."""
    s = _host(scales, np.uint16)
    a, b = np.empty_like(s), np.empty_like(s)
    _check("bonsai_q1_to_affine", _lib.bonsai_q1_to_affine(s.ctypes.data, s.size, a.ctypes.data, b.ctypes.data))
    return a, b


def q1_from_affine(mlx_scales: np.ndarray, biases: np.ndarray) -> np.ndarray:
    """MLX (scale, bias) with scale == -2 bias exactly -> binary scales (bonsai_q1_from_affine)."""
    a, b = _host(mlx_scales, np.uint16), _host(biases, np.uint16)
    if a.shape != b.shape:
        raise ValueError("scales and biases must have the same shape")
    s = np.empty_like(a)
    _check("bonsai_q1_from_affine", _lib.bonsai_q1_from_affine(a.ctypes.data, b.ctypes.data, a.size, s.ctypes.data))
    return s


def t5_pack(trits: np.ndarray) -> np.ndarray:
    """int8 trits [N, K] in {-1, 0, +1} -> base-3 bytes [N, 32 ceil(K/160)] (bonsai_t5_pack)."""
    t = _host(trits, np.int8)
    N, K = t.shape
    out = np.zeros((N, t5_row_bytes(K)), dtype=np.uint8)
    _check("bonsai_t5_pack", _lib.bonsai_t5_pack(t.ctypes.data, N, K, out.ctypes.data))
    return out


def t5_unpack(codes: np.ndarray, K: int) -> np.ndarray:
    c = _host(codes, np.uint8)
    N = c.shape[0]
    if c.shape[1] != t5_row_bytes(K):
        raise ValueError("codes must be [N, 32 ceil(K/160)]")
    out = np.empty((N, K), dtype=np.int8)
    _check("bonsai_t5_unpack", _lib.bonsai_t5_unpack(c.ctypes.data, N, K, out.ctypes.data))
    return out


def q2t_to_t5(wcodes: np.ndarray, K: int) -> np.ndarray:
    """2-bit ternary words [N, K/16] -> base-3 bytes [N, 32 ceil(K/160)] (bonsai_q2t_to_t5)."""
    w = _host(wcodes, np.uint32)
    N = w.shape[0]
    if w.shape[1] * 16 != K:
        raise ValueError("wcodes must be [N, K/16]")
    out = np.zeros((N, t5_row_bytes(K)), dtype=np.uint8)
    _check("bonsai_q2t_to_t5", _lib.bonsai_q2t_to_t5(w.ctypes.data, N, K, out.ctypes.data))
    return out


def t5_to_q2t(codes: np.ndarray, K: int) -> np.ndarray:
    """Base-3 bytes [N, 32 ceil(K/160)] -> 2-bit ternary words [N, K/16] (bonsai_t5_to_q2t)."""
    c = _host(codes, np.uint8)
    N = c.shape[0]
    if c.shape[1] != t5_row_bytes(K) or K % 16:
        raise ValueError("codes must be [N, 32 ceil(K/160)] and K a multiple of 16")
    out = np.empty((N, K // 16), dtype=np.uint32)
    _check("bonsai_t5_to_q2t", _lib.bonsai_t5_to_q2t(c.ctypes.data, N, K, out.ctypes.data))
    return out


def q1_pack(signs: np.ndarray) -> np.ndarray:
    """int8 signs [N, K] in {-1, +1} -> uint32 words [N, K/32] (bonsai_q1_pack)."""
    s = _host(signs, np.int8)
    N, K = s.shape
    out = np.empty((N, K // 32 if K % 32 == 0 else 0), dtype=np.uint32)
    _check("bonsai_q1_pack", _lib.bonsai_q1_pack(s.ctypes.data, N, K, out.ctypes.data))
    return out


def q1_unpack(wbits: np.ndarray, K: int) -> np.ndarray:
    w = _host(wbits, np.uint32)
    N = w.shape[0]
    out = np.empty((N, K), dtype=np.int8)
    if w.shape[1] * 32 != K:
        raise ValueError("wbits must be [N, K/32]")
    _check("bonsai_q1_unpack", _lib.bonsai_q1_unpack(w.ctypes.data, N, K, out.ctypes.data))
    return out


def q2t_pack(trits: np.ndarray) -> np.ndarray:
    """int8 trits [N, K] in {-1, 0, +1} -> uint32 words [N, K/16] (bonsai_q2t_pack)."""
    t = _host(trits, np.int8)
    N, K = t.shape
    out = np.empty((N, K // 16 if K % 16 == 0 else 0), dtype=np.uint32)
    _check("bonsai_q2t_pack", _lib.bonsai_q2t_pack(t.ctypes.data, N, K, out.ctypes.data))
    return out


def q2t_unpack(wcodes: np.ndarray, K: int) -> np.ndarray:
    w = _host(wcodes, np.uint32)
    N = w.shape[0]
    out = np.empty((N, K), dtype=np.int8)
    if w.shape[1] * 16 != K:
        raise ValueError("wcodes must be [N, K/16]")
    _check("bonsai_q2t_unpack", _lib.bonsai_q2t_unpack(w.ctypes.data, N, K, out.ctypes.data))
    return out
