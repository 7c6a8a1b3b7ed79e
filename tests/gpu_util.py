"""Helpers of the GPU tests: device transfer, calls through the C ABI, comparison."""
from __future__ import annotations

import sys

import numpy as np

import oracle


def torch_dev():
    import torch
    return torch, torch.device("cuda:0")


def to_dev(a: np.ndarray):
    """Host array -> contiguous device tensor with the same bytes (uint32 -> int32, uint16 -> int16)."""
    torch, dev = torch_dev()
    a = np.ascontiguousarray(a)
    view = {np.dtype(np.uint32): np.int32, np.dtype(np.uint16): np.int16}.get(a.dtype, a.dtype)
    return torch.from_numpy(a.view(view)).to(dev)


def note(msg: str):
    """Name the case before a GPU step, flushed, so a crash still says what ran."""
    sys.stdout.write(f"[gpu] {msg}\n")
    sys.stdout.flush()


def call(kind: str, w: np.ndarray, s: np.ndarray, x: np.ndarray, out=None):
    """Run one entry point on device copies of (w, s, x); returns the float32 result on the host."""
    import ternary_weight_quantized_bonsai_amd as bonsai
    torch, _ = torch_dev()
    fn = {"q1_gemv": bonsai.q1_gemv, "q1_gemm": bonsai.q1_gemm, "q2t_gemv": bonsai.q2t_gemv,
          "q2t_gemm": bonsai.q2t_gemm}[kind]
    note(f"{kind} M={x.shape[0]} N={w.shape[0]} K={x.shape[1]}")
    y = fn(to_dev(w), to_dev(s), to_dev(x), out=out)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def ref(kind: str, orc, w, s, x, m_idx=None, n_idx=None):
    K = x.shape[1]
    if kind.startswith("q1"):
        return orc.q1_matmul(w, s, x, K, m_idx, n_idx)
    return orc.q2t_matmul(w, s, x, K, m_idx, n_idx)


def exact(kind: str, orc, w, s, x, m_idx=None, n_idx=None):
    K = x.shape[1]
    if kind.startswith("q1"):
        return orc.q1_exact(w, s, x, K, m_idx, n_idx)
    return orc.q2t_exact(w, s, x, K, m_idx, n_idx)


def assert_close(y: np.ndarray, yref: np.ndarray, a: np.ndarray, what: str):
    """|y - y_ref| <= 1e-3 * sum|w x| + 1e-6 elementwise (the acceptance bound)."""
    assert y.shape == yref.shape, (what, y.shape, yref.shape)
    err = np.abs(y.astype(np.float64) - yref)
    tol = oracle.tolerance(a)
    bad = ~(err <= tol)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {y.size} out of tolerance; first at {tuple(i)}: "
                             f"got {y[tuple(i)]!r} want {yref[tuple(i)]!r} tol {tol[tuple(i)]:.3e}")
    return float((err / np.maximum(tol, 1e-300)).max())
