"""Seeded synthetic inputs for the binary / ternary g128 matmul.

This module is the only code shared by the oracle side and the GPU side.  It
draws random numbers and nothing else: it holds none of the method's
arithmetic (no sign mapping, no scale lookup, no bit order).  Every array is
returned in its storage form:

* sign words   - uint32, each bit an independent fair coin.  The generator does
                 not know which bit belongs to which k; every bit is iid.
* trit words   - uint32, each aligned 2-bit field independently one of the
                 patterns 0b00 / 0b01 / 0b11 with probabilities 0.4 / 0.3 / 0.3.
                 The fields are iid, so no field-to-k assignment is implied.
* scales       - IEEE binary16 bit patterns (uint16) of |N(0, 0.02)| + 1e-3,
                 rounded to nearest-even by numpy's float16 conversion.
* activations  - IEEE binary16 bit patterns (uint16) of N(0, 1).
* biases       - IEEE binary16 bit patterns (uint16) of N(0, 0.02), for the
                 affine (scale, bias) form of the binary words.
* base-3 bytes - uint8, each byte independently uniform over 0..242 (every
                 value below 243 is a valid byte; the generator knows only the
                 row length, 32 bytes per 160 weights).

The workload shapes are those of the model card ("1-bit Bonsai 27B",
model-overview table and the config summary on the Bonsai-27B article):
hidden size 5120, vocabulary 248,320, group size 128; the prefill length 512
comes from the pp512 column of the cross-platform throughput table.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Config", "CONFIGS", "rng_for", "sign_words", "trit_words", "scales_f16",
    "activations_f16", "biases_f16", "trits_i8", "t5_bytes", "make_q1", "make_q2t", "make_q1a", "make_t5",
    "make_t5_trits", "digest",
]


@dataclass(frozen=True)
class Config:
    name: str
    kind: str          # "q1_gemv" | "q1_gemm" | "q2t_gemv"
    M: int
    N: int
    K: int
    note: str


# The five workload shapes.  C1 is the small case the oracle finishes in
# well under a second; the others are the real decode / prefill shapes.
CONFIGS = {
    "C1": Config("C1", "q1_gemv", 1, 256, 512, "binary GEMV, 4 groups per row"),
    "C2a": Config("C2a", "q1_gemv", 1, 13824, 5120, "binary decode GEMV, MLP-shaped"),
    "C2b": Config("C2b", "q1_gemv", 1, 5120, 5120, "binary decode GEMV, attention-shaped"),
    "C3": Config("C3", "q1_gemv", 1, 248320, 5120, "binary LM-head GEMV, vocab rows"),
    "C4": Config("C4", "q1_gemm", 512, 13824, 5120, "binary prefill GEMM, pp512"),
    "C5": Config("C5", "q2t_gemv", 1, 5120, 5120, "ternary decode GEMV, M=1"),
    "C5m8": Config("C5m8", "q2t_gemv", 8, 5120, 5120, "ternary decode GEMV, M=8"),
    # beyond the five workloads: the ternary prefill at the binary prefill's shape (pp512)
    "C6": Config("C6", "q2t_gemm", 512, 13824, 5120, "ternary prefill GEMM, pp512"),
}


def rng_for(seed: int, tag: str) -> np.random.Generator:
    """An independent PCG64 stream for (seed, tag); tag names shape and array."""
    digest = hashlib.sha256(f"{seed}/{tag}".encode()).digest()
    return np.random.Generator(np.random.PCG64(int.from_bytes(digest[:16], "little")))


def sign_words(n_rows: int, n_words: int, seed: int, tag: str) -> np.ndarray:
    """uint32 [n_rows, n_words]; every bit an independent fair coin."""
    rng = rng_for(seed, tag + "/signs")
    return rng.integers(0, 1 << 32, size=(n_rows, n_words), dtype=np.uint64).astype(np.uint32)


def trit_words(n_rows: int, n_words: int, seed: int, tag: str,
               p_zero: float = 0.4, p_plus: float = 0.3) -> np.ndarray:
    """uint32 [n_rows, n_words] of 16 aligned 2-bit fields each.

    Each field is independently 0b00 (p_zero), 0b01 (p_plus) or 0b11 (the rest).
    The pattern 0b10 is never drawn.
    """
    rng = rng_for(seed, tag + "/trits")
    u = rng.random(size=(n_rows, n_words, 16))
    field = np.where(u < 1.0 - p_zero - p_plus, 3, np.where(u < 1.0 - p_zero, 1, 0)).astype(np.uint32)
    shifts = (2 * np.arange(16, dtype=np.uint32))
    return np.bitwise_or.reduce(field << shifts, axis=2).astype(np.uint32)


def scales_f16(n_rows: int, n_groups: int, seed: int, tag: str) -> np.ndarray:
    """uint16 [n_rows, n_groups]: binary16 bits of |N(0, 0.02)| + 1e-3."""
    rng = rng_for(seed, tag + "/scales")
    v = np.abs(rng.standard_normal(size=(n_rows, n_groups)) * 0.02) + 1e-3
    return v.astype(np.float16).view(np.uint16)


def activations_f16(m: int, k: int, seed: int, tag: str) -> np.ndarray:
    """uint16 [m, k]: binary16 bits of N(0, 1)."""
    rng = rng_for(seed, tag + "/x")
    return rng.standard_normal(size=(m, k)).astype(np.float16).view(np.uint16)


def biases_f16(n_rows: int, n_groups: int, seed: int, tag: str) -> np.ndarray:
    """uint16 [n_rows, n_groups]: binary16 bits of N(0, 0.02) (either sign)."""
    rng = rng_for(seed, tag + "/biases")
    return (rng.standard_normal(size=(n_rows, n_groups)) * 0.02).astype(np.float16).view(np.uint16)


def trits_i8(n_rows: int, k: int, seed: int, tag: str, p_zero: float = 0.4, p_plus: float = 0.3) -> np.ndarray:
    """int8 [n_rows, k]: each entry independently 0 (p_zero), +1 (p_plus) or -1."""
    rng = rng_for(seed, tag + "/trits8")
    u = rng.random(size=(n_rows, k))
    return np.where(u < 1.0 - p_zero - p_plus, -1, np.where(u < 1.0 - p_zero, 1, 0)).astype(np.int8)


def t5_bytes(n_rows: int, k: int, seed: int, tag: str) -> np.ndarray:
    """uint8 [n_rows, 32 ceil(k/160)]: each byte uniform over 0..242."""
    rng = rng_for(seed, tag + "/t5")
    return rng.integers(0, 243, size=(n_rows, 32 * ((k + 159) // 160)), dtype=np.uint8)


def make_q1(M: int, N: int, K: int, seed: int = 0, tag: str | None = None):
    """(sign words [N, K/32], scales [N, K/128], x [M, K]) for a binary matmul."""
    tag = tag or f"{N}x{K}"
    return (sign_words(N, K // 32, seed, tag), scales_f16(N, K // 128, seed, tag),
            activations_f16(M, K, seed, f"{tag}/M{M}"))


def make_q2t(M: int, N: int, K: int, seed: int = 0, tag: str | None = None):
    """(trit words [N, K/16], scales [N, K/128], x [M, K]) for a ternary matmul."""
    tag = tag or f"t{N}x{K}"
    return (trit_words(N, K // 16, seed, tag), scales_f16(N, K // 128, seed, tag),
            activations_f16(M, K, seed, f"{tag}/M{M}"))


def make_q1a(M: int, N: int, K: int, seed: int = 0, tag: str | None = None):
    """(sign words, scales, biases [N, K/128], x) for an affine 1-bit matmul."""
    tag = tag or f"a{N}x{K}"
    w, s, x = make_q1(M, N, K, seed, tag)
    return w, s, biases_f16(N, K // 128, seed, tag), x


def make_t5(M: int, N: int, K: int, seed: int = 0, tag: str | None = None):
    """(base-3 bytes [N, 32 ceil(K/160)], scales [N, K/128], x [M, K]) for a base-3 matmul."""
    tag = tag or f"t5{N}x{K}"
    return (t5_bytes(N, K, seed, tag), scales_f16(N, K // 128, seed, tag),
            activations_f16(M, K, seed, f"{tag}/M{M}"))


def make_t5_trits(M: int, N: int, K: int, seed: int = 0, tag: str | None = None):
    """(trits int8 [N, K], scales [N, K/128], x [M, K]) for a ternary matmul in any layout; the
    caller packs the trits (the packers hold the layouts, this module holds none)."""
    tag = tag or f"t5{N}x{K}"
    return (trits_i8(N, K, seed, tag), scales_f16(N, K // 128, seed, tag),
            activations_f16(M, K, seed, f"{tag}/M{M}"))


def digest(buf: np.ndarray) -> str:
    """Short SHA-256 of an array's bytes, so two hosts can show identical inputs."""
    return hashlib.sha256(np.ascontiguousarray(buf).view(np.uint8).tobytes()).hexdigest()[:16]
