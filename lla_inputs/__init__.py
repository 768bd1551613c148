"""Seeded synthetic inputs for the causal Local Linear Attention (LLA) forward.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic.  Both the fp64 oracle tests and the GPU path (tests,
``bench.py``, ``smoke()``) take their inputs from here, so the two sides see
bit-identical values.

Workloads (the shapes of the pages' settings, synthetic stand-ins for their data):

* ``tiny``      B1 H1 n64 d16, fp32, q,k,v ~ N(0,1); h = 4, lambda = 1e-2.
                Variant ``tiny_affine``: same q,k, v = k A^T + c exactly (A, c ~ N(0,1)),
                lambda = 0 (exact affine recovery on rows i >= d).
* ``halfnormal`` B1 H4 n1024 d64, fp32, q,k ~ N(0,1)/d^(1/4), v ~ N(0,1), key coordinate 0
                folded to |.| so about half of the queries sit outside the key support
                along e_0 (boundary queries); h = 8, lambda = 1e-1.
* ``d12``       B4 H12 n2048 d64, bf16, q,k RMS-normalised, v ~ N(0,1); h = 8, lambda = 1e-1
                (head shape of a 12-layer, 768-wide, 12-head model).
* ``d24``       B2 H16 n4096 d64, bf16, q,k RMS-normalised, v = k A^T + c + 0.1 N(0,1) per
                head; h = 8, lambda = 1e-2 (head shape of a 1024-wide, 16-head model; the
                headline throughput workload).
* ``long``      B1 H8 n16384 d128, bf16, q,k RMS-normalised, v ~ N(0,1); h = sqrt(128),
                lambda = 1e-1 (long context, large head).
* ``parallax_d12``, ``parallax_d24``: the q, k, v of ``d12`` and ``d24`` (same seeds and
                recipes, so bit-identical) plus a Parallax probe rho (``generate_probe``);
                h as there, lambda unused.

Decode workloads (``DECODE_WORKLOADS``, Parallax decode: one query per (batch, head) against a
key-value cache of L positions; batch and context sizes from the pages' decode sweep):

* ``decode_b8_l8192``  B8 H16 L8192 d64 bf16 (seed 5); h = 8.
* ``decode_b1_l32768`` B1 H16 L32768 d64 bf16 (seed 6): the sweep's longest context.
* ``decode_b64_l1024`` B64 H16 L1024 d64 bf16 (seed 7): many short caches.
* ``decode_d128``      B8 H8 L8192 d128 bf16 (seed 8); h = sqrt(128): the I/O-matched head size.
* ``lla_decode_b8_l8192`` the q, k, v of ``decode_b8_l8192`` (same seed, bit-identical) for the
                LLA decode step, lambda = 1e-2 (as the headline forward workload).
Decode recipe: ``default_rng(seed)`` draws, in fp64 and in this order, q ``[B,H,d]``, k and v
``[B,H,L,d]`` (standard normal), then rho ``[B,H,d]``; q, k and rho are RMS-normalised, v is
left as drawn; all four are cast once to the storage dtype.

Probe recipe (Parallax workloads): ``numpy.random.default_rng([seed, 1])`` -- a stream of
its own, so drawing rho changes none of q, k, v -- draws rho ``[B,H,n,d]`` standard normal
in fp64; rho is RMS-normalised like q and k (the pages' Parallax layers apply RMSNorm to
rho) and cast once to the workload's storage dtype.

Recipe: ``numpy.random.default_rng(seed)`` draws, in fp64 and in this order, q, k, v
(each ``[B,H,n,d]`` standard normal) and then the workload's extras (A ``[B,H,d,d]``,
c ``[B,H,d]``).  RMS normalisation is ``x / sqrt(mean(x^2, -1) + 1e-6)`` in fp64 with no
gain.  Values are then cast once: fp32 by ``astype``; bf16 by round-to-nearest-even of
the fp32 value (done here on the bit pattern, identical to ``torch``'s cast).  Arrays are
returned as float32 numpy arrays whose values are exactly representable in the stated
storage dtype.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_probe", "make_cotangent", "round_to_bf16", "generate",
           "generate_probe", "generate_cotangent", "DecodeWorkload", "DECODE_WORKLOADS", "generate_decode"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    n: int
    d: int
    dtype: str  # storage dtype of q, k, v: "f32" or "bf16"
    h: float
    lam: float
    seed: int
    recipe: str  # "normal", "affine_exact", "halfnormal", "rms", "rms_affine_noisy"

    @property
    def queries(self) -> int:
        return self.B * self.H * self.n

    @property
    def pairs(self) -> int:
        return self.B * self.H * self.n * (self.n + 1) // 2

    def with_shape(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 64, 16, "f32", 4.0, 1e-2, 0, "normal"),
    "tiny_affine": Workload("tiny_affine", 1, 1, 64, 16, "f32", 4.0, 0.0, 0, "affine_exact"),
    "halfnormal": Workload("halfnormal", 1, 4, 1024, 64, "f32", 8.0, 1e-1, 1, "halfnormal"),
    "d12": Workload("d12", 4, 12, 2048, 64, "bf16", 8.0, 1e-1, 2, "rms"),
    "d24": Workload("d24", 2, 16, 4096, 64, "bf16", 8.0, 1e-2, 3, "rms_affine_noisy"),
    "long": Workload("long", 1, 8, 16384, 128, "bf16", math.sqrt(128.0), 1e-1, 4, "rms"),
    "parallax_d12": Workload("parallax_d12", 4, 12, 2048, 64, "bf16", 8.0, 0.0, 2, "rms"),
    "parallax_d24": Workload("parallax_d24", 2, 16, 4096, 64, "bf16", 8.0, 0.0, 3, "rms_affine_noisy"),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(x.shape)


def _rms(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + 1e-6)


def make_inputs(B: int, H: int, n: int, d: int, seed: int, recipe: str, extras: bool = False):
    """Draw the fp64 (pre-cast) q, k, v of one workload recipe.

    With ``extras=True`` also return a dict holding the recipe's extra draws (A, c)."""
    rng = np.random.default_rng(seed)
    shape = (B, H, n, d)
    ex = {}
    q = rng.standard_normal(shape)
    k = rng.standard_normal(shape)
    v = rng.standard_normal(shape)
    if recipe == "normal":
        pass
    elif recipe == "affine_exact":
        A = rng.standard_normal((B, H, d, d))
        c = rng.standard_normal((B, H, d))
        v = np.einsum("bhjd,bhed->bhje", k, A) + c[:, :, None, :]
        ex = dict(A=A, c=c)
    elif recipe == "halfnormal":
        q = q / d ** 0.25
        k = k / d ** 0.25
        k[..., 0] = np.abs(k[..., 0])
    elif recipe == "rms":
        q = _rms(q)
        k = _rms(k)
    elif recipe == "rms_affine_noisy":
        q = _rms(q)
        k = _rms(k)
        A = rng.standard_normal((B, H, d, d))
        c = rng.standard_normal((B, H, d))
        v = np.einsum("bhjd,bhed->bhje", k, A) + c[:, :, None, :] + 0.1 * v
        ex = dict(A=A, c=c)
    else:
        raise ValueError(f"unknown recipe {recipe!r}")
    if extras:
        return q, k, v, ex
    return q, k, v


def cast(x: np.ndarray, dtype: str) -> np.ndarray:
    """Cast fp64 values once to the storage dtype; returned as float32 holding exact values."""
    x32 = x.astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return round_to_bf16(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


def generate(w: Workload):
    """Return (q, k, v) of workload ``w`` as float32 arrays holding the cast values,
    plus the fp64 pre-cast arrays: ``(q, k, v, (q64, k64, v64))``."""
    q64, k64, v64 = make_inputs(w.B, w.H, w.n, w.d, w.seed, w.recipe)
    return cast(q64, w.dtype), cast(k64, w.dtype), cast(v64, w.dtype), (q64, k64, v64)


def make_probe(B: int, H: int, n: int, d: int, seed: int) -> np.ndarray:
    """Draw the fp64 (pre-cast) Parallax probe rho ``[B,H,n,d]``: standard normal from the
    stream ``default_rng([seed, 1])``, RMS-normalised."""
    rng = np.random.default_rng([seed, 1])
    return _rms(rng.standard_normal((B, H, n, d)))


def generate_probe(w: Workload):
    """Return the probe of workload ``w`` as a float32 array holding the cast values, plus
    the fp64 pre-cast array: ``(rho, rho64)``."""
    rho64 = make_probe(w.B, w.H, w.n, w.d, w.seed)
    return cast(rho64, w.dtype), rho64


def make_cotangent(B: int, H: int, n: int, d: int, seed: int) -> np.ndarray:
    """Draw the fp64 (pre-cast) output cotangent dout ``[B,H,n,d]`` for backward tests and
    benchmarks: standard normal from the stream ``default_rng([seed, 2])``."""
    return np.random.default_rng([seed, 2]).standard_normal((B, H, n, d))


def generate_cotangent(w: Workload):
    """The cotangent of workload ``w`` as float32 holding the cast values, plus the fp64
    pre-cast array: ``(dout, dout64)``."""
    d64 = make_cotangent(w.B, w.H, w.n, w.d, w.seed)
    return cast(d64, w.dtype), d64


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    H: int
    L: int   # cached positions; the query is the newest one and sees all of them
    d: int
    dtype: str
    h: float
    seed: int
    lam: float = 0.0   # ridge of the LLA decode step (unused by Parallax)

    @property
    def queries(self) -> int:
        return self.B * self.H

    def with_shape(self, **kw) -> "DecodeWorkload":
        return dataclasses.replace(self, **kw)


DECODE_WORKLOADS = {
    "decode_b8_l8192": DecodeWorkload("decode_b8_l8192", 8, 16, 8192, 64, "bf16", 8.0, 5),
    "decode_b1_l32768": DecodeWorkload("decode_b1_l32768", 1, 16, 32768, 64, "bf16", 8.0, 6),
    "decode_b64_l1024": DecodeWorkload("decode_b64_l1024", 64, 16, 1024, 64, "bf16", 8.0, 7),
    "decode_d128": DecodeWorkload("decode_d128", 8, 8, 8192, 128, "bf16", math.sqrt(128.0), 8),
    "lla_decode_b8_l8192": DecodeWorkload("lla_decode_b8_l8192", 8, 16, 8192, 64, "bf16", 8.0, 5, 1e-2),
}


def generate_decode(w: DecodeWorkload):
    """Return (q [B,H,d], k [B,H,L,d], v [B,H,L,d], rho [B,H,d]) of a decode workload as
    float32 arrays holding the cast values."""
    rng = np.random.default_rng(w.seed)
    q = _rms(rng.standard_normal((w.B, w.H, w.d)))
    k = _rms(rng.standard_normal((w.B, w.H, w.L, w.d)))
    v = rng.standard_normal((w.B, w.H, w.L, w.d))
    rho = _rms(rng.standard_normal((w.B, w.H, w.d)))
    return tuple(cast(x, w.dtype) for x in (q, k, v, rho))
