"""Seeded synthetic inputs for the causal LLA forward pass.

This module only draws random tensors and casts them. It holds none of the
method's arithmetic (no weights, moments, solves or outputs), so that the GPU
path and the float64 CPU oracle can both be fed from it without sharing any
part of the computation.

Five workloads are defined. Each one takes the shape of a workload on the
pages and nothing else:

* ``tiny``      B=1 H=1 n=256  d=16,  fp32. Gaussian q,k,v; q,k unit rows.
* ``piecewise`` B=1 H=2 n=1024 d=64,  fp32. Keys uniform on the unit sphere,
  8 equal segments, each with its own linear map A_s ~ N(0, 1/d); values
  v_j = A_s k_j + 0.01 noise; the query at position i is the key of position
  i+1 (one extra key is drawn for the last position). Shape of the test-time
  piecewise regression study in the LLA paper (Sec. 4, Figs. 3-4: d=64,
  L=1024); no sequence from that study is reproduced.
* ``standard``  B=4 H=8 n=4096 d=128, bf16. Gaussian q,k,v; q,k unit rows
  scaled by 4.
* ``long``      B=1 H=16 n=16384 d=128, bf16. Gaussian q,k,v; q,k unit rows.
  Shape of the peak-memory curve (LLA paper, Sec. 3.2, Fig. 2: d=128).
* ``recall``    B=8 H=16 n=2048 d=128, bf16. Keys and queries are one of 256
  unit centres plus N(0, 0.05^2 I) noise (centre drawn independently for each
  key and each query); values are rows of a shared N(0,1) codebook with 8192
  entries. Shape of the MQAR recall task (LLA paper, Sec. 4, vocabulary
  8192); no MQAR item is reproduced.

Draw order: one ``numpy.random.default_rng(seed)`` per workload; shared
tensors first (the recall codebook), then per (b, h) in loop order b, h; within
a head q, k, v (for ``piecewise``: keys, maps, noise). All draws are float64,
then cast: fp32 by round-to-nearest, bf16 by float64 -> float32 -> bf16 with
round-to-nearest-even. The float64 widening of the cast values is what both
the GPU and the oracle see.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "make_workload",
    "make_scaled",
    "f64_to_bf16_bits",
    "bf16_bits_to_f64",
]


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    B: int
    H: int
    n: int
    d: int
    dtype: str          # "f32" or "bf16": the element type handed to the GPU
    lam: float
    cg_max_iters: int
    cg_rel_tol: float


SPECS = {
    "tiny": Spec("tiny", 1, 1, 256, 16, "f32", 0.1, 32, 1e-8),
    "piecewise": Spec("piecewise", 1, 2, 1024, 64, "f32", 0.1, 64, 1e-8),
    "standard": Spec("standard", 4, 8, 4096, 128, "bf16", 1.0, 16, 0.0),
    "long": Spec("long", 1, 16, 16384, 128, "bf16", 1.0, 24, 1e-4),
    "recall": Spec("recall", 8, 16, 2048, 128, "bf16", 1e-3, 64, 1e-4),
}
WORKLOADS = tuple(SPECS)


@dataclasses.dataclass
class Workload:
    """One generated workload.

    ``q, k, v`` are the exact values the GPU receives, widened to float64,
    shaped [B, H, n, d]. ``q_dev, k_dev, v_dev`` are the arrays to upload:
    float32 for fp32 workloads, uint16 bf16 bit patterns for bf16 workloads.
    """

    spec: Spec
    B: int
    H: int
    n: int
    d: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_dev: np.ndarray
    k_dev: np.ndarray
    v_dev: np.ndarray

    @property
    def name(self) -> str:
        return self.spec.name

    @property
    def dtype(self) -> str:
        return self.spec.dtype

    @property
    def lam(self) -> float:
        # lambda is passed to the library as a C float; this is its exact value
        return float(np.float32(self.spec.lam))

    @property
    def cg_max_iters(self) -> int:
        return self.spec.cg_max_iters

    @property
    def cg_rel_tol(self) -> float:
        return float(np.float32(self.spec.cg_rel_tol))


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (nearest) -> bfloat16 (nearest-even) bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    u = (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16))
    return u.view(np.float32).astype(np.float64)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _head_gaussian(rng, n, d, norm_scale):
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    if norm_scale is not None:
        q = _unit_rows(q) * norm_scale
        k = _unit_rows(k) * norm_scale
    return q, k, v


def _head_piecewise(rng, n, d, n_segments=8, noise=0.01):
    keys = _unit_rows(rng.standard_normal((n + 1, d)))
    seg_len = max(1, n // n_segments)
    maps = rng.standard_normal((n_segments, d, d)) / np.sqrt(d)
    eps = rng.standard_normal((n, d))
    k = keys[:n]
    seg = np.minimum(np.arange(n) // seg_len, n_segments - 1)
    v = np.einsum("jab,jb->ja", maps[seg], k) + noise * eps
    q = keys[1:n + 1]
    return q, k, v


def _head_recall(rng, n, d, codebook, n_centres=256, noise=0.05):
    centres = _unit_rows(rng.standard_normal((n_centres, d)))
    q = centres[rng.integers(0, n_centres, n)] + noise * rng.standard_normal((n, d))
    k = centres[rng.integers(0, n_centres, n)] + noise * rng.standard_normal((n, d))
    v = codebook[rng.integers(0, codebook.shape[0], n)]
    return q, k, v


def make_workload(name: str, seed: int = 0, B: Optional[int] = None,
                  H: Optional[int] = None, n: Optional[int] = None,
                  d: Optional[int] = None) -> Workload:
    """Generate workload ``name``; B, H, n, d may be overridden for smaller
    cases built by the same recipe (n must stay a multiple of 8 for
    ``piecewise`` segments to be equal; other workloads take any n >= 1)."""
    spec = SPECS[name]
    B = spec.B if B is None else B
    H = spec.H if H is None else H
    n = spec.n if n is None else n
    d = spec.d if d is None else d
    rng = np.random.default_rng(seed)
    codebook = rng.standard_normal((8192, d)) if name == "recall" else None
    q = np.empty((B, H, n, d))
    k = np.empty((B, H, n, d))
    v = np.empty((B, H, n, d))
    for b in range(B):
        for h in range(H):
            if name == "tiny" or name == "long":
                qh, kh, vh = _head_gaussian(rng, n, d, 1.0)
            elif name == "standard":
                qh, kh, vh = _head_gaussian(rng, n, d, 4.0)
            elif name == "piecewise":
                qh, kh, vh = _head_piecewise(rng, n, d)
            elif name == "recall":
                qh, kh, vh = _head_recall(rng, n, d, codebook)
            else:  # pragma: no cover
                raise KeyError(name)
            q[b, h], k[b, h], v[b, h] = qh, kh, vh
    if spec.dtype == "f32":
        dev = [x.astype(np.float32) for x in (q, k, v)]
        exact = [x.astype(np.float64) for x in dev]
    else:
        dev = [f64_to_bf16_bits(x) for x in (q, k, v)]
        exact = [bf16_bits_to_f64(x) for x in dev]
    return Workload(spec, B, H, n, d, *exact, *dev)


def make_random(B: int, H: int, n: int, d: int, dtype: str = "f32",
                seed: int = 0, qk_scale: Optional[float] = 1.0,
                key_ramp: Optional[float] = None) -> Workload:
    """Gaussian q,k,v of any shape (q,k unit rows times ``qk_scale``, or raw
    Gaussian when ``qk_scale`` is None), for edge-case tests. With
    ``key_ramp`` the key of position j is further scaled by
    1 + key_ramp * j / (n - 1), so that scores grow along the sequence."""
    rng = np.random.default_rng(seed)
    q = np.empty((B, H, n, d))
    k = np.empty((B, H, n, d))
    v = np.empty((B, H, n, d))
    ramp = None
    if key_ramp is not None:
        ramp = 1.0 + key_ramp * np.arange(n) / max(n - 1, 1)
    for b in range(B):
        for h in range(H):
            q[b, h], k[b, h], v[b, h] = _head_gaussian(rng, n, d, qk_scale)
            if ramp is not None:
                k[b, h] *= ramp[:, None]
    spec = Spec("random", B, H, n, d, dtype, 1.0, 16, 0.0)
    if dtype == "f32":
        dev = [x.astype(np.float32) for x in (q, k, v)]
        exact = [x.astype(np.float64) for x in dev]
    else:
        dev = [f64_to_bf16_bits(x) for x in (q, k, v)]
        exact = [bf16_bits_to_f64(x) for x in dev]
    return Workload(spec, B, H, n, d, *exact, *dev)


def make_scaled(B: int, H: int, n: int, d: int, dtype: str = "bf16", seed: int = 0,
                span_log2: float = 0.0, log2_q: int = 0, log2_k: int = 0, log2_v: int = 0,
                lam: float = 1.0, qk_scale: float = 2.0) -> Workload:
    """Inputs with widely varying magnitudes, for range tests: Gaussian q,k,v
    as in ``make_random`` (q,k unit rows times ``qk_scale``); then every row of
    q, k and v is multiplied by its own 2^u, u ~ U(-span_log2, 0) (drawn per
    head after its q,k,v, in the order q rows, k rows, v rows), and the whole
    of q, k, v by 2^log2_q, 2^log2_k, 2^log2_v. ``lam`` is the ridge the
    workload is run with (scale it by 4^log2_k to keep the fit's balance)."""
    rng = np.random.default_rng(seed)
    q = np.empty((B, H, n, d))
    k = np.empty((B, H, n, d))
    v = np.empty((B, H, n, d))
    for b in range(B):
        for h in range(H):
            qh, kh, vh = _head_gaussian(rng, n, d, qk_scale)
            rows = 2.0 ** rng.uniform(-span_log2, 0.0, size=(3, n, 1))
            q[b, h] = qh * rows[0] * 2.0 ** log2_q
            k[b, h] = kh * rows[1] * 2.0 ** log2_k
            v[b, h] = vh * rows[2] * 2.0 ** log2_v
    spec = Spec("scaled", B, H, n, d, dtype, lam, 16, 0.0)
    if dtype == "f32":
        dev = [x.astype(np.float32) for x in (q, k, v)]
        exact = [x.astype(np.float64) for x in dev]
    else:
        dev = [f64_to_bf16_bits(x) for x in (q, k, v)]
        exact = [bf16_bits_to_f64(x) for x in dev]
    return Workload(spec, B, H, n, d, *exact, *dev)


def make_cotangent(B: int, H: int, n: int, d: int, seed: int = 1) -> np.ndarray:
    """A seeded upstream gradient dL/dout for the backward pass: N(0, 1)
    entries, drawn in float64 from ``default_rng(seed)`` and rounded to
    float32 (the float64 widening of those values is what both sides see).
    Shape [B, H, n, d]."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((B, H, n, d)).astype(np.float32)
