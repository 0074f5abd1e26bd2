"""Seeded synthetic video-shaped Q/K/V for the block-sparse attention path.

This module is shared by the tests, the benchmark and the smoke check. It holds
no arithmetic of the attention method itself: it only defines the workload
shapes and draws the inputs that both the CPU oracle and the HIP library
consume.

The AB-Attention abstract (paperdot search page, query "Xing Ma") evaluates on
Wan2.1 and HunyuanVideo activations; no weights or prompts are available, so a
smooth 3D positional field stands in for post-RoPE queries and keys of a video
latent. Recipe:

* Token n of a T x Hg x W latent grid sits at (t, y, x) with n = (t*Hg + y)*W + x
  (raster order; tokens are never permuted).
* Per head h, channel c and term r = 0..3: integer frequencies k_t, k_y, k_x
  drawn uniformly from -3..3 (cycles per axis length) and a phase phi drawn
  uniformly from [0, 2*pi).
* F[h, n, c] = A * sqrt(2/4) * sum_r sin(2*pi*(k_t t/T + k_y y/Hg + k_x x/W) + phi),
  which has unit RMS per channel at A = 1.
* Q = F + sigma * eps_q and K = F + sigma * eps_k share the field, so attention
  is local in 3D the way video attention is.
* V is an independent field G + sigma * eps_v for the tiny case and a standard
  normal otherwise.
* Draw order from numpy's PCG64 (default_rng(seed)): F parameters, G parameters
  (tiny case only), then eps_q, eps_k, eps_v as [B, H, N, d] standard normals.
* bf16 workloads are rounded to bf16 (round to nearest even); every consumer
  sees exactly the rounded values.
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = ["Workload", "WORKLOADS", "generate", "round_to_bf16", "get"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    grid: tuple  # (T, Hg, W)
    d: int
    dtype: str  # "fp32" | "bf16"
    q_block: int
    k_block: int
    n_clusters: int
    density: float
    sigma: float
    v_field: bool  # True: V is an independent smooth field plus noise
    amplitude: float = 1.0
    kmeans_iters: int = 4

    @property
    def N(self) -> int:
        t, y, x = self.grid
        return t * y * x

    @property
    def nqb(self) -> int:
        return -(-self.N // self.q_block)

    @property
    def nkb(self) -> int:
        return -(-self.N // self.k_block)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def dense_flops(self) -> float:
        """4*B*H*N^2*d: the non-causal dense attention forward (two GEMMs)."""
        return 4.0 * self.B * self.H * float(self.N) ** 2 * self.d


WORKLOADS = {
    # Tiny CPU-checkable case (density sweep 1.0 / 0.25).
    "tiny": Workload("tiny", 1, 1, (4, 8, 8), 64, "fp32", 64, 16, 4, 0.25, 0.5, True),
    # Wan2.1-1.3B-shaped layer.
    "wan1.3b": Workload("wan1.3b", 1, 12, (21, 30, 52), 128, "bf16", 128, 32, 8, 0.10, 0.5, False),
    # Wan2.1-14B-shaped layer.
    "wan14b": Workload("wan14b", 1, 40, (21, 45, 80), 128, "bf16", 128, 32, 8, 0.08, 0.5, False),
    # HunyuanVideo-shaped layer, more peaked attention.
    "hunyuan": Workload("hunyuan", 1, 24, (33, 45, 80), 128, "bf16", 128, 16, 8, 0.08, 0.3, False),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def _field(rng: np.random.Generator, H: int, d: int, grid, amplitude: float) -> np.ndarray:
    """Sum of four random integer-frequency sinusoids over (t, y, x), [H, N, d] float32."""
    T, Hg, W = grid
    freqs = rng.integers(-3, 4, size=(H, d, 4, 3))
    phases = rng.uniform(0.0, 2.0 * math.pi, size=(H, d, 4))
    t = np.arange(T, dtype=np.float64)
    y = np.arange(Hg, dtype=np.float64)
    x = np.arange(W, dtype=np.float64)
    amp = np.float32(amplitude * math.sqrt(2.0 / 4.0))
    out = np.zeros((H, T, Hg, W, d), dtype=np.float32)

    def head(h):  # every random number is drawn above, so heads are independent
        for r in range(4):
            kt, ky, kx = freqs[h, :, r, 0], freqs[h, :, r, 1], freqs[h, :, r, 2]
            # angle = 2*pi*(kt t/T + ky y/Hg + kx x/W) + phi, split as a (t, y) part and an x part
            a_ty = 2.0 * math.pi * (np.outer(t / T, kt)[:, None, :] + np.outer(y / Hg, ky)[None, :, :]) + phases[h, :, r]
            a_x = 2.0 * math.pi * np.outer(x / W, kx)
            s_ty = np.sin(a_ty).astype(np.float32)[:, :, None, :]
            c_ty = np.cos(a_ty).astype(np.float32)[:, :, None, :]
            s_x = np.sin(a_x).astype(np.float32)[None, None, :, :]
            c_x = np.cos(a_x).astype(np.float32)[None, None, :, :]
            # sin(a + b) = sin a cos b + cos a sin b
            out[h] += s_ty * c_x
            out[h] += c_ty * s_x
        out[h] *= amp

    # the heads on threads (numpy releases the interpreter lock in these array
    # operations); each head's values are the same as in a sequential loop
    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1, H))) as ex:
        list(ex.map(head, range(H)))
    return out.reshape(H, T * Hg * W, d)


def generate(w: Workload, seed: int = 0):
    """Return (q, k, v) as float32 numpy arrays [B, H, N, d].

    For bf16 workloads the values are already rounded to bf16, so converting
    them to a bf16 tensor is exact and the oracle sees the same numbers.
    """
    rng = np.random.default_rng(seed)
    B, H, N, d = w.B, w.H, w.N, w.d
    F = _field(rng, H, d, w.grid, w.amplitude)
    G = _field(rng, H, d, w.grid, w.amplitude) if w.v_field else None
    sig = np.float32(w.sigma)
    q = np.empty((B, H, N, d), dtype=np.float32)
    k = np.empty((B, H, N, d), dtype=np.float32)
    v = np.empty((B, H, N, d), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            q[b, h] = F[h] + sig * rng.standard_normal((N, d), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            k[b, h] = F[h] + sig * rng.standard_normal((N, d), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            e = rng.standard_normal((N, d), dtype=np.float32)
            v[b, h] = (G[h] + sig * e) if G is not None else e
    del F, G
    if w.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return q, k, v
