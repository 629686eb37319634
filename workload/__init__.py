"""Seeded synthetic inputs for the Dobb step -- shared by the oracle side and the HIP side.

This module holds none of the optimizer's arithmetic.  It builds inputs with the shapes and spectra
of the Dobb pages' workloads ("Dobb: Shard-Local Preconditioning in Block-Diagonal Eigenbases",
thelatestinai.com listing):

* Table 1 builds 768 x 768 matrices with a prescribed entropy effective rank.  The construction
  appendix is not on the pages; the reading used here is a power-law spectrum sigma_i = i^-alpha
  with alpha solved so that exp(-sum p_i log p_i)/dim hits the target, p_i = sigma_i / sum sigma,
  and Haar-random singular vectors.  It reproduces Table 1(a)'s printed orthogonality of Y exactly.
* Activations have a prescribed population second moment: x_t = V diag(sqrt(lambda)) z_t with
  z_t ~ N(0, I), Haar V and lambda_i = i^-alpha solved for the effective-rank target (15 % in
  Table 1(b) and in the weight-matrix workloads).
* Matrix sets: GPT-2 Small / XL and a Llama-7B-style stack with the m x n shapes of each layer.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# ------------------------------------------------------------------------------------------------
# spectra


def _entropy_rank(p: np.ndarray) -> float:
    p = p / p.sum()
    return float(np.exp(-np.sum(p * np.log(p))) / len(p))


def power_law_alpha(n: int, target: float) -> float:
    """alpha such that p_i proportional to i^-alpha (i = 1..n) has entropy effective rank `target`."""
    i = np.arange(1, n + 1, dtype=np.float64)
    lo, hi = 0.0, 20.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if _entropy_rank(i ** -mid) > target:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def power_law(n: int, target: float) -> np.ndarray:
    i = np.arange(1, n + 1, dtype=np.float64)
    return i ** -power_law_alpha(n, target)


# ------------------------------------------------------------------------------------------------
# random matrices


def haar(n: int, rng: np.random.Generator) -> np.ndarray:
    """Haar-distributed orthogonal matrix: QR of a Gaussian matrix with R's diagonal made positive."""
    q, r = np.linalg.qr(rng.standard_normal((n, n)))
    return q * np.sign(np.diag(r))


def table1_matrix(n: int, target: float, rng: np.random.Generator) -> np.ndarray:
    """Y = U diag(sigma) V^T with power-law sigma of entropy effective rank `target` (Table 1(a))."""
    s = power_law(n, target)
    return (haar(n, rng) * s) @ haar(n, rng).T


def activations(N: int, n: int, target: float, rng: np.random.Generator,
                basis: np.ndarray | None = None) -> np.ndarray:
    """N x n activations (rows are tokens) whose population second moment V diag(lambda) V^T has
    power-law eigenvalues of effective rank `target`, distinct and decaying (fp64)."""
    lam = power_law(n, target)
    V = haar(n, rng) if basis is None else basis
    Z = rng.standard_normal((N, n))
    return (Z * np.sqrt(lam)) @ V.T


def activations_torch(N: int, n: int, target: float, seed: int, device, dtype, basis=None):
    """Same construction with torch on `device` (used for multi-GB matrix sets)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    lam = torch.from_numpy(power_law(n, target)).to(device=device, dtype=torch.float32)
    if basis is None:  # Haar basis from a CPU QR (keeps GPU solver libraries out of the picture)
        gc = torch.Generator()
        gc.manual_seed(int(seed))
        q, r = torch.linalg.qr(torch.randn(n, n, generator=gc, dtype=torch.float64))
        basis = (q * torch.sign(torch.diagonal(r))).to(device=device, dtype=torch.float32)
    Z = torch.randn(N, n, generator=g, device=device, dtype=torch.float32)
    X = (Z * lam.sqrt()) @ basis.T
    return X.to(dtype), basis


# ------------------------------------------------------------------------------------------------
# matrix sets


@dataclass(frozen=True)
class MatrixSpec:
    name: str
    m: int
    n: int
    nb: int


def _set(layers: int, shapes, blocks_of) -> list[MatrixSpec]:
    out = []
    for layer in range(layers):
        for name, m, n in shapes:
            out.append(MatrixSpec(f"h{layer}.{name}", m, n, blocks_of(n)))
    return out


def gpt2_small_set(B: int = 16) -> list[MatrixSpec]:
    """12 layers x {qkv 2304x768, attn-proj 768x768, fc 3072x768, fc-proj 768x3072}, B blocks."""
    shapes = [("qkv", 2304, 768), ("proj", 768, 768), ("fc", 3072, 768), ("fcproj", 768, 3072)]
    return _set(12, shapes, lambda n: n // B)


def gpt2_xl_set(B: int = 16) -> list[MatrixSpec]:
    """48 layers x {qkv 4800x1600, proj 1600x1600, fc 6400x1600, fc-proj 1600x6400}, B blocks."""
    shapes = [("qkv", 4800, 1600), ("proj", 1600, 1600), ("fc", 6400, 1600), ("fcproj", 1600, 6400)]
    return _set(48, shapes, lambda n: n // B)


def llama7b_set(nb: int = 128) -> list[MatrixSpec]:
    """32 layers x {q,k,v,o 4096x4096, gate/up 11008x4096, down 4096x11008}, block size nb."""
    shapes = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
              ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)]
    return _set(32, shapes, lambda n: nb)


def single_768_set(B: int = 4) -> list[MatrixSpec]:
    """One 768x768 weight with B blocks (the single-matrix configurations: B = 4, and B = 1, 4, 16 for
    the Table 1(b) gradients)."""
    return [MatrixSpec("w", 768, 768, 768 // B)]


def seed_for(config: int, layer: int, index: int) -> int:
    return 1000 * config + 10 * layer + index


def param_count(specs) -> int:
    return sum(s.m * s.n for s in specs)


__all__ = ["power_law_alpha", "power_law", "haar", "table1_matrix", "activations",
           "activations_torch", "MatrixSpec", "gpt2_small_set", "gpt2_xl_set", "llama7b_set", "single_768_set",
           "seed_for", "param_count"]
