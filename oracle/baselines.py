"""Baselines and the logit-fidelity measure for the oracle (test infrastructure only).

The page "RoPE-Aware Bit Allocation for KV-Cache Quantization" (abstract) compares
Block-GTQ against uniform TQ-MSE at the same budget by the per-layer mean absolute
error of RoPE query-key logits.  Two uniform baselines are built here:

* U_same: the same per-token-norm / per-block-scale quantizer with every block at
  budget/(d/2) bits (the allocator is the only difference);
* U_rot: TurboQuant-MSE proper -- per-token L2 norm, a seeded random-sign
  normalised Walsh-Hadamard rotation, the Gaussian Lloyd-Max codebook scaled by
  1/sqrt(d) for every rotated coordinate, then the inverse rotation.  The
  related-papers page for "Quantization Dominates Rank Reduction for KV-Cache"
  lists a KV/KQV/QKQV analysis whose key path is exactly "WHT + MSE".
"""
from __future__ import annotations

import numpy as np

from . import GREEDY, UNIFORM, allocate, block_energy, codebook, dequant, encode, per_coord


def hadamard(d: int) -> np.ndarray:
    H = np.array([[1.0]])
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    return H / np.sqrt(d)


def quantize_blockgtq(k16: np.ndarray, budget: int, mode: int = GREEDY, pairing: int = 0) -> np.ndarray:
    """Dequantized keys [n, d] (fp64) of one head under the (greedy or uniform) allocation."""
    n, d = k16.shape
    e = block_energy(k16.reshape(n, 1, d), pairing)
    bits, sig = allocate(e, budget, mode)
    w = per_coord(bits[0].astype(np.int32), d, pairing)
    s = per_coord(sig[0], d, pairing)
    codes, scale = encode(k16, w, s)
    return dequant(codes, w, s, scale)


def quantize_rot(k16: np.ndarray, bits_per_dim: int, seed: int = 0, signs: np.ndarray | None = None) -> np.ndarray:
    """TurboQuant-MSE style: norm, random-sign WHT, per-coordinate Lloyd-Max, inverse.
    signs: the +-1 diagonal (drawn from `seed` when not given)."""
    n, d = k16.shape
    x = k16.astype(np.float64)
    if signs is None:
        rng = np.random.default_rng(seed)
        signs = rng.choice([-1.0, 1.0], size=d)
    R = hadamard(d) * signs[None, :]          # y = R x  (orthogonal)
    norm = np.linalg.norm(x, axis=1)
    safe = np.where(norm > 0, norm, 1.0)
    y = (x / safe[:, None]) @ R.T
    cb = codebook(bits_per_dim)
    lev = cb["levels_h"] / np.sqrt(d)
    idx = np.abs(y[:, :, None] - lev[None, None, :]).argmin(-1)
    yq = lev[idx]
    return (yq @ R) * norm[:, None]


def logit_mae(q16: np.ndarray, k16: np.ndarray, khat: np.ndarray) -> float:
    """Mean over (query head, token) of |q.khat - q.k| (unscaled), fp64."""
    q = q16.astype(np.float64)
    k = k16.astype(np.float64)
    return float(np.mean(np.abs(q @ khat.T - q @ k.T)))


def mae_report(q16, k16, budget: int, pairing: int = 0) -> dict:
    d = k16.shape[1]
    g = quantize_blockgtq(k16, budget, GREEDY, pairing)
    u = quantize_blockgtq(k16, budget, UNIFORM, pairing)
    r = quantize_rot(k16, budget // (d // 2))
    return {"blockgtq": logit_mae(q16, k16, g), "u_same": logit_mae(q16, k16, u), "u_rot": logit_mae(q16, k16, r)}
