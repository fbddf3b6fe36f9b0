"""Brute-force, structurally different formulation of the MoE layer (NumPy, fp64).

TEST INFRASTRUCTURE ONLY: pins the C oracle, never used by the GPU path.

Where the C oracle loops over the selected experts of each token, this module
computes EVERY expert's output for every token, builds a dense [B][E] routing
matrix that is zero outside the selected set, and contracts the two.  The
selected set is found by enumerating all k-subsets of the E experts and
keeping the one with the largest logit sum (ties: the lexicographically
smallest index tuple), so it only suits tiny E.
"""
from __future__ import annotations

import itertools

import numpy as np


def bf16_bits_to_f64(a) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, via the float32 bit layout."""
    a = np.asarray(a, dtype=np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def silu(v):
    return v / (1.0 + np.exp(-v))


def best_subset(z_row: np.ndarray, k: int) -> tuple[int, ...]:
    """Exhaustive search: the k-subset with the largest sum of logits."""
    best, best_sum = None, -np.inf
    for sub in itertools.combinations(range(len(z_row)), k):
        s = float(np.sum(z_row[list(sub)]))
        if s > best_sum:
            best, best_sum = sub, s
    return best


def dense_weights(z: np.ndarray, k: int, score_fn: int, renormalize: int,
                  routed_scale: float = 1.0) -> np.ndarray:
    """[B][E] routing matrix from logits: score every expert, keep the best subset."""
    B, E = z.shape
    D = np.zeros((B, E))
    for t in range(B):
        sub = list(best_subset(z[t], k))
        if score_fn == 0:
            p = np.exp(z[t] - z[t].max())
            p = p / p.sum()                       # softmax over all experts
        else:
            p = 1.0 / (1.0 + np.exp(-z[t]))       # sigmoid per expert
        sel = p[sub]
        if renormalize:
            sel = sel / sel.sum()
        D[t, sub] = sel * routed_scale
    return D


def layer(x, wr, w13, w2, s13=None, s2=None, bias=None, *, k, score_fn, renormalize=1,
          routed_scale=1.0, add_residual=1):
    """Dense all-experts layer.  Arguments are bf16 bit arrays with the oracle's layout."""
    X = bf16_bits_to_f64(x)                      # [B][H]
    Wr = bf16_bits_to_f64(wr)                    # [E][H]
    W13 = bf16_bits_to_f64(w13)                  # [E][2I][H]
    W2 = bf16_bits_to_f64(w2)                    # [E][H][I]
    E, I2, H = W13.shape
    I = I2 // 2
    z = X @ Wr.T
    if bias is not None:
        z = z + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    D = dense_weights(z, k, score_fn, renormalize, routed_scale)
    G = np.einsum("eih,bh->bei", W13[:, :I, :], X)     # gate pre-activations
    U = np.einsum("eih,bh->bei", W13[:, I:, :], X)     # up pre-activations
    Hh = silu(G) * U                                   # [B][E][I]
    Y = np.einsum("eri,bei->ber", W2, Hh)              # every expert's output
    out = np.einsum("be,ber->br", D, Y)
    if s13 is not None:
        S13 = bf16_bits_to_f64(s13)
        S2 = bf16_bits_to_f64(s2)
        Is = S13.shape[0] // 2
        hs = silu(X @ S13[:Is].T) * (X @ S13[Is:].T)
        out = out + hs @ S2.T
    if add_residual:
        out = out + X
    return out, D, z
