"""Work accounting for the HSTU attention path (host logic, no GPU).

Convention: only visible (i, j) pairs are counted.  Each visible pair costs
2*d_qk FLOPs for its QK^T entry and 2*d_v for its share of A.V, per head.
The dense count of the worked example on the page "4.3 用户行为序列建模"
(section "实例演算", 2*2*T^2*d for both products) is the same convention
applied to all T^2 pairs; a causal mask keeps L(L+1)/2 of them.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def visible_pairs(lengths: Sequence[int], num_candidates: Optional[Sequence[int]] = None) -> int:
    """Visible (query, key) pairs of a jagged batch.

    Causal sequence of L rows: L(L+1)/2.  Sequence with n history rows and c
    candidates (M-FALCON): n(n+1)/2 causal history pairs plus c(n+1), since
    every candidate sees the n history rows and itself.
    """
    L = np.asarray(lengths, dtype=np.int64)
    if num_candidates is None:
        return int(np.sum(L * (L + 1) // 2))
    c = np.asarray(num_candidates, dtype=np.int64)
    n = L - c
    return int(np.sum(n * (n + 1) // 2 + c * (n + 1)))


def grad_blocks(lengths, num_candidates=None) -> int:
    """32x32 blocks (query tile q, key tile k) holding a visible pair, per
    head: k <= q with history keys in tile k, or the diagonal tile of
    candidate keys (each candidate is seen by its own row alone).  The
    gradient kernels store G = dLoss/dS for exactly these blocks."""
    L = np.asarray(lengths, dtype=np.int64)
    c = np.zeros_like(L) if num_candidates is None else np.asarray(num_candidates, dtype=np.int64)
    total = 0
    for Lb, cb in zip(L.tolist(), c.tolist()):
        nq = -(-Lb // 32)
        nh = -(-(Lb - cb) // 32)
        q = np.arange(nq, dtype=np.int64)
        total += int(np.sum(np.where(q < nh, q + 1, nh + 1)))
    return total


def attn_flops(lengths, H: int, d_qk: int, d_v: int, num_candidates=None) -> int:
    """Unmasked attention FLOPs: sum over heads of (2*d_qk + 2*d_v) per visible pair."""
    return int(visible_pairs(lengths, num_candidates)) * H * (2 * d_qk + 2 * d_v)


def attn_bwd_flops(lengths, H: int, d: int, num_candidates=None) -> int:
    """Algorithmic FLOPs of the attention gradients: the four products over
    visible pairs (dV = A^T dO, dO V^T, dQ = G K, dK = G^T Q), 2*d each per
    pair and head -- twice the forward's count.  Recomputing S is not counted."""
    return int(visible_pairs(lengths, num_candidates)) * H * 8 * d


def layer_bwd_flops(lengths, H: int, d: int, D: int) -> int:
    """Algorithmic FLOPs of one layer's gradients: the attention gradients
    plus four products -- dY = dX_out W2 and dW2 = dX_out^T Y (2*T*D*H*d
    each), dX = dP W1 and dW1 = dP^T X (2*T*4*H*d*D each).  The recomputed
    forward is not counted."""
    T = int(np.sum(np.asarray(lengths, dtype=np.int64)))
    return attn_bwd_flops(lengths, H, d) + 2 * gemm_flops(T, D, H * d) + 2 * gemm_flops(T, 4 * H * d, D)


def dense_attn_flops(T: int, d: int) -> int:
    """Dense count of both products over all T^2 pairs: 2 * 2 * T^2 * d."""
    return 2 * 2 * T * T * d


def gemm_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def layer_flops(lengths, H: int, d: int, D: int) -> dict:
    """FLOPs of one HSTU layer: f1 (D -> 4Hd), attention, f2 (Hd -> D)."""
    T = int(np.sum(np.asarray(lengths, dtype=np.int64)))
    return {
        "f1": gemm_flops(T, 4 * H * d, D),
        "attn": attn_flops(lengths, H, d, d),
        "f2": gemm_flops(T, D, H * d),
    }


def attn_min_bytes(T: int, H: int, d_qk: int, d_v: int, elem_bytes: int) -> int:
    """Algorithmic HBM bytes of the attention core: Q, K, V read once, O written once."""
    return T * H * (2 * d_qk + 2 * d_v) * elem_bytes


def ln_gate_bytes(T: int, width: int, elem_bytes: int) -> int:
    """Algorithmic bytes of the LN*U epilogue: O and U read, Y written."""
    return 3 * T * width * elem_bytes
