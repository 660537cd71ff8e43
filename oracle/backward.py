"""fp64 reference for the backward pass of attention and its per-chunk share.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this module;
only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of the
benchmark call it. It shares no code with the HIP library.

Context. The Ulysses Sequence Parallelism article is about training with
long contexts (summary; detailed notes 1, 2 and 6-8): the local attention
between the two all-to-alls runs forward and backward on each rank. Its
detailed notes 2 add that FlashAttention never stores the score matrix, so
the backward recomputes the softmax weights from the saved row log-sum-exp.
The pages print no gradient formulas. The reading taken here is the plain
one: the gradients are the derivatives of the forward output O (the
``attention`` function of this package) against an upstream gradient dO,
that is of the scalar L = sum over b, i, h, d of dO * O.

Notation as in ``attention.py``: BSHD tensors, ``scale`` multiplies the dot
products, positions are explicit integer arrays. With the softmax weights
P_ij = exp(S_ij - LSE_i) of the keys row i may see (0 for the others):
    dV_j  = sum_i P_ij dO_i
    dP_ij = <dO_i, v_j>
    Delta_i = sum_j P_ij dP_ij            (= <dO_i, O_i>)
    dS_ij = P_ij (dP_ij - Delta_i)        (derivative through the softmax)
    dQ_i  = scale * sum_j dS_ij k_j
    dK_j  = scale * sum_i dS_ij q_i
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .attention import attention

Grads = Tuple[np.ndarray, np.ndarray, np.ndarray]


def _positions(n: int, pos: Optional[np.ndarray]) -> np.ndarray:
    p = np.arange(n, dtype=np.int64) if pos is None else np.asarray(pos, dtype=np.int64)
    assert p.shape == (n,)
    return p


def attention_grad(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
                   causal: bool = False, q_pos: Optional[np.ndarray] = None,
                   k_pos: Optional[np.ndarray] = None) -> Grads:
    """dQ, dK, dV of full attention by the chain rule, from Q, K, V and dO only.

    The softmax weights are formed from scratch (row max, exponentials, row
    sum) rather than from a saved LSE, and Delta is sum_j P_ij dP_ij, the
    softmax Jacobian's own form: nothing here depends on the forward's stored
    statistics. A row that sees no key has P = 0 and contributes nothing.
    Shapes as ``attention``; returns float64 dq ``[B][Sq][H][D]``, dk and dv
    ``[B][Skv][H][D]``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    assert k.shape == (B, Skv, H, D) and v.shape == (B, Skv, H, D) and do.shape == q.shape
    qp, kp = _positions(Sq, q_pos), _positions(Skv, k_pos)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    if Sq == 0 or Skv == 0:
        return dq, dk, dv
    allowed = (kp[None, :] <= qp[:, None]) if causal else np.ones((Sq, Skv), dtype=bool)
    for b in range(B):
        for h in range(H):
            Q, K, V, dO = q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h]
            S = np.where(allowed, scale * (Q @ K.T), -np.inf)
            m = S.max(axis=1, keepdims=True)
            seen = np.isfinite(m)
            E = np.where(allowed, np.exp(S - np.where(seen, m, 0.0)), 0.0)
            Z = E.sum(axis=1, keepdims=True)
            P = E / np.where(seen, Z, 1.0)
            dP = dO @ V.T
            Delta = (P * dP).sum(axis=1, keepdims=True)
            dS = P * (dP - Delta)
            dv[b, :, h] = P.T @ dO
            dq[b, :, h] = scale * (dS @ K)
            dk[b, :, h] = scale * (dS.T @ Q)
    return dq, dk, dv


def backward_delta(o: np.ndarray, do: np.ndarray) -> np.ndarray:
    """Delta_i = <dO_i, O_i> per row, ``[B][H][Sq]``.

    For the exact O this equals sum_j P_ij dP_ij (O_i is the P-weighted mean of
    the value rows), which is what lets the per-chunk share below use one
    number per row instead of the row's whole softmax.
    """
    o = np.asarray(o, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    assert o.shape == do.shape
    return np.transpose((o * do).sum(axis=3), (0, 2, 1))


def chunk_grad(q: np.ndarray, k_c: np.ndarray, v_c: np.ndarray, do: np.ndarray,
               lse: np.ndarray, delta: np.ndarray, scale: float, causal: bool = False,
               q_pos: Optional[np.ndarray] = None,
               k_pos: Optional[np.ndarray] = None) -> Grads:
    """One K/V chunk's share of the backward, from the saved LSE and Delta.

    This is what a ring rank computes when chunk c passes by (Context
    parallelism guide (diffusers), section Ring Attention, run in reverse for
    the gradients): with the full rows' LSE and Delta the weights of the
    chunk's keys are P_ij = exp(S_ij - LSE_i) exactly, so
      dQ_c = scale * dS_c K_c   (summed over the chunks, the full dQ)
      dK_c = scale * dS_c^T Q,  dV_c = P_c^T dO   (this Q shard's share of the
                                                   chunk's key gradients)
    A row whose LSE is -inf saw no key anywhere and gets P = 0.

    Shapes: q, do ``[B][Sq][H][D]``; k_c, v_c ``[B][L][H][D]``; lse, delta
    ``[B][H][Sq]``. Returns float64 dq_c, dk_c, dv_c.
    """
    q = np.asarray(q, dtype=np.float64)
    k_c = np.asarray(k_c, dtype=np.float64)
    v_c = np.asarray(v_c, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    delta = np.asarray(delta, dtype=np.float64)
    B, Sq, H, D = q.shape
    L = k_c.shape[1]
    assert k_c.shape == (B, L, H, D) and v_c.shape == k_c.shape and do.shape == q.shape
    assert lse.shape == (B, H, Sq) and delta.shape == (B, H, Sq)
    qp, kp = _positions(Sq, q_pos), _positions(L, k_pos)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k_c), np.zeros_like(v_c)
    if Sq == 0 or L == 0:
        return dq, dk, dv
    allowed = (kp[None, :] <= qp[:, None]) if causal else np.ones((Sq, L), dtype=bool)
    for b in range(B):
        for h in range(H):
            Q, K, V, dO = q[b, :, h], k_c[b, :, h], v_c[b, :, h], do[b, :, h]
            lse_i = lse[b, h][:, None]
            ok = allowed & np.isfinite(lse_i)
            S = scale * (Q @ K.T)
            P = np.where(ok, np.exp(S - np.where(np.isfinite(lse_i), lse_i, 0.0)), 0.0)
            dP = dO @ V.T
            dS = P * (dP - delta[b, h][:, None])
            dv[b, :, h] = P.T @ dO
            dq[b, :, h] = scale * (dS @ K)
            dk[b, :, h] = scale * (dS.T @ Q)
    return dq, dk, dv


def forward_for_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                         causal: bool = False, q_pos: Optional[np.ndarray] = None,
                         k_pos: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """The forward's (O, LSE) that a training step saves for the backward, in fp64."""
    return attention(q, k, v, scale, causal, q_pos, k_pos)
