"""fp64 reference for block-wise softmax attention, its per-chunk partials and their merge.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this module;
only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of the
benchmark call it. It shares no code with the HIP library.

Everything here is float64 numpy, written as the plain definition rather than
a fast algorithm, so that a reader can check it against the pages by eye.

Notation: tensors are BSHD, ``q[b][i][h][d]``, ``k[b][j][h][d]``,
``v[b][j][h][d]``; ``scale`` multiplies the dot products; positions are
explicit integer arrays, one per query row and one per key row.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              causal: bool = False, q_pos: Optional[np.ndarray] = None,
              k_pos: Optional[np.ndarray] = None,
              row_block: int = 512) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention by brute force, with the row log-sum-exp.

    For each batch b, head h and query row i, over the keys j it may see:
        S_ij  = scale * <q_i, k_j>
        LSE_i = ln sum_j exp(S_ij)              (natural log, scale included)
        O_i   = sum_j exp(S_ij - LSE_i) * v_j
    This is ordinary full attention, the result every context-parallel variant
    must reproduce (Context parallelism guide (diffusers), section Ring
    Attention: after a full turn of the ring every GPU has seen every token's
    K/V; Ulysses Sequence Parallelism article, detailed notes 2: tiling never
    changes what is computed, only what is stored).

    Causal masking follows positions, not a 4-D mask (Ulysses Sequence
    Parallelism article, detailed notes 7: position_ids drive causal masking):
    key j is visible to query i iff ``k_pos[j] <= q_pos[i]``.

    A row that sees no key at all gets O = 0 and LSE = -inf.

    Shapes: q ``[B][Sq][H][D]``, k and v ``[B][Skv][H][D]`` (any float dtype; they
    are upcast to float64). Returns ``o`` float64 ``[B][Sq][H][D]`` and ``lse``
    float64 ``[B][H][Sq]``. Rows are processed in blocks of ``row_block`` only to
    bound memory; each block is the same formula.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    assert k.shape == (B, Skv, H, D) and v.shape == (B, Skv, H, D)
    if q_pos is None:
        q_pos = np.arange(Sq, dtype=np.int64)
    if k_pos is None:
        k_pos = np.arange(Skv, dtype=np.int64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    assert q_pos.shape == (Sq,) and k_pos.shape == (Skv,)

    o = np.zeros((B, Sq, H, D), dtype=np.float64)
    lse = np.full((B, H, Sq), NEG_INF, dtype=np.float64)
    if Skv == 0 or Sq == 0:
        return o, lse
    for b in range(B):
        for h in range(H):
            K = k[b, :, h, :]          # [Skv][D]
            V = v[b, :, h, :]          # [Skv][D]
            for i0 in range(0, Sq, row_block):
                i1 = min(Sq, i0 + row_block)
                Qb = q[b, i0:i1, h, :]  # [rows][D]
                S = scale * (Qb @ K.T)  # [rows][Skv]
                if causal:
                    allowed = k_pos[None, :] <= q_pos[i0:i1, None]
                else:
                    allowed = np.ones(S.shape, dtype=bool)
                S = np.where(allowed, S, NEG_INF)
                m = S.max(axis=1)                       # row max over allowed keys
                seen = np.isfinite(m)                   # rows with at least one key
                m_safe = np.where(seen, m, 0.0)
                E = np.where(allowed, np.exp(S - m_safe[:, None]), 0.0)
                Z = E.sum(axis=1)
                row_lse = np.where(seen, m_safe + np.log(np.where(seen, Z, 1.0)), NEG_INF)
                lse[b, h, i0:i1] = row_lse
                Zs = np.where(seen, Z, 1.0)
                o[b, i0:i1, h, :] = np.where(seen[:, None], (E @ V) / Zs[:, None], 0.0)
    return o, lse


def chunk_partial(q: np.ndarray, k_chunk: np.ndarray, v_chunk: np.ndarray, scale: float,
                  causal: bool = False, q_pos: Optional[np.ndarray] = None,
                  k_pos: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """One ring hop's partial result: attention of Q over one K/V chunk only.

    Returns the chunk's own (O_c, LSE_c), normalised within the chunk, which is
    the (output, LSE) pair that the ring converts to fp32 and merges (diffusers
    parallel API, ContextParallelConfig: convert_to_fp32). ``k_pos`` carries the
    chunk's global key positions so causal masking still uses global order.
    """
    return attention(q, k_chunk, v_chunk, scale, causal, q_pos, k_pos)


def lse_merge(o_parts: np.ndarray, lse_parts: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Merge P partial (O_c, LSE_c) pairs into the result over the union of their keys.

    All at once, per row (Sequence Parallelism (SGLang Diffusion), section
    Numerics across node boundaries: the ring merges hops by online softmax;
    here the merge is written in its closed form):
        M   = max_c LSE_c
        LSE = M + ln sum_c exp(LSE_c - M)
        O   = sum_c exp(LSE_c - LSE) * O_c
    exp(LSE_c) is the chunk's own softmax normaliser, so the weights
    exp(LSE_c - LSE) are exactly each chunk's share of the full normaliser. If
    every LSE_c is -inf the row saw no key: O = 0, LSE = -inf.

    Shapes: o_parts ``[P][B][Sq][H][D]``, lse_parts ``[P][B][H][Sq]``.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    P, B, Sq, H, D = o_parts.shape
    assert lse_parts.shape == (P, B, H, Sq)
    M = lse_parts.max(axis=0)                          # [B][H][Sq]
    seen = np.isfinite(M)
    M_safe = np.where(seen, M, 0.0)
    W = np.exp(lse_parts - M_safe[None])               # exp(LSE_c - M); -inf -> 0
    Z = W.sum(axis=0)
    lse = np.where(seen, M_safe + np.log(np.where(seen, Z, 1.0)), NEG_INF)
    lse_safe = np.where(seen, lse, 0.0)
    w = np.where(seen[None], np.exp(lse_parts - lse_safe[None]), 0.0)  # [P][B][H][Sq]
    w_bshd = np.transpose(w, (0, 1, 3, 2))[..., None]  # [P][B][Sq][H][1]
    o = (w_bshd * o_parts).sum(axis=0)
    return o, lse


def ring_attention(q: np.ndarray, chunks: Sequence[Tuple[np.ndarray, np.ndarray, np.ndarray]],
                   order: Sequence[int], scale: float, causal: bool = False,
                   q_pos: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """One ring rank's result: its Q attends every K/V chunk in ring order, then merge.

    ``chunks[c] = (k_c, v_c, k_pos_c)`` in sequence order; ``order`` lists the
    chunk indices in the order this rank receives them (Context parallelism
    guide (diffusers), section Ring Attention: each GPU attends the block it
    holds, then passes it on). Each hop gives a partial (O_c, LSE_c), and the
    partials are merged in fp64 with ``lse_merge``. Uneven chunk lengths are
    allowed: ring-anything pads for the exchange and slices back before the
    attention, so padding never enters the math (same guide, section Ring
    Anything Attention).
    """
    parts_o, parts_l = [], []
    for c in order:
        k_c, v_c, kp = chunks[c]
        o_c, l_c = chunk_partial(q, k_c, v_c, scale, causal, q_pos, kp)
        parts_o.append(o_c)
        parts_l.append(l_c)
    return lse_merge(np.stack(parts_o), np.stack(parts_l))


def softmax_matrix(q: np.ndarray, k: np.ndarray, scale: float, causal: bool = False,
                   q_pos: Optional[np.ndarray] = None,
                   k_pos: Optional[np.ndarray] = None) -> np.ndarray:
    """The explicit softmax weights exp(S_ij - LSE_i), ``[B][H][Sq][Skv]`` (tiny inputs)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    q_pos = np.arange(Sq) if q_pos is None else np.asarray(q_pos)
    k_pos = np.arange(Skv) if k_pos is None else np.asarray(k_pos)
    _, lse = attention(q, k, np.zeros_like(k), scale, causal, q_pos, k_pos)
    out = np.zeros((B, H, Sq, Skv))
    for b in range(B):
        for h in range(H):
            S = scale * (q[b, :, h, :] @ k[b, :, h, :].T)
            allowed = (k_pos[None, :] <= q_pos[:, None]) if causal else np.ones_like(S, bool)
            L = lse[b, h][:, None]
            ok = allowed & np.isfinite(L)
            out[b, h] = np.where(ok, np.exp(S - np.where(np.isfinite(L), L, 0.0)), 0.0)
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16/int16 words) to float64 exactly.

    A bf16 value is the upper half of an IEEE binary32 word, so the decode is a
    16-bit shift into a float32 followed by an exact widening.
    """
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)

