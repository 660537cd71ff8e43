"""Reference Ulysses relayouts (sequence shard <-> head shard), as index mappings.

TEST INFRASTRUCTURE ONLY; nothing in the product path imports it.

The Ulysses exchange regroups data so that each rank holds every token for a
subset of heads, and a second exchange regroups the attention output back by
token (Context parallelism guide (diffusers), section Ulysses Attention;
Ulysses Sequence Parallelism article, detailed notes 3 and 4). On one GPU the
transport is gone and what remains is the pack/unpack permutation of all P
ranks' shards:

    seq2head:  out[p][b][q*S_l + s][h][d] = in[q][b][s][p*H_l + h][d]
    head2seq:  out[q][b][s][p*H_l + h][d] = in[p][b][q*S_l + s][h][d]

with P ranks, S_l = S/P tokens per sequence shard (source rank q holds tokens
[q*S_l, (q+1)*S_l)), and H_l = H/P heads per head group (destination rank p
gets heads [p*H_l, (p+1)*H_l)). Both are pure copies: values are moved, never
computed, so any dtype's bits survive unchanged.
"""
from __future__ import annotations

import numpy as np


def seq2head(x: np.ndarray, P: int) -> np.ndarray:
    """``[P][B][S_l][H][D]`` -> ``[P][B][P*S_l][H/P][D]`` by reshape/transpose."""
    Pq, B, S_l, H, D = x.shape
    assert Pq == P and H % P == 0
    H_l = H // P
    t = x.reshape(P, B, S_l, P, H_l, D)          # [q][b][s][p][h][d]
    t = np.transpose(t, (3, 1, 0, 2, 4, 5))      # [p][b][q][s][h][d]
    return np.ascontiguousarray(t).reshape(P, B, P * S_l, H_l, D)


def head2seq(y: np.ndarray, P: int) -> np.ndarray:
    """``[P][B][P*S_l][H_l][D]`` -> ``[P][B][S_l][P*H_l][D]``, the inverse of seq2head."""
    Pp, B, S, H_l, D = y.shape
    assert Pp == P and S % P == 0
    S_l = S // P
    t = y.reshape(P, B, P, S_l, H_l, D)          # [p][b][q][s][h][d]
    t = np.transpose(t, (2, 1, 3, 0, 4, 5))      # [q][b][s][p][h][d]
    return np.ascontiguousarray(t).reshape(P, B, S_l, P * H_l, D)


def seq2head_loop(x: np.ndarray, P: int) -> np.ndarray:
    """The same mapping written as explicit loops over every index (tiny shapes only)."""
    _, B, S_l, H, D = x.shape
    H_l = H // P
    out = np.empty((P, B, P * S_l, H_l, D), dtype=x.dtype)
    for p in range(P):
        for b in range(B):
            for q in range(P):
                for s in range(S_l):
                    for h in range(H_l):
                        for d in range(D):
                            out[p, b, q * S_l + s, h, d] = x[q, b, s, p * H_l + h, d]
    return out


def head2seq_loop(y: np.ndarray, P: int) -> np.ndarray:
    """Explicit-loop form of head2seq (tiny shapes only)."""
    _, B, S, H_l, D = y.shape
    S_l = S // P
    out = np.empty((P, B, S_l, P * H_l, D), dtype=y.dtype)
    for q in range(P):
        for b in range(B):
            for s in range(S_l):
                for p in range(P):
                    for h in range(H_l):
                        for d in range(D):
                            out[q, b, s, p * H_l + h, d] = y[p, b, q * S_l + s, h, d]
    return out
