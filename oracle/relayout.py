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

and, for the value tensor only, a key-contiguous form of seq2head (seq2head_vt:
each head's values in tiles of 64 tokens, each tile [D][64]), the operand order
of the P.V product.

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


VT_TILE = 64   # keys per tile of the key-contiguous value layout


def seq2head_vt(x: np.ndarray, P: int) -> np.ndarray:
    """``[P][B][S_l][H][D]`` -> ``[P][B][H/P][ceil(T/64)][D][64]``, T = P*S_l: the
    seq2head regrouping of the value tensor, delivered in tiles of 64 tokens with
    each (group, batch, head, tile, feature) a row of the tile's 64 tokens (keys
    contiguous). Token t = q*S_l + s sits in tile t // 64 at column t % 64;
    columns past T in the last tile are zero. A permutation plus zero padding:

        out[p][b][h][t // 64][d][t % 64] = in[q][b][s][p*H_l + h][d]
    """
    y = seq2head(x, P)                                  # [p][b][t][h][d]
    Pp, B, T, H_l, D = y.shape
    nt = -(-T // VT_TILE)
    pad = np.zeros((Pp, B, nt * VT_TILE, H_l, D), dtype=y.dtype)
    pad[:, :, :T] = y
    t = pad.reshape(Pp, B, nt, VT_TILE, H_l, D)         # [p][b][tile][j][h][d]
    return np.ascontiguousarray(np.transpose(t, (0, 1, 4, 2, 5, 3)))


def seq2head_vt_loop(x: np.ndarray, P: int) -> np.ndarray:
    """The tiled key-contiguous regrouping as explicit loops (tiny shapes only)."""
    _, B, S_l, H, D = x.shape
    H_l = H // P
    T = P * S_l
    nt = -(-T // VT_TILE)
    out = np.zeros((P, B, H_l, nt, D, VT_TILE), dtype=x.dtype)
    for p in range(P):
        for b in range(B):
            for h in range(H_l):
                for d in range(D):
                    for q in range(P):
                        for s in range(S_l):
                            t = q * S_l + s
                            out[p, b, h, t // VT_TILE, d, t % VT_TILE] = x[q, b, s, p * H_l + h, d]
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


# ---------------------------------------------------------------------------
# Ulysses Anything: per-rank token counts and head counts need not be equal
# (Context parallelism guide (diffusers), section Ulysses Anything Attention:
# the mode drops both divisibility requirements; diffusers parallel API,
# ContextParallelConfig: ulysses_anything). Source rank q holds tokens
# [off_q, off_q + S_q) of the sequence, destination rank p receives the
# contiguous heads [h0_p, h0_p + H_p):
#
#   seq2head:  out[p][b][off_q + s][h][d] = in[q][b][s][h0_p + h][d]
#   head2seq:  out[q][b][s][h0_p + h][d] = in[p][b][off_q + s][h][d]
#
# Shards are given as lists, one array per rank.


def even_split(n: int, P: int) -> list:
    """Split n items over P ranks: the first n mod P ranks get one more."""
    return [n // P + (1 if r < n % P else 0) for r in range(P)]


def _offsets(sizes) -> list:
    out = [0]
    for x in sizes:
        out.append(out[-1] + int(x))
    return out


def anything_seq2head(shards, h_counts):
    """list of ``[B][S_q][H][D]`` -> list of ``[B][S][H_p][D]`` (sum S_q = S, sum H_p = H)."""
    h0 = _offsets(h_counts)
    return [np.ascontiguousarray(np.concatenate([x[:, :, h0[p]:h0[p + 1], :] for x in shards],
                                                axis=1))
            for p in range(len(h_counts))]


def anything_head2seq(groups, s_lens):
    """list of ``[B][S][H_p][D]`` -> list of ``[B][S_q][H][D]``, the inverse of anything_seq2head."""
    off = _offsets(s_lens)
    return [np.ascontiguousarray(np.concatenate([y[:, off[q]:off[q + 1], :, :] for y in groups],
                                                axis=2))
            for q in range(len(s_lens))]


def anything_seq2head_loop(shards, h_counts):
    """Explicit-loop form of anything_seq2head (tiny shapes only)."""
    B, _, H, D = shards[0].shape
    s_lens = [x.shape[1] for x in shards]
    S = sum(s_lens)
    off, h0 = _offsets(s_lens), _offsets(h_counts)
    out = [np.empty((B, S, hp, D), dtype=shards[0].dtype) for hp in h_counts]
    for p in range(len(h_counts)):
        for q in range(len(shards)):
            for b in range(B):
                for s in range(s_lens[q]):
                    for h in range(h_counts[p]):
                        for d in range(D):
                            out[p][b, off[q] + s, h, d] = shards[q][b, s, h0[p] + h, d]
    return out


def anything_head2seq_loop(groups, s_lens):
    """Explicit-loop form of anything_head2seq (tiny shapes only)."""
    B, S, _, D = groups[0].shape
    h_counts = [y.shape[2] for y in groups]
    H = sum(h_counts)
    off, h0 = _offsets(s_lens), _offsets(h_counts)
    out = [np.empty((B, sq, H, D), dtype=groups[0].dtype) for sq in s_lens]
    for q in range(len(s_lens)):
        for p in range(len(groups)):
            for b in range(B):
                for s in range(s_lens[q]):
                    for h in range(h_counts[p]):
                        for d in range(D):
                            out[q][b, s, h0[p] + h, d] = groups[p][b, off[q] + s, h, d]
    return out


# ---------------------------------------------------------------------------
# K/V gather: queries stay sequence-sharded, keys and values are all-gathered
# and each rank attends its own query shard to the full K/V (Sequence
# Parallelism page (SGLang Diffusion), section Choosing The Attention
# Exchange, kv_gather). On one GPU the all-gather's unpack joins the P
# sequence shards into one sequence:  out[b][off_q + s][h][d] = in_q[b][s][h][d]


def kv_gather(shards):
    """list of ``[B][S_q][H][D]`` -> ``[B][S][H][D]`` (shards joined in rank order)."""
    return np.ascontiguousarray(np.concatenate(shards, axis=1))


def kv_gather_loop(shards):
    """Explicit-loop form of kv_gather (tiny shapes only)."""
    B, _, H, D = shards[0].shape
    s_lens = [x.shape[1] for x in shards]
    off = _offsets(s_lens)
    out = np.empty((B, off[-1], H, D), dtype=shards[0].dtype)
    for q, x in enumerate(shards):
        for b in range(B):
            for s in range(s_lens[q]):
                for h in range(H):
                    for d in range(D):
                        out[b, off[q] + s, h, d] = x[b, s, h, d]
    return out


def kv_gather_vt(shards):
    """list of ``[B][S_q][H][D]`` -> ``[B][H][ceil(S/64)][D][64]``: the all-gather's
    unpack of the value tensor delivered key-contiguous in tiles of 64 tokens
    (the layout of seq2head_vt), zero padding past the last token:

        out[b][h][t // 64][d][t % 64] = shard_q[b][s][h][d],  t = off_q + s
    """
    full = kv_gather(shards)                            # [b][t][h][d]
    B, S, H, D = full.shape
    nt = -(-S // VT_TILE)
    pad = np.zeros((B, nt * VT_TILE, H, D), dtype=full.dtype)
    pad[:, :S] = full
    return np.ascontiguousarray(
        np.transpose(pad.reshape(B, nt, VT_TILE, H, D), (0, 3, 1, 4, 2)))
