"""Pins of the fp64 CPU oracle against facts fixed outside the oracle itself.

Each test checks the oracle against something it cannot agree with by
construction: hand-derived exact values (tests/golden/), closed forms, exact
identities of the method (chunk + merge == full attention for every ring
degree and order), a library routine (torch's fp64 scaled_dot_product_attention
and logsumexp), and explicit index loops. A last group plants plausible
mistakes in copies of the oracle and checks that these pins catch them.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-12


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _sym(x):
    return {"0": 0.0, "1": 1.0, "ln2": math.log(2), "ln3": math.log(3), "ln5": math.log(5)}[x]


def _frac(s):
    return float(Fraction(s))


def _tiny_inputs():
    g = _golden("tiny_attention.json")
    q = np.array(g["q"], dtype=np.float64)[None, :, None, :]           # [1][4][1][4]
    k = np.array([[_sym(x) for x in row] for row in g["k_symbolic"]])[None, :, None, :]
    v = np.array(g["v"], dtype=np.float64)[None, :, None, :]
    return g, q, k, v


def _check_golden_attention(attn_fn):
    """True iff ``attn_fn`` reproduces the hand-derived tiny example (both mask modes)."""
    g, q, k, v = _tiny_inputs()
    o, lse = attn_fn(q, k, v, g["scale"])
    exp_o = np.array([[_frac(x) for x in r] for r in g["noncausal"]["O"]])
    exp_l = np.array([math.log(_frac(z)) for z in g["noncausal"]["Z"]])
    ok = np.allclose(o[0, :, 0, :], exp_o, atol=TOL, rtol=0) and \
        np.allclose(lse[0, 0], exp_l, atol=TOL, rtol=0)
    c = g["causal"]
    o, lse = attn_fn(q, k, v, g["scale"], True, np.array(c["q_pos"]), np.array(c["k_pos"]))
    exp_o = np.array([[_frac(x) for x in r] for r in c["O"]])
    exp_l = np.array([math.log(_frac(z)) if z != "none" else -np.inf for z in c["Z"]])
    ok = ok and np.allclose(o[0, :, 0, :], exp_o, atol=TOL, rtol=0)
    ok = ok and np.array_equal(np.isinf(lse[0, 0]), np.isinf(exp_l)) and \
        np.allclose(lse[0, 0][np.isfinite(exp_l)], exp_l[np.isfinite(exp_l)], atol=TOL, rtol=0)
    return bool(ok)


# ---------------------------------------------------------------- golden values

def test_golden_tiny_attention():
    assert _check_golden_attention(oracle.attention)


def test_golden_tiny_merge():
    g, q, k, v = _tiny_inputs()
    m = g["merge"]
    o_a = np.array([_frac(x) for x in m["O_A"]])
    o_b = np.array([_frac(x) for x in m["O_B"]])
    o_parts = np.stack([o_a, o_b])[:, None, None, None, :]           # [2][1][1][1][4]
    l_parts = np.array([math.log(_frac(m["Z_A"])), math.log(_frac(m["Z_B"]))])[:, None, None, None]
    o, lse = oracle.lse_merge(o_parts, l_parts)
    assert np.allclose(o[0, 0, 0], [_frac(x) for x in m["O"]], atol=TOL, rtol=0)
    assert abs(lse[0, 0, 0] - math.log(_frac(m["Z"]))) < TOL
    # the same split through the per-chunk path, in both orders
    chunks = [(k[:, :2], v[:, :2], np.arange(2)), (k[:, 2:], v[:, 2:], np.arange(2, 3))]
    for order in ([0, 1], [1, 0]):
        o2, l2 = oracle.ring_attention(q[:, :1], chunks, order, g["scale"])
        assert np.allclose(o2[0, 0, 0], [_frac(x) for x in m["O"]], atol=TOL, rtol=0)
        assert abs(l2[0, 0, 0] - math.log(8)) < TOL


def test_golden_tiny_relayout():
    g = _golden("tiny_relayout.json")
    x = np.array(g["in"], dtype=np.int64)
    assert list(x.shape) == g["in_shape"]
    want = np.array(g["seq2head"], dtype=np.int64)
    assert np.array_equal(oracle.seq2head(x, g["P"]), want)
    assert np.array_equal(oracle.seq2head_loop(x, g["P"]), want)
    assert np.array_equal(oracle.head2seq(want, g["P"]), x)
    assert np.array_equal(oracle.head2seq_loop(want, g["P"]), x)


# ------------------------------------------------------------------ closed forms

def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_uniform_weights_when_q_zero():
    k, v = _rand((1, 7, 2, 8), 1), _rand((1, 7, 2, 8), 2)
    q = np.zeros((1, 5, 2, 8))
    o, lse = oracle.attention(q, k, v, 0.3)
    assert np.allclose(o, v.mean(axis=1, keepdims=True).repeat(5, axis=1), atol=TOL)
    assert np.allclose(lse, math.log(7), atol=TOL)


def test_uniform_weights_when_keys_equal():
    q, v = _rand((1, 5, 1, 8), 3), _rand((1, 6, 1, 8), 4)
    k = np.repeat(_rand((1, 1, 1, 8), 5), 6, axis=1)
    scale = 0.25
    o, lse = oracle.attention(q, k, v, scale)
    s0 = scale * (q[0, :, 0, :] @ k[0, 0, 0, :])
    assert np.allclose(o[0, :, 0, :], v[0, :, 0, :].mean(axis=0), atol=TOL)
    assert np.allclose(lse[0, 0], math.log(6) + s0, atol=TOL)


def test_constant_values_give_constant_output():
    q, k = _rand((1, 9, 3, 16), 6), _rand((1, 11, 3, 16), 7)
    c = _rand((16,), 8)
    v = np.broadcast_to(c, (1, 11, 3, 16)).copy()
    for causal in (False, True):
        o, _ = oracle.attention(q, k, v, 0.25, causal)
        rows = slice(None) if not causal else slice(0, 9)
        assert np.allclose(o[:, rows], c, atol=1e-12)


def test_single_key():
    q, k, v = _rand((1, 4, 2, 8), 9), _rand((1, 1, 2, 8), 10), _rand((1, 1, 2, 8), 11)
    o, lse = oracle.attention(q, k, v, 0.5)
    assert np.allclose(o, np.broadcast_to(v, o.shape), atol=TOL)
    want = 0.5 * np.einsum("bihd,bjhd->bhi", q, k)
    assert np.allclose(lse, want, atol=TOL)


def test_causal_first_row_is_first_value():
    q, k, v = _rand((1, 6, 2, 8), 12), _rand((1, 6, 2, 8), 13), _rand((1, 6, 2, 8), 14)
    o, lse = oracle.attention(q, k, v, 0.5, causal=True)
    assert np.allclose(o[:, 0], v[:, 0], atol=TOL)
    assert np.allclose(lse[:, :, 0], 0.5 * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0]), atol=TOL)


def test_fully_masked_rows():
    q, k, v = _rand((1, 3, 1, 4), 15), _rand((1, 5, 1, 4), 16), _rand((1, 5, 1, 4), 17)
    o, lse = oracle.attention(q, k, v, 0.5, True, np.array([-1, -5, 10]), np.arange(5))
    assert np.all(o[0, :2] == 0) and np.all(np.isneginf(lse[0, 0, :2]))
    assert np.isfinite(lse[0, 0, 2]) and not np.any(np.isnan(o))
    o, lse = oracle.attention(q, k[:, :0], v[:, :0], 0.5)   # no keys at all
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_merge_two_identical_partials():
    o1, l1 = _rand((1, 1, 5, 2, 8), 18), _rand((1, 1, 2, 5), 19)
    o, lse = oracle.lse_merge(np.concatenate([o1, o1]), np.concatenate([l1, l1]))
    assert np.allclose(o, o1[0], atol=TOL)
    assert np.allclose(lse, l1[0] + math.log(2), atol=TOL)


def test_merge_single_partial_is_identity():
    o1, l1 = _rand((1, 2, 5, 3, 8), 20), _rand((1, 2, 3, 5), 21)
    o, lse = oracle.lse_merge(o1, l1)
    assert np.allclose(o, o1[0], atol=TOL) and np.allclose(lse, l1[0], atol=TOL)


def test_merge_masked_partials():
    o_parts = _rand((3, 1, 2, 1, 4), 22)
    l_parts = np.array([[[[-np.inf, 0.5]]], [[[-np.inf, -np.inf]]], [[[-np.inf, 1.0]]]])
    o, lse = oracle.lse_merge(o_parts, l_parts)
    assert np.all(o[0, 0] == 0) and np.isneginf(lse[0, 0, 0])
    w0, w2 = math.exp(0.5), math.exp(1.0)
    assert abs(lse[0, 0, 1] - math.log(w0 + w2)) < TOL
    assert np.allclose(o[0, 1, 0], (w0 * o_parts[0, 0, 1, 0] + w2 * o_parts[2, 0, 1, 0]) / (w0 + w2),
                       atol=TOL)


# ------------------------------------------------------- identities of the method

S_ID = 48   # divisible by 1, 2, 3, 4 and 8


@pytest.fixture(scope="module")
def qkv48():
    return _rand((1, S_ID, 2, 16), 30), _rand((1, S_ID, 2, 16), 31), _rand((1, S_ID, 2, 16), 32)


def _chunks(k, v, lens):
    out, acc = [], 0
    for n in lens:
        out.append((k[:, acc:acc + n], v[:, acc:acc + n], np.arange(acc, acc + n)))
        acc += n
    return out


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("P", [1, 2, 3, 4, 8])
def test_chunk_merge_equals_full_attention(qkv48, P, causal):
    q, k, v = qkv48
    scale = 1 / math.sqrt(16)
    o_ref, l_ref = oracle.attention(q, k, v, scale, causal)
    chunks = _chunks(k, v, [S_ID // P] * P)
    if P <= 4:
        orders = list(itertools.permutations(range(P)))
    else:
        rng = np.random.default_rng(P)
        orders = [list(rng.permutation(P)) for _ in range(100)]
    for order in orders:
        o, l = oracle.ring_attention(q, chunks, order, scale, causal)
        assert np.max(np.abs(o - o_ref)) < TOL
        fin = np.isfinite(l_ref)
        assert np.array_equal(fin, np.isfinite(l))
        assert np.max(np.abs(l[fin] - l_ref[fin])) < TOL


@pytest.mark.parametrize("lens", [(13, 13, 13, 9), (1, 46, 1), (5, 7, 11, 2, 23),
                                  synthetic.random_splits(48, 6, seed=3)])
@pytest.mark.parametrize("causal", [False, True])
def test_uneven_chunks_equal_full_attention(qkv48, lens, causal):
    q, k, v = qkv48
    o_ref, l_ref = oracle.attention(q, k, v, 0.25, causal)
    chunks = _chunks(k, v, lens)
    for order in [list(range(len(lens))), list(reversed(range(len(lens))))]:
        o, l = oracle.ring_attention(q, chunks, order, 0.25, causal)
        assert np.max(np.abs(o - o_ref)) < TOL
        assert np.max(np.abs(l - l_ref)) < TOL


def test_ring_ranks_union_is_full_attention(qkv48):
    """Every ring rank's share (its Q shard, all chunks in its order) tiles full attention."""
    q, k, v = qkv48
    P, n = 4, S_ID // 4
    o_ref, l_ref = oracle.attention(q, k, v, 0.25, True)
    chunks = _chunks(k, v, [n] * P)
    for r in range(P):
        qs = q[:, r * n:(r + 1) * n]
        o, l = oracle.ring_attention(qs, chunks, synthetic.ring_order(r, P), 0.25, True,
                                     np.arange(r * n, (r + 1) * n))
        assert np.max(np.abs(o - o_ref[:, r * n:(r + 1) * n])) < TOL
        assert np.max(np.abs(l - l_ref[:, :, r * n:(r + 1) * n])) < TOL


def test_softmax_rows_sum_to_one(qkv48):
    q, k, _ = qkv48
    for causal in (False, True):
        P = oracle.softmax_matrix(q[:, :20], k, 0.25, causal)
        assert np.max(np.abs(P.sum(axis=-1) - 1.0)) < TOL
        if causal:   # nothing after the diagonal
            assert np.all(np.triu(P[0, 0], 1)[:, :20] == 0)


def test_ring_anything_split_of_4099_matches():
    """The uneven 1025/1025/1025/1024 split merges to full attention (small head dim)."""
    lens = synthetic.even_split(4099, 4)
    assert lens == (1025, 1025, 1025, 1024)
    rng = np.random.default_rng(40)
    q = rng.standard_normal((1, 64, 1, 8))
    k = rng.standard_normal((1, 4099, 1, 8))
    v = rng.standard_normal((1, 4099, 1, 8))
    qpos = np.arange(2000, 2064)
    o_ref, l_ref = oracle.attention(q, k, v, 0.35, True, qpos)
    o, l = oracle.ring_attention(q, _chunks(k, v, lens), [1, 0, 3, 2], 0.35, True, qpos)
    assert np.max(np.abs(o - o_ref)) < TOL and np.max(np.abs(l - l_ref)) < TOL


# -------------------------------------------------- library routine cross-check

@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_sdpa_fp64(causal):
    g = torch.Generator().manual_seed(50)
    B, S, H, D = 2, 37, 3, 16
    q, k, v = (torch.randn(B, S, H, D, generator=g, dtype=torch.float64) for _ in range(3))
    scale = 1 / math.sqrt(D)
    o, lse = oracle.attention(q.numpy(), k.numpy(), v.numpy(), scale, causal)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2), is_causal=causal, scale=scale)
    assert np.max(np.abs(o - ref.transpose(1, 2).numpy())) < 1e-12
    s = scale * torch.einsum("bihd,bjhd->bhij", q, k)
    if causal:
        s = s.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
    assert np.max(np.abs(lse - torch.logsumexp(s, dim=-1).numpy())) < 1e-12


def test_bf16_decode():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x8000, 0x4049], dtype=np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    assert got[0] == 1.0 and got[1] == -2.0 and np.isposinf(got[2]) and np.isneginf(got[3])
    assert got[4] == 2.0 ** -133 and got[5] == 0.0 and math.copysign(1, got[5]) < 0
    assert got[6] == 3.140625
    t = synthetic.make_tensor((1000,), torch.bfloat16, 7)
    assert np.array_equal(oracle.bf16_bits_to_f64(t.view(torch.int16).numpy()),
                          t.to(torch.float64).numpy())


# ------------------------------------------------------------------- relayout

@pytest.mark.parametrize("P,S_l,H,D", [(1, 3, 2, 4), (2, 3, 4, 2), (4, 2, 8, 3), (3, 5, 6, 1)])
def test_relayout_loops_and_roundtrip(P, S_l, H, D):
    x = np.arange(P * 2 * S_l * H * D).reshape(P, 2, S_l, H, D)
    y = oracle.seq2head(x, P)
    assert np.array_equal(y, oracle.seq2head_loop(x, P))
    assert np.array_equal(oracle.head2seq(y, P), x)
    assert np.array_equal(oracle.head2seq_loop(y, P), x)
    z = np.arange(y.size).reshape(y.shape)
    assert np.array_equal(oracle.seq2head(oracle.head2seq(z, P), P), z)
    if P == 1:
        assert np.array_equal(y, x)


@pytest.mark.parametrize("P,S_l,H,D", [(1, 3, 2, 4), (2, 3, 4, 2), (4, 2, 8, 3), (3, 5, 6, 1),
                                       (2, 40, 2, 2), (1, 128, 1, 1)])
def test_relayout_vt_loop_and_index_formula(P, S_l, H, D):
    """Tiled key-contiguous seq2head against its loop form and, element by
    element, out[p][b][h][t // 64][d][t % 64] = in[q][b][s][p*H_l + h][d] with
    t = q*S_l + s; the padding columns past T = P*S_l are zero."""
    x = np.arange(1, P * 2 * S_l * H * D + 1).reshape(P, 2, S_l, H, D)
    y = oracle.seq2head_vt(x, P)
    T = P * S_l
    nt = -(-T // 64)
    assert y.shape == (P, 2, H // P, nt, D, 64)
    assert np.array_equal(y, oracle.seq2head_vt_loop(x, P))
    H_l = H // P
    for (p, b, h, tile, d, j), val in np.ndenumerate(y):
        t = 64 * tile + j
        if t >= T:
            assert val == 0
        else:
            q, s = divmod(t, S_l)
            assert val == x[q, b, s, p * H_l + h, d]
    # every value moved exactly once, the rest is padding
    nz = y[y != 0]
    assert sorted(nz.tolist()) == sorted(x.ravel().tolist())


@pytest.mark.parametrize("lens", [(3, 4), (64, 64, 1), (5,), (30, 30, 30, 30)])
def test_kv_gather_vt_index_formula(lens):
    """Key-contiguous gather: element by element out[b][h][t // 64][d][t % 64] =
    shard_q[b][s][h][d] with t = off_q + s, zero padding; and for equal shards the
    same array as the key-contiguous Ulysses regrouping with one head group of all
    the gathered tokens."""
    B, H, D = 2, 3, 2
    shards = [np.arange(1, B * n * H * D + 1).reshape(B, n, H, D) + 1000 * q
              for q, n in enumerate(lens)]
    y = oracle.kv_gather_vt(shards)
    S = sum(lens)
    assert y.shape == (B, H, -(-S // 64), D, 64)
    off = np.cumsum((0,) + tuple(lens))
    for (b, h, tile, d, j), val in np.ndenumerate(y):
        t = 64 * tile + j
        if t >= S:
            assert val == 0
            continue
        q = int(np.searchsorted(off, t, side="right") - 1)
        assert val == shards[q][b, t - off[q], h, d]
    full = np.concatenate(shards, axis=1)[None]      # one shard of all S tokens
    assert np.array_equal(y, oracle.seq2head_vt(full, 1)[0])


def test_relayout_moves_bits_unchanged():
    bits = synthetic.random_bits((4, 1, 6, 8, 16), 2, seed=60).numpy()
    y = oracle.seq2head(bits, 4)
    assert sorted(y.ravel().tolist()) == sorted(bits.ravel().tolist())
    assert np.array_equal(oracle.head2seq(y, 4), bits)
    assert np.array_equal(y, oracle.seq2head_loop(bits, 4))


def test_relayout_shard_semantics():
    """Rank p's head-sharded tensor is heads [p*H_l, (p+1)*H_l) of the full sequence."""
    P, S_l, H, D = 4, 5, 8, 3
    full = _rand((1, P * S_l, H, D), 61)                 # [1][S][H][D]
    shards = full.reshape(P, 1, S_l, H, D)               # contiguous sequence shards
    y = oracle.seq2head(shards, P)
    for p in range(P):
        assert np.array_equal(y[p], full[:, :, p * 2:(p + 1) * 2, :])


# ------------------------------------------------------ relayout: Ulysses Anything

def test_anything_golden():
    g = _golden("tiny_relayout_anything.json")
    ins = [np.array(x, dtype=np.int64) for x in g["in"]]
    want = [np.array(x, dtype=np.int64) for x in g["seq2head"]]
    for f in (oracle.anything_seq2head, oracle.anything_seq2head_loop):
        got = f(ins, g["h_counts"])
        assert all(np.array_equal(a, b) for a, b in zip(got, want))
    for f in (oracle.anything_head2seq, oracle.anything_head2seq_loop):
        back = f(want, g["s_lens"])
        assert all(np.array_equal(a, b) for a, b in zip(back, ins))


@pytest.mark.parametrize("s_lens,h_counts,B,D", [
    ([3, 2, 2], [2, 1, 1], 1, 2),      # uneven tokens and heads
    ([1, 0, 4], [0, 3, 1], 2, 1),      # empty shard, empty head group
    ([5], [3], 2, 3),                  # one rank: a plain copy
    ([2, 2, 1, 1], [1, 1, 1, 1], 1, 2),
])
def test_anything_loops_and_roundtrip(s_lens, h_counts, B, D):
    H = sum(h_counts)
    rng = np.random.default_rng(sum(s_lens) * 7 + H)
    ins = [rng.integers(0, 1 << 16, size=(B, sq, H, D)) for sq in s_lens]
    out = oracle.anything_seq2head(ins, h_counts)
    assert [o.shape for o in out] == [(B, sum(s_lens), hp, D) for hp in h_counts]
    assert all(np.array_equal(a, b) for a, b in zip(out, oracle.anything_seq2head_loop(ins, h_counts)))
    back = oracle.anything_head2seq(out, s_lens)
    assert all(np.array_equal(a, b) for a, b in zip(back, ins))
    assert all(np.array_equal(a, b) for a, b in zip(oracle.anything_head2seq_loop(out, s_lens), ins))
    if len(s_lens) == 1:
        assert np.array_equal(out[0], ins[0])


def test_anything_even_split_is_standard_ulysses():
    """With equal shards and head groups the mode is ordinary Ulysses."""
    P, S_l, H, D = 4, 3, 8, 2
    x = np.arange(P * 1 * S_l * H * D).reshape(P, 1, S_l, H, D)
    got = oracle.anything_seq2head([x[q] for q in range(P)], [H // P] * P)
    want = oracle.seq2head(x, P)
    assert all(np.array_equal(got[p], want[p]) for p in range(P))


def test_anything_shard_semantics_and_split_rule():
    """Rank p's group is heads [h0_p, h0_p + H_p) of the full sequence; the
    default split gives the first n mod P ranks one extra item."""
    assert oracle.even_split(4481, 4) == [1121, 1120, 1120, 1120]
    assert oracle.even_split(30, 4) == [8, 8, 7, 7]
    assert oracle.even_split(3, 5) == [1, 1, 1, 0, 0]
    S, H, D = 11, 7, 2
    full = _rand((1, S, H, D), 62)
    s_lens, h_counts = oracle.even_split(S, 3), oracle.even_split(H, 3)
    off = np.cumsum([0] + s_lens)
    ins = [full[:, off[q]:off[q + 1]] for q in range(3)]
    out = oracle.anything_seq2head(ins, h_counts)
    h0 = np.cumsum([0] + h_counts)
    for p in range(3):
        assert np.array_equal(out[p], full[:, :, h0[p]:h0[p + 1], :])


def test_anything_pins_catch_planted_mistakes():
    g = _golden("tiny_relayout_anything.json")
    ins = [np.array(x, dtype=np.int64) for x in g["in"]]
    want = [np.array(x, dtype=np.int64) for x in g["seq2head"]]
    # head groups assigned in reverse rank order
    bad = oracle.anything_seq2head(ins, g["h_counts"][::-1])
    assert not all(a.shape == b.shape and np.array_equal(a, b) for a, b in zip(bad, want))
    # tokens concatenated in reverse source-rank order
    bad = oracle.anything_seq2head(ins[::-1], g["h_counts"])
    assert not all(np.array_equal(a, b) for a, b in zip(bad, want))


# ----------------------------------------------------------- relayout: K/V gather

@pytest.mark.parametrize("s_lens,B,H,D", [([3, 1, 2], 2, 2, 3), ([4], 1, 3, 2), ([0, 2, 0, 1], 1, 1, 1)])
def test_kv_gather_loop_and_special_case(s_lens, B, H, D):
    rng = np.random.default_rng(len(s_lens) * 11 + H)
    shards = [rng.integers(0, 1 << 16, size=(B, sq, H, D)) for sq in s_lens]
    out = oracle.kv_gather(shards)
    assert np.array_equal(out, oracle.kv_gather_loop(shards))
    # the gather is the uneven regrouping with one destination holding every head
    one_group = oracle.anything_seq2head(shards, [H] + [0] * (len(s_lens) - 1))
    assert np.array_equal(out, one_group[0])


def test_kv_gather_rank_share_is_full_attention_rows():
    """A K/V-gather rank's output is full attention restricted to its query shard."""
    S, H, D, P = 12, 2, 4, 3
    q, k, v = (_rand((1, S, H, D), 70 + i) for i in range(3))
    lens = oracle.even_split(S, P)
    off = np.cumsum([0] + lens)
    full_o, full_l = oracle.attention(q, k, v, 0.5)
    kg = oracle.kv_gather([k[:, off[r]:off[r + 1]] for r in range(P)])
    vg = oracle.kv_gather([v[:, off[r]:off[r + 1]] for r in range(P)])
    for r in range(P):
        o, l = oracle.attention(q[:, off[r]:off[r + 1]], kg, vg, 0.5)
        assert np.allclose(o, full_o[:, off[r]:off[r + 1]], atol=1e-12)
        assert np.allclose(l, full_l[:, :, off[r]:off[r + 1]], atol=1e-12)


# -------------------------------------------------- unified (Ulysses x ring) composition

@pytest.mark.parametrize("U,R,causal", [(2, 2, False), (2, 3, True), (3, 2, False)])
def test_unified_sp_composition_is_full_attention(U, R, causal):
    """Unified SP (Context parallelism guide (diffusers), section Unified
    Attention): the sequence is cut into R ring segments, each spread over U
    Ulysses ranks. Within a segment the Ulysses regrouping gives each rank the
    whole segment for H/U heads; ring attention over the R segments (same head
    group) then the inverse regrouping give every rank full attention for its
    tokens."""
    S_sub, H, D = 2, 2 * U, 3
    S = U * R * S_sub
    q, k, v = (_rand((1, S, H, D), 80 + i) for i in range(3))
    full_o, _ = oracle.attention(q, k, v, 0.5, causal)
    seg = U * S_sub

    def regroup(x, r):  # segment r's U sub-shards -> U head groups over the segment
        shards = x[:, r * seg:(r + 1) * seg].reshape(1, U, S_sub, H, D).transpose(1, 0, 2, 3, 4)
        return oracle.seq2head(np.ascontiguousarray(shards), U)     # [U][1][seg][H/U][D]

    qh = [regroup(q, r) for r in range(R)]
    kh = [regroup(k, r) for r in range(R)]
    vh = [regroup(v, r) for r in range(R)]
    for r in range(R):
        outs = []
        for u in range(U):
            chunks = [(kh[c][u], vh[c][u], np.arange(c * seg, (c + 1) * seg)) for c in range(R)]
            order = [(r - t) % R for t in range(R)]
            o, _ = oracle.ring_attention(qh[r][u], chunks, order, 0.5, causal,
                                         q_pos=np.arange(r * seg, (r + 1) * seg))
            outs.append(o)
        back = oracle.head2seq(np.stack(outs), U)                    # [U][1][S_sub][H][D]
        got = np.concatenate([back[u] for u in range(U)], axis=1)    # the segment's tokens
        assert np.allclose(got, full_o[:, r * seg:(r + 1) * seg], atol=1e-12)


# ---------------------------------------- planted mistakes are caught by the pins

def _mutant(kind):
    def attn(q, k, v, scale, causal=False, q_pos=None, k_pos=None):
        if kind == "no_scale":
            return oracle.attention(q, k, v, 1.0, causal, q_pos, k_pos)
        if kind == "neg_scale":
            return oracle.attention(q, k, v, -scale, causal, q_pos, k_pos)
        if kind == "swap_qk":    # transposed operands: scores from K against Q
            return oracle.attention(q, k, v, scale, causal, q_pos, k_pos) if q.shape != k.shape \
                else oracle.attention(k, q, v, scale, causal, k_pos, q_pos)
        if kind == "log2_lse":
            o, l = oracle.attention(q, k, v, scale, causal, q_pos, k_pos)
            return o, l / math.log(2)
        if kind == "strict_causal":   # diagonal excluded
            qp = None if q_pos is None else np.asarray(q_pos) - 1
            return oracle.attention(q, k, v, scale, causal, qp, k_pos)
        if kind == "v_transposed":    # values taken from the keys
            return oracle.attention(q, k, k, scale, causal, q_pos, k_pos)
        raise ValueError(kind)
    return attn


@pytest.mark.parametrize("kind", ["no_scale", "neg_scale", "log2_lse", "strict_causal",
                                  "v_transposed"])
def test_golden_catches_planted_attention_mistakes(kind):
    assert not _check_golden_attention(_mutant(kind))


def test_merge_pins_catch_planted_mistakes(qkv48):
    q, k, v = qkv48
    o_ref, l_ref = oracle.attention(q, k, v, 0.25)
    chunks = _chunks(k, v, [12] * 4)
    parts = [oracle.chunk_partial(q, *chunks[c][:2], 0.25, False, None, chunks[c][2])
             for c in range(4)]
    po = np.stack([p[0] for p in parts])
    pl = np.stack([p[1] for p in parts])
    # weights without the max shift but forgetting to renormalise
    bad_o = (np.exp(np.transpose(pl, (0, 1, 3, 2)))[..., None] * po).sum(0)
    assert np.max(np.abs(bad_o - o_ref)) > 1e-3
    # averaging partials instead of LSE weighting
    assert np.max(np.abs(po.mean(0) - o_ref)) > 1e-3
    # max instead of log-sum-exp for the merged LSE
    assert np.max(np.abs(pl.max(0) - l_ref)) > 1e-3


def test_relayout_pins_catch_planted_mistakes():
    g = _golden("tiny_relayout.json")
    x = np.array(g["in"], dtype=np.int64)
    want = np.array(g["seq2head"], dtype=np.int64)
    P = g["P"]
    # head group and sequence shard axes swapped
    t = np.transpose(x.reshape(P, 1, 2, P, 1, 1), (0, 1, 3, 2, 4, 5)).reshape(P, 1, 4, 1, 1)
    assert not np.array_equal(t, want)
    # tokens interleaved (local index major) instead of source-rank major
    t = np.transpose(x.reshape(P, 1, 2, P, 1, 1), (3, 1, 2, 0, 4, 5)).reshape(P, 1, 4, 1, 1)
    assert not np.array_equal(t, want)
