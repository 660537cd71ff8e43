"""Pins for the fp64 backward oracle (``oracle/backward.py``): CPU only.

The gradients are tied to facts other than the oracle's own formulas: a
hand-derived worked example (``tests/golden/tiny_backward.json``), torch's
fp64 autograd through its own attention routine, central finite differences
of the (separately pinned) forward, closed forms and identities of the
softmax derivative, and the decomposition over K/V chunks that the ring's
backward relies on. Each plausible mistake planted below must fail a pin.
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
from oracle import backward as bwd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-12


def _frac(s):
    return float(Fraction(s))


def _sym(x):
    return {"0": 0.0, "2ln2": 2 * math.log(2), "2ln3": 2 * math.log(3)}[x]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _golden_inputs():
    with open(os.path.join(GOLDEN, "tiny_backward.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], dtype=np.float64)[None, :, None, :]
    k = np.array([[_sym(x) for x in r] for r in g["k_symbolic"]])[None, :, None, :]
    v = np.array(g["v"], dtype=np.float64)[None, :, None, :]
    do = np.array(g["do"], dtype=np.float64)[None, :, None, :]
    return g, q, k, v, do


def _check_golden_grad(grad_fn):
    """True iff ``grad_fn`` reproduces the hand-derived example in both mask modes."""
    g, q, k, v, do = _golden_inputs()
    logs = np.array([math.log(3), math.log(2)])
    ok = True
    for mode in ("noncausal", "causal"):
        e = g[mode]
        if mode == "causal":
            dq, dk, dv = grad_fn(q, k, v, do, g["scale"], True, np.array(e["q_pos"]),
                                 np.array(e["k_pos"]))
        else:
            dq, dk, dv = grad_fn(q, k, v, do, g["scale"])
        want_dq = np.array([[_frac(c) for c in r] for r in e["dq_coeffs"]]) * logs[None, :]
        want_dk = np.array([[_frac(c) for c in r] for r in e["dk"]])
        want_dv = np.array([[_frac(c) for c in r] for r in e["dv"]])
        ok = ok and np.allclose(dq[0, :, 0], want_dq, atol=TOL, rtol=0)
        ok = ok and np.allclose(dk[0, :, 0], want_dk, atol=TOL, rtol=0)
        ok = ok and np.allclose(dv[0, :, 0], want_dv, atol=TOL, rtol=0)
    return bool(ok)


def _via_saved_stats(q, k, v, do, scale, causal=False, q_pos=None, k_pos=None):
    """The chunk form with one chunk, fed the fp64 forward's LSE and Delta."""
    o, lse = bwd.forward_for_backward(q, k, v, scale, causal, q_pos, k_pos)
    return bwd.chunk_grad(q, k, v, do, lse, bwd.backward_delta(o, do), scale, causal,
                          q_pos, k_pos)


# ---------------------------------------------------------------- golden values

def test_golden_tiny_backward():
    assert _check_golden_grad(bwd.attention_grad)


def test_golden_tiny_backward_from_saved_stats():
    assert _check_golden_grad(_via_saved_stats)


def test_golden_intermediates():
    """P, O, dP, Delta and dS of the worked example, row by row."""
    g, q, k, v, do = _golden_inputs()
    e = g["noncausal"]
    P = oracle.softmax_matrix(q, k, g["scale"])[0, 0]
    assert np.allclose(P, [[_frac(x) for x in r] for r in e["P"]], atol=TOL)
    o, _ = oracle.attention(q, k, v, g["scale"])
    assert np.allclose(o[0, :, 0], [[_frac(x) for x in r] for r in e["O"]], atol=TOL)
    delta = bwd.backward_delta(o, do)[0, 0]
    assert np.allclose(delta, [_frac(x) for x in e["Delta"]], atol=TOL)
    dP = do[0, :, 0] @ v[0, :, 0].T
    assert np.allclose(dP, [[_frac(x) for x in r] for r in e["dP"]], atol=TOL)
    assert np.allclose(P * (dP - delta[:, None]), [[_frac(x) for x in r] for r in e["dS"]],
                       atol=TOL)


# -------------------------------------------------- library routine cross-check

def _torch_grads(q, k, v, do, scale, mask=None, is_causal=False):
    tq, tk, tv = (torch.tensor(x).transpose(1, 2).requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                         is_causal=is_causal, scale=scale)
    o.backward(torch.tensor(do).transpose(1, 2))
    return tuple(t.grad.transpose(1, 2).numpy() for t in (tq, tk, tv))


@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_autograd_fp64(causal):
    B, S, H, D = 2, 29, 3, 16
    q, k, v, do = (_rand((B, S, H, D), 60 + n) for n in range(4))
    scale = 1 / math.sqrt(D)
    want = _torch_grads(q, k, v, do, scale, is_causal=causal)
    for got in (bwd.attention_grad(q, k, v, do, scale, causal),
                _via_saved_stats(q, k, v, do, scale, causal)):
        for a, b in zip(got, want):
            assert np.max(np.abs(a - b)) < 1e-12


def test_against_torch_autograd_positions_and_rectangular():
    """Sq != Skv, offset positions (a later query shard against earlier keys)."""
    B, Sq, Skv, H, D = 1, 11, 23, 2, 8
    q, do = _rand((B, Sq, H, D), 70), _rand((B, Sq, H, D), 71)
    k, v = _rand((B, Skv, H, D), 72), _rand((B, Skv, H, D), 73)
    q_pos, k_pos = np.arange(15, 15 + Sq), np.arange(Skv)
    allowed = torch.tensor(k_pos[None, :] <= q_pos[:, None])
    want = _torch_grads(q, k, v, do, 0.3, mask=allowed)
    got = bwd.attention_grad(q, k, v, do, 0.3, True, q_pos, k_pos)
    for a, b in zip(got, want):
        assert np.max(np.abs(a - b)) < 1e-12


# ------------------------------------------------------------ finite differences

def test_finite_differences_of_the_forward():
    """Central differences of L = sum dO*O, with O from the forward oracle."""
    B, S, H, D = 1, 5, 1, 3
    q, k, v, do = (_rand((B, S, H, D), 80 + n) for n in range(4))
    scale, h = 0.7, 1e-6
    for causal in (False, True):
        grads = bwd.attention_grad(q, k, v, do, scale, causal)

        def loss(qq, kk, vv):
            return float((oracle.attention(qq, kk, vv, scale, causal)[0] * do).sum())

        for which, g in zip(range(3), grads):
            for idx in itertools.product(range(B), range(S), range(H), range(D)):
                args = [q.copy(), k.copy(), v.copy()]
                args[which][idx] += h
                up = loss(*args)
                args[which][idx] -= 2 * h
                dn = loss(*args)
                assert abs((up - dn) / (2 * h) - g[idx]) < 1e-7


# --------------------------------------------------------- closed forms, identities

def test_key_gradients_sum_to_zero_and_value_gradients_to_dout():
    """Rows of dS sum to 0 (softmax Jacobian), rows of P to 1."""
    q, k, v, do = (_rand((2, 19, 2, 8), 90 + n) for n in range(4))
    for causal in (False, True):
        dq, dk, dv = bwd.attention_grad(q, k, v, do, 0.4, causal)
        assert np.max(np.abs(dk.sum(axis=1))) < 1e-12
        assert np.max(np.abs(dv.sum(axis=1) - do.sum(axis=1))) < 1e-12


def test_single_key_and_equal_values():
    q, do = _rand((1, 6, 2, 4), 100), _rand((1, 6, 2, 4), 101)
    k, v = _rand((1, 1, 2, 4), 102), _rand((1, 1, 2, 4), 103)
    dq, dk, dv = bwd.attention_grad(q, k, v, do, 0.5)
    assert np.all(dq == 0) and np.max(np.abs(dk)) < 1e-15
    assert np.allclose(dv, do.sum(axis=1, keepdims=True), atol=1e-12)
    # equal value rows: O does not depend on the weights, so dQ = dK = 0
    k = _rand((1, 9, 2, 4), 104)
    v = np.broadcast_to(_rand((1, 1, 2, 4), 105), (1, 9, 2, 4)).copy()
    dq, dk, dv = bwd.attention_grad(q, k, v, do, 0.5)
    assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12


def test_delta_equals_weighted_dp():
    q, k, v, do = (_rand((1, 13, 2, 8), 110 + n) for n in range(4))
    o, _ = oracle.attention(q, k, v, 0.35)
    P = oracle.softmax_matrix(q, k, 0.35)
    dP = np.einsum("bihd,bjhd->bhij", do, v)
    assert np.max(np.abs(bwd.backward_delta(o, do) - (P * dP).sum(-1))) < 1e-12


def test_rows_without_keys_get_zero():
    q, do = _rand((1, 4, 1, 8), 120), _rand((1, 4, 1, 8), 121)
    k, v = _rand((1, 6, 1, 8), 122), _rand((1, 6, 1, 8), 123)
    q_pos, k_pos = np.array([-3, -1, 2, 9]), np.arange(6)   # rows 0, 1 see no key
    dq, dk, dv = bwd.attention_grad(q, k, v, do, 0.5, True, q_pos, k_pos)
    o, lse = oracle.attention(q, k, v, 0.5, True, q_pos, k_pos)
    assert np.all(np.isneginf(lse[0, 0, :2]))
    cq, ck, cv = bwd.chunk_grad(q, k, v, do, lse, bwd.backward_delta(o, do), 0.5, True,
                                q_pos, k_pos)
    for a, b in ((dq, cq), (dk, ck), (dv, cv)):
        assert np.all(np.isfinite(b)) and np.max(np.abs(a - b)) < 1e-12
    assert np.all(dq[:, :2] == 0) and np.all(cq[:, :2] == 0)


# ------------------------------------------------- decomposition over chunks

S_ID = 48


@pytest.mark.parametrize("lens,causal", [([48], False), ([12] * 4, False), ([12] * 4, True),
                                         ([17, 5, 0, 26], True), ([6] * 8, False)])
def test_chunk_shares_sum_to_full_gradient(lens, causal):
    """dQ = sum_c dQ_c; dK, dV are the chunks' slices (ring backward, any split)."""
    q, k, v, do = (_rand((1, S_ID, 2, 16), 130 + n) for n in range(4))
    scale = 0.25
    dq, dk, dv = bwd.attention_grad(q, k, v, do, scale, causal)
    o, lse = oracle.attention(q, k, v, scale, causal)
    delta = bwd.backward_delta(o, do)
    acc, k_parts, v_parts, at = np.zeros_like(q), [], [], 0
    for n in lens:
        sl = slice(at, at + n)
        cq, ck, cv = bwd.chunk_grad(q, k[:, sl], v[:, sl], do, lse, delta, scale, causal,
                                    None, np.arange(at, at + n))
        acc += cq
        k_parts.append(ck)
        v_parts.append(cv)
        at += n
    assert np.max(np.abs(acc - dq)) < 1e-12
    assert np.max(np.abs(np.concatenate(k_parts, axis=1) - dk)) < 1e-12
    assert np.max(np.abs(np.concatenate(v_parts, axis=1) - dv)) < 1e-12


def test_query_shards_sum_to_key_gradients():
    """Each ring rank adds its Q shard's share into the travelling dK, dV."""
    q, k, v, do = (_rand((1, S_ID, 2, 16), 140 + n) for n in range(4))
    scale = 0.25
    for causal in (False, True):
        dq, dk, dv = bwd.attention_grad(q, k, v, do, scale, causal)
        o, lse = oracle.attention(q, k, v, scale, causal)
        delta = bwd.backward_delta(o, do)
        sk, sv = np.zeros_like(k), np.zeros_like(v)
        for r in range(4):
            sl = slice(12 * r, 12 * r + 12)
            cq, ck, cv = bwd.chunk_grad(q[:, sl], k, v, do[:, sl], lse[:, :, sl],
                                        delta[:, :, sl], scale, causal, np.arange(12 * r, 12 * r + 12))
            assert np.max(np.abs(cq - dq[:, sl])) < 1e-12
            sk += ck
            sv += cv
        assert np.max(np.abs(sk - dk)) < 1e-12 and np.max(np.abs(sv - dv)) < 1e-12


# ---------------------------------------- planted mistakes are caught by the pins

def _mutant(kind):
    """The chain rule with one plausible mistake, for the pins to catch."""
    def grad(q, k, v, do, scale, causal=False, q_pos=None, k_pos=None):
        if kind == "strict_causal":
            q_pos = None if q_pos is None else np.asarray(q_pos) - 1
        P = oracle.softmax_matrix(q, k, scale, causal, q_pos, k_pos)[0, 0]
        Q, K, V, dO = q[0, :, 0], k[0, :, 0], v[0, :, 0], do[0, :, 0]
        dP = dO @ (K.T if kind == "dp_from_k" else V.T)
        delta = (P * dP).sum(1, keepdims=True)
        dS = {"no_delta": P * dP, "delta_sign": P * (dP + delta)}.get(kind, P * (dP - delta))
        s = 1.0 if kind == "no_scale" else scale
        dq = s * (dS @ K)
        dk = s * ((dS if kind == "dk_transposed" else dS.T) @ Q)
        dv = (P if kind == "dv_transposed" else P.T) @ dO
        return tuple(x[None, :, None, :] for x in (dq, dk, dv))
    return grad


@pytest.mark.parametrize("kind", ["no_delta", "delta_sign", "no_scale", "dk_transposed",
                                  "dv_transposed", "dp_from_k", "strict_causal"])
def test_golden_catches_planted_backward_mistakes(kind):
    assert _check_golden_grad(_mutant("none"))
    assert not _check_golden_grad(_mutant(kind))


def test_chunk_form_catches_dropped_delta_and_stale_lse():
    q, k, v, do = (_rand((1, 16, 1, 8), 150 + n) for n in range(4))
    want = bwd.attention_grad(q, k, v, do, 0.3)
    o, lse = oracle.attention(q, k, v, 0.3)
    delta = bwd.backward_delta(o, do)
    good = bwd.chunk_grad(q, k, v, do, lse, delta, 0.3)
    assert all(np.max(np.abs(a - b)) < 1e-12 for a, b in zip(good, want))
    no_delta = bwd.chunk_grad(q, k, v, do, lse, np.zeros_like(delta), 0.3)
    assert max(np.max(np.abs(a - b)) for a, b in zip(no_delta, want)) > 1e-3
    # a chunk's own LSE in place of the full row's (forgetting the merge)
    _, lse_half = oracle.attention(q, k[:, :8], v[:, :8], 0.3)
    half = bwd.chunk_grad(q, k[:, :8], v[:, :8], do, lse_half, delta, 0.3)
    assert np.max(np.abs(half[1] - want[1][:, :8])) > 1e-3
