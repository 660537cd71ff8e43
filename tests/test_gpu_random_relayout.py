"""GPU bit-exactness of the layout transforms on seeded random shapes.

Each case draws the rank count P, batch B, head width D (odd widths included,
so the narrow-word paths run too), the element size, and random bit
patterns, then checks against the oracle:

* the standard Ulysses regroupings, on a stack of 1..3 tensors (one launch),
  and their round trip;
* the uneven (Ulysses Anything) regroupings with a random split of the tokens
  and of the heads over the ranks (ranks with no tokens or no heads allowed),
  and their round trip, on one tensor and on the same stack of tensors;
* the K/V gather over the same random token split, on one tensor and stacked.

The transforms are pure copies, so every comparison is on raw bits.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests._parity import say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import context_attention_dit_amd as cp
DEV = "cuda:0"

N_CASES = 32


def _split_counts(rng, total, parts):
    cuts = np.sort(rng.integers(0, total + 1, size=parts - 1))
    return tuple(int(x) for x in np.diff(np.concatenate([[0], cuts, [total]])))


def _case(seed):
    rng = np.random.default_rng(30_000 + seed)
    P = int(rng.integers(1, 9))
    B = int(rng.integers(1, 3))
    D = int(rng.choice([1, 3, 8, 12, 64, 72, 128]))
    isz = int(rng.choice([2, 4]))
    n = int(rng.integers(1, 4))
    S_l = int(rng.integers(1, 40))
    H = P * int(rng.integers(1, 5))
    S_any = int(rng.integers(1, 300))
    H_any = int(rng.integers(1, 25))
    s_lens = _split_counts(rng, S_any, P)
    h_counts = _split_counts(rng, H_any, P)
    return P, B, D, isz, n, S_l, H, s_lens, h_counts


def _pieces(flat, shapes):
    out, o = [], 0
    for shp in shapes:
        m = int(np.prod(shp))
        out.append(flat[o:o + m].reshape(shp))
        o += m
    return out


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_relayouts_bit_exact(seed):
    P, B, D, isz, n, S_l, H, s_lens, h_counts = _case(seed)
    dt = torch.bfloat16 if isz == 2 else torch.float32
    say(f"random relayout {seed}: P={P} B={B} D={D} bytes={isz} n={n} S_l={S_l} H={H} "
        f"s_lens={s_lens} h_counts={h_counts}")

    # standard regroupings on n stacked tensors
    bits = synthetic.random_bits((n, P, B, S_l, H, D), isz, seed=40_000 + seed)
    y = cp.ulysses_seq2head(bits.view(dt).to(DEV), P)
    z = cp.ulysses_head2seq(y, P)
    torch.cuda.synchronize()
    yb = y.cpu().view(bits.dtype).numpy()
    for t in range(n):
        assert np.array_equal(yb[t], oracle.seq2head(bits[t].numpy(), P)), f"seq2head tensor {t}"
    assert np.array_equal(z.cpu().view(bits.dtype).numpy(), bits.numpy()), "round trip"
    # head2seq on its own random input
    hb = synthetic.random_bits(tuple(yb.shape), isz, seed=41_000 + seed)
    w = cp.ulysses_head2seq(hb.view(dt).to(DEV), P)
    torch.cuda.synchronize()
    wb = w.cpu().view(bits.dtype).numpy()
    for t in range(n):
        assert np.array_equal(wb[t], oracle.head2seq(hb[t].numpy(), P)), f"head2seq tensor {t}"

    # uneven regroupings
    S, Ht = sum(s_lens), sum(h_counts)
    flat = synthetic.random_bits((B * S * Ht * D,), isz, seed=42_000 + seed)
    g = cp.ulysses_anything_seq2head(flat.view(dt).to(DEV), s_lens, h_counts, B, D)
    back = cp.ulysses_anything_head2seq(g, s_lens, h_counts, B, D)
    torch.cuda.synchronize()
    shards = _pieces(flat.numpy(), [(B, s, Ht, D) for s in s_lens])
    want = oracle.anything_seq2head(shards, list(h_counts))
    got = _pieces(g.cpu().view(flat.dtype).numpy(), [(B, S, h, D) for h in h_counts])
    for p, (a, b) in enumerate(zip(got, want)):
        assert np.array_equal(a, b), f"anything seq2head group {p}"
    assert torch.equal(back.cpu().view(flat.dtype), flat), "anything round trip"
    gb = synthetic.random_bits((B * S * Ht * D,), isz, seed=43_000 + seed)
    r = cp.ulysses_anything_head2seq(gb.view(dt).to(DEV), s_lens, h_counts, B, D)
    torch.cuda.synchronize()
    groups = _pieces(gb.numpy(), [(B, S, h, D) for h in h_counts])
    want = oracle.anything_head2seq(groups, list(s_lens))
    got = _pieces(r.cpu().view(gb.dtype).numpy(), [(B, s, Ht, D) for s in s_lens])
    for q, (a, b) in enumerate(zip(got, want)):
        assert np.array_equal(a, b), f"anything head2seq shard {q}"

    # K/V gather over the same token split (Ht heads)
    kv = cp.kv_gather(flat.view(dt).to(DEV), s_lens, B, Ht, D)
    torch.cuda.synchronize()
    assert np.array_equal(kv.cpu().view(flat.dtype).numpy(), oracle.kv_gather(shards)), "gather"

    # the same three on a stack of n tensors, one launch each
    stack = synthetic.random_bits((n, B * S * Ht * D), isz, seed=44_000 + seed)
    sd = stack.view(dt).to(DEV)
    gs = cp.ulysses_anything_seq2head(sd, s_lens, h_counts, B, D)
    hs = cp.ulysses_anything_head2seq(sd, s_lens, h_counts, B, D)
    ks = cp.kv_gather(sd, s_lens, B, Ht, D)
    torch.cuda.synchronize()
    gsb, hsb, ksb = (t.cpu().view(stack.dtype).numpy() for t in (gs, hs, ks))
    for t in range(n):
        sh = _pieces(stack[t].numpy(), [(B, s, Ht, D) for s in s_lens])
        want = np.concatenate([w.ravel() for w in oracle.anything_seq2head(sh, list(h_counts))])
        assert np.array_equal(gsb[t], want), f"stacked anything seq2head tensor {t}"
        gr = _pieces(stack[t].numpy(), [(B, S, h, D) for h in h_counts])
        want = np.concatenate([w.ravel() for w in oracle.anything_head2seq(gr, list(s_lens))])
        assert np.array_equal(hsb[t], want), f"stacked anything head2seq tensor {t}"
        assert np.array_equal(ksb[t], oracle.kv_gather(sh)), f"stacked gather tensor {t}"
