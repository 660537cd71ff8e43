"""Seeded random shapes built to take each multi-launch or chunk-list plan of
the bf16 forward, checked against the fp64 oracle on sampled rows:

* the short-last-tile plan (non-causal ring, B = 1, last query tile of 1-32
  rows just past the CU count): random head counts, tail lengths, chunk
  splits (some empty) and visit orders;
* the last-round plan (non-causal, one chunk, more 256-row blocks than CUs
  with the last round at most half full): random batch, heads, rows, keys;
* the chunk-list ping-pong kernel (causal ring, D = 128, at least as many
  256-row blocks as CUs): random chunk splits, positions and orders.
"""
import math

import numpy as np
import pytest
import torch

import context_attention_dit_amd as cp
import oracle
import synthetic
from tests._parity import check_lse, check_o, say, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 128


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _rows(rng, Sq):
    sel = set(range(min(12, Sq))) | set(range(max(0, Sq - 40), Sq))
    for r in range(128, Sq, 128):
        sel |= {r - 1, r}
    sel |= set(rng.choice(Sq, size=min(16, Sq), replace=False).tolist())
    return np.array(sorted(sel))


def _split(rng, total, parts):
    cuts = np.sort(rng.choice(np.arange(total + 1), size=parts - 1, replace=True))
    edges = np.concatenate([[0], cuts, [total]])
    return [int(x) for x in np.diff(edges)]


def _ring_case(seed, B, H, Sq, lens, pos, order, causal, q0):
    q = synthetic.make_tensor((B, Sq, H, D), torch.bfloat16, seed)
    ks = [synthetic.make_tensor((B, n, H, D), torch.bfloat16, seed + 1 + 2 * c)
          for c, n in enumerate(lens)]
    vs = [synthetic.make_tensor((B, n, H, D), torch.bfloat16, seed + 2 + 2 * c)
          for c, n in enumerate(lens)]
    dev = [(ks[c].to(DEV), vs[c].to(DEV), pos[c]) for c in range(len(lens))]
    o, lse = cp.ring_attention(q.to(DEV), [dev[c] for c in order], causal=causal, q_pos0=q0)
    torch.cuda.synchronize()
    rows = _rows(np.random.default_rng(seed), Sq)
    ref = [(to_f64(ks[c]), to_f64(vs[c]), pos[c] + np.arange(lens[c])) for c in range(len(lens))]
    wo, wl = oracle.ring_attention(to_f64(q)[:, rows], ref, order, 1 / math.sqrt(D), causal,
                                   q0 + rows)
    check_o(o[:, rows], wo, "bf16", "O")
    check_lse(lse[:, :, rows], wl, "LSE")


@pytest.mark.parametrize("seed", range(6))
def test_random_short_last_tile(seed):
    rng = np.random.default_rng(7000 + seed)
    cus = _cus()
    H = int(rng.choice([32, 40, 48, 64, 80, 96, 128]))
    full = cus // H                       # full 128-row tiles that fit one per CU
    Sq = full * 128 + int(rng.integers(1, 33))
    P = int(rng.integers(1, 6))
    lens = _split(rng, int(rng.integers(300, 2500)), P)
    pos = np.cumsum([0] + lens[:-1]).tolist()
    order = rng.permutation(P).tolist()
    tiles = sum((n + 63) // 64 for n in lens)
    assert ((Sq + 127) // 128) * H > cus >= full * H and tiles >= 4
    say(f"random short last tile #{seed}: H={H} Sq={Sq} lens={lens} order={order}")
    _ring_case(7100 + seed, 1, H, Sq, lens, pos, order, False, 0)


@pytest.mark.parametrize("seed", range(6))
def test_random_last_round(seed):
    rng = np.random.default_rng(8000 + seed)
    cus = _cus()
    while True:
        B = int(rng.choice([1, 2]))
        H = int(rng.integers(8, 97))
        Sq = int(rng.integers(300, 2200))
        units = B * H * ((Sq + 255) // 256)
        if units > cus and 0 < 2 * (units % cus) <= cus:
            break
    Skv = int(rng.integers(1, 1600))
    out_dtype = torch.float32 if seed % 3 == 2 else torch.bfloat16
    say(f"random last round #{seed}: B={B} H={H} Sq={Sq} Skv={Skv} ({units} blocks) {out_dtype}")
    q = synthetic.make_tensor((B, Sq, H, D), torch.bfloat16, 8100 + seed)
    k = synthetic.make_tensor((B, Skv, H, D), torch.bfloat16, 8200 + seed)
    v = synthetic.make_tensor((B, Skv, H, D), torch.bfloat16, 8300 + seed)
    o, lse = cp.attn_chunk_partial(q.to(DEV), k.to(DEV), v.to(DEV), out_dtype=out_dtype)
    torch.cuda.synchronize()
    rows = _rows(rng, Sq)
    wo, wl = oracle.chunk_partial(to_f64(q)[:, rows], to_f64(k), to_f64(v), 1 / math.sqrt(D),
                                  False, rows, np.arange(Skv))
    check_o(o[:, rows], wo, "bf16", "O")
    check_lse(lse[:, :, rows], wl, "LSE")


@pytest.mark.parametrize("seed", range(6))
def test_random_causal_chunk_list(seed):
    rng = np.random.default_rng(9000 + seed)
    cus = _cus()
    while True:
        B = int(rng.choice([1, 2]))
        H = int(rng.integers(8, 65))
        Sq = int(rng.integers(256, 2600))
        if B * H * ((Sq + 255) // 256) >= cus and B * H * ((Sq + 127) // 128) > cus:
            break
    P = int(rng.integers(2, 6))
    lens = _split(rng, int(rng.integers(400, 3000)), P)
    pos = np.cumsum([0] + lens[:-1]).tolist()
    order = rng.permutation(P).tolist()
    q0 = int(rng.integers(0, sum(lens)))
    say(f"random causal chunk list #{seed}: B={B} H={H} Sq={Sq} lens={lens} order={order} q0={q0}")
    _ring_case(9100 + seed, B, H, Sq, lens, pos, order, True, q0)
