"""GPU parity of ring calls whose last query tile is short, on single-batch
grids just past the CU count (the 1025-row ranks of a 4099-token ring are the
model case). Non-causal, the full query tiles run as one round of two-group
blocks and the last tile's rows as a launch of their own with their keys
split, merged into the same O and LSE rows; causal calls keep one launch
(their blocks already fit one round), and run here as controls. Shapes put 1, 8 and 32 rows in the last tile
(33 as a control that takes the plain path), D = 128 and 64 and chunks in
ring order; causal controls include a last row that sees every key and rows
that see none. Each is checked
against the fp64 oracle on sampled rows that include every row of the last
tile.
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


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _rows(Sq):
    last = (Sq - 1) // 128 * 128
    sel = set(range(min(40, Sq))) | set(range(max(0, last - 8), Sq))
    for r in range(128, Sq, 128):
        sel |= {r - 1, r}
    return np.array(sorted(sel))


def _run(H, Sq, lens, pos, order, causal, q0, seed, D=128):
    B = 1
    tiles = sum((n + 63) // 64 for n in lens)
    nqt = (Sq + 127) // 128
    planned = (not causal and Sq - (nqt - 1) * 128 <= 32 and nqt * H > _cus() >= (nqt - 1) * H
               and tiles >= 4)
    say(f"ring with a short last tile: H={H} Sq={Sq} D={D} lens={lens} order={order} "
        f"causal={causal} q0={q0} (split last tile: {planned})")
    q = synthetic.make_tensor((B, Sq, H, D), torch.bfloat16, seed)
    ks = [synthetic.make_tensor((B, n, H, D), torch.bfloat16, seed + 1 + 2 * c)
          for c, n in enumerate(lens)]
    vs = [synthetic.make_tensor((B, n, H, D), torch.bfloat16, seed + 2 + 2 * c)
          for c, n in enumerate(lens)]
    dev = [(ks[c].to(DEV), vs[c].to(DEV), pos[c]) for c in range(len(lens))]
    o, lse = cp.ring_attention(q.to(DEV), [dev[c] for c in order], causal=causal, q_pos0=q0)
    torch.cuda.synchronize()
    rows = _rows(Sq)
    ref = [(to_f64(ks[c]), to_f64(vs[c]), pos[c] + np.arange(lens[c])) for c in range(len(lens))]
    wo, wl = oracle.ring_attention(to_f64(q)[:, rows], ref, order, 1 / math.sqrt(D), causal,
                                   q0 + rows)
    check_o(o[:, rows], wo, "bf16", "O")
    check_lse(lse[:, :, rows], wl, "LSE")
    return o, lse, planned


@pytest.mark.parametrize("H,Sq,lens,pos,order,causal,q0", [
    # 4099-token ring rank shape, shorter chunks: one row in the last tile
    (32, 1025, (300, 200, 100, 50), (0, 300, 500, 600), (2, 0, 3, 1), False, 0),
    # causal (one launch: control), queries after most keys
    (32, 1025, (300, 200, 100, 50), (0, 300, 500, 600), (3, 2, 1, 0), True, 400),
    # 8 rows in the last tile, one chunk
    (64, 520, (777,), (0,), (0,), False, 0),
    # 32 rows in the last tile (the longest that is split off)
    (128, 288, (250, 260), (0, 250), (1, 0), False, 0),
    # 33 rows: the plain path (control)
    (128, 289, (250, 260), (0, 250), (1, 0), False, 0),
])
def test_ring_short_last_tile(H, Sq, lens, pos, order, causal, q0):
    _run(H, Sq, lens, pos, order, causal, q0, seed=7 * H + Sq)


def test_ring_short_last_tile_d64():
    _run(32, 1025, (300, 200, 100, 50), (0, 300, 500, 600), (2, 0, 3, 1), False, 0, seed=77,
         D=64)


def test_ring_short_last_tile_rows_without_keys():
    """Causal (one launch), keys placed after some queries: the first rows
    and, in a second call, every row including the last tile's see no key
    (O = 0, LSE = -inf)."""
    H, Sq = 32, 1025
    _run(H, Sq, (512, 300), (600, 1112), (1, 0), True, 0, seed=501)
    o, lse, _ = _run(H, Sq, (512, 300), (5000, 5512), (1, 0), True, 0, seed=502)
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))

