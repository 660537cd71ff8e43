"""GPU parity of one-chunk non-causal ring calls whose 256-row query tiles
take more than one round of the compute units, with the last round at most
half full. With the workspace cp_ring_attention_workspace_bytes reports, that
round's tiles run with their keys split over blocks (fp32 partials merged
after); the Wan 21x30x52 Ulysses rank (640 tiles, 128 in the last round) is
the model case. Shapes put the round's first tile inside a head, a short last
tile, two batches, ragged key counts and 2 to 8 splits. Controls: a workspace
below that size (the last round then runs unsplit), too few key tiles to
split, a causal call. Every case is checked against the fp64 oracle on
sampled rows that include rows of the split tiles and of the full rounds,
and the split and unsplit runs of one shape are compared with each other.
The Qwen-Image rank (one round of tiles, no split) runs through the same call
as the benchmark times it, at full size.
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


def _splits(B, H, Sq, Skv, causal):
    """The key splits the library's plan gives the last round (0: no split)."""
    cus = _cus()
    nitems = (Sq + 255) // 256 * B * H
    rest = nitems % cus
    if causal or nitems <= cus or rest == 0 or 2 * rest > cus:
        return 0
    s = min(8, cus // rest, ((Skv + 63) // 64) // 4)
    return s if s >= 2 else 0


def _rows(Sq, seed, n_rand=40, tile_stride=1):
    sel = set(range(min(8, Sq))) | set(range(max(0, Sq - 8), Sq))
    for r in range(256, Sq, 256 * tile_stride):
        sel |= {r - 1, r}
    rng = np.random.default_rng(seed)
    sel |= set(rng.integers(0, Sq, n_rand).tolist())
    return np.array(sorted(sel))


def _check(q, k, v, o, lse, causal, rows, what):
    D = q.shape[-1]
    wo, wl = oracle.ring_attention(to_f64(q)[:, rows], [(to_f64(k), to_f64(v), np.arange(k.shape[1]))],
                                   [0], 1 / math.sqrt(D), causal, rows)
    check_o(o[:, torch.from_numpy(rows).to(o.device)], wo, "bf16", f"{what} O")
    check_lse(lse[:, :, torch.from_numpy(rows).to(lse.device)], wl, f"{what} LSE")


def _run(B, H, Sq, Skv, causal, seed, expect_split=None):
    D = 128
    s = _splits(B, H, Sq, Skv, causal)
    if expect_split is not None and _cus() == 256:
        assert (s > 0) == expect_split, s
    say(f"one-chunk ring, B={B} H={H} Sq={Sq} Skv={Skv} causal={causal}: last-round splits {s}")
    q = synthetic.make_tensor((B, Sq, H, D), torch.bfloat16, seed)
    k = synthetic.make_tensor((B, Skv, H, D), torch.bfloat16, seed + 1)
    v = synthetic.make_tensor((B, Skv, H, D), torch.bfloat16, seed + 2)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    need = cp.ring_attention_workspace_bytes(1, B, H, Sq, D)
    o, lse = cp.ring_attention(qd, [(kd, vd, 0)], causal=causal)   # the reported workspace
    # a workspace too small for the split: the last round runs unsplit
    o2, lse2 = cp.ring_attention(qd, [(kd, vd, 0)], causal=causal,
                                 workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    if s:
        assert need > 0
    rows = _rows(Sq, seed)
    _check(q, k, v, o, lse, causal, rows, "split")
    _check(q, k, v, o2, lse2, causal, rows, "unsplit")
    # the two plans agree to bf16 rounding everywhere
    assert (o.float() - o2.float()).abs().max().item() <= 2 ** -6
    assert (lse - lse2).abs().max().item() <= 1e-4
    if not s:
        assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("B,H,Sq,Skv,seed", [
    (1, 40, 1792, 2100, 11),   # 280 tiles: 24 in the last round, from inside head 36; 8 splits
    (1, 40, 1790, 1000, 12),   # a 254-row last tile; 16 key tiles -> 4 splits
    (2, 20, 1792, 700, 13),    # two batches; 11 key tiles -> 2 splits
])
def test_last_round_key_split(B, H, Sq, Skv, seed):
    _run(B, H, Sq, Skv, False, seed, expect_split=True)


def test_last_round_controls():
    # too few key tiles to split (4), and a causal call: one plan either way
    _run(1, 40, 1792, 200, False, 21, expect_split=False)
    _run(1, 40, 1792, 2100, True, 22, expect_split=False)


@pytest.mark.parametrize("wname,splits", [
    ("wan-21x30x52-ulysses8-rank0", 2),       # 640 tiles, 128 in the last round
    ("qwen-image-1536-ulysses4-rank0", 0),    # 222 tiles: one round, no split
])
def test_ulysses_rank0_ring_one_chunk(wname, splits):
    """A Ulysses rank 0's attention through the ring call with one chunk (the
    call the benchmark times): Wan 21x30x52 (32760 rows, 5 heads, its last
    round split 2 ways) and Qwen-Image 1536 (9472 rows, 6 heads, the
    ping-pong plan of cp_attn_chunk_partial), sampled rows against the
    oracle."""
    w = synthetic.WORKLOADS[wname]
    H, D = w.H_local, w.D
    say(f"{w.name}: inputs")
    q, k, v = (x[:, :, :H].contiguous() for x in synthetic.make_qkv(w))  # rank 0's heads
    if _cus() == 256:
        assert _splits(1, H, w.S, w.S, False) == splits
    say(f"{w.name}: ring call with one chunk")
    o, lse = cp.ring_attention(q.to(DEV), [(k.to(DEV), v.to(DEV), 0)])
    torch.cuda.synchronize()
    rows = _rows(w.S, w.seed, n_rand=64, tile_stride=8)
    say(f"{w.name}: oracle on {len(rows)} rows x {H} heads")
    _check(q, k, v, o, lse, False, rows, f"{w.name} rank 0")
