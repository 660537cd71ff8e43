"""GPU parity of the ping-pong attention kernels against the fp64 oracle.

attn_pp_kernel: one K/V chunk on grids of more query tiles than CUs (8-wave
blocks over 256 query rows, two groups half a step apart). Shapes put the
last 256-row block's second group partly or wholly past Sq, make keys
ragged, empty or shorter than a tile, and cover causal offsets, D = 64, fp32
outputs, a negative scale and the ring entry point with one chunk. Its
chunk-list form (causal rings whose 256-row blocks fill the CUs) is checked
on ragged, empty and reordered chunks, two batches, and blocks that see no
key; non-causal grids whose last round of 256-row blocks is at most half
full (its rows then run as two-group blocks) on split points inside a head,
a short last block, two batches and fp32 outputs.

attn_g2pp_kernel: small grids (no more query tiles than CUs, at least four
key tiles, D = 128): 8-wave blocks over one 128-row query tile whose two
groups take the two halves of its key tiles. Shapes give each group one,
two or three tiles, none at all (a query tile that sees one key tile, or
none), ragged and empty chunks in ring order, and fp32 outputs.

Rows are sampled: the first rows, both sides of every block and group
boundary, and the last rows.
"""
import math

import numpy as np
import pytest
import torch

import context_attention_dit_amd as cp
import oracle
import synthetic
from tests._parity import check_lse, check_o, check_o_scaled, say, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rows(Sq):
    edges = [0, Sq - 1]
    for r in range(128, Sq, 128):
        edges += [r - 1, r]
    sel = set(range(min(40, Sq))) | set(range(max(0, Sq - 40), Sq))
    sel |= {e for e in edges if 0 <= e < Sq}
    return np.array(sorted(sel))


def _check(o, lse, q, k, v, scale, causal, q0, k0, out_dtype, peaky=False):
    Sq, Skv = q.shape[1], k.shape[1]
    rows = _rows(Sq)
    wo, wl = oracle.chunk_partial(to_f64(q)[:, rows], to_f64(k), to_f64(v), scale, causal,
                                  q0 + rows, k0 + np.arange(Skv))
    got = o[:, rows]
    if out_dtype == torch.float32:
        check_o(got, wo, "bf16", "O")          # fp32 output of bf16 inputs: the bf16 bars
    elif peaky:
        check_o_scaled(got, wo, "O")
    else:
        check_o(got, wo, "bf16", "O")
    check_lse(lse[:, :, rows], wl, "LSE")


@pytest.mark.parametrize("B,H,Sq,Skv,D,causal,q0,k0,out_dtype", [
    (1, 40, 1000, 777, 128, False, 0, 0, torch.bfloat16),     # ragged keys
    (1, 40, 1000, 1700, 128, True, 500, 0, torch.bfloat16),   # causal, queries mid-sequence
    (2, 32, 612, 900, 128, False, 0, 0, torch.float32),       # last block: group 1 past Sq
    (1, 48, 712, 300, 128, True, 0, 0, torch.bfloat16),       # last block: group 1 partly valid
    (2, 24, 700, 1500, 64, True, 800, 0, torch.bfloat16),     # D = 64
    (1, 40, 1000, 37, 128, False, 0, 0, torch.bfloat16),      # keys shorter than a tile
    (1, 40, 1000, 65, 128, True, 0, 935, torch.bfloat16),     # causal, keys after most queries
])
def test_pingpong_chunk_partial(B, H, Sq, Skv, D, causal, q0, k0, out_dtype):
    say(f"ping-pong chunk partial B={B} H={H} Sq={Sq} Skv={Skv} D={D} causal={causal} "
        f"q0={q0} k0={k0} {out_dtype}")
    assert B * H * ((Sq + 127) // 128) > 256   # more query tiles than CUs: this kernel
    q = synthetic.make_tensor((B, Sq, H, D), torch.bfloat16, Sq + Skv + H)
    k = synthetic.make_tensor((B, Skv, H, D), torch.bfloat16, Sq + Skv + H + 1)
    v = synthetic.make_tensor((B, Skv, H, D), torch.bfloat16, Sq + Skv + H + 2)
    o, lse = cp.attn_chunk_partial(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, q_pos0=q0,
                                   kv_pos0=k0, out_dtype=out_dtype)
    torch.cuda.synchronize()
    _check(o, lse, q, k, v, 1 / math.sqrt(D), causal, q0, k0, out_dtype)


def test_pingpong_no_keys_and_negative_scale():
    B, H, Sq, D = 1, 40, 1000, 128
    q = synthetic.make_tensor((B, Sq, H, D), torch.bfloat16, 61)
    say("ping-pong: no keys")
    k0 = torch.empty((B, 0, H, D), dtype=torch.bfloat16, device=DEV)
    o, lse = cp.attn_chunk_partial(q.to(DEV), k0, k0)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    say("ping-pong: negative scale, causal")
    k = synthetic.make_tensor((B, 600, H, D), torch.bfloat16, 62)
    v = synthetic.make_tensor((B, 600, H, D), torch.bfloat16, 63)
    scale = -0.37
    o, lse = cp.attn_chunk_partial(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale, causal=True,
                                   q_pos0=100)
    torch.cuda.synchronize()
    _check(o, lse, q, k, v, scale, True, 100, 0, torch.bfloat16, peaky=True)


def test_pingpong_through_the_ring_with_one_chunk():
    """cp_ring_attention with one chunk on a grid of more than two query tiles
    per CU (no key splits) runs the same kernel."""
    B, H, Sq, Skv, D = 1, 64, 1100, 1234, 128
    say(f"ping-pong through the ring: H={H} Sq={Sq} Skv={Skv}")
    assert B * H * ((Sq + 127) // 128) > 512
    q = synthetic.make_tensor((B, Sq, H, D), torch.bfloat16, 71)
    k = synthetic.make_tensor((B, Skv, H, D), torch.bfloat16, 72)
    v = synthetic.make_tensor((B, Skv, H, D), torch.bfloat16, 73)
    o, lse = cp.ring_attention(q.to(DEV), [(k.to(DEV), v.to(DEV), 0)], causal=True, q_pos0=300)
    torch.cuda.synchronize()
    _check(o, lse, q, k, v, 1 / math.sqrt(D), True, 300, 0, torch.bfloat16)


def _small_grid(B, H, Sq, tiles):
    # the launcher's choice of the two-group kernel on a 256-CU part
    return B * H * ((Sq + 127) // 128) <= 256 and tiles >= 4


@pytest.mark.parametrize("B,H,Sq,Skv,causal,q0,k0,out_dtype", [
    (1, 24, 300, 256, False, 0, 0, torch.bfloat16),     # 4 key tiles: 2 per group
    (1, 24, 300, 300, True, 0, 0, torch.bfloat16),      # first query tile: 1 tile per group
    (2, 12, 640, 320, False, 0, 0, torch.float32),      # 5 tiles: 2 and 3, fp32 out
    (1, 24, 700, 900, True, 0, 64, torch.bfloat16),     # first query tile: 1 tile, group 0 none
    (1, 24, 700, 900, True, 0, 200, torch.bfloat16),    # first query tile sees no key at all
    (1, 20, 1000, 4000, True, 3000, 0, torch.bfloat16), # long, ragged last query tile
])
def test_two_group_chunk_partial(B, H, Sq, Skv, causal, q0, k0, out_dtype):
    D = 128
    say(f"two-group ping-pong chunk partial B={B} H={H} Sq={Sq} Skv={Skv} causal={causal} "
        f"q0={q0} k0={k0} {out_dtype}")
    assert _small_grid(B, H, Sq, (Skv + 63) // 64)
    q = synthetic.make_tensor((B, Sq, H, D), torch.bfloat16, 3 * Sq + Skv + H)
    k = synthetic.make_tensor((B, Skv, H, D), torch.bfloat16, 3 * Sq + Skv + H + 1)
    v = synthetic.make_tensor((B, Skv, H, D), torch.bfloat16, 3 * Sq + Skv + H + 2)
    o, lse = cp.attn_chunk_partial(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, q_pos0=q0,
                                   kv_pos0=k0, out_dtype=out_dtype)
    torch.cuda.synchronize()
    _check(o, lse, q, k, v, 1 / math.sqrt(D), causal, q0, k0, out_dtype)


@pytest.mark.parametrize("H,Sq,lens,pos,order,causal,q0", [
    # FLUX-like rank: four chunks in ring order, one ragged and one short
    (24, 1152, (1152, 1000, 77, 1152), (0, 1152, 2152, 2229), (2, 0, 3, 1), False, 0),
    # causal, reversed visit order, an empty chunk, the diagonal chunk last
    (8, 900, (512, 0, 700, 300), (0, 512, 512, 1212), (3, 2, 1, 0), True, 700),
    # causal from position 0: the first query tiles see few keys
    (16, 500, (400, 400), (0, 400), (1, 0), True, 0),
])
def test_two_group_ring(H, Sq, lens, pos, order, causal, q0):
    B, D = 1, 128
    say(f"two-group ping-pong ring H={H} Sq={Sq} lens={lens} order={order} causal={causal} "
        f"q0={q0}")
    assert _small_grid(B, H, Sq, sum((n + 63) // 64 for n in lens))
    q = synthetic.make_tensor((B, Sq, H, D), torch.bfloat16, 81 + H)
    ks = [synthetic.make_tensor((B, n, H, D), torch.bfloat16, 90 + 3 * c) for c, n in enumerate(lens)]
    vs = [synthetic.make_tensor((B, n, H, D), torch.bfloat16, 91 + 3 * c) for c, n in enumerate(lens)]
    dev = [(ks[c].to(DEV), vs[c].to(DEV), pos[c]) for c in range(len(lens))]
    o, lse = cp.ring_attention(q.to(DEV), [dev[c] for c in order], causal=causal, q_pos0=q0)
    torch.cuda.synchronize()
    rows = _rows(Sq)
    ref = [(to_f64(ks[c]), to_f64(vs[c]), pos[c] + np.arange(lens[c])) for c in range(len(lens))]
    wo, wl = oracle.ring_attention(to_f64(q)[:, rows], ref, order, 1 / math.sqrt(D), causal,
                                   q0 + rows)
    check_o(o[:, rows], wo, "bf16", "O")
    check_lse(lse[:, :, rows], wl, "LSE")


@pytest.mark.parametrize("B,H,Sq,lens,pos,order,q0", [
    # 8 blocks of 256 rows x 32 heads: ragged and empty chunks, reversed order,
    # the diagonal inside the last chunk visited
    (1, 32, 2048, (700, 0, 1000, 900, 500), (0, 700, 700, 1700, 2600), (4, 3, 2, 1, 0), 1100),
    # two batches, last 256-row block partly past Sq
    (2, 16, 1900, (1200, 1300), (0, 1200), (1, 0), 600),
    # keys placed after the first queries: the first blocks see no key at all
    (1, 32, 2048, (800, 800), (1000, 1800), (0, 1), 0),
])
def test_pingpong_causal_chunk_list(B, H, Sq, lens, pos, order, q0):
    """The large-grid ping-pong kernel walks a causal chunk list (D = 128,
    at least as many 256-row blocks as CUs, no key splits)."""
    D = 128
    say(f"ping-pong causal chunk list B={B} H={H} Sq={Sq} lens={lens} order={order} q0={q0}")
    assert B * H * ((Sq + 255) // 256) >= torch.cuda.get_device_properties(0).multi_processor_count
    assert B * H * ((Sq + 127) // 128) > 256   # no two-group blocks (causal: never split)
    q = synthetic.make_tensor((B, Sq, H, D), torch.bfloat16, 91 + Sq)
    ks = [synthetic.make_tensor((B, n, H, D), torch.bfloat16, 92 + 2 * c) for c, n in enumerate(lens)]
    vs = [synthetic.make_tensor((B, n, H, D), torch.bfloat16, 93 + 2 * c) for c, n in enumerate(lens)]
    dev = [(ks[c].to(DEV), vs[c].to(DEV), pos[c]) for c in range(len(lens))]
    o, lse = cp.ring_attention(q.to(DEV), [dev[c] for c in order], causal=True, q_pos0=q0)
    torch.cuda.synchronize()
    rows = _rows(Sq)
    ref = [(to_f64(ks[c]), to_f64(vs[c]), pos[c] + np.arange(lens[c])) for c in range(len(lens))]
    wo, wl = oracle.ring_attention(to_f64(q)[:, rows], ref, order, 1 / math.sqrt(D), True,
                                   q0 + rows)
    check_o(o[:, rows], wo, "bf16", "O")
    check_lse(lse[:, :, rows], wl, "LSE")


@pytest.mark.parametrize("B,H,Sq,Skv,out_dtype", [
    (1, 80, 1000, 777, torch.bfloat16),    # 320 blocks: the last 64 as two-group blocks
    (1, 96, 900, 500, torch.bfloat16),     # 384: the last 128 (a half round exactly)
    (1, 72, 850, 1300, torch.bfloat16),    # 288; last 256-row block of a head has 82 rows
    (2, 36, 900, 700, torch.float32),      # two batches, fp32 out
])
def test_pingpong_last_round_as_two_group_blocks(B, H, Sq, Skv, out_dtype):
    """Non-causal, one chunk, more 256-row blocks than CUs with a last round at
    most half full: that round's rows run as 128-row two-group blocks in a
    second launch (the split point falls inside a head, so one head's rows
    come from both kernels)."""
    D = 128
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units = B * H * ((Sq + 255) // 256)
    assert units > cus and 0 < 2 * (units % cus) <= cus
    say(f"ping-pong last round as two-group blocks: B={B} H={H} Sq={Sq} Skv={Skv} {out_dtype}")
    q = synthetic.make_tensor((B, Sq, H, D), torch.bfloat16, 131 + H)
    k = synthetic.make_tensor((B, Skv, H, D), torch.bfloat16, 132 + H)
    v = synthetic.make_tensor((B, Skv, H, D), torch.bfloat16, 133 + H)
    o, lse = cp.attn_chunk_partial(q.to(DEV), k.to(DEV), v.to(DEV), out_dtype=out_dtype)
    torch.cuda.synchronize()
    # every head at the split point and the last head, sampled rows
    _check(o, lse, q, k, v, 1 / math.sqrt(D), False, 0, 0, out_dtype)
    if out_dtype == torch.bfloat16:   # the ring with this one chunk (its own plan)
        ro, rl = cp.ring_attention(q.to(DEV), [(k.to(DEV), v.to(DEV), 0)])
        torch.cuda.synchronize()
        _check(ro, rl, q, k, v, 1 / math.sqrt(D), False, 0, 0, out_dtype)
