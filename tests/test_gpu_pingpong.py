"""GPU parity of the ping-pong attention kernel (one K/V chunk on grids of
more query tiles than CUs: 8-wave blocks over 256 query rows, two groups half
a step apart) against the fp64 oracle.

Shapes put the last 256-row block's second group partly or wholly past Sq,
make keys ragged, empty or shorter than a tile, and cover causal offsets,
D = 64, fp32 outputs, a negative scale and the ring entry point with one
chunk. Rows are sampled: the first rows, both sides of every block and group
boundary near the end, and the last rows.
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
