"""Calls on different HIP streams run concurrently and independently.

The library keeps no device state between calls (every buffer is the
caller's), so a relayout on one stream can overlap attention on another, as a
Ulysses layer pipeline does with the next layer's regrouping. The test issues
several such pairs on two streams (default priority) without waiting between
them, then checks every result bit for bit against the same calls run one after
another.
"""
import pytest
import torch

import synthetic
from tests._parity import say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import context_attention_dit_amd as cp
DEV = "cuda:0"


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_attention_and_relayout_on_two_streams():
    P, S_l, H, D, L = 4, 512, 8, 128, 3
    Hl, S = H // P, P * S_l
    bf = torch.bfloat16
    say(f"two streams: {L} layers of seq2head (P={P}, S_l={S_l}, H={H}) beside attention")
    qkv = [synthetic.make_tensor((3, P, 1, S_l, H, D), bf, 2400 + l).to(DEV) for l in range(L)]
    heads = [torch.empty((3, P, 1, S, Hl, D), dtype=bf, device=DEV) for _ in range(L)]
    o = [torch.empty((1, S, Hl, D), dtype=bf, device=DEV) for _ in range(L)]
    lse = [torch.empty((1, Hl, S), dtype=torch.float32, device=DEV) for _ in range(L)]

    def attend(l, stream=None):
        cp.attn_chunk_partial(heads[l][0, 0], heads[l][1, 0], heads[l][2, 0], o[l], lse[l],
                              out_dtype=bf, stream=stream)

    # sequential reference
    for l in range(L):
        cp.ulysses_seq2head(qkv[l], P, heads[l])
        attend(l)
    torch.cuda.synchronize()
    want = [(heads[l].clone(), o[l].clone(), lse[l].clone()) for l in range(L)]
    for t in heads + o + lse:
        t.zero_()
    torch.cuda.synchronize()

    # pipelined: layer l+1's regrouping on stream B while layer l attends on stream A
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    ready = [torch.cuda.Event() for _ in range(L)]
    with torch.cuda.stream(sb):
        cp.ulysses_seq2head(qkv[0], P, heads[0], stream=sb)
        ready[0].record(sb)
    for l in range(L):
        sa.wait_event(ready[l])
        attend(l, stream=sa)
        if l + 1 < L:
            cp.ulysses_seq2head(qkv[l + 1], P, heads[l + 1], stream=sb)
            ready[l + 1].record(sb)
    torch.cuda.synchronize()
    for l in range(L):
        for name, got, exp in zip(("heads", "O", "LSE"), (heads[l], o[l], lse[l]), want[l]):
            assert torch.equal(_bits(got), _bits(exp)), f"layer {l}: {name}"


def test_ring_own_workspace_on_side_stream():
    """ring_attention() allocating its own key-split workspace while launching on a
    side stream: the current stream immediately reallocates and overwrites freed
    blocks of the same size, which must not reach the ring's partials."""
    import math

    import numpy as np

    import oracle
    from tests._parity import BF16_MAX, LSE_MAX, to_f64

    H, Sq, D, lens = 32, 1025, 128, [1025, 1025, 1025, 1024]
    bf = torch.bfloat16
    need = cp.ring_attention_workspace_bytes(len(lens), 1, H, Sq, D)
    assert need > 0
    say(f"ring on a side stream, binding-allocated workspace of {need} bytes")
    q = synthetic.make_tensor((1, Sq, H, D), bf, 2500).to(DEV)
    k = synthetic.make_tensor((1, sum(lens), H, D), bf, 2501).to(DEV)
    v = synthetic.make_tensor((1, sum(lens), H, D), bf, 2502).to(DEV)
    chunks, s0 = [], 0
    for n in lens:
        chunks.append((k[:, s0:s0 + n].contiguous(), v[:, s0:s0 + n].contiguous(), s0))
        s0 += n
    ref_o, ref_l = cp.ring_attention(q, chunks)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    outs = []
    for rep in range(4):
        o = torch.empty_like(q)
        lse = torch.empty((1, H, Sq), dtype=torch.float32, device=DEV)
        side.wait_stream(torch.cuda.current_stream())
        cp.ring_attention(q, chunks, o, lse, stream=side)
        # the binding's workspace is out of scope now: grab blocks of its size on
        # the current stream and fill them while the side stream still runs
        junk = [torch.full((need // 4,), float("nan"), device=DEV) for _ in range(4)]
        outs.append((o, lse, junk))
    torch.cuda.synchronize()
    for o, lse, _ in outs:
        assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16))
        assert torch.equal(lse, ref_l)
    rows = np.array([0, 1, 511, 1024])
    wo, wl = oracle.attention(to_f64(q)[:, rows], to_f64(k), to_f64(v), 1 / math.sqrt(D))
    assert np.abs(to_f64(ref_o)[:, rows] - wo).max() <= BF16_MAX
    assert np.abs(to_f64(ref_l)[:, :, rows] - wl).max() <= LSE_MAX
