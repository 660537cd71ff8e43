"""HIP graph capture of whole steps of the hot path.

The entry points allocate nothing, synchronise nothing and record no memset,
so a caller can capture a step on its stream and replay it. Each test captures
one step, then replays it several times. Between replays it copies new inputs
into the captured buffers, runs the same step eagerly and synchronises. Every
replay must equal the eager step bit for bit: the kernels are deterministic.
"""
import pytest
import torch

import synthetic
from tests._parity import say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import context_attention_dit_amd as cp
DEV = "cuda:0"
REPLAYS = 4


def _capture(step):
    """Warm the step up on a side stream, then capture it; returns (graph, outputs)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step()
    return g, outs


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_graph_ulysses_step():
    """Q, K, V regrouped in one launch, every rank's local attention, O regrouped back."""
    P, B, S_l, H, D = 4, 1, 96, 8, 128
    Hl, S = H // P, P * S_l
    bf = torch.bfloat16
    qkv = torch.empty((3, P, B, S_l, H, D), dtype=bf, device=DEV)
    heads = torch.empty((3, P, B, S, Hl, D), dtype=bf, device=DEV)
    o = torch.empty((P, B, S, Hl, D), dtype=bf, device=DEV)
    lse = torch.empty((P, B, Hl, S), dtype=torch.float32, device=DEV)
    back = torch.empty((P, B, S_l, H, D), dtype=bf, device=DEV)

    def step():
        cp.ulysses_seq2head(qkv, P, heads)
        for p in range(P):
            cp.attn_chunk_partial(heads[0, p], heads[1, p], heads[2, p], o[p], lse[p],
                                  out_dtype=bf)
        cp.ulysses_head2seq(o, P, back)
        return back.clone(), lse.clone()

    qkv.copy_(synthetic.make_tensor(tuple(qkv.shape), bf, 2100).to(DEV))
    say(f"graph capture: Ulysses step P={P} S_l={S_l} H={H} D={D}")
    g, (g_back, g_lse) = _capture(step)
    for r in range(REPLAYS):
        qkv.copy_(synthetic.make_tensor(tuple(qkv.shape), bf, 2101 + r).to(DEV))
        g.replay()
        torch.cuda.synchronize()
        got_back, got_lse = g_back.clone(), g_lse.clone()
        want_back, want_lse = step()
        torch.cuda.synchronize()
        assert torch.equal(_bits(got_back), _bits(want_back)), f"replay {r}: O"
        assert torch.equal(_bits(got_lse), _bits(want_lse)), f"replay {r}: LSE"


@pytest.mark.parametrize("H,Sq,lens,causal", [
    (2, 200, (70, 0, 131), True),        # causal ring with an empty chunk (one launch)
    (40, 800, (600, 500), False),        # 280 query tiles: keys split across blocks + merge
])
def test_graph_ring_forward_backward(H, Sq, lens, causal):
    """A ring rank's forward, Delta and backward, captured as one graph."""
    B, D = 1, 128
    bf, f32 = torch.bfloat16, torch.float32
    q = torch.empty((B, Sq, H, D), dtype=bf, device=DEV)
    do = torch.empty_like(q)
    ks = [torch.empty((B, n, H, D), dtype=bf, device=DEV) for n in lens]
    vs = [torch.empty_like(k) for k in ks]
    starts = [sum(lens[:c]) for c in range(len(lens))]
    chunks = list(zip(ks, vs, starts))
    q_pos0 = sum(lens) - Sq if causal else 0
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=f32, device=DEV)
    delta = torch.empty_like(lse)
    dq = torch.empty((B, Sq, H, D), dtype=f32, device=DEV)
    grads = [(torch.empty(k.shape, dtype=f32, device=DEV), torch.empty(k.shape, dtype=f32,
                                                                      device=DEV)) for k in ks]
    need = cp.ring_attention_workspace_bytes(len(lens), B, H, Sq, D)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)

    def fill(seed):
        for t, x in enumerate([q, do] + ks + vs):
            x.copy_(synthetic.make_tensor(tuple(x.shape), bf, seed + t).to(DEV))

    def step():
        cp.ring_attention(q, chunks, o, lse, causal=causal, q_pos0=q_pos0, workspace=ws)
        cp.attn_backward_delta(o, do, delta)
        cp.ring_attention_backward(q, chunks, do, lse, delta, dq, grads, causal=causal,
                                   q_pos0=q_pos0)
        return [t.clone() for t in (o, lse, dq)] + [t.clone() for gr in grads for t in gr]

    fill(2200)
    say(f"graph capture: ring rank H={H} Sq={Sq} lens={lens} causal={causal} "
        f"workspace={need} B")
    g, g_outs = _capture(step)
    names = ["O", "LSE", "dQ"] + [f"chunk {c} d{x}" for c in range(len(lens)) for x in "KV"]
    for r in range(REPLAYS):
        fill(2300 + 10 * r)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in g_outs]
        want = step()
        torch.cuda.synchronize()
        for name, a, b in zip(names, got, want):
            assert torch.equal(_bits(a), _bits(b)), f"replay {r}: {name}"
