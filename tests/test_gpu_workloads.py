"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

Outputs the oracle can afford are compared in full (FLUX ring rank, the
ring-anything split of 4099 tokens); for the long Ulysses sequences, and the
128K sequence as a ring of 8, the oracle computes a sample of query rows one
by one (first rows, last rows and seeded random rows of every head) against
the full K/V, with explicit positions. Relayouts are compared bit for bit with the oracle's permutation.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests._parity import check_lse, check_o, say, to_f64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import context_attention_dit_amd as cp
DEV = "cuda:0"


def _rows(S, n_edge, n_rand, seed):
    rng = np.random.default_rng(seed)
    r = set(range(min(n_edge, S))) | set(range(max(0, S - n_edge), S))
    r |= set(rng.choice(S, size=min(n_rand, S), replace=False).tolist())
    return np.array(sorted(r))


def _ring_chunks(w, k, v):
    starts = w.chunk_starts()
    return [(k[:, s:s + n].contiguous(), v[:, s:s + n].contiguous(), s)
            for s, n in zip(starts, w.chunk_lens)]


def test_flux_ring_rank0_full():
    """FLUX 1024x1024 ring rank 0: 1152 query rows over 4 chunks in order [0,3,2,1]."""
    w = synthetic.FLUX_RING
    say(f"{w.name}: generating inputs")
    q, k, v = synthetic.make_qkv(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    chunks = _ring_chunks(w, kd, vd)
    order = synthetic.ring_order(0, w.P)
    assert order == [0, 3, 2, 1]
    n = w.chunk_lens[0]
    q0 = qd[:, :n].contiguous()
    say(f"{w.name}: fused ring")
    o, lse = cp.ring_attention(q0, [chunks[c] for c in order])
    say(f"{w.name}: partials + merge")
    parts = [cp.attn_chunk_partial(q0, chunks[c][0], chunks[c][1]) for c in order]
    mo, ml = cp.lse_merge(torch.stack([p[0] for p in parts]), torch.stack([p[1] for p in parts]),
                          out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    say(f"{w.name}: oracle")
    wo, wl = oracle.attention(to_f64(q[:, :n]), to_f64(k), to_f64(v), 1 / math.sqrt(w.D))
    check_o(o, wo, "bf16", "ring O")
    check_lse(lse, wl, "ring LSE")
    check_o(mo, wo, "bf16", "merged O")
    check_lse(ml, wl, "merged LSE")


@pytest.mark.parametrize("causal", [True, False])
def test_ring_anything_4099_all_ranks(causal):
    """S = 4099 split 1025/1025/1025/1024, every rank in its ring order."""
    w = synthetic.LLM_RING_ANYTHING
    say(f"{w.name} causal={causal}: inputs")
    q, k, v = synthetic.make_qkv(w)
    kd, vd = k.to(DEV), v.to(DEV)
    chunks = _ring_chunks(w, kd, vd)
    starts = w.chunk_starts()
    outs = []
    for r in range(w.P):
        s0, n = starts[r], w.chunk_lens[r]
        say(f"{w.name} causal={causal}: rank {r}")
        outs.append(cp.ring_attention(q[:, s0:s0 + n].contiguous().to(DEV),
                                      [chunks[c] for c in synthetic.ring_order(r, w.P)],
                                      causal=causal, q_pos0=s0))
    torch.cuda.synchronize()
    say(f"{w.name} causal={causal}: oracle")
    wo, wl = oracle.attention(to_f64(q), to_f64(k), to_f64(v), 1 / math.sqrt(w.D), causal)
    for r, (o, lse) in enumerate(outs):
        s0, n = starts[r], w.chunk_lens[r]
        check_o(o, wo[:, s0:s0 + n], "bf16", f"rank {r} O")
        check_lse(lse, wl[:, :, s0:s0 + n], f"rank {r} LSE")


@pytest.mark.parametrize("wname,n_edge,n_rand", [
    ("qwen-image-1536-ulysses4-rank0", 192, 384),
    ("wan-21x30x52-ulysses8-rank0", 96, 192),
    ("llm-128k-causal-ulysses8-rank0", 96, 160),
])
def test_ulysses_rank0(wname, n_edge, n_rand):
    """seq2head of Q, K, V for all ranks; rank 0's local attention; head2seq back."""
    w = synthetic.WORKLOADS[wname]
    P, S_l, H, D = w.P, w.S_local, w.H, w.D
    say(f"{w.name}: generating inputs")
    q, k, v = synthetic.make_qkv(w)
    shards = [x.view(P, 1, S_l, H, D).to(DEV) for x in (q, k, v)]
    say(f"{w.name}: seq2head x3")
    qh, kh, vh = (cp.ulysses_seq2head(x, P) for x in shards)
    torch.cuda.synchronize()
    say(f"{w.name}: seq2head vs oracle (Q)")
    want = oracle.seq2head(q.view(torch.int16).numpy().reshape(P, 1, S_l, H, D), P)
    assert np.array_equal(qh.cpu().view(torch.int16).numpy(), want)
    del want
    say(f"{w.name}: rank 0 attention (causal={w.causal})")
    o, lse = cp.attn_chunk_partial(qh[0], kh[0], vh[0], causal=w.causal, out_dtype=torch.bfloat16)
    say(f"{w.name}: head2seq")
    back = cp.ulysses_head2seq(kh, P)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), shards[1].view(torch.int16))
    del back, shards
    rows = _rows(w.S, n_edge, n_rand, seed=w.seed)
    say(f"{w.name}: oracle on {len(rows)} rows x {w.H_local} heads")
    heads = slice(0, w.H_local)
    qf = to_f64(q[:, rows][:, :, heads])
    wo, wl = oracle.attention(qf, to_f64(k[:, :, heads]), to_f64(v[:, :, heads]),
                              1 / math.sqrt(D), w.causal, q_pos=rows, k_pos=np.arange(w.S))
    got_o = o[:, torch.from_numpy(rows).to(DEV)]
    got_l = lse[:, :, torch.from_numpy(rows).to(DEV)]
    check_o(got_o, wo, "bf16", "rank 0 O (sampled rows)")
    check_lse(got_l, wl, "rank 0 LSE (sampled rows)")


def test_llm_128k_causal_ring8_rank7():
    """The 128K causal sequence split as a ring of 8 instead: rank 7 (query
    rows 114688-131071, all 32 heads) over the 8 key chunks in ring order
    7, 6, ..., 0, one ring call (the chunk-list ping-pong kernel); sampled rows
    against the oracle over every key up to the row's position."""
    w = synthetic.LLM_ULYSSES
    P, D = w.P, w.D
    S_l = w.S // P
    say(f"{w.name} as a ring of {P}, rank {P - 1}: generating inputs")
    q, k, v = synthetic.make_qkv(w)
    r = P - 1
    kd, vd = k.to(DEV), v.to(DEV)
    chunks = [(kd[:, c * S_l:(c + 1) * S_l].contiguous(), vd[:, c * S_l:(c + 1) * S_l].contiguous(),
               c * S_l) for c in range(r, -1, -1)]
    del kd, vd
    say(f"ring rank {r}: attention")
    o, lse = cp.ring_attention(q[:, r * S_l:(r + 1) * S_l].contiguous().to(DEV), chunks, causal=True,
                               q_pos0=r * S_l)
    torch.cuda.synchronize()
    del chunks
    rows = _rows(S_l, 8, 24, seed=w.seed + 7)
    say(f"ring rank {r}: oracle on {len(rows)} rows x {w.H} heads")
    pos = r * S_l + rows
    wo, wl = oracle.attention(to_f64(q[:, pos]), to_f64(k), to_f64(v), 1 / math.sqrt(D), True,
                              q_pos=pos, k_pos=np.arange(w.S))
    idx = torch.from_numpy(rows).to(DEV)
    check_o(o[:, idx], wo, "bf16", f"ring rank {r} O (sampled rows)")
    check_lse(lse[:, :, idx], wl, f"ring rank {r} LSE (sampled rows)")


def test_ulysses_anything_flux1008_rank0():
    """FLUX 1008x1008 (4481 tokens) over a Ulysses degree of 4: uneven sequence
    shards 1121/1120/1120/1120. The packed shards of a batch-1 sequence are the
    full tensor itself; rank 0's head group is the first slice of the output."""
    w = synthetic.FLUX_ANYTHING
    s_lens, h_counts = list(w.chunk_lens), list(w.head_counts)
    S, H, D = w.S, w.H, w.D
    say(f"{w.name}: generating inputs")
    q, k, v = synthetic.make_qkv(w)
    say(f"{w.name}: anything seq2head x3")
    qh, kh, vh = (cp.ulysses_anything_seq2head(x.to(DEV).reshape(-1), s_lens, h_counts, 1, D)
                  for x in (q, k, v))
    torch.cuda.synchronize()
    shards = []
    for s0, n in zip(w.chunk_starts(), s_lens):
        shards.append(q[:, s0:s0 + n].contiguous().view(torch.int16).numpy())
    want = np.concatenate([g.ravel() for g in oracle.anything_seq2head(shards, h_counts)])
    assert np.array_equal(qh.cpu().view(torch.int16).numpy(), want)
    del want, shards
    n0 = S * h_counts[0] * D
    say(f"{w.name}: rank 0 attention over {h_counts[0]} heads")
    o, lse = cp.attn_chunk_partial(qh[:n0].view(1, S, h_counts[0], D), kh[:n0].view(1, S, h_counts[0], D),
                                   vh[:n0].view(1, S, h_counts[0], D), out_dtype=torch.bfloat16)
    say(f"{w.name}: anything head2seq")
    back = cp.ulysses_anything_head2seq(kh, s_lens, h_counts, 1, D)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16).cpu(), k.reshape(-1).view(torch.int16))
    rows = _rows(S, 64, 192, seed=w.seed)
    heads = slice(0, h_counts[0])
    say(f"{w.name}: oracle on {len(rows)} rows x {h_counts[0]} heads")
    wo, wl = oracle.attention(to_f64(q[:, rows][:, :, heads]), to_f64(k[:, :, heads]),
                              to_f64(v[:, :, heads]), 1 / math.sqrt(D))
    idx = torch.from_numpy(rows).to(DEV)
    check_o(o[:, idx], wo, "bf16", "rank 0 O (sampled rows)")
    check_lse(lse[:, :, idx], wl, "rank 0 LSE (sampled rows)")


def test_kv_gather_wan_rank0():
    """Wan 21x30x52 with a K/V-gather degree of 4: rank 0 keeps its 8190 query
    rows and attends to the K/V gathered from all shards. Computed both from
    the gathered tensors and from the shards in place (ring call); each is
    checked against the oracle on sampled rows."""
    w = synthetic.WAN_KV_GATHER
    S, H, D, lens = w.S, w.H, w.D, list(w.chunk_lens)
    say(f"{w.name}: generating inputs")
    q, k, v = synthetic.make_qkv(w)
    kd, vd = k.to(DEV), v.to(DEV)
    say(f"{w.name}: gather K and V")
    kg = cp.kv_gather(kd.reshape(-1), lens, 1, H, D)
    vg = cp.kv_gather(vd.reshape(-1), lens, 1, H, D)
    torch.cuda.synchronize()
    assert torch.equal(kg.view(torch.int16), kd.view(torch.int16))
    n0 = lens[0]
    q0 = q[:, :n0].contiguous().to(DEV)
    say(f"{w.name}: rank 0 attention over the gathered K/V")
    o1, l1 = cp.attn_chunk_partial(q0, kg, vg, out_dtype=torch.bfloat16)
    say(f"{w.name}: rank 0 attention over the shards in place")
    shards = [(kd[:, s:s + n].contiguous(), vd[:, s:s + n].contiguous(), s)
              for s, n in zip(w.chunk_starts(), lens)]
    o2, l2 = cp.ring_attention(q0, shards)
    torch.cuda.synchronize()
    rows = _rows(n0, 32, 96, seed=w.seed)
    say(f"{w.name}: oracle on {len(rows)} rows x {H} heads")
    wo, wl = oracle.attention(to_f64(q[:, rows]), to_f64(k), to_f64(v), 1 / math.sqrt(D))
    idx = torch.from_numpy(rows).to(DEV)
    for o, lse, tag in ((o1, l1, "gathered"), (o2, l2, "shards")):
        check_o(o[:, idx], wo, "bf16", f"rank 0 O ({tag})")
        check_lse(lse[:, :, idx], wl, f"rank 0 LSE ({tag})")


def test_unified_flux_both_segments():
    """FLUX 1024x1024 as Ulysses 2 x ring 2. Ring segment r (2304 tokens) is
    spread over U = 2 Ulysses ranks; within the segment the Ulysses regrouping
    gives each rank all 2304 tokens for 12 heads, ring attention runs over
    both segments' K/V for those heads, and the inverse regrouping returns
    every rank its own 1152 tokens for all 24 heads. Checked for all four
    ranks (both ranks of both segments): O after the inverse regrouping and
    each rank's LSE, against the oracle on sampled rows."""
    w = synthetic.FLUX_UNIFIED
    R = len(w.chunk_lens)
    U = w.P // R
    S, H, D, seg = w.S, w.H, w.D, w.chunk_lens[0]
    sub, Hu = seg // U, H // U
    say(f"{w.name}: generating inputs")
    q, k, v = synthetic.make_qkv(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    # per segment: [U][1][sub][H][D] sub-shards -> [U][1][seg][H/U][D] head groups
    say(f"{w.name}: Ulysses regrouping inside each segment")
    grp = {}
    for name, x in (("q", qd), ("k", kd), ("v", vd)):
        grp[name] = [cp.ulysses_seq2head(x[:, r * seg:(r + 1) * seg].reshape(U, 1, sub, H, D), U)
                     for r in range(R)]
    rows = _rows(seg, 32, 96, seed=w.seed)
    say(f"{w.name}: oracle on {len(rows)} rows of each segment x {H} heads")
    for r in range(R):
        outs, lses = [], []
        for u in range(U):
            chunks = [(grp["k"][c][u], grp["v"][c][u], c * seg) for c in range(R)]
            say(f"{w.name}: ring attention for rank (ring {r}, ulysses {u})")
            o, lse = cp.ring_attention(grp["q"][r][u].contiguous(),
                                       [chunks[c] for c in synthetic.ring_order(r, R)])
            outs.append(o)
            lses.append(lse)
        back = cp.ulysses_head2seq(torch.stack(outs), U)          # [U][1][sub][H][D]
        torch.cuda.synchronize()
        got = torch.cat([back[u] for u in range(U)], dim=1)        # segment r's tokens
        wo, wl = oracle.attention(to_f64(q[:, r * seg + rows]), to_f64(k), to_f64(v),
                                  1 / math.sqrt(D))
        check_o(got[:, torch.from_numpy(rows).to(DEV)], wo, "bf16",
                f"segment {r} O (sampled rows)")
        for u in range(U):
            check_lse(lses[u][:, :, torch.from_numpy(rows).to(DEV)],
                      wl[:, u * Hu:(u + 1) * Hu], f"segment {r} rank {u} LSE")
