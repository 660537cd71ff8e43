"""GPU parity of the key-contiguous V path: cp_ulysses_seq2head_vt (bit-exact
against the oracle's index permutation) and cp_attn_chunk_partial_vt (O and
LSE bit-identical to cp_attn_chunk_partial on the same values, and within the
bf16 bars of the fp64 oracle), on every launch plan of the attention call:
two-group blocks (small grids), ping-pong blocks (large grids, causal and
not) and the non-causal last-round plan; ragged query and key tails, two
batches, causal offsets, fp32 and bf16 outputs.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests._parity import check_lse, check_o, check_o_scaled, say, to_f64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import context_attention_dit_amd as cp
DEV = "cuda:0"


def _vt_of(v: torch.Tensor) -> torch.Tensor:
    """[B][S][H][D] -> [B][H][ceil(S/64)][D][64], zero padding (test-side
    marshalling of the same values)."""
    B, S, H, D = v.shape
    nt = (S + 63) // 64
    pad = torch.zeros((B, nt * 64, H, D), dtype=v.dtype, device=v.device)
    pad[:, :S] = v
    return pad.view(B, nt, 64, H, D).permute(0, 3, 1, 4, 2).contiguous()


@pytest.mark.parametrize("P,B,S_l,H,D", [(2, 1, 5, 4, 128), (3, 2, 5, 6, 128), (4, 2, 67, 8, 128),
                                         (8, 1, 4095, 40, 128), (1, 1, 130, 2, 128),
                                         (2, 1, 128, 2, 128), (8, 1, 2048, 32, 128)])
def test_seq2head_vt_bit_exact(P, B, S_l, H, D):
    say(f"seq2head_vt P={P} B={B} S_l={S_l} H={H} D={D}")
    bits = synthetic.random_bits((P, B, S_l, H, D), 2, seed=700 + S_l)
    x = bits.view(torch.bfloat16).to(DEV)
    y = cp.ulysses_seq2head_vt(x, P)
    torch.cuda.synchronize()
    want = oracle.seq2head_vt(bits.numpy(), P)
    assert np.array_equal(y.cpu().view(torch.int16).numpy(), want)


def test_seq2head_vt_leaves_out_untouched_beyond_its_extent():
    """Ragged token count (T = 15): the one tile is written whole (zeros past T),
    nothing after it."""
    P, B, S_l, H, D = 3, 1, 5, 3, 128
    bits = synthetic.random_bits((P, B, S_l, H, D), 2, seed=711)
    n = P * B * (H // P) * 1 * D * 64
    buf = torch.full((n + 64,), -1, dtype=torch.int16, device=DEV)
    out = buf[:n].view(torch.bfloat16).view(P, B, H // P, 1, D, 64)
    cp.ulysses_seq2head_vt(bits.view(torch.bfloat16).to(DEV), P, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().view(torch.int16).numpy(), oracle.seq2head_vt(bits.numpy(), P))
    assert torch.all(buf[n:] == -1)


# (B, H, Sq, Skv, causal, q_pos0, kv_pos0): two-group grids, ping-pong grids,
# the non-causal last-round plan (320 blocks of 256 rows: 64 in the last round)
PLANS = [
    (1, 2, 300, 1001, False, 0, 0),        # two-group blocks, ragged query and key tails
    (2, 3, 129, 520, True, 0, 0),          # two-group, two batches, causal
    (1, 2, 200, 1016, True, 900, 0),       # causal offsets: every row sees >= 901 keys
    (1, 2, 200, 1016, True, 0, 100),       # causal offsets: rows 0..99 see no key
    (1, 16, 1100, 1107, False, 0, 0),      # ping-pong blocks, ragged
    (1, 4, 2056, 2056, True, 0, 0),        # ping-pong, causal
    (1, 10, 8192, 264, False, 0, 0),       # last-round plan: 320 units
    (1, 3, 64, 0, False, 0, 0),            # empty chunk
]


@pytest.mark.parametrize("B,H,Sq,Skv,causal,q0,k0", PLANS)
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_chunk_partial_vt_matches_bshd_call_bitwise(B, H, Sq, Skv, causal, q0, k0, out_dtype):
    D = 128
    say(f"chunk_partial_vt B={B} H={H} Sq={Sq} Skv={Skv} causal={causal} q0={q0} k0={k0} "
        f"out={out_dtype}")
    q = synthetic.make_tensor((B, Sq, H, D), torch.bfloat16, 820).to(DEV)
    k = synthetic.make_tensor((B, Skv, H, D), torch.bfloat16, 821).to(DEV)
    v = synthetic.make_tensor((B, Skv, H, D), torch.bfloat16, 822).to(DEV)
    vt = _vt_of(v)
    kw = dict(causal=causal, q_pos0=q0, kv_pos0=k0, out_dtype=out_dtype)
    o1, l1 = cp.attn_chunk_partial(q, k, v, **kw)
    o2, l2 = cp.attn_chunk_partial_vt(q, k, vt, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.uint8), o2.view(torch.uint8)), "O bits differ"
    assert torch.equal(l1.view(torch.uint8), l2.view(torch.uint8)), "LSE bits differ"
    if Sq * Skv * H * B <= 2_000_000:   # small enough for the oracle on every row
        want_o, want_l = oracle.chunk_partial(to_f64(q), to_f64(k), to_f64(v), 1 / np.sqrt(D),
                                              causal, np.arange(q0, q0 + Sq),
                                              np.arange(k0, k0 + Skv))
        check_o_scaled(o2, want_o)
        check_lse(l2, want_l)


def test_ulysses_rank_through_vt_path_against_oracle():
    """A whole Ulysses rank step on the key-contiguous path: Q and K regrouped by
    cp_ulysses_seq2head_n, V by cp_ulysses_seq2head_vt, rank p's attention by
    cp_attn_chunk_partial_vt, O back by cp_ulysses_head2seq; every rank, every
    row against the oracle's full attention."""
    P, B, S_l, H, D = 4, 1, 96, 8, 128
    say(f"ulysses vt step P={P} S_l={S_l} H={H}")
    qkv = [synthetic.make_tensor((P, B, S_l, H, D), torch.bfloat16, 840 + t) for t in range(3)]
    g = [x.to(DEV) for x in qkv]
    qk = cp.ulysses_seq2head(torch.stack(g[:2]), P)       # [2][P][B][S][H_l][D]
    vt = cp.ulysses_seq2head_vt(g[2], P)                  # [P][B][H_l][tiles][D][64]
    o = torch.empty((P, B, P * S_l, H // P, D), dtype=torch.bfloat16, device=DEV)
    for p in range(P):
        cp.attn_chunk_partial_vt(qk[0, p], qk[1, p], vt[p], o[p], out_dtype=torch.bfloat16)
    back = cp.ulysses_head2seq(o, P)                      # [P][B][S_l][H][D]
    torch.cuda.synchronize()
    full = [to_f64(x).transpose(1, 0, 2, 3, 4).reshape(B, P * S_l, H, D) for x in qkv]
    want, _ = oracle.chunk_partial(full[0], full[1], full[2], 1 / np.sqrt(D))
    got = to_f64(back).transpose(1, 0, 2, 3, 4).reshape(B, P * S_l, H, D)
    err = np.abs(got - want)
    assert err.max() <= 1e-2 and err.mean() <= 1e-3, (err.max(), err.mean())


@pytest.mark.parametrize("wname,n_edge,n_rand", [
    ("qwen-image-1536-ulysses4-rank0", 64, 128),
    ("wan-21x30x52-ulysses8-rank0", 48, 96),
    ("llm-128k-causal-ulysses8-rank0", 48, 80),
])
def test_ulysses_rank0_full_size_vt(wname, n_edge, n_rand):
    """The benchmark's path at full size: V of all ranks regrouped key-contiguous
    (bit-exact against the oracle on rank 0's group), rank 0's attention through
    cp_attn_chunk_partial_vt, equal bit for bit to the token-major call, and
    sampled rows against the oracle."""
    from tests.test_gpu_workloads import _rows
    import math
    w = synthetic.WORKLOADS[wname]
    P, S_l, H, D = w.P, w.S_local, w.H, w.D
    say(f"{w.name}: generating inputs")
    q, k, v = synthetic.make_qkv(w)
    shards = [x.view(P, 1, S_l, H, D).to(DEV) for x in (q, k, v)]
    say(f"{w.name}: seq2head (Q, K), seq2head_vt (V)")
    qk = cp.ulysses_seq2head(torch.stack(shards[:2]), P)
    vt = cp.ulysses_seq2head_vt(shards[2], P)
    vh = cp.ulysses_seq2head(shards[2], P)
    torch.cuda.synchronize()
    say(f"{w.name}: seq2head_vt vs oracle (rank 0's group)")
    want = oracle.seq2head_vt(v.view(torch.int16).numpy().reshape(P, 1, S_l, H, D), P)
    assert np.array_equal(vt[0].cpu().view(torch.int16).numpy(), want[0])
    del want, shards
    say(f"{w.name}: rank 0 attention, both V layouts (causal={w.causal})")
    o, lse = cp.attn_chunk_partial_vt(qk[0, 0], qk[1, 0], vt[0], causal=w.causal,
                                      out_dtype=torch.bfloat16)
    o2, lse2 = cp.attn_chunk_partial(qk[0, 0], qk[1, 0], vh[0], causal=w.causal,
                                     out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), "O bits differ"
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32)), "LSE bits differ"
    del o2, lse2, vh, vt, qk
    rows = _rows(w.S, n_edge, n_rand, seed=w.seed)
    say(f"{w.name}: oracle on {len(rows)} rows x {w.H_local} heads")
    heads = slice(0, w.H_local)
    wo, wl = oracle.attention(to_f64(q[:, rows][:, :, heads]), to_f64(k[:, :, heads]),
                              to_f64(v[:, :, heads]), 1 / math.sqrt(D), w.causal, q_pos=rows,
                              k_pos=np.arange(w.S))
    idx = torch.from_numpy(rows).to(DEV)
    check_o(o[:, idx], wo, "bf16", "rank 0 O (sampled rows)")
    check_lse(lse[:, :, idx], wl, "rank 0 LSE (sampled rows)")


@pytest.mark.parametrize("P,B,S_l,H", [(4, 1, 8190, 40), (3, 2, 37, 5), (1, 1, 64, 2)])
def test_kv_gather_vt_bit_exact_and_attention(P, B, S_l, H):
    """The gathered V, key-contiguous, bit for bit against the oracle; a Q shard's
    attention over the gathered K and V equal bit for bit through both layouts."""
    D = 128
    say(f"kv_gather_vt P={P} B={B} S_l={S_l} H={H}")
    bits = synthetic.random_bits((P, B, S_l, H, D), 2, seed=900 + S_l)
    y = cp.kv_gather_vt(bits.view(torch.bfloat16).to(DEV))
    torch.cuda.synchronize()
    want = oracle.kv_gather_vt([bits[q].numpy() for q in range(P)])
    assert np.array_equal(y.cpu().view(torch.int16).numpy(), want)
    Sq = min(S_l, 600)
    q = synthetic.make_tensor((B, Sq, H, D), torch.bfloat16, 910).to(DEV)
    kv = [synthetic.make_tensor((P, B, S_l, H, D), torch.bfloat16, 911 + t).to(DEV)
          for t in range(2)]
    k_full, v_full = (cp.kv_gather(x.reshape(-1), [S_l] * P, B, H, D) for x in kv)
    vt = cp.kv_gather_vt(kv[1])
    o1, l1 = cp.attn_chunk_partial(q, k_full, v_full, out_dtype=torch.bfloat16)
    o2, l2 = cp.attn_chunk_partial_vt(q, k_full, vt, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
