"""GPU parity at the documented limits of the C ABI.

* Widest head stride: H*D = 2^24 (131072 heads of D = 128), the largest the
  entry points accept. A 64-row tile then spans 2^31 bytes, so any 32-bit
  overflow in the kernels' offset arithmetic would show in the last heads.
  The tensors are zero except for seeded inputs on a few heads at both ends of
  the head range; the oracle computes those heads (heads are independent).
* Most chunks: a ring of 64 chunks (CP_MAX_RING_CHUNKS), forward and backward.
* Longest chunk: 2^21 keys of 8 heads in one chunk (4 GiB per K or V, so a
  chunk's own offsets pass 2^31 bytes) and the same keys as a ring of two
  chunks, causal and not; the running fp32 sums cover 2^21 keys per row. The
  oracle computes two sampled heads (the others are zero).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests._parity import check_lse, check_o, say, to_f64
from tests.test_gpu_backward import check_grad

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import context_attention_dit_amd as cp
DEV = "cuda:0"


def test_widest_head_stride_forward_and_backward():
    D = 128
    H = (1 << 24) // D
    Sq, Skv = 130, 65           # two query tiles (the second ragged), one full + one ragged key tile
    heads = [0, 1, H // 2, H - 2, H - 1]
    say(f"max head stride: H={H} D={D} Sq={Sq} Skv={Skv}, sampled heads {heads}")
    scale = 1 / math.sqrt(D)
    bf = torch.bfloat16
    q = torch.zeros((1, Sq, H, D), dtype=bf, device=DEV)
    k = torch.zeros((1, Skv, H, D), dtype=bf, device=DEV)
    v = torch.zeros((1, Skv, H, D), dtype=bf, device=DEV)
    do = torch.zeros((1, Sq, H, D), dtype=bf, device=DEV)
    n = len(heads)
    src = [synthetic.make_tensor(shape, bf, 1500 + t) for t, shape in
           enumerate([(1, Sq, n, D), (1, Skv, n, D), (1, Skv, n, D), (1, Sq, n, D)])]
    hidx = torch.tensor(heads, device=DEV)
    for dst, s in zip((q, k, v, do), src):
        dst[:, :, hidx] = s.to(DEV)
    o, lse = cp.attn_chunk_partial(q, k, v, out_dtype=torch.bfloat16, causal=True)
    half = Skv // 2
    ro, rl = cp.ring_attention(q, [(k[:, half:].contiguous(), v[:, half:].contiguous(), half),
                                   (k[:, :half].contiguous(), v[:, :half].contiguous(), 0)],
                               causal=True)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = (to_f64(x) for x in src)
    wo, wl = oracle.attention(q64, k64, v64, scale, causal=True)
    check_o(o[:, :, hidx], wo, "bf16", "chunk O, sampled heads")
    check_lse(lse[:, hidx], wl, "chunk LSE, sampled heads")
    check_o(ro[:, :, hidx], wo, "bf16", "ring O, sampled heads")
    check_lse(rl[:, hidx], wl, "ring LSE, sampled heads")
    del ro, rl
    # backward from the oracle's saved statistics on the sampled heads (the
    # other heads' rows get LSE = ln(visible keys), Delta = 0: any finite input)
    lse_in = torch.log(torch.arange(1, Sq + 1, device=DEV, dtype=torch.float32).clamp(max=Skv))
    lse_in = lse_in.expand(1, H, Sq).contiguous()
    lse_in[:, hidx] = torch.tensor(wl, dtype=torch.float32, device=DEV)
    o_bf = torch.zeros_like(q)
    o_bf[:, :, hidx] = torch.tensor(wo, dtype=torch.float32).to(bf).to(DEV)
    delta = cp.attn_backward_delta(o_bf, do)
    del o_bf
    dq, dk, dv = cp.attn_chunk_backward(q, k, v, do, lse_in, delta, causal=True)
    torch.cuda.synchronize()
    wq, wk, wv = oracle.chunk_grad(q64, k64, v64, do64, wl, oracle.backward_delta(wo, do64),
                                   scale, causal=True)
    check_grad(dq[:, :, hidx], wq, "dQ, sampled heads")
    check_grad(dk[:, :, hidx], wk, "dK, sampled heads")
    check_grad(dv[:, :, hidx], wv, "dV, sampled heads")


def test_ring_of_64_chunks_forward_and_backward():
    P, H, D = 64, 2, 64
    lens = synthetic.random_splits(40 * P, P, seed=64, min_len=0)
    S = sum(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(int)
    say(f"ring of {P} chunks, S={S}, lens {min(lens)}..{max(lens)}")
    q, k, v, do = (synthetic.make_tensor((1, S, H, D), torch.bfloat16, 1600 + t)
                   for t in range(4))
    q64, k64, v64, do64 = (to_f64(x) for x in (q, k, v, do))
    scale = 1 / math.sqrt(D)
    r = 5
    q0, n = int(starts[r]), S - int(starts[r])  # the query shard: every row from chunk 5 on
    kd, vd = k.to(DEV), v.to(DEV)
    chunks = [(kd[:, s:s + m].contiguous(), vd[:, s:s + m].contiguous(), int(s))
              for s, m in zip(starts, lens)]
    order = synthetic.ring_order(r, P)
    qd, dod = q[:, q0:].contiguous().to(DEV), do[:, q0:].contiguous().to(DEV)
    o, lse = cp.ring_attention(qd, [chunks[c] for c in order], causal=True, q_pos0=q0)
    torch.cuda.synchronize()
    q_pos = np.arange(q0, S)
    wo, wl = oracle.attention(q64[:, q0:], k64, v64, scale, True, q_pos, np.arange(S))
    check_o(o, wo, "bf16", "ring O")
    check_lse(lse, wl, "ring LSE")
    o_bf = torch.tensor(wo, dtype=torch.float32).to(torch.bfloat16).to(DEV)
    delta = cp.attn_backward_delta(o_bf, dod)
    dq, grads = cp.ring_attention_backward(qd, [chunks[c] for c in order], dod,
                                           torch.tensor(wl, dtype=torch.float32).to(DEV), delta,
                                           causal=True, q_pos0=q0)
    torch.cuda.synchronize()
    wq, wk, wv = oracle.chunk_grad(q64[:, q0:], k64, v64, do64[:, q0:], wl,
                                   oracle.backward_delta(wo, do64[:, q0:]), scale, True, q_pos,
                                   np.arange(S))
    check_grad(dq, wq, "dQ")
    got_k = torch.cat([grads[order.index(c)][0] for c in range(P)], dim=1)
    got_v = torch.cat([grads[order.index(c)][1] for c in range(P)], dim=1)
    check_grad(got_k, wk, "dK")
    check_grad(got_v, wv, "dV")


def test_longest_chunk_forward_and_ring():
    D, H, Sq, Skv = 128, 8, 200, 1 << 21
    heads = [0, H - 1]
    n = len(heads)
    say(f"longest chunk: Skv={Skv} H={H} D={D} Sq={Sq}, sampled heads {heads}")
    bf = torch.bfloat16
    src = [synthetic.make_tensor(shape, bf, 1700 + t) for t, shape in
           enumerate([(1, Sq, n, D), (1, Skv, n, D), (1, Skv, n, D)])]
    hidx = torch.tensor(heads, device=DEV)
    q = torch.zeros((1, Sq, H, D), dtype=bf, device=DEV)
    k = torch.zeros((1, Skv, H, D), dtype=bf, device=DEV)
    v = torch.zeros((1, Skv, H, D), dtype=bf, device=DEV)
    for dst, x in zip((q, k, v), src):
        dst[:, :, hidx] = x.to(DEV)
    scale = 1 / math.sqrt(D)
    q64, k64, v64 = (to_f64(x) for x in src)
    # one chunk holding every key, non-causal
    o, lse = cp.attn_chunk_partial(q, k, v, out_dtype=bf)
    torch.cuda.synchronize()
    wo, wl = oracle.attention(q64, k64, v64, scale)
    check_o(o[:, :, hidx], wo, "bf16", "one chunk O, sampled heads")
    check_lse(lse[:, hidx], wl, "one chunk LSE, sampled heads")
    del o, lse
    # the same keys as a ring of two chunks, queries at the end of the sequence
    half = Skv // 2
    chunks = [(k[:, half:].contiguous(), v[:, half:].contiguous(), half),
              (k[:, :half].contiguous(), v[:, :half].contiguous(), 0)]
    del k, v
    q0 = Skv - Sq + 7          # row i sees keys 0 .. q0 + i; the last 7 rows see all of them
    for causal in (False, True):
        ro, rl = cp.ring_attention(q, chunks, causal=causal, q_pos0=q0)
        torch.cuda.synchronize()
        if causal:
            wo, wl = oracle.attention(q64, k64, v64, scale, True, np.arange(q0, q0 + Sq),
                                      np.arange(Skv))
        check_o(ro[:, :, hidx], wo, "bf16", f"ring O (causal={causal}), sampled heads")
        check_lse(rl[:, hidx], wl, f"ring LSE (causal={causal}), sampled heads")
        del ro, rl
