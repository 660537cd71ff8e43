"""GPU parity of the attention backward at the workloads' full sizes, in the
launch configuration the benchmark times.

* FLUX 1024x1024 ring rank 0: Delta, then one cp_attn_chunk_backward per chunk
  in ring order [0, 3, 2, 1] with dQ accumulated; every head, every output is
  compared with the fp64 oracle. The saved O (rounded to bf16) and LSE are the
  oracle's own forward.
* The whole FLUX ring, all 4 ranks: each rank's forward (cp_ring_attention)
  and backward (cp_ring_attention_backward, its chunks in its ring order), the
  dK/dV shares accumulated across ranks into each chunk owner's buffers. The
  summed gradients of two sampled heads are compared with the oracle's full
  backward (attention_grad, from Q, K, V and dO alone), causal and not.
* Wan and the 128K causal LLM Ulysses ranks: one call over the whole
  sequence. The oracle cannot afford every row's forward statistics there, so
  the kernel is fed the oracle's exact LSE and Delta for a sample of query rows
  (first rows, last rows, seeded random rows) and, for every other row, the
  stand-in LSE = ln(visible keys) + 1/2 (the expected log-normaliser of N(0,1)
  logits) with Delta = 0. Sampled dQ rows depend only on their own statistics
  and are true gradients; dK and dV of a sample of keys are compared with the
  oracle's chunk_grad evaluated on exactly the same inputs, summing over all
  query rows.
Tolerance as in test_gpu_backward.py.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests._parity import say, to_f64
from tests.test_gpu_backward import check_grad

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import context_attention_dit_amd as cp
DEV = "cuda:0"


def _sample(S, n_edge, n_rand, seed):
    rng = np.random.default_rng(seed)
    r = set(range(min(n_edge, S))) | set(range(max(0, S - n_edge), S))
    r |= set(rng.choice(S, size=min(n_rand, S), replace=False).tolist())
    return np.array(sorted(r))


def _f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a bf16 tensor (every bf16 value is an fp32 value)."""
    return t.detach().cpu().to(torch.float32).to(torch.float64).numpy()


def test_flux_ring_rank0_backward_full():
    w = synthetic.FLUX_RING
    say(f"{w.name} backward: inputs")
    q, k, v = synthetic.make_qkv(w)
    n, H, D = w.chunk_lens[0], w.H, w.D
    scale = 1 / math.sqrt(D)
    q0 = q[:, :n].contiguous()
    do = synthetic.make_tensor((1, n, H, D), torch.bfloat16, 1077)
    q64, k64, v64, do64 = _f64(q0), _f64(k), _f64(v), _f64(do)
    say(f"{w.name} backward: oracle forward")
    o, lse = oracle.attention(q64, k64, v64, scale)
    delta = oracle.backward_delta(o, do64)
    o_bf = torch.tensor(o, dtype=torch.float32).to(torch.bfloat16).to(DEV)
    lse_d = torch.tensor(lse, dtype=torch.float32).to(DEV)
    starts = w.chunk_starts()
    order = synthetic.ring_order(0, w.P)
    kd, vd = k.to(DEV), v.to(DEV)
    chunks = [(kd[:, s:s + m].contiguous(), vd[:, s:s + m].contiguous(), s)
              for s, m in zip(starts, w.chunk_lens)]
    say(f"{w.name} backward: GPU, chunks in order {order}")
    qd, dod = q0.to(DEV), do.to(DEV)
    delta_d = cp.attn_backward_delta(o_bf, dod)
    dq = torch.empty((1, n, H, D), dtype=torch.float32, device=DEV)
    grads = {}
    for step, c in enumerate(order):
        kc, vc, s0 = chunks[c]
        grads[c] = cp.attn_chunk_backward(qd, kc, vc, dod, lse_d, delta_d, dq, scale=scale,
                                          kv_pos0=s0, accumulate_dq=step > 0)[1:]
    torch.cuda.synchronize()
    say(f"{w.name} backward: oracle gradients")
    want_dq = np.zeros_like(q64)
    for c in order:
        s0, m = starts[c], w.chunk_lens[c]
        gq, gk, gv = oracle.chunk_grad(q64, k64[:, s0:s0 + m], v64[:, s0:s0 + m], do64, lse,
                                       delta, scale, False, None, np.arange(s0, s0 + m))
        want_dq += gq
        check_grad(grads[c][0], gk, f"dK chunk {c}")
        check_grad(grads[c][1], gv, f"dV chunk {c}")
    check_grad(dq, want_dq, "dQ")


@pytest.mark.parametrize("causal", [False, True])
def test_flux_ring_all_ranks_backward_accumulated(causal):
    w = synthetic.FLUX_RING
    say(f"{w.name}: every rank's forward and backward, causal={causal}")
    q, k, v = synthetic.make_qkv(w)
    H, D, P = w.H, w.D, w.P
    do = synthetic.make_tensor((1, w.S, H, D), torch.bfloat16, 1078)
    starts, lens = w.chunk_starts(), w.chunk_lens
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    chunks = [(kd[:, s:s + m].contiguous(), vd[:, s:s + m].contiguous(), s)
              for s, m in zip(starts, lens)]
    f32 = torch.float32
    acc = [(torch.zeros((1, m, H, D), dtype=f32, device=DEV),
            torch.zeros((1, m, H, D), dtype=f32, device=DEV)) for m in lens]
    dq = torch.empty((1, w.S, H, D), dtype=f32, device=DEV)
    for r in range(P):
        s0, m = starts[r], lens[r]
        order = synthetic.ring_order(r, P)
        visit = [chunks[c] for c in order]
        q_r, do_r = qd[:, s0:s0 + m].contiguous(), dod[:, s0:s0 + m].contiguous()
        o_r, lse_r = cp.ring_attention(q_r, visit, causal=causal, q_pos0=s0)
        delta_r = cp.attn_backward_delta(o_r, do_r)
        dq_r, _ = cp.ring_attention_backward(q_r, visit, do_r, lse_r, delta_r,
                                             grads=[acc[c] for c in order], causal=causal,
                                             q_pos0=s0, accumulate_dkv=True)
        dq[:, s0:s0 + m] = dq_r
    torch.cuda.synchronize()
    heads = [0, H - 1]
    say(f"{w.name}: oracle backward on heads {heads}")
    hs = torch.tensor(heads)
    q64, k64, v64, do64 = (_f64(x[:, :, hs]) for x in (q, k, v, do))
    wq, wk, wv = oracle.attention_grad(q64, k64, v64, do64, 1 / math.sqrt(D), causal)
    hd = hs.to(DEV)
    check_grad(dq[:, :, hd], wq, "dQ, all ranks")
    check_grad(torch.cat([a[0] for a in acc], dim=1)[:, :, hd], wk, "dK summed over ranks")
    check_grad(torch.cat([a[1] for a in acc], dim=1)[:, :, hd], wv, "dV summed over ranks")


@pytest.mark.parametrize("wname", [synthetic.WAN_ULYSSES.name, synthetic.LLM_ULYSSES.name])
def test_ulysses_rank_backward_sampled(wname):
    w = synthetic.WORKLOADS[wname]
    S, Hl, D, causal = w.S, w.H_local, w.D, w.causal
    scale = 1 / math.sqrt(D)
    say(f"{w.name} backward: inputs")
    q, k, v, do = (synthetic.make_tensor((1, S, Hl, D), torch.bfloat16, 1100 + t)
                   for t in range(4))
    q64, k64, v64, do64 = (_f64(x) for x in (q, k, v, do))
    pos = np.arange(S)
    rows = _sample(S, 3, 13, seed=S)
    say(f"{w.name} backward: oracle statistics of {len(rows)} rows")
    o_r, lse_r = oracle.attention(q64[:, rows], k64, v64, scale, causal, rows, pos)
    delta_r = oracle.backward_delta(o_r, do64[:, rows])
    visible = (pos + 1) if causal else np.full(S, S)
    lse = np.broadcast_to(np.log(visible) + 0.5, (1, Hl, S)).astype(np.float32).copy()
    delta = np.zeros((1, Hl, S), dtype=np.float32)
    lse[:, :, rows] = lse_r.astype(np.float32)
    delta[:, :, rows] = delta_r.astype(np.float32)
    say(f"{w.name} backward: GPU (one call over the whole sequence, causal={causal})")
    dq, dk, dv = cp.attn_chunk_backward(q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV),
                                        torch.from_numpy(lse).to(DEV),
                                        torch.from_numpy(delta).to(DEV), scale=scale,
                                        causal=causal)
    torch.cuda.synchronize()
    say(f"{w.name} backward: oracle dQ rows")
    lse64, delta64 = lse.astype(np.float64), delta.astype(np.float64)
    wq = oracle.chunk_grad(q64[:, rows], k64, v64, do64[:, rows], lse64[:, :, rows],
                           delta64[:, :, rows], scale, causal, rows, pos)[0]
    check_grad(dq[:, torch.from_numpy(rows).to(DEV)], wq, "dQ sampled rows")
    keys = _sample(S, 3, 13, seed=S + 1)
    say(f"{w.name} backward: oracle dK, dV of {len(keys)} keys over all {S} rows")
    _, wk, wv = oracle.chunk_grad(q64, k64[:, keys], v64[:, keys], do64, lse64, delta64, scale,
                                  causal, pos, keys)
    kt = torch.from_numpy(keys).to(DEV)
    check_grad(dk[:, kt], wk, "dK sampled keys")
    check_grad(dv[:, kt], wv, "dV sampled keys")
