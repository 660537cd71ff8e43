"""GPU parity on seeded random shapes: forward ring, per-hop partials + merge,
and ring backward, against the fp64 oracle.

Each case draws B, H, D in {64, 128}, ragged Sq and a key length split into a
random number of chunks (empty chunks allowed), causal or not, with random
query and key position offsets and a random ring visit order; about half the
cases run the backward with both accumulate flags into pre-filled buffers. The
draws are seeded, so every run checks the same cases.

Tolerances: LSE max-abs 1e-4, gradients as in the other backward tests. The
per-hop fp32 partials (cp_attn_chunk_partial, no final rounding) are held to
the absolute bars, max-abs 1e-2 and mean-abs 1e-3. For bf16 outputs: max-abs <= 1e-2 * max(1, max|ref|) and
mean-abs <= max(1e-3, 2^-8 * mean|ref|). With only a few visible keys O is
close to single value rows (|O| up to ~4), and bf16 itself rounds such values
by up to 2^-8 of their size (half a bf16 step is 0.0078 at |O| = 2; about a
quarter step on average), before the 2^-8 rounding of P. The absolute bars
(1e-2, 1e-3) hold for outputs well below 1, which is what averages over many
keys give, as in every workload.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests._parity import check_lse, check_o, check_o_scaled, say, to_f64
from tests.test_gpu_backward import check_grad

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import context_attention_dit_amd as cp
DEV = "cuda:0"

N_CASES = 64
# mean-abs bar relative to mean|ref|: 2^-8 (the sweep measures at most ~2^-8.8,
# about the mean bf16 rounding of O plus that of P), so a systematic bias of
# 0.4% or more fails
MEAN_REL = 2.0 ** -8


def _case(seed):
    rng = np.random.default_rng(10_000 + seed)
    B = int(rng.integers(1, 3))
    H = int(rng.integers(1, 5))
    D = int(rng.choice([64, 128]))
    Sq = int(rng.integers(1, 300))
    Skv = int(rng.integers(1, 400))
    P = int(rng.integers(1, 6))
    causal = bool(rng.integers(0, 2))
    cuts = np.sort(rng.integers(0, Skv + 1, size=P - 1))
    lens = tuple(int(x) for x in np.diff(np.concatenate([[0], cuts, [Skv]])))
    q_pos0 = int(rng.integers(0, Skv + 64)) if causal else 0
    kv_pos0 = int(rng.integers(0, 32)) if causal else 0
    order = [int(x) for x in rng.permutation(P)]
    accumulate = bool(rng.integers(0, 2))   # backward adds into pre-filled buffers
    return B, H, D, Sq, lens, causal, q_pos0, kv_pos0, order, accumulate


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape_forward_and_backward(seed):
    B, H, D, Sq, lens, causal, q_pos0, kv_pos0, order, accumulate = _case(seed)
    Skv = sum(lens)
    say(f"random case {seed}: B={B} H={H} D={D} Sq={Sq} lens={lens} causal={causal} "
        f"q_pos0={q_pos0} kv_pos0={kv_pos0} order={order} accumulate={accumulate}")
    bf = torch.bfloat16
    q = synthetic.make_tensor((B, Sq, H, D), bf, 20_000 + 4 * seed)
    k = synthetic.make_tensor((B, Skv, H, D), bf, 20_001 + 4 * seed)
    v = synthetic.make_tensor((B, Skv, H, D), bf, 20_002 + 4 * seed)
    do = synthetic.make_tensor((B, Sq, H, D), bf, 20_003 + 4 * seed)
    q64, k64, v64, do64 = (to_f64(x) for x in (q, k, v, do))
    scale = 1 / math.sqrt(D)
    q_pos = np.arange(q_pos0, q_pos0 + Sq)
    k_pos = np.arange(kv_pos0, kv_pos0 + Skv)
    wo, wl = oracle.attention(q64, k64, v64, scale, causal, q_pos, k_pos)

    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(int)
    kd, vd = k.to(DEV), v.to(DEV)
    chunks = [(kd[:, s:s + m].contiguous(), vd[:, s:s + m].contiguous(), kv_pos0 + int(s))
              for s, m in zip(starts, lens)]
    visit = [chunks[c] for c in order]
    qd, dod = q.to(DEV), do.to(DEV)
    o, lse = cp.ring_attention(qd, visit, causal=causal, q_pos0=q_pos0)
    parts = [cp.attn_chunk_partial(qd, kc, vc, causal=causal, q_pos0=q_pos0, kv_pos0=p0)
             for kc, vc, p0 in visit]
    mo, ml = cp.lse_merge(torch.stack([p[0] for p in parts]), torch.stack([p[1] for p in parts]),
                          out_dtype=bf)
    torch.cuda.synchronize()
    check_o_scaled(o, wo, "ring O", mean_rel=MEAN_REL)
    check_lse(lse, wl, "ring LSE")
    check_o_scaled(mo, wo, "partials + merge O", mean_rel=MEAN_REL)
    check_lse(ml, wl, "partials + merge LSE")
    # each hop's fp32 partial (no final bf16 rounding) at the absolute bars
    for (kc, vc, p0), (po, pl) in zip(visit, parts):
        n = kc.shape[1]
        cwo, cwl = oracle.chunk_partial(q64, to_f64(kc), to_f64(vc), scale, causal, q_pos,
                                        np.arange(p0, p0 + n))
        check_o(po, cwo, "bf16", f"chunk at {p0} (+{n}) fp32 partial O")
        check_lse(pl, cwl, f"chunk at {p0} (+{n}) LSE")
    err = np.abs(to_f64(o) - wo)
    say(f"  ring O mean-abs / mean|ref| = {err.mean() / max(np.abs(wo).mean(), 1e-30):.2e}")

    # backward of the same rank from the oracle's saved statistics
    o_bf = torch.tensor(wo, dtype=torch.float32).to(bf).to(DEV)
    delta = cp.attn_backward_delta(o_bf, dod)
    f32 = torch.float32
    if accumulate:
        # running sums from earlier ranks or chunks, 0.1 N(0, 1): the call must add to
        # them (a skipped addition would leave an error ~0.1, far above the bars), and
        # the fp32 rounding of the sum stays ~1e-8, below the bars of small gradients
        gen = torch.Generator().manual_seed(30_000 + seed)
        pre_q = (0.1 * torch.randn((B, Sq, H, D), generator=gen)).to(DEV)
        pre_kv = [((0.1 * torch.randn(kc.shape, generator=gen)).to(DEV),
                   (0.1 * torch.randn(kc.shape, generator=gen)).to(DEV)) for kc, _, _ in visit]
        dq_in, grads_in = pre_q.clone(), [(a.clone(), b.clone()) for a, b in pre_kv]
    else:
        dq_in, grads_in = None, None
    dq, grads = cp.ring_attention_backward(qd, visit, dod,
                                           torch.tensor(wl, dtype=f32).to(DEV), delta,
                                           dq_in, grads_in, causal=causal, q_pos0=q_pos0,
                                           accumulate_dq=accumulate, accumulate_dkv=accumulate)
    torch.cuda.synchronize()
    if accumulate:   # the call's share, the prefill taken off exactly (in fp64)
        dq = dq.double() - pre_q.double()
        grads = [(a.double() - pa.double(), b.double() - pb.double())
                 for (a, b), (pa, pb) in zip(grads, pre_kv)]
    # the kernel's contract: gradients for the Delta of the O it is given (the
    # oracle's O rounded to bf16, as stored); with few keys O is not small and
    # that rounding alone moves Delta by more than the kernel's own arithmetic
    wq, wk, wv = oracle.chunk_grad(q64, k64, v64, do64, wl,
                                   oracle.backward_delta(to_f64(o_bf), do64), scale, causal,
                                   q_pos, k_pos)
    check_grad(dq, wq, "dQ")
    got_k = torch.cat([grads[order.index(c)][0] for c in range(len(lens))], dim=1)
    got_v = torch.cat([grads[order.index(c)][1] for c in range(len(lens))], dim=1)
    check_grad(got_k, wk, "dK")
    check_grad(got_v, wv, "dV")
