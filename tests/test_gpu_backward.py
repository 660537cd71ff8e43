"""GPU parity of the attention backward (cp_attn_backward_delta, cp_attn_chunk_backward).

Inputs: seeded bf16 Q, K, V and dO from ``synthetic``. The saved forward
statistics come from the fp64 oracle, never from the HIP path: O is the
oracle's output rounded to bf16 (what a training step stores) and LSE the
oracle's, rounded to fp32. Expected gradients are ``oracle.chunk_grad`` with
the exact fp64 LSE and Delta.

Tolerance (gradients are fp32 sums of bf16 products): the kernels round P and
dS to bf16 (unit roundoff u = 2^-8) before their products, as the forward does
for P. Each gradient element is a sum of random-sign terms, each perturbed by
at most u relative, so its error is about u/3 of its own size on average; a
CPU emulation of exactly these roundings gives mean|err| = 1.3e-3 * rms(ref)
and max|err| <= 3.3e-3 * max|ref| on these shapes. The bar:
  max|err| <= 1e-2 * max|ref|   and   mean|err| <= 3e-3 * rms(ref).
Delta is an fp32 dot product of D terms: max-abs 1e-5.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests._parity import F32_MAX, say, to_f64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import context_attention_dit_amd as cp
DEV = "cuda:0"

GRAD_MAX, GRAD_MEAN = 1e-2, 3e-3


def check_grad(got: torch.Tensor, want: np.ndarray, what: str) -> None:
    g = to_f64(got)
    assert g.shape == want.shape, (what, g.shape, want.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    err = np.abs(g - want)
    ref_max = np.abs(want).max()
    ref_rms = math.sqrt((want ** 2).mean())
    if ref_max == 0:
        assert err.max() == 0, f"{what}: expected exact zeros, max-abs {err.max():.3e}"
        return
    print(f"  {what}: max-abs/max|ref| {err.max() / ref_max:.2e}, "
          f"mean-abs/rms {err.mean() / ref_rms:.2e}", flush=True)
    assert err.max() <= GRAD_MAX * ref_max, \
        f"{what}: max-abs {err.max():.3e} > {GRAD_MAX} * {ref_max:.3e}"
    assert err.mean() <= GRAD_MEAN * ref_rms, \
        f"{what}: mean-abs {err.mean():.3e} > {GRAD_MEAN} * rms {ref_rms:.3e}"


def _inputs(B, Sq, Skv, H, D, seed):
    q = synthetic.make_tensor((B, Sq, H, D), torch.bfloat16, seed)
    k = synthetic.make_tensor((B, Skv, H, D), torch.bfloat16, seed + 1)
    v = synthetic.make_tensor((B, Skv, H, D), torch.bfloat16, seed + 2)
    do = synthetic.make_tensor((B, Sq, H, D), torch.bfloat16, seed + 3)
    return q, k, v, do


def _saved_stats(q64, k64, v64, do64, scale, causal, q_pos, k_pos):
    """Oracle forward: exact (O, LSE, Delta) and the stored bf16 O / fp32 LSE."""
    o, lse = oracle.attention(q64, k64, v64, scale, causal, q_pos, k_pos)
    delta = oracle.backward_delta(o, do64)
    o_bf = torch.tensor(o, dtype=torch.float32).to(torch.bfloat16)
    lse_f = torch.tensor(lse, dtype=torch.float32)
    return o, lse, delta, o_bf, lse_f


def _run(q, k, v, do, o_bf, lse_f, scale, causal, q_pos0, kv_pos0):
    dd = [x.to(DEV) for x in (q, k, v, do)]
    delta = cp.attn_backward_delta(o_bf.to(DEV), dd[3])
    dq, dk, dv = cp.attn_chunk_backward(*dd, lse_f.to(DEV), delta, scale=scale, causal=causal,
                                        q_pos0=q_pos0, kv_pos0=kv_pos0)
    torch.cuda.synchronize()
    return delta, dq, dk, dv


CASES = [
    # B, Sq, Skv, H, D, causal, q_pos0, kv_pos0
    (1, 200, 333, 2, 128, False, 0, 0),     # several tiles, ragged both ways
    (2, 130, 70, 3, 64, False, 0, 0),
    (1, 256, 256, 2, 128, True, 0, 0),      # diagonal tiles
    (1, 300, 190, 2, 64, True, 0, 0),       # Sq > Skv, causal
    (1, 150, 400, 2, 128, True, 250, 0),    # later query shard against earlier keys
    (2, 77, 129, 1, 128, True, 60, 0),      # partly masked rectangle
    (1, 33, 17, 4, 64, False, 0, 0),        # below one tile
    (1, 1, 1, 1, 128, False, 0, 0),         # one query, one key
]


@pytest.mark.parametrize("B,Sq,Skv,H,D,causal,q_pos0,kv_pos0", CASES)
def test_chunk_backward_matches_oracle(B, Sq, Skv, H, D, causal, q_pos0, kv_pos0):
    say(f"backward B={B} Sq={Sq} Skv={Skv} H={H} D={D} causal={causal} "
        f"q_pos0={q_pos0} kv_pos0={kv_pos0}")
    q, k, v, do = _inputs(B, Sq, Skv, H, D, seed=Sq * 7 + Skv)
    q64, k64, v64, do64 = (to_f64(x) for x in (q, k, v, do))
    scale = 1 / math.sqrt(D)
    q_pos, k_pos = np.arange(q_pos0, q_pos0 + Sq), np.arange(kv_pos0, kv_pos0 + Skv)
    o, lse, delta, o_bf, lse_f = _saved_stats(q64, k64, v64, do64, scale, causal, q_pos, k_pos)
    d_gpu, dq, dk, dv = _run(q, k, v, do, o_bf, lse_f, scale, causal, q_pos0, kv_pos0)
    want_delta = oracle.backward_delta(to_f64(o_bf), do64)
    assert np.abs(to_f64(d_gpu) - want_delta).max() <= F32_MAX
    wq, wk, wv = oracle.chunk_grad(q64, k64, v64, do64, lse, delta, scale, causal, q_pos, k_pos)
    check_grad(dq, wq, "dQ")
    check_grad(dk, wk, "dK")
    check_grad(dv, wv, "dV")


@pytest.mark.parametrize("scale,causal", [(-0.1, False), (-0.1, True), (0.0, True)])
def test_negative_and_zero_scale(scale, causal):
    say(f"backward scale={scale} causal={causal}")
    B, Sq, Skv, H, D = 1, 96, 160, 2, 128
    q, k, v, do = _inputs(B, Sq, Skv, H, D, seed=900)
    q64, k64, v64, do64 = (to_f64(x) for x in (q, k, v, do))
    q_pos, k_pos = np.arange(64, 64 + Sq), np.arange(Skv)
    o, lse, delta, o_bf, lse_f = _saved_stats(q64, k64, v64, do64, scale, causal, q_pos, k_pos)
    _, dq, dk, dv = _run(q, k, v, do, o_bf, lse_f, scale, causal, 64, 0)
    wq, wk, wv = oracle.chunk_grad(q64, k64, v64, do64, lse, delta, scale, causal, q_pos, k_pos)
    check_grad(dq, wq, "dQ")
    check_grad(dk, wk, "dK")
    check_grad(dv, wv, "dV")


def test_rows_without_keys_and_fully_masked_chunk():
    """Queries positioned before every key: LSE = -inf rows give exact zeros."""
    say("backward rows without keys")
    B, Sq, Skv, H, D = 1, 70, 90, 2, 64
    q, k, v, do = _inputs(B, Sq, Skv, H, D, seed=910)
    q64, k64, v64, do64 = (to_f64(x) for x in (q, k, v, do))
    scale = 1 / math.sqrt(D)
    q_pos, k_pos = np.arange(-40, -40 + Sq), np.arange(Skv)   # rows 0..39 see no key
    o, lse, delta, o_bf, lse_f = _saved_stats(q64, k64, v64, do64, scale, True, q_pos, k_pos)
    assert np.all(np.isneginf(lse[:, :, :40]))
    _, dq, dk, dv = _run(q, k, v, do, o_bf, lse_f, scale, True, -40, 0)
    wq, wk, wv = oracle.chunk_grad(q64, k64, v64, do64, lse, delta, scale, True, q_pos, k_pos)
    assert torch.all(dq[:, :40] == 0)
    check_grad(dq, wq, "dQ")
    check_grad(dk, wk, "dK")
    check_grad(dv, wv, "dV")
    # a chunk entirely in the future of every query contributes exact zeros
    qq, kk, vv, dd = (x.to(DEV) for x in (q, k, v, do))
    lse_d = lse_f.to(DEV)
    delta_d = cp.attn_backward_delta(o_bf.to(DEV), dd)
    dq2, dk2, dv2 = cp.attn_chunk_backward(qq, kk, vv, dd, lse_d, delta_d, causal=True, q_pos0=0,
                                           kv_pos0=10_000)
    torch.cuda.synchronize()
    assert torch.all(dq2 == 0) and torch.all(dk2 == 0) and torch.all(dv2 == 0)


def test_ring_accumulation_over_chunks_and_shards():
    """dQ summed over a rank's chunks, dK/dV summed over the ranks' Q shards,
    equal the full gradient (the ring backward's bookkeeping)."""
    say("backward ring accumulation")
    B, S, H, D, P = 1, 4 * 96, 2, 128, 4
    q, k, v, do = _inputs(B, S, S, H, D, seed=920)
    q64, k64, v64, do64 = (to_f64(x) for x in (q, k, v, do))
    scale = 1 / math.sqrt(D)
    for causal in (False, True):
        o, lse, delta, o_bf, lse_f = _saved_stats(q64, k64, v64, do64, scale, causal, None, None)
        wq, wk, wv = oracle.attention_grad(q64, k64, v64, do64, scale, causal)
        qd, kd, vd, dd = (x.to(DEV) for x in (q, k, v, do))
        delta_d = cp.attn_backward_delta(o_bf.to(DEV), dd)
        lse_d = lse_f.to(DEV)
        n = S // P
        dq = torch.full((B, S, H, D), float("nan"), device=DEV)
        dk = torch.zeros((B, S, H, D), device=DEV)
        dv = torch.zeros((B, S, H, D), device=DEV)
        for r in range(P):                                  # rank r owns Q shard r
            qs = slice(r * n, (r + 1) * n)
            dq_r = dq[:, qs]
            dq_r = torch.empty_like(dq_r)
            for step, c in enumerate(synthetic.ring_order(r, P)):   # chunks in ring order
                ks = slice(c * n, (c + 1) * n)
                dk_c = torch.empty((B, n, H, D), device=DEV)
                dv_c = torch.empty((B, n, H, D), device=DEV)
                cp.attn_chunk_backward(
                    qd[:, qs].contiguous(), kd[:, ks].contiguous(), vd[:, ks].contiguous(),
                    dd[:, qs].contiguous(), lse_d[:, :, qs].contiguous(),
                    delta_d[:, :, qs].contiguous(), dq_r, dk_c, dv_c, causal=causal,
                    q_pos0=r * n, kv_pos0=c * n, accumulate_dq=step > 0)
                dk[:, ks] += dk_c
                dv[:, ks] += dv_c
            dq[:, qs] = dq_r
        torch.cuda.synchronize()
        check_grad(dq, wq, f"dQ causal={causal}")
        check_grad(dk, wk, f"dK causal={causal}")
        check_grad(dv, wv, f"dV causal={causal}")


def test_accumulate_flags_add_to_existing_buffers():
    say("backward accumulate flags")
    B, Sq, Skv, H, D = 1, 100, 140, 2, 128
    q, k, v, do = (x.to(DEV) for x in _inputs(B, Sq, Skv, H, D, seed=930))
    lse = torch.randn((B, H, Sq), device=DEV) + 8.0
    delta = torch.randn((B, H, Sq), device=DEV)
    dq0, dk0, dv0 = cp.attn_chunk_backward(q, k, v, do, lse, delta)
    base = [torch.randn_like(x) for x in (dq0, dk0, dv0)]
    acc = [x.clone() for x in base]
    cp.attn_chunk_backward(q, k, v, do, lse, delta, *acc, accumulate_dq=True, accumulate_dkv=True)
    torch.cuda.synchronize()
    for a, b0, x in zip(acc, base, (dq0, dk0, dv0)):
        assert torch.allclose(a, b0 + x, rtol=0, atol=1e-6)


def test_empty_sides():
    say("backward Sq = 0 / Skv = 0")
    B, H, D = 1, 2, 64
    q, k, v, do = (x.to(DEV) for x in _inputs(B, 0, 50, H, D, seed=940))
    lse = torch.empty((B, H, 0), device=DEV)
    dq, dk, dv = cp.attn_chunk_backward(q, k, v, do, lse, lse.clone())
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)
    q, k, v, do = (x.to(DEV) for x in _inputs(B, 30, 0, H, D, seed=950))
    lse = torch.full((B, H, 30), float("-inf"), device=DEV)
    dq, dk, dv = cp.attn_chunk_backward(q, k, v, do, lse, torch.zeros_like(lse))
    torch.cuda.synchronize()
    assert torch.all(dq == 0)
    keep = torch.randn_like(dq)
    dq2 = keep.clone()
    cp.attn_chunk_backward(q, k, v, do, lse, torch.zeros_like(lse), dq2, dk, dv,
                           accumulate_dq=True)
    torch.cuda.synchronize()
    assert torch.equal(dq2, keep)


def test_backward_is_deterministic():
    say("backward determinism")
    B, Sq, Skv, H, D = 1, 300, 500, 3, 128
    q, k, v, do = (x.to(DEV) for x in _inputs(B, Sq, Skv, H, D, seed=960))
    lse = torch.randn((B, H, Sq), device=DEV) + 9.0
    delta = torch.randn((B, H, Sq), device=DEV)
    a = cp.attn_chunk_backward(q, k, v, do, lse, delta, causal=True, q_pos0=200)
    b = cp.attn_chunk_backward(q, k, v, do, lse, delta, causal=True, q_pos0=200)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_delta_dtypes(dtype):
    say(f"backward delta {dtype}")
    B, Sq, H, D = 2, 37, 3, 128
    o = synthetic.make_tensor((B, Sq, H, D), dtype, 970)
    do = synthetic.make_tensor((B, Sq, H, D), dtype, 971)
    got = cp.attn_backward_delta(o.to(DEV), do.to(DEV))
    torch.cuda.synchronize()
    want = oracle.backward_delta(to_f64(o), to_f64(do))
    assert np.abs(to_f64(got) - want).max() <= F32_MAX


@pytest.mark.parametrize("lens,causal,H", [
    ((96, 96, 96, 96), False, 2),          # even ring of 4
    ((130, 0, 257, 64), True, 2),          # uneven, an empty chunk, causal
    ((1025, 1025, 1025, 1024), True, 1),   # the ring-anything split of 4099
    ((300,), False, 3),                    # P = 1
])
def test_ring_backward_matches_oracle(lens, causal, H):
    """cp_ring_attention_backward: dQ over every chunk, each chunk's dK/dV share,
    in ring order (rank 1 of the ring: its own chunk first)."""
    say(f"ring backward lens={lens} causal={causal} H={H}")
    D = 128
    S = sum(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(int)
    r = 1 if len(lens) > 1 else 0
    q0, n = int(starts[r]), lens[r] if lens[r] > 0 else lens[0]
    q, k, v, do = _inputs(1, n, S, H, D, seed=S + H)
    q64, k64, v64, do64 = (to_f64(x) for x in (q, k, v, do))
    scale = 1 / math.sqrt(D)
    q_pos = np.arange(q0, q0 + n)
    o, lse, delta, o_bf, lse_f = _saved_stats(q64, k64, v64, do64, scale, causal, q_pos,
                                              np.arange(S))
    wq, wk, wv = oracle.chunk_grad(q64, k64, v64, do64, lse, delta, scale, causal, q_pos,
                                   np.arange(S))
    kd, vd = k.to(DEV), v.to(DEV)
    order = synthetic.ring_order(r, len(lens))
    chunks = [(kd[:, s:s + m].contiguous(), vd[:, s:s + m].contiguous(), int(s))
              for s, m in zip(starts, lens)]
    qd, dod = q.to(DEV), do.to(DEV)
    delta_d = cp.attn_backward_delta(o_bf.to(DEV), dod)
    dq, grads = cp.ring_attention_backward(qd, [chunks[c] for c in order], dod, lse_f.to(DEV),
                                           delta_d, scale=scale, causal=causal, q_pos0=q0)
    torch.cuda.synchronize()
    check_grad(dq, wq, "dQ")
    got_k = torch.cat([grads[order.index(c)][0] for c in range(len(lens))], dim=1)
    got_v = torch.cat([grads[order.index(c)][1] for c in range(len(lens))], dim=1)
    check_grad(got_k, wk, "dK")
    check_grad(got_v, wv, "dV")
    # the same through per-chunk calls with dQ accumulated: identical bytes for
    # dK/dV (the same blocks do the same work), dQ within rounding of the
    # summation order
    dq2 = torch.empty_like(dq)
    for step, c in enumerate(order):
        kc, vc, s0 = chunks[c]
        _, dk2, dv2 = cp.attn_chunk_backward(qd, kc, vc, dod, lse_f.to(DEV), delta_d, dq2,
                                             scale=scale, causal=causal, q_pos0=q0, kv_pos0=s0,
                                             accumulate_dq=step > 0)
        gk, gv = grads[step]
        assert torch.equal(dk2, gk) and torch.equal(dv2, gv)
    torch.cuda.synchronize()
    check_grad(dq2, wq, "dQ per chunk")


def _nan_padded(x: torch.Tensor) -> torch.Tensor:
    """x ([1][S][H][D]) on the GPU as a view whose memory continues with 64 NaN rows."""
    buf = torch.full((1, x.shape[1] + 64) + tuple(x.shape[2:]), float("nan"), dtype=x.dtype)
    buf[:, :x.shape[1]] = x
    return buf.to(DEV)[:, :x.shape[1]]


@pytest.mark.parametrize("causal", [False, True])
def test_ring_backward_never_reads_past_its_tensors(causal):
    """Q, dO and every K/V chunk are views followed by NaN rows. The backward
    kernels must not read past any of them (a ragged tile's missing rows come
    in as zeros through the load's range check): a NaN row that entered a
    product would turn gradients into NaN."""
    lens, H, D = (201, 64, 150, 37), 2, 128
    say(f"ring backward, NaN rows after every tensor, causal={causal}")
    S = sum(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(int)
    r = 2
    q0, n = int(starts[r]), lens[r]
    q, k, v, do = _inputs(1, n, S, H, D, seed=77)
    q64, k64, v64, do64 = (to_f64(x) for x in (q, k, v, do))
    scale = 1 / math.sqrt(D)
    q_pos = np.arange(q0, q0 + n)
    o, lse, delta, o_bf, lse_f = _saved_stats(q64, k64, v64, do64, scale, causal, q_pos,
                                              np.arange(S))
    wq, wk, wv = oracle.chunk_grad(q64, k64, v64, do64, lse, delta, scale, causal, q_pos,
                                   np.arange(S))
    chunks = [(_nan_padded(k[:, s:s + m]), _nan_padded(v[:, s:s + m]), int(s))
              for s, m in zip(starts, lens)]
    order = synthetic.ring_order(r, len(lens))
    qd, dod = _nan_padded(q), _nan_padded(do)
    delta_d = cp.attn_backward_delta(_nan_padded(o_bf), dod)
    dq, grads = cp.ring_attention_backward(qd, [chunks[c] for c in order], dod, lse_f.to(DEV),
                                           delta_d, scale=scale, causal=causal, q_pos0=q0)
    torch.cuda.synchronize()
    check_grad(dq, wq, "dQ")
    check_grad(torch.cat([grads[order.index(c)][0] for c in range(len(lens))], dim=1), wk, "dK")
    check_grad(torch.cat([grads[order.index(c)][1] for c in range(len(lens))], dim=1), wv, "dV")


def test_ring_backward_accumulates_into_existing_buffers():
    say("ring backward accumulate flags")
    B, Sq, H, D = 1, 100, 2, 128
    lens = (70, 130)
    q, do = (x.to(DEV) for x in _inputs(B, Sq, 1, H, D, seed=990)[::3])
    kv = [(synthetic.make_tensor((B, m, H, D), torch.bfloat16, 991 + c).to(DEV),
           synthetic.make_tensor((B, m, H, D), torch.bfloat16, 995 + c).to(DEV), 70 * c)
          for c, m in enumerate(lens)]
    lse = torch.randn((B, H, Sq), device=DEV) + 8.0
    delta = torch.randn((B, H, Sq), device=DEV)
    dq0, g0 = cp.ring_attention_backward(q, kv, do, lse, delta)
    base_q = torch.randn_like(dq0)
    base_g = [(torch.randn_like(a), torch.randn_like(b)) for a, b in g0]
    dq1 = base_q.clone()
    g1 = [(a.clone(), b.clone()) for a, b in base_g]
    cp.ring_attention_backward(q, kv, do, lse, delta, dq1, g1, accumulate_dq=True,
                               accumulate_dkv=True)
    torch.cuda.synchronize()
    assert torch.allclose(dq1, base_q + dq0, rtol=0, atol=1e-6)
    for (a, b), (a0, b0), (x, y) in zip(g1, base_g, g0):
        assert torch.allclose(a, a0 + x, rtol=0, atol=1e-6)
        assert torch.allclose(b, b0 + y, rtol=0, atol=1e-6)


F32_GRAD_MAX = 1e-5


@pytest.mark.parametrize("Sq,Skv,H,D,causal,q_pos0", [
    (64, 256, 2, 64, False, 0),     # the tiny fp32 workload's ring rank against all keys
    (64, 256, 2, 64, True, 64),     # the same rank, causal
    (70, 133, 3, 128, True, 40),    # ragged, D = 128
    (0, 40, 2, 64, False, 0),       # no queries: dK = dV = 0
])
def test_f32_backward_matches_oracle(Sq, Skv, H, D, causal, q_pos0):
    """fp32 inputs: every step in fp32; max-abs 1e-5 (relative to max(1, max|ref|))."""
    say(f"fp32 backward Sq={Sq} Skv={Skv} H={H} D={D} causal={causal}")
    q, k, v, do = (synthetic.make_tensor(shape, torch.float32, 1300 + n)
                   for n, shape in enumerate([(1, Sq, H, D), (1, Skv, H, D), (1, Skv, H, D),
                                              (1, Sq, H, D)]))
    q64, k64, v64, do64 = (to_f64(x) for x in (q, k, v, do))
    scale = 1 / math.sqrt(D)
    q_pos, k_pos = np.arange(q_pos0, q_pos0 + Sq), np.arange(Skv)
    o, lse = oracle.attention(q64, k64, v64, scale, causal, q_pos, k_pos)
    delta = oracle.backward_delta(o, do64)
    dd = [x.to(DEV) for x in (q, k, v, do)]
    if Sq > 0:
        delta_d = cp.attn_backward_delta(torch.tensor(o, dtype=torch.float32).to(DEV), dd[3])
    else:
        delta_d = torch.empty((1, H, 0), device=DEV)
    dq, dk, dv = cp.attn_chunk_backward(*dd, torch.tensor(lse, dtype=torch.float32).to(DEV),
                                        delta_d, scale=scale, causal=causal, q_pos0=q_pos0)
    torch.cuda.synchronize()
    want = oracle.chunk_grad(q64, k64, v64, do64, lse, delta, scale, causal, q_pos, k_pos)
    for got, w, name in zip((dq, dk, dv), want, ("dQ", "dK", "dV")):
        g = to_f64(got)
        assert np.all(np.isfinite(g))
        if w.size == 0:
            continue
        err = np.abs(g - w).max()
        print(f"  {name}: max-abs {err:.2e} (max|ref| {np.abs(w).max():.2e})", flush=True)
        assert err <= F32_GRAD_MAX * max(1.0, np.abs(w).max()), f"{name}: max-abs {err:.3e}"


def test_f32_ring_backward_tiny_workload():
    """The tiny fp32 workload (S 256, H 2, D 64, ring of 4): every rank's
    backward through cp_ring_attention_backward; dK/dV summed over the ranks."""
    w = synthetic.TINY
    say(f"{w.name}: fp32 ring backward, all ranks")
    q, k, v = synthetic.make_qkv(w)
    do = synthetic.make_tensor(tuple(q.shape), torch.float32, 1400)
    q64, k64, v64, do64 = (to_f64(x) for x in (q, k, v, do))
    scale = 1 / math.sqrt(w.D)
    o, lse = oracle.attention(q64, k64, v64, scale)
    delta = oracle.backward_delta(o, do64)
    wq, wk, wv = oracle.attention_grad(q64, k64, v64, do64, scale)
    starts = w.chunk_starts()
    kd, vd = k.to(DEV), v.to(DEV)
    chunks = [(kd[:, s:s + m].contiguous(), vd[:, s:s + m].contiguous(), s)
              for s, m in zip(starts, w.chunk_lens)]
    dq = torch.empty(q.shape, device=DEV)
    dk = torch.zeros(k.shape, device=DEV)
    dv = torch.zeros(v.shape, device=DEV)
    o_d = torch.tensor(o, dtype=torch.float32).to(DEV)
    lse_d = torch.tensor(lse, dtype=torch.float32).to(DEV)
    for r in range(w.P):
        s0, n = starts[r], w.chunk_lens[r]
        rows = slice(s0, s0 + n)
        order = synthetic.ring_order(r, w.P)
        qr, dor = q[:, rows].contiguous().to(DEV), do[:, rows].contiguous().to(DEV)
        dl = cp.attn_backward_delta(o_d[:, rows].contiguous(), dor)
        dq_r, grads = cp.ring_attention_backward(qr, [chunks[c] for c in order], dor,
                                                 lse_d[:, :, rows].contiguous(), dl, scale=scale,
                                                 q_pos0=s0)
        dq[:, rows] = dq_r
        for c, (gk, gv) in zip(order, grads):
            dk[:, starts[c]:starts[c] + w.chunk_lens[c]] += gk
            dv[:, starts[c]:starts[c] + w.chunk_lens[c]] += gv
    torch.cuda.synchronize()
    for got, want, name in ((dq, wq, "dQ"), (dk, wk, "dK"), (dv, wv, "dV")):
        err = np.abs(to_f64(got) - want).max()
        print(f"  {name}: max-abs {err:.2e}", flush=True)
        assert err <= F32_GRAD_MAX * max(1.0, np.abs(want).max()), f"{name}: max-abs {err:.3e}"
