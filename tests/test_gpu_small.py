"""GPU parity at small sizes: several tiles, ragged tails, edge cases.

Every case draws seeded inputs from ``synthetic``, runs the HIP library
through the C ABI, and compares element by element with the fp64 oracle.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests._parity import (check_lse, check_o, check_o_scaled, kind_of, say, to_f64)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import context_attention_dit_amd as cp
DEV = "cuda:0"


def _qkv(B, Sq, Skv, H, D, dtype, seed):
    q = synthetic.make_tensor((B, Sq, H, D), dtype, seed)
    k = synthetic.make_tensor((B, Skv, H, D), dtype, seed + 1)
    v = synthetic.make_tensor((B, Skv, H, D), dtype, seed + 2)
    return q, k, v


# ------------------------------------------------------------------- relayout

@pytest.mark.parametrize("P,B,S_l,H,D,dtype", [
    (2, 1, 128, 2, 64, torch.float32),     # the tiny workload's relayout
    (4, 1, 37, 8, 128, torch.bfloat16),
    (4, 2, 5, 24, 128, torch.bfloat16),
    (8, 1, 3, 40, 128, torch.bfloat16),
    (1, 2, 7, 3, 64, torch.bfloat16),      # P = 1 is a copy
    (3, 2, 4, 6, 3, torch.bfloat16),       # 2-byte words
    (2, 1, 9, 4, 5, torch.float32),        # 4-byte words
    (4, 1, 6, 8, 2, torch.bfloat16),       # 4-byte runs
])
def test_relayout_bit_exact(P, B, S_l, H, D, dtype):
    say(f"relayout P={P} B={B} S_l={S_l} H={H} D={D} {dtype}")
    isz = 2 if dtype == torch.bfloat16 else 4
    bits = synthetic.random_bits((P, B, S_l, H, D), isz, seed=P * 100 + D)
    x = bits.view(dtype).to(DEV)
    y = cp.ulysses_seq2head(x, P)
    z = cp.ulysses_head2seq(y, P)
    torch.cuda.synchronize()
    want = oracle.seq2head(bits.numpy(), P)
    assert np.array_equal(y.cpu().view(bits.dtype).numpy(), want)
    assert np.array_equal(z.cpu().view(bits.dtype).numpy(), bits.numpy())
    # head2seq on independent random bits against its own oracle
    bits2 = synthetic.random_bits(tuple(want.shape), isz, seed=P * 100 + D + 1)
    w2 = cp.ulysses_head2seq(bits2.view(dtype).to(DEV), P)
    torch.cuda.synchronize()
    assert np.array_equal(w2.cpu().view(bits.dtype).numpy(), oracle.head2seq(bits2.numpy(), P))


def test_relayout_misaligned_base_uses_narrow_words():
    say("relayout with 2-byte-offset base pointers")
    P, B, S_l, H, D = 2, 1, 4, 4, 64
    bits = synthetic.random_bits((P * B * S_l * H * D + 1,), 2, seed=5)
    buf = bits.view(torch.bfloat16).to(DEV)
    x = buf[1:].view(P, B, S_l, H, D)           # base is 2 bytes off 16-byte alignment
    out = torch.empty(P * B * S_l * H * D + 1, dtype=torch.bfloat16, device=DEV)
    y = out[1:].view(P, B, P * S_l, H // P, D)
    cp._check("cp_ulysses_seq2head", cp._seq2head(x.data_ptr(), y.data_ptr(), P, B, S_l, H, D,
                                                  0, torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    want = oracle.seq2head(bits.numpy()[1:].reshape(P, B, S_l, H, D), P)
    assert np.array_equal(y.cpu().view(torch.int16).numpy(), want)


# ------------------------------------------------------- relayout: Ulysses Anything

def _shard_sizes(B, s_lens, h_counts, D):
    S, H = sum(s_lens), sum(h_counts)
    return [B * sq * H * D for sq in s_lens], [B * S * hp * D for hp in h_counts]


def _split(flat, sizes, shapes):
    out, o = [], 0
    for n, shp in zip(sizes, shapes):
        out.append(flat[o:o + n].reshape(shp))
        o += n
    return out


@pytest.mark.parametrize("s_lens,h_counts,B,D,itemsize", [
    ((5, 3, 4), (3, 2, 3), 2, 128, 2),          # uneven tokens and heads
    ((7, 0, 2), (0, 4, 1), 1, 64, 2),           # a rank with no tokens, a rank with no heads
    ((3, 3), (1, 2), 1, 12, 4),                 # fp32, D not a multiple of 16 bytes
    ((9,), (5,), 2, 32, 2),                     # one rank: a plain copy
    ((1121, 1120, 1120, 1120), (8, 8, 7, 7), 1, 128, 2),  # 4481 tokens, 30 heads over 4
])
def test_anything_relayout_bit_exact(s_lens, h_counts, B, D, itemsize):
    say(f"anything relayout s={s_lens} h={h_counts} B={B} D={D} bytes={itemsize}")
    S, H = sum(s_lens), sum(h_counts)
    ssz, gsz = _shard_sizes(B, s_lens, h_counts, D)
    bits = synthetic.random_bits((B * S * H * D,), itemsize, seed=S + H)
    dt = torch.bfloat16 if itemsize == 2 else torch.float32
    x = bits.view(dt).to(DEV)
    y = cp.ulysses_anything_seq2head(x, s_lens, h_counts, B, D)
    back = cp.ulysses_anything_head2seq(y, s_lens, h_counts, B, D)
    torch.cuda.synchronize()
    ints = torch.int16 if itemsize == 2 else torch.int32
    shards = _split(bits.numpy(), ssz, [(B, sq, H, D) for sq in s_lens])
    want = oracle.anything_seq2head(shards, list(h_counts))
    got = _split(y.cpu().view(ints).numpy(), gsz, [(B, S, hp, D) for hp in h_counts])
    assert all(np.array_equal(a, b) for a, b in zip(got, want))
    assert torch.equal(back.view(ints).cpu(), bits)


def test_anything_relayout_even_split_matches_standard():
    P, B, S_l, H, D = 4, 2, 6, 8, 128
    x = synthetic.random_bits((P, B, S_l, H, D), 2, seed=33).view(torch.bfloat16).to(DEV)
    say("anything relayout with even counts vs standard Ulysses")
    a = cp.ulysses_anything_seq2head(x.reshape(-1), [S_l] * P, [H // P] * P, B, D)
    b = cp.ulysses_seq2head(x, P)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.reshape(-1).view(torch.int16))


def test_anything_relayout_misaligned_base_uses_narrow_words():
    s_lens, h_counts, B, D = (3, 2), (2, 1), 1, 64
    S, H = sum(s_lens), sum(h_counts)
    n = B * S * H * D
    bits = synthetic.random_bits((n + 1,), 2, seed=6)
    say("anything relayout with 2-byte-offset base pointers")
    buf = bits.view(torch.bfloat16).to(DEV)
    out = torch.empty(n + 1, dtype=torch.bfloat16, device=DEV)
    cp.ulysses_anything_seq2head(buf[1:], s_lens, h_counts, B, D, out[1:])
    torch.cuda.synchronize()
    ssz, gsz = _shard_sizes(B, s_lens, h_counts, D)
    shards = _split(bits.numpy()[1:], ssz, [(B, sq, H, D) for sq in s_lens])
    want = np.concatenate([w.ravel() for w in oracle.anything_seq2head(shards, list(h_counts))])
    assert np.array_equal(out[1:].cpu().view(torch.int16).numpy(), want)


@pytest.mark.parametrize("s_lens,B,H,D", [((5, 3, 4), 2, 3, 128), ((0, 7, 2), 1, 2, 64),
                                         ((6,), 2, 1, 32)])
def test_kv_gather_bit_exact(s_lens, B, H, D):
    say(f"kv gather s={s_lens} B={B} H={H} D={D}")
    S = sum(s_lens)
    bits = synthetic.random_bits((B * S * H * D,), 2, seed=S * 3 + H)
    x = bits.view(torch.bfloat16).to(DEV)
    y = cp.kv_gather(x, s_lens, B, H, D)
    torch.cuda.synchronize()
    sizes = [B * sq * H * D for sq in s_lens]
    shards = _split(bits.numpy(), sizes, [(B, sq, H, D) for sq in s_lens])
    assert np.array_equal(y.cpu().view(torch.int16).numpy(), oracle.kv_gather(shards))


# ---------------------------------------------------------------------- merge

@pytest.mark.parametrize("P,D", [(1, 128), (2, 128), (4, 128), (7, 128), (8, 64),
                                 (11, 128),          # more partials than the unrolled fast path
                                 (3, 12), (9, 4),    # D not a multiple of 8: one column per lane
                                 (2, 1000), (3, 4096), (2, 4092)])  # wide rows: R = 2, 1, 1
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_merge_matches_oracle(P, D, out_dtype):
    say(f"merge P={P} D={D} out={out_dtype}")
    B, Sq, H = 2, 77, 3
    o_parts = synthetic.make_tensor((P, B, Sq, H, D), torch.float32, 10 + P)
    lse_parts = synthetic.make_tensor((P, B, H, Sq), torch.float32, 20 + P) * 3.0
    lse_parts[:, 0, 1, :5] = -math.inf           # rows no chunk saw
    if P > 1:
        lse_parts[0, 1, 2, 10:20] = -math.inf    # rows one chunk did not see
    o, lse = cp.lse_merge(o_parts.to(DEV), lse_parts.to(DEV), out_dtype=out_dtype)
    torch.cuda.synchronize()
    wo, wl = oracle.lse_merge(o_parts.numpy(), lse_parts.numpy())
    if out_dtype == torch.float32:
        check_o(o, wo, "f32")
    else:
        # bf16 output is the fp32 merge (held to the fp32 merge tolerance 1e-5)
        # rounded once to bf16: within 1e-5 plus half a bf16 spacing of the
        # oracle (the partials here reach |x| ~ 5, where bf16's own spacing
        # exceeds the attention tolerance)
        spacing = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(wo), 2.0 ** -126))) - 7)
        assert np.all(np.abs(to_f64(o) - wo) <= 1e-5 + 0.5 * spacing)
    check_lse(lse, wl)
    assert np.all(to_f64(o)[0, :5, 1] == 0)


# -------------------------------------------------------- chunk partial attention

CASES = [
    # B, Sq, Skv, H, D, causal, q_pos0, kv_pos0
    (1, 256, 256, 2, 64, False, 0, 0),
    (2, 300, 333, 3, 128, False, 0, 0),
    (1, 129, 65, 2, 128, True, 64, 0),
    (1, 200, 200, 2, 128, True, 0, 0),
    (2, 77, 190, 2, 64, True, 150, 40),
    (1, 1, 1, 1, 128, False, 0, 0),
    (1, 130, 70, 1, 128, True, 0, 100),   # many rows see nothing
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("in_dtype,out_dtype", [(torch.bfloat16, torch.float32),
                                                (torch.bfloat16, torch.bfloat16),
                                                (torch.float32, torch.float32)])
def test_chunk_partial(case, in_dtype, out_dtype):
    B, Sq, Skv, H, D, causal, qp, kp = case
    say(f"chunk_partial {case} {in_dtype}->{out_dtype}")
    q, k, v = _qkv(B, Sq, Skv, H, D, in_dtype, seed=Sq * 7 + Skv)
    scale = 1 / math.sqrt(D)
    o, lse = cp.attn_chunk_partial(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale, causal=causal,
                                   q_pos0=qp, kv_pos0=kp, out_dtype=out_dtype)
    torch.cuda.synchronize()
    wo, wl = oracle.chunk_partial(to_f64(q), to_f64(k), to_f64(v), scale, causal,
                                  np.arange(qp, qp + Sq), np.arange(kp, kp + Skv))
    kind = "bf16" if (in_dtype == torch.bfloat16) else "f32"
    check_o(o, wo, kind)
    check_lse(lse, wl)


@pytest.mark.parametrize("scale_of", [lambda D: -1 / math.sqrt(D), lambda D: 0.0,
                                      lambda D: -0.37])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("in_dtype,out_dtype", [(torch.bfloat16, torch.float32),
                                                (torch.bfloat16, torch.bfloat16),
                                                (torch.float32, torch.float32)])
def test_forward_negative_and_zero_scale(scale_of, causal, in_dtype, out_dtype):
    """A negative scale flips the sign of every score (the bf16 kernel folds it
    into Q); a zero scale gives uniform weights over the visible keys (O is
    their V mean, LSE = ln of their count). Per-hop partial and ring. The fp32
    partials of bf16 inputs are held to the absolute bf16 bars; bf16-rounded
    outputs (the ring's O, bf16 partials) to the scaled bars."""
    B, Sq, Skv, H, D = 1, 150, 211, 2, 128
    scale = scale_of(D)
    say(f"forward scale={scale:.4f} causal={causal} {in_dtype}->{out_dtype}")
    q, k, v = _qkv(B, Sq, Skv, H, D, in_dtype, seed=911)
    qp, kp = (60, 0) if causal else (0, 0)
    o, lse = cp.attn_chunk_partial(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale, causal=causal,
                                   q_pos0=qp, kv_pos0=kp, out_dtype=out_dtype)
    lens = (90, 121)
    kd, vd = k.to(DEV), v.to(DEV)
    chunks = [(kd[:, :lens[0]].contiguous(), vd[:, :lens[0]].contiguous(), kp),
              (kd[:, lens[0]:].contiguous(), vd[:, lens[0]:].contiguous(), kp + lens[0])]
    ro, rl = cp.ring_attention(q.to(DEV), chunks[::-1], scale=scale, causal=causal, q_pos0=qp)
    torch.cuda.synchronize()
    wo, wl = oracle.chunk_partial(to_f64(q), to_f64(k), to_f64(v), scale, causal,
                                  np.arange(qp, qp + Sq), np.arange(kp, kp + Skv))
    # bf16-rounded outputs: the scaled bars (a large |scale| makes the softmax
    # peaky and O close to single V rows, not small); fp32 outputs: absolute
    if out_dtype == torch.bfloat16:
        check_o_scaled(o, wo, "partial O")
    else:
        check_o(o, wo, "bf16" if in_dtype == torch.bfloat16 else "f32", "partial O")
    check_lse(lse, wl)
    if in_dtype == torch.bfloat16:
        check_o_scaled(ro, wo, "ring O")
    else:
        check_o(ro, wo, "f32", "ring O")
    check_lse(rl, wl, "ring LSE")
    if scale == 0.0:   # closed form: uniform weights over the visible keys
        counts = np.array([min(Skv, qp + i - kp + 1) if causal else Skv for i in range(Sq)])
        assert np.abs(to_f64(lse)[0, 0] - np.log(np.maximum(counts, 1))).max() <= 1e-4


@pytest.mark.parametrize("in_dtype", [torch.bfloat16, torch.float32])
def test_chunk_partial_no_keys(in_dtype):
    say(f"chunk_partial Skv=0 {in_dtype}")
    q = synthetic.make_tensor((1, 70, 2, 128), in_dtype, 3).to(DEV)
    k = torch.empty((1, 0, 2, 128), dtype=in_dtype, device=DEV)
    o = torch.full((1, 70, 2, 128), 7.0, device=DEV)
    lse = torch.full((1, 2, 70), 7.0, device=DEV)
    cp.attn_chunk_partial(q, k, k, o, lse)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_stress_inputs():
    """Peaky softmax (Q x 8) and all-equal keys (uniform closed form)."""
    w = synthetic.FLUX_RING
    q, k, v = synthetic.make_qkv(w, S=320, H=2, scale_q=8.0)
    say("stress: peaky softmax")
    o, lse = cp.attn_chunk_partial(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    wo, wl = oracle.attention(to_f64(q), to_f64(k), to_f64(v), 1 / math.sqrt(128))
    check_o(o, wo, "bf16")
    check_lse(lse, wl)
    say("stress: all keys equal")
    k_eq = k[:, :1].expand_as(k).contiguous()
    o, lse = cp.attn_chunk_partial(q.to(DEV), k_eq.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    mean_v = to_f64(v).mean(axis=1, keepdims=True)
    check_o(o, np.broadcast_to(mean_v, wo.shape), "bf16")


# ------------------------------------------------------------------------ ring

def _chunk_tensors(k, v, lens):
    out, acc = [], 0
    for n in lens:
        out.append((k[:, acc:acc + n].contiguous(), v[:, acc:acc + n].contiguous(), acc))
        acc += n
    return out


def test_tiny_ring_all_ranks_all_orders():
    """The tiny fp32 workload: ring degree 4, every rank, all 24 visit orders."""
    w = synthetic.TINY
    q, k, v = synthetic.make_qkv(w)
    scale = 1 / math.sqrt(w.D)
    wo, wl = oracle.attention(to_f64(q), to_f64(k), to_f64(v), scale)
    chunks = _chunk_tensors(k.to(DEV), v.to(DEV), w.chunk_lens)
    n = w.S // w.P
    for r in range(w.P):
        qs = q[:, r * n:(r + 1) * n].contiguous().to(DEV)
        for order in itertools.permutations(range(w.P)):
            say(f"tiny ring rank {r} order {order}")
            o, lse = cp.ring_attention(qs, [chunks[c] for c in order], scale=scale)
            torch.cuda.synchronize()
            check_o(o, wo[:, r * n:(r + 1) * n], "f32")
            check_lse(lse, wl[:, :, r * n:(r + 1) * n])
    # the whole Q in one call
    o, lse = cp.ring_attention(q.to(DEV), chunks, scale=scale)
    torch.cuda.synchronize()
    check_o(o, wo, "f32")
    check_lse(lse, wl)


@pytest.mark.parametrize("lens,causal,in_dtype", [
    ((100, 100, 100, 100), False, torch.bfloat16),
    ((129, 0, 64, 200), True, torch.bfloat16),     # an empty chunk
    ((7, 300, 1, 65, 33), True, torch.bfloat16),
    ((250,), False, torch.bfloat16),
    ((90, 90, 91), True, torch.float32),
    ((64, 64), False, torch.float32),
])
def test_ring_uneven_chunks(lens, causal, in_dtype):
    S = sum(lens)
    P = len(lens)
    H, D = 2, 128
    q, k, v = _qkv(1, S, S, H, D, in_dtype, seed=S + P)
    scale = 1 / math.sqrt(D)
    wo, wl = oracle.attention(to_f64(q), to_f64(k), to_f64(v), scale, causal)
    chunks = _chunk_tensors(k.to(DEV), v.to(DEV), lens)
    starts = [0] + list(np.cumsum(lens)[:-1])
    for r in range(P):
        if lens[r] == 0:
            continue
        s0, n = starts[r], lens[r]
        order = synthetic.ring_order(r, P)
        say(f"ring lens={lens} rank={r} causal={causal} {in_dtype}")
        o, lse = cp.ring_attention(q[:, s0:s0 + n].contiguous().to(DEV), [chunks[c] for c in order],
                                   scale=scale, causal=causal, q_pos0=int(s0))
        torch.cuda.synchronize()
        check_o(o, wo[:, s0:s0 + n], kind_of(in_dtype))
        check_lse(lse, wl[:, :, s0:s0 + n])


@pytest.mark.parametrize("causal", [False, True])
def test_ring_small_grid_two_groups(causal):
    """2 query tiles x 2 heads: each tile gets a whole CU, its keys split
    between two wave groups and merged in LDS, so no workspace is needed."""
    lens = (700, 513, 0, 811)
    S, H, D = sum(lens), 2, 128
    q, k, v = _qkv(1, S, S, H, D, torch.bfloat16, seed=321)
    chunks = _chunk_tensors(k.to(DEV), v.to(DEV), lens)
    q0, n = 900, 200
    assert cp.ring_attention_workspace_bytes(4, 1, H, n, D) == 0
    say(f"ring with two-group blocks causal={causal}")
    o, lse = cp.ring_attention(q[:, q0:q0 + n].contiguous().to(DEV), [chunks[c] for c in (3, 1, 0, 2)],
                               causal=causal, q_pos0=q0)
    torch.cuda.synchronize()
    wo, wl = oracle.attention(to_f64(q), to_f64(k), to_f64(v), 1 / math.sqrt(D), causal)
    check_o(o, wo[:, q0:q0 + n], "bf16")
    check_lse(lse, wl[:, :, q0:q0 + n])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq,Skv,H,D", [(200, 2000, 2, 128), (1, 700, 3, 64), (300, 256, 1, 128),
                                        (129, 1111, 4, 128)])
def test_chunk_partial_small_grid_two_groups(causal, Sq, Skv, H, D):
    """A single chunk over few query tiles: each tile's keys are split between
    the two wave groups of one block and merged in LDS (no workspace)."""
    q, k, v = _qkv(1, Sq, Skv, H, D, torch.bfloat16, seed=Sq + Skv)
    say(f"chunk partial two groups Sq={Sq} Skv={Skv} H={H} D={D} causal={causal}")
    o, lse = cp.attn_chunk_partial(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal,
                                   q_pos0=Skv - Sq if causal else 0)
    torch.cuda.synchronize()
    qp = np.arange(Sq) + (Skv - Sq if causal else 0)
    wo, wl = oracle.attention(to_f64(q), to_f64(k), to_f64(v), 1 / math.sqrt(D), causal,
                              q_pos=qp, k_pos=np.arange(Skv))
    check_o(o, wo, "bf16")
    check_lse(lse, wl)


@pytest.mark.parametrize("Sq", [
    128 * 75,        # 300 query tiles
    128 * 100 - 3,   # 400 query tiles, the last ragged
])
def test_ring_key_splits_across_blocks(Sq):
    """Between one and two query tiles per CU: each tile's keys are split over
    two blocks whose fp32 partials go through the workspace."""
    lens = (1024, 1040)
    S, H, D = sum(lens), 4, 128
    q = synthetic.make_tensor((1, Sq, H, D), torch.bfloat16, 41)
    k = synthetic.make_tensor((1, S, H, D), torch.bfloat16, 42)
    v = synthetic.make_tensor((1, S, H, D), torch.bfloat16, 43)
    chunks = _chunk_tensors(k.to(DEV), v.to(DEV), lens)
    ws = cp.ring_attention_workspace_bytes(2, 1, H, Sq, D)
    assert ws > 0, "expected a split across blocks for this grid"
    say(f"ring with key splits across blocks, Sq={Sq}, workspace {ws} bytes")
    o, lse = cp.ring_attention(q.to(DEV), chunks)
    torch.cuda.synchronize()
    rows = np.arange(0, Sq, 37)
    wo, wl = oracle.attention(to_f64(q[:, rows]), to_f64(k), to_f64(v), 1 / math.sqrt(D))
    check_o(o[:, torch.from_numpy(rows).to(DEV)], wo, "bf16")
    check_lse(lse[:, :, torch.from_numpy(rows).to(DEV)], wl)
    with pytest.raises(cp.CpAttnError) as e:
        cp.ring_attention(q.to(DEV), chunks,
                          workspace=torch.empty(ws - 16, dtype=torch.uint8, device=DEV))
    assert e.value.status == 4


@pytest.mark.parametrize("Sq,H,D,lens", [
    (1, 1, 64, (4000,)),                   # one query row
    (300, 3, 128, (1025, 1025, 1024)),     # 9 ragged query tiles
    (130, 2, 64, (64, 0, 900, 77)),        # empty and one-tile chunks
])
def test_ring_small_grids(Sq, H, D, lens):
    """Grids smaller than the GPU: each query tile's keys are split between the
    two wave groups of its block and merged in LDS. Checked against the oracle,
    with a garbage-filled workspace, and for byte-identical repeats."""
    S = sum(lens)
    q, k, v = _qkv(1, Sq, S, H, D, torch.bfloat16, seed=Sq + S)
    chunks = _chunk_tensors(k.to(DEV), v.to(DEV), lens)
    qd = q.to(DEV)
    need = cp.ring_attention_workspace_bytes(len(lens), 1, H, Sq, D)
    ws = torch.full((max(need, 16),), 255, dtype=torch.uint8, device=DEV)
    say(f"small grid Sq={Sq} H={H} D={D} lens={lens}")
    o1, l1 = cp.ring_attention(qd, chunks, workspace=ws)
    o2, l2 = cp.ring_attention(qd, chunks, workspace=ws)
    o3, l3 = cp.ring_attention(qd, chunks, workspace=torch.zeros_like(ws))
    torch.cuda.synchronize()
    wo, wl = oracle.attention(to_f64(q), to_f64(k), to_f64(v), 1 / math.sqrt(D))
    check_o(o1, wo, "bf16")
    check_lse(l1, wl)
    for o, l in ((o2, l2), (o3, l3)):
        assert torch.equal(o.view(torch.uint8), o1.view(torch.uint8))
        assert torch.equal(l.view(torch.uint8), l1.view(torch.uint8))


@pytest.mark.parametrize("B,H,Sq,lens,causal,q0", [
    (2, 16, 1025, (600, 555), False, 0),      # a 1-row last tile
    (2, 16, 1041, (1041, 200), True, 0),      # 17 rows, causal: the tail sees part of the keys
    (1, 32, 1056, (700, 0, 900), False, 0),   # 32 rows, an empty chunk
    (1, 32, 1030, (1030, 1030), True, 1030),  # causal, queries in the second chunk
])
def test_ring_short_last_tile(B, H, Sq, lens, causal, q0):
    """Grids of one to two query tiles per CU (non-causal: keys split across
    blocks through the workspace) whose last tile holds at most 32 rows. The
    first rows, the rows before the last tile and the last tile itself
    against the oracle."""
    D = 128
    say(f"ring short last tile B={B} H={H} Sq={Sq} lens={lens} causal={causal}")
    q, k, v = _qkv(B, Sq, sum(lens), H, D, torch.bfloat16, seed=Sq + H)
    kd, vd = k.to(DEV), v.to(DEV)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(int)
    chunks = [(kd[:, s:s + n].contiguous(), vd[:, s:s + n].contiguous(), int(s))
              for s, n in zip(starts, lens)]
    o, lse = cp.ring_attention(q.to(DEV), chunks[::-1], causal=causal, q_pos0=q0)
    torch.cuda.synchronize()
    rows = np.r_[0:40, Sq - 200:Sq]   # first rows, the rows before the seam, the tail
    wo, wl = oracle.chunk_partial(to_f64(q)[:, rows], to_f64(k), to_f64(v), 1 / math.sqrt(D),
                                  causal, q0 + rows, np.arange(sum(lens)))
    check_o(o[:, rows], wo, "bf16", "O")
    check_lse(lse[:, :, rows], wl, "LSE")


def test_ring_zero_chunks():
    say("ring with P = 0")
    q = synthetic.make_tensor((1, 40, 2, 64), torch.bfloat16, 1).to(DEV)
    o, lse = cp.ring_attention(q, [])
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_partials_plus_merge_equal_ring():
    """Per-hop partials merged by cp_lse_merge agree with the fused ring (bf16)."""
    lens = (96, 160, 128, 64)
    S, H, D = sum(lens), 3, 128
    q, k, v = _qkv(1, S, S, H, D, torch.bfloat16, seed=99)
    chunks = _chunk_tensors(k.to(DEV), v.to(DEV), lens)
    qd = q[:, 96:256].contiguous().to(DEV)
    order = synthetic.ring_order(1, 4)
    say("partials + merge vs fused ring")
    parts = [cp.attn_chunk_partial(qd, chunks[c][0], chunks[c][1], causal=True, q_pos0=96,
                                   kv_pos0=chunks[c][2]) for c in order]
    po = torch.stack([p[0] for p in parts])
    pl = torch.stack([p[1] for p in parts])
    mo, ml = cp.lse_merge(po, pl, out_dtype=torch.bfloat16)
    ro, rl = cp.ring_attention(qd, [chunks[c] for c in order], causal=True, q_pos0=96)
    torch.cuda.synchronize()
    wo, wl = oracle.attention(to_f64(q), to_f64(k), to_f64(v), 1 / math.sqrt(D), True)
    for o, l in ((mo, ml), (ro, rl)):
        check_o(o, wo[:, 96:256], "bf16")
        check_lse(l, wl[:, :, 96:256])
    # the GPU partials themselves against the oracle's per-chunk partials
    for (o_c, l_c), c in zip(parts, order):
        kc, vc, p0 = chunks[c]
        w_o, w_l = oracle.chunk_partial(to_f64(q[:, 96:256]), to_f64(kc), to_f64(vc),
                                        1 / math.sqrt(D), True, np.arange(96, 256),
                                        np.arange(p0, p0 + lens[c]))
        check_o(o_c, w_o, "bf16", f"O_{c}")
        check_lse(l_c, w_l, f"LSE_{c}")


# ----------------------------------------------------------- determinism / guards

def test_repeat_runs_are_byte_identical():
    q, k, v = _qkv(1, 333, 500, 3, 128, torch.bfloat16, seed=7)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    chunks = _chunk_tensors(k, v, (200, 300))
    say("determinism")
    a = [cp.attn_chunk_partial(q, k, v, causal=True), cp.ring_attention(q, chunks, causal=True)]
    b = [cp.attn_chunk_partial(q, k, v, causal=True), cp.ring_attention(q, chunks, causal=True)]
    parts_o = torch.stack([a[0][0], a[0][0]])
    parts_l = torch.stack([a[0][1], a[0][1] - 1.0])
    m1 = cp.lse_merge(parts_o, parts_l)
    m2 = cp.lse_merge(parts_o, parts_l)
    torch.cuda.synchronize()
    for (o1, l1), (o2, l2) in zip(a + [m1], b + [m2]):
        assert torch.equal(o1.view(torch.uint8), o2.view(torch.uint8))
        assert torch.equal(l1.view(torch.uint8), l2.view(torch.uint8))


def test_outputs_stay_inside_their_buffers():
    """Canary regions around every output are untouched (no out-of-bounds writes)."""
    B, Sq, Skv, H, D = 1, 157, 201, 2, 128
    q, k, v = _qkv(B, Sq, Skv, H, D, torch.bfloat16, seed=11)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    pad = 4096
    n_o, n_l = B * Sq * H * D, B * H * Sq
    o_buf = torch.full((n_o + 2 * pad,), 12345.0, device=DEV)
    l_buf = torch.full((n_l + 2 * pad,), 12345.0, device=DEV)
    o = o_buf[pad:pad + n_o].view(B, Sq, H, D)
    lse = l_buf[pad:pad + n_l].view(B, H, Sq)
    say("canaries")
    cp.attn_chunk_partial(q, k, v, o, lse, causal=True, q_pos0=50)
    x = synthetic.make_tensor((4, 1, 13, 8, 128), torch.bfloat16, 2).to(DEV)
    y_buf = torch.full((x.numel() + 2 * pad,), 3.0, dtype=torch.bfloat16, device=DEV)
    cp.ulysses_seq2head(x, 4, y_buf[pad:pad + x.numel()].view(4, 1, 52, 2, 128))
    torch.cuda.synchronize()
    for buf, n, val in ((o_buf, n_o, 12345.0), (l_buf, n_l, 12345.0), (y_buf, x.numel(), 3.0)):
        assert torch.all(buf[:pad] == val) and torch.all(buf[pad + n:] == val)


@pytest.mark.parametrize("causal", [False, True])
def test_keys_past_a_chunk_are_never_read(causal):
    """Each K/V chunk is a view whose memory continues with NaN rows. The
    kernels must not read past a chunk's length (a ragged last tile's missing
    keys come in as zeros through the load's range check): any NaN V row
    read would turn O into NaN, as would a NaN K row that escaped the mask."""
    B, Sq, H, D = 1, 150, 3, 128
    lens = (201, 64, 1000, 37)
    say(f"NaN rows after every chunk, causal={causal}")
    q, k, v = _qkv(B, Sq, sum(lens), H, D, torch.bfloat16, seed=41)
    chunks, k_parts, v_parts, pos = [], [], [], 0
    for n in lens:
        kb = torch.full((B, n + 64, H, D), float("nan"), dtype=torch.bfloat16)
        vb = torch.full((B, n + 64, H, D), float("nan"), dtype=torch.bfloat16)
        kb[:, :n] = k[:, pos:pos + n]
        vb[:, :n] = v[:, pos:pos + n]
        kb, vb = kb.to(DEV), vb.to(DEV)
        chunks.append((kb[:, :n], vb[:, :n], pos))
        pos += n
    qd = q.to(DEV)
    qp = 700 if causal else 0
    ro, rl = cp.ring_attention(qd, chunks[::-1], causal=causal, q_pos0=qp)
    po, pl = cp.attn_chunk_partial(qd, chunks[2][0], chunks[2][1], causal=causal, q_pos0=qp,
                                   kv_pos0=chunks[2][2], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(ro.float()).all() and torch.isfinite(po).all()
    wo, wl = oracle.chunk_partial(to_f64(q), to_f64(k), to_f64(v), 1.0 / math.sqrt(D), causal,
                                  np.arange(qp, qp + Sq), np.arange(0, pos))
    check_o(ro, wo, "bf16", "ring O")
    check_lse(rl, wl, "ring LSE")
    p0 = chunks[2][2]
    wpo, wpl = oracle.chunk_partial(to_f64(q), to_f64(k[:, p0:p0 + lens[2]]),
                                    to_f64(v[:, p0:p0 + lens[2]]), 1.0 / math.sqrt(D), causal,
                                    np.arange(qp, qp + Sq), np.arange(p0, p0 + lens[2]))
    check_o(po, wpo, "bf16", "partial O")
    check_lse(pl, wpl, "partial LSE")


def test_rejected_call_leaves_outputs_untouched():
    q = synthetic.make_tensor((1, 64, 6, 128), torch.bfloat16, 1).to(DEV)
    o = torch.full((1, 64, 6, 128), 5.0, device=DEV)
    lse = torch.full((1, 6, 64), 5.0, device=DEV)
    say("rejected calls")
    with pytest.raises(cp.CpAttnError):
        cp.attn_chunk_partial(q, q, q, o, lse, scale=float("nan"))
    x = synthetic.make_tensor((4, 1, 8, 6, 128), torch.bfloat16, 2).to(DEV)
    y = torch.full((4, 1, 32, 1, 128), 5.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(cp.CpAttnError) as e:
        cp._check("cp_ulysses_seq2head", cp._seq2head(x.data_ptr(), y.data_ptr(), 4, 1, 8, 6, 128,
                                                      0, None))
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert torch.all(o == 5.0) and torch.all(lse == 5.0) and torch.all(y == 5.0)


@pytest.mark.parametrize("n,P,B,S_l,H,D,dtype", [
    (3, 4, 1, 37, 8, 128, torch.bfloat16),    # a rank's Q, K, V
    (2, 8, 2, 5, 40, 128, torch.bfloat16),
    (3, 2, 1, 9, 4, 5, torch.float32),        # 4-byte words
    (3, 3, 2, 4, 6, 3, torch.bfloat16),       # 2-byte words
])
def test_relayout_stacked_tensors_bit_exact(n, P, B, S_l, H, D, dtype):
    """One launch over n tensors back to back equals n single-tensor relayouts."""
    say(f"stacked relayout n={n} P={P} B={B} S_l={S_l} H={H} D={D} {dtype}")
    isz = 2 if dtype == torch.bfloat16 else 4
    bits = synthetic.random_bits((n, P, B, S_l, H, D), isz, seed=n * 1000 + P * 10 + D)
    x = bits.view(dtype).to(DEV)
    y = cp.ulysses_seq2head(x, P)
    z = cp.ulysses_head2seq(y, P)
    torch.cuda.synchronize()
    yb = y.cpu().view(bits.dtype).numpy()
    for t in range(n):
        assert np.array_equal(yb[t], oracle.seq2head(bits[t].numpy(), P)), f"tensor {t}"
    assert np.array_equal(z.cpu().view(bits.dtype).numpy(), bits.numpy())
