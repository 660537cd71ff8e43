"""cp_ring_attention_noalloc against cp_ring_attention through the C ABI.

The no-alloc entry point keeps the key-split partials in the library's static
device scratch instead of a caller workspace; it shares the kernels, so its
outputs must equal cp_ring_attention's bit for bit. Two calls in a row, the
second on a smaller input, both large enough to split keys (so both use the
scratch, and the second finds the first's leftovers there), then an fp32 call
(no scratch) and a call whose scratch need exceeds the built-in limit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from _parity import BF16_MAX, LSE_MAX, say, to_f64

pytestmark = pytest.mark.gpu

cp = pytest.importorskip("context_attention_dit_amd")


def _case(H, Sq, lens, seed, dtype=torch.bfloat16, D=128):
    S = sum(lens)
    q = synthetic.make_tensor((1, Sq, H, D), dtype, seed).cuda()
    k = synthetic.make_tensor((1, S, H, D), dtype, seed + 1).cuda()
    v = synthetic.make_tensor((1, S, H, D), dtype, seed + 2).cuda()
    chunks, s0 = [], 0
    for n in lens:
        chunks.append((k[:, s0:s0 + n].contiguous(), v[:, s0:s0 + n].contiguous(), s0))
        s0 += n
    return q, k, v, chunks


def _compare(q, k, v, chunks, causal=False, q_pos0=0):
    B, Sq, H, D = q.shape
    need = cp.ring_attention_workspace_bytes(len(chunks), B, H, Sq, D)
    o_ref, l_ref = cp.ring_attention(q, chunks, causal=causal, q_pos0=q_pos0)
    o = torch.full_like(o_ref, 7.0)
    lse = torch.full_like(l_ref, 7.0)
    cp.ring_attention_noalloc(q, chunks, o, lse, causal=causal, q_pos0=q_pos0)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o,
                       o_ref.view(torch.int16) if o.dtype == torch.bfloat16 else o_ref)
    assert torch.equal(lse, l_ref)
    # a few rows against the oracle as well
    rows = np.unique(np.linspace(0, Sq - 1, 6).astype(int))
    qf = to_f64(q)[:, rows]
    wo, wl = oracle.attention(qf, to_f64(k), to_f64(v), 1 / math.sqrt(D), causal=causal,
                              q_pos=q_pos0 + rows, k_pos=np.arange(k.shape[1]))
    err = np.abs(to_f64(o)[:, rows] - wo).max()
    bar = BF16_MAX if q.dtype == torch.bfloat16 else 1e-5
    assert err <= bar, f"O max-abs {err:.3e}"
    assert np.abs(to_f64(lse)[:, :, rows] - wl).max() <= LSE_MAX
    return need


def test_noalloc_matches_ring_twice_then_smaller():
    # ring-anything rank 0 (S 4099, H 32, chunks 1025/1025/1025/1024): 288 query
    # tiles, the last one a single row: the 256 full tiles as two-group blocks,
    # the last row's keys split 8 ways with their partials in the scratch
    say("noalloc: call 1, Sq 1025 H 32, chunks 1025/1025/1025/1024")
    q, k, v, ch = _case(32, 1025, [1025, 1025, 1025, 1024], 4100)
    need1 = _compare(q, k, v, ch)
    assert 0 < need1 <= cp.NOALLOC_SCRATCH_BYTES
    del q, k, v, ch
    # 260 query tiles, two key splits over blocks
    say("noalloc: call 2 (smaller), Sq 1250 H 26, chunks 1250/777/513")
    q, k, v, ch = _case(26, 1250, [1250, 777, 513], 4200)
    need2 = _compare(q, k, v, ch)
    assert 0 < need2 < need1


def test_noalloc_one_chunk_last_round_split():
    # one chunk, 280 query tiles of 256 rows: the last round's 24 tiles split
    # their keys 8 ways, partials in the scratch (ring call: in its workspace)
    say("noalloc: one chunk, Sq 1792 H 40, 2100 keys (last round split)")
    q, k, v, ch = _case(40, 1792, [2100], 4300)
    need = _compare(q, k, v, ch)
    assert 0 < need <= cp.NOALLOC_SCRATCH_BYTES
    del q, k, v, ch


def test_noalloc_causal_and_fp32():
    say("noalloc: causal ring-anything rank 2 shape, Sq 1025 H 32")
    q, k, v, ch = _case(32, 1025, [1025, 1025, 1025, 1024], 4250)
    _compare(q, k, v, ch, causal=True, q_pos0=2050)
    del q, k, v, ch
    say("noalloc: causal ragged ring (no split), Sq 700 H 8")
    q, k, v, ch = _case(8, 700, [300, 500, 211], 4300)
    _compare(q, k, v, ch, causal=True, q_pos0=250)
    say("noalloc: fp32 ring, Sq 96 H 2 D 64")
    q, k, v, ch = _case(2, 96, [64, 40], 4400, dtype=torch.float32, D=64)
    _compare(q, k, v, ch)


def test_noalloc_rejects_sizes_beyond_scratch():
    # one head, 511 query tiles, a list of two chunks: two key splits of
    # 65408 x 128 fp32 partials exceed 64 MiB (one chunk would not split)
    B, H, D = 1, 1, 128
    Sq = 511 * 128
    need = cp.ring_attention_workspace_bytes(2, B, H, Sq, D)
    assert need > cp.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, Sq, H, D), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((B, 4096, H, D), dtype=torch.bfloat16, device="cuda")
    o, lse = torch.empty_like(q), torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
    with pytest.raises(cp.CpAttnError) as e:
        cp.ring_attention_noalloc(q, [(kv, kv, 0), (kv, kv, 4096)], o, lse)
    assert e.value.status == 4
