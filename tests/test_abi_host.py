"""Host-only checks of the C ABI: the library loads, exports what the header
declares, and rejects bad arguments before anything reaches the GPU.

No call here launches work: every call either fails validation or is a
zero-sized no-op, both of which return before any HIP call.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cp_attn.h")

cp = pytest.importorskip("context_attention_dit_amd")
lib = ctypes.CDLL(cp.LIB_PATH)

OK, INVALID, UNSUPPORTED, DIVISIBILITY, WORKSPACE = 0, 1, 2, 3, 4
BF16, F32 = 0, 1
FAKE = 0x7f0000000000      # a 16-byte aligned address that is never dereferenced
FAKE2 = 0x7f1000000000
FAKE3 = 0x7f2000000000
FAKE4 = 0x7f3000000000
FAKE5 = 0x7f4000000000
FAKE6 = 0x7f5000000000     # fake workspace


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(cp_\w+)\s*\(", text, re.M)))


def test_header_functions_exported():
    names = _declared_functions()
    assert {"cp_attn_chunk_partial", "cp_lse_merge", "cp_ring_attention",
            "cp_ring_attention_workspace_bytes", "cp_ulysses_seq2head", "cp_ulysses_head2seq",
            "cp_last_error", "cp_abi_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in cp_attn.h but not exported"


def test_abi_version_matches_header():
    m = re.search(r"#define\s+CP_ATTN_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert cp.abi_version() == int(m.group(1))


def test_max_chunks_matches_header():
    m = re.search(r"#define\s+CP_MAX_RING_CHUNKS\s+(\d+)", open(HEADER).read())
    assert cp.MAX_RING_CHUNKS == int(m.group(1))


def _partial(q=FAKE, k=FAKE2, v=FAKE3, o=FAKE4, lse=FAKE5, B=1, H=2, Sq=8, Skv=8, D=128,
             dt=BF16, odt=F32, scale=0.1, causal=0, qp=0, kp=0):
    return cp._chunk_partial(q, k, v, o, lse, B, H, Sq, Skv, D, dt, odt, scale, causal, qp, kp, None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=96), UNSUPPORTED),
    (dict(D=0), UNSUPPORTED),
    (dict(B=-1), INVALID),
    (dict(Sq=-3), INVALID),
    (dict(Skv=-1), INVALID),
    (dict(q=None), INVALID),
    (dict(o=None), INVALID),
    (dict(k=None), INVALID),
    (dict(q=FAKE + 8), INVALID),
    (dict(lse=FAKE5 + 2), INVALID),
    (dict(o=FAKE + 64), INVALID),           # output overlaps q
    (dict(lse=FAKE2 + 16), INVALID),        # lse overlaps k
    (dict(dt=F32, odt=BF16), UNSUPPORTED),
    (dict(dt=7), INVALID),
    (dict(odt=9), INVALID),
    (dict(causal=2), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(Sq=1 << 30), UNSUPPORTED),
    (dict(Skv=1 << 30), UNSUPPORTED),
    (dict(B=1 << 20, H=1 << 20), UNSUPPORTED),
])
def test_chunk_partial_rejects(kw, status):
    assert _partial(**kw) == status
    assert cp.last_error().startswith("cp_attn_chunk_partial")


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(Sq=0), dict(Sq=0, q=None, o=None)])
def test_chunk_partial_zero_size_is_noop(kw):
    assert _partial(**kw) == OK
    assert cp.last_error() == ""


def _merge(o_parts=FAKE, lse_parts=FAKE2, P=4, o=FAKE3, lse=FAKE4, B=1, H=2, Sq=8, D=128, odt=F32):
    return cp._lse_merge(o_parts, lse_parts, P, o, lse, B, H, Sq, D, odt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(P=0), INVALID), (dict(P=-1), INVALID), (dict(D=6), UNSUPPORTED), (dict(o=None), INVALID),
    (dict(D=4100), UNSUPPORTED),
    (dict(lse_parts=FAKE2 + 2), INVALID), (dict(o=FAKE + 128), INVALID), (dict(odt=3), INVALID),
    (dict(B=-2), INVALID),
])
def test_merge_rejects(kw, status):
    assert _merge(**kw) == status
    assert cp.last_error().startswith("cp_lse_merge")


def test_merge_zero_size_is_noop():
    assert _merge(Sq=0) == OK


def _ring(P=4, chunks=None, q=FAKE, o=FAKE4, lse=FAKE5, B=1, H=2, Sq=8, D=128, dt=BF16, scale=0.1,
          causal=0, ws=FAKE6, ws_bytes=1 << 30):
    if chunks is None:
        chunks = [(FAKE2 + c * 4096, FAKE3 + c * 4096, 8, 8 * c) for c in range(max(P, 0))]
    arr = (cp.KVChunk * max(1, len(chunks)))(*[cp.KVChunk(*c) for c in chunks])
    return cp._ring(q, arr, P, o, lse, B, H, Sq, D, dt, scale, causal, 0, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(P=-1), INVALID), (dict(P=65), UNSUPPORTED), (dict(D=32), UNSUPPORTED),
    (dict(q=None), INVALID), (dict(o=FAKE + 16), INVALID),
    (dict(chunks=[(FAKE2, None, 8, 0)], P=1), INVALID),
    (dict(chunks=[(FAKE2, FAKE3, -1, 0)], P=1), INVALID),
    (dict(chunks=[(FAKE2 + 4, FAKE3, 8, 0)], P=1), INVALID),
    (dict(chunks=[(FAKE4, FAKE3, 8, 0)], P=1), INVALID),      # output overlaps a chunk
    (dict(dt=F32, D=96), UNSUPPORTED),
    # 300 query tiles (between one and two per CU): the grid needs a workspace
    (dict(H=300, ws=FAKE6 + 8), INVALID),                      # misaligned workspace
    (dict(H=300, ws=FAKE4 + 64), INVALID),                     # workspace overlaps the output
])
def test_ring_rejects(kw, status):
    assert _ring(**kw) == status
    assert cp.last_error().startswith("cp_ring_attention")


def test_ring_zero_size_is_noop_and_workspace_query():
    assert _ring(Sq=0) == OK
    # at most one query tile per CU: keys are split inside the block, no workspace
    assert cp.ring_attention_workspace_bytes(4, 1, 24, 1152, 128) == 0
    # 300 query tiles: split across blocks through the workspace
    n = cp.ring_attention_workspace_bytes(4, 1, 300, 8, 128)
    assert n > 0
    assert _ring(H=300, ws=None, ws_bytes=0) == WORKSPACE
    assert _ring(H=300, ws_bytes=n - 16) == WORKSPACE


def test_workspace_query_one_chunk_last_round():
    # one chunk: the query also covers the optional key split of a last round
    # of 256-row tiles that is at most half full. Wan rank (5 heads x 128
    # tiles = 640 on 256 CUs, 128 in the last round): 2 splits x 128 tiles x
    # 256 rows x (128 + 1) fp32; with two chunks (or none of that) nothing
    assert cp.ring_attention_workspace_bytes(1, 1, 5, 32760, 128) == 2 * 128 * 256 * 129 * 4
    assert cp.ring_attention_workspace_bytes(2, 1, 5, 32760, 128) == 0
    # 280 tiles (24 in the last round): up to 8 splits
    assert cp.ring_attention_workspace_bytes(1, 1, 40, 1792, 128) == 8 * 24 * 256 * 129 * 4
    # exactly 5 rounds (K/V-gather rank), or a last round more than half full
    # (400 tiles, 144 in the last round): no split
    assert cp.ring_attention_workspace_bytes(1, 1, 10, 32760, 128) == 0
    assert cp.ring_attention_workspace_bytes(1, 1, 100, 1024, 128) == 0
    # D = 64 keeps the two-group last round
    assert cp.ring_attention_workspace_bytes(1, 1, 5, 32760, 64) == 0
    # between one and two 128-row tiles per CU (Qwen-Image rank, 444 tiles): a
    # chunk list splits keys across blocks, one chunk does not
    assert cp.ring_attention_workspace_bytes(2, 1, 6, 9472, 128) > 0
    assert cp.ring_attention_workspace_bytes(1, 1, 6, 9472, 128) == 0
    # one chunk with a one-row last tile (4099-token ring rank): that row's split
    assert 0 < cp.ring_attention_workspace_bytes(1, 1, 32, 1025, 128) < 8 * 32 * 129 * 4 + 1


def test_ring_fp32_needs_no_workspace():
    # the fp32 path never splits keys: at a size where bf16 needs a workspace, an
    # fp32 call without one passes the workspace check (and here fails on the
    # misaligned LSE that follows it, so nothing is launched)
    assert cp.ring_attention_workspace_bytes(4, 1, 300, 8, 128) > 0
    assert _ring(H=300, dt=BF16, ws=None, ws_bytes=0, lse=FAKE5 + 2) == WORKSPACE
    assert _ring(H=300, dt=F32, ws=None, ws_bytes=0, lse=FAKE5 + 2) == INVALID
    assert "misaligned" in cp.last_error()


def test_noalloc_scratch_size_matches_header():
    m = re.search(r"#define\s+CP_NOALLOC_SCRATCH_BYTES\s+(\d+)", open(HEADER).read())
    assert cp.NOALLOC_SCRATCH_BYTES == int(m.group(1))


def _ring_noalloc(P=4, q=FAKE, o=FAKE4, lse=FAKE5, B=1, H=2, Sq=8, D=128, dt=BF16, scale=0.1,
                  causal=0):
    chunks = [(FAKE2 + c * 4096, FAKE3 + c * 4096, 8, 8 * c) for c in range(max(P, 0))]
    arr = (cp.KVChunk * max(1, len(chunks)))(*[cp.KVChunk(*c) for c in chunks])
    return cp._ring_noalloc(q, arr, P, o, lse, B, H, Sq, D, dt, scale, causal, 0, None)


def test_noalloc_rejects_before_any_launch():
    assert _ring_noalloc(Sq=0) == OK
    assert _ring_noalloc(P=-1) == INVALID
    assert cp.last_error().startswith("cp_ring_attention_noalloc")
    assert _ring_noalloc(q=None) == INVALID
    # sizes whose key-split partials exceed the static scratch: rejected with
    # CP_E_WORKSPACE, whatever the chunks
    Sq = next(t * 128 for t in range(257, 100000)
              if cp.ring_attention_workspace_bytes(4, 1, 1, t * 128, 128)
              > cp.NOALLOC_SCRATCH_BYTES)
    assert _ring_noalloc(H=1, Sq=Sq) == WORKSPACE
    assert "scratch" in cp.last_error()


def _relayout(fn, inp=FAKE, out=FAKE2, P=4, B=1, S=8, H=8, D=128, dt=BF16):
    return fn(inp, out, P, B, S, H, D, dt, None)


@pytest.mark.parametrize("name", ["_seq2head", "_head2seq"])
@pytest.mark.parametrize("kw,status", [
    (dict(H=6), DIVISIBILITY), (dict(H=10, P=3), DIVISIBILITY), (dict(P=0), INVALID),
    (dict(B=-1), INVALID), (dict(inp=None), INVALID), (dict(out=FAKE + 256), INVALID),
    (dict(dt=5), INVALID), (dict(inp=FAKE + 1), INVALID),
])
def test_relayout_rejects(name, kw, status):
    fn = getattr(cp, name)
    assert _relayout(fn, **kw) == status
    assert cp.last_error().startswith("cp_ulysses")


def test_relayout_zero_size_is_noop():
    assert _relayout(cp._seq2head, S=0) == OK
    assert _relayout(cp._head2seq, D=0, inp=None, out=None) == OK


def _anything(fn, inp=FAKE, out=FAKE2, P=3, B=1, s_lens=(4, 3, 3), h_counts=(2, 2, 1), D=128,
              dt=BF16):
    sa, sp = cp._counts(s_lens) if s_lens is not None else (None, None)
    ha, hp = cp._counts(h_counts) if h_counts is not None else (None, None)
    return fn(inp, out, P, B, sp, hp, D, dt, None)


@pytest.mark.parametrize("name", ["_any_seq2head", "_any_head2seq"])
@pytest.mark.parametrize("kw,status", [
    (dict(P=0), INVALID), (dict(P=65, s_lens=[1] * 65, h_counts=[1] * 65), UNSUPPORTED),
    (dict(s_lens=None), INVALID), (dict(h_counts=None), INVALID),
    (dict(s_lens=(4, -1, 3)), INVALID), (dict(h_counts=(2, 2, -3)), INVALID),
    (dict(B=-1), INVALID), (dict(D=-2), INVALID), (dict(dt=5), INVALID),
    (dict(inp=None), INVALID), (dict(out=FAKE + 512), INVALID), (dict(inp=FAKE + 1), INVALID),
    (dict(B=1 << 16), UNSUPPORTED),
])
def test_anything_relayout_rejects(name, kw, status):
    assert _anything(getattr(cp, name), **kw) == status
    assert cp.last_error().startswith("cp_ulysses_anything")


@pytest.mark.parametrize("kw", [dict(B=0), dict(D=0), dict(s_lens=(0, 0, 0)),
                                dict(h_counts=(0, 0, 0), inp=None, out=None)])
def test_anything_relayout_zero_size_is_noop(kw):
    assert _anything(cp._any_seq2head, **kw) == OK
    assert _anything(cp._any_head2seq, **kw) == OK


@pytest.mark.parametrize("kw,status", [
    (dict(P=0), INVALID), (dict(P=65), UNSUPPORTED), (dict(H=-1), INVALID),
    (dict(s_lens=None), INVALID), (dict(inp=None), INVALID), (dict(dt=9), INVALID),
    (dict(out=FAKE + 64), INVALID),
])
def test_kv_gather_rejects(kw, status):
    args = dict(inp=FAKE, out=FAKE2, P=3, B=1, s_lens=(4, 3, 3), H=4, D=128, dt=BF16)
    args.update(kw)
    lens = args["s_lens"]
    if lens is not None and len(lens) != args["P"] and args["P"] > 0:
        lens = [1] * args["P"]
    arr, ptr = cp._counts(lens) if lens is not None else (None, None)
    assert cp._kv_gather(args["inp"], args["out"], args["P"], args["B"], ptr, args["H"], args["D"],
                         args["dt"], None) == status
    assert cp.last_error().startswith("cp_kv_gather")


def _anything_n(fn, count, inp=FAKE, out=FAKE2, P=3, B=1, s_lens=(4, 3, 3), h_counts=(2, 2, 1),
                D=128, dt=BF16):
    sa, sp = cp._counts(s_lens)
    ha, hp = cp._counts(h_counts)
    return fn(inp, out, count, P, B, sp, hp, D, dt, None)


# one tensor of the default shape: B*S*H*D*2 = 1*10*5*128*2 bytes
ANY_BYTES = 10 * 5 * 128 * 2


@pytest.mark.parametrize("name", ["_any_seq2head_n", "_any_head2seq_n"])
@pytest.mark.parametrize("kw,status", [
    (dict(count=0), INVALID), (dict(count=-1), INVALID), (dict(count=65536), UNSUPPORTED),
    (dict(count=256, B=256), UNSUPPORTED),                  # B*count must stay below 2^16
    (dict(count=2, out=FAKE + ANY_BYTES), INVALID),         # the second input overlaps out
    (dict(count=3, P=0), INVALID), (dict(count=3, inp=None), INVALID),
])
def test_anything_relayout_n_rejects(name, kw, status):
    kw = dict(kw)
    assert _anything_n(getattr(cp, name), kw.pop("count"), **kw) == status
    assert cp.last_error().startswith("cp_ulysses_anything")


def test_anything_relayout_n_zero_size_is_noop():
    assert _anything_n(cp._any_seq2head_n, 3, B=0) == OK
    assert _anything_n(cp._any_head2seq_n, 3, s_lens=(0, 0, 0), inp=None, out=None) == OK


@pytest.mark.parametrize("count,kw,status", [
    (0, {}, INVALID), (65536, {}, UNSUPPORTED), (2, dict(B=40000), UNSUPPORTED),
    (2, dict(out=FAKE + 10 * 4 * 128 * 2), INVALID),        # overlap from the second tensor on
    (2, dict(H=-1), INVALID),
])
def test_kv_gather_n_rejects(count, kw, status):
    args = dict(inp=FAKE, out=FAKE2, P=3, B=1, H=4, D=128, dt=BF16)
    args.update(kw)
    arr, ptr = cp._counts((4, 3, 3))
    assert cp._kv_gather_n(args["inp"], args["out"], count, args["P"], args["B"], ptr, args["H"],
                           args["D"], args["dt"], None) == status
    assert cp.last_error().startswith("cp_kv_gather_n")


# ---- the Python binding checks the buffers the C ABI only sees as addresses
# (these raise before any pointer is taken, so they run on CPU tensors)

def test_binding_rejects_wrong_output_buffers():
    import torch
    bf = torch.bfloat16
    x = torch.zeros((2, 1, 3, 4, 8), dtype=bf)
    with pytest.raises(ValueError, match="out must be"):
        cp.ulysses_seq2head(x, 2, torch.zeros((2, 1, 6, 2, 7), dtype=bf))     # short last dim
    with pytest.raises(ValueError, match="out must be"):
        cp.ulysses_seq2head(x, 2, torch.zeros((2, 1, 6, 2, 8), dtype=torch.float32))
    y = torch.zeros((2, 1, 6, 2, 8), dtype=bf)
    with pytest.raises(ValueError, match="out must be"):
        cp.ulysses_head2seq(y, 2, torch.zeros((2, 1, 3, 4, 4), dtype=bf))
    flat = torch.zeros(1 * 5 * 3 * 8, dtype=bf)
    with pytest.raises(ValueError, match="out must be"):
        cp.ulysses_anything_seq2head(flat, (2, 3), (1, 2), 1, 8, torch.zeros(119, dtype=bf))
    with pytest.raises(ValueError, match="packed tensor"):
        cp.ulysses_anything_seq2head(flat[:-1], (2, 3), (1, 2), 1, 8)
    with pytest.raises(ValueError, match="out must be"):
        cp.kv_gather(flat, (2, 3), 1, 3, 8, torch.zeros((1, 5, 3, 4), dtype=bf))
    q = torch.zeros((1, 4, 2, 64), dtype=bf)
    with pytest.raises(ValueError, match="o must be"):
        cp.attn_chunk_partial(q, q, q, torch.zeros((1, 4, 2, 32)))
    with pytest.raises(ValueError, match="lse must be"):
        cp.attn_chunk_partial(q, q, q, None, torch.zeros((1, 2, 4), dtype=bf))
    with pytest.raises(ValueError, match="o must be"):
        cp.ring_attention(q, [(q, q, 0)], torch.zeros((1, 4, 2, 64)))        # not q's dtype
    parts = torch.zeros((2, 1, 4, 2, 64))
    with pytest.raises(ValueError, match="lse must be"):
        cp.lse_merge(parts, torch.zeros((2, 1, 2, 4)), None, torch.zeros((1, 2, 3)))


def test_binding_rejects_wrong_backward_inputs():
    import torch
    bf = torch.bfloat16
    q = torch.zeros((1, 4, 2, 64), dtype=bf)
    lse32 = torch.zeros((1, 2, 4))
    with pytest.raises(ValueError, match="lse must be"):
        cp.attn_chunk_backward(q, q, q, q, lse32.to(bf), lse32)
    with pytest.raises(ValueError, match="dout must be"):
        cp.attn_chunk_backward(q, q, q, q.float(), lse32, lse32)
    with pytest.raises(ValueError, match="delta must be"):
        cp.ring_attention_backward(q, [(q, q, 0)], q, lse32, lse32.to(bf))
    with pytest.raises(ValueError, match="delta must be"):
        cp.attn_backward_delta(q, q, torch.zeros((1, 2, 4), dtype=bf))
    with pytest.raises(ValueError, match="chunk 0 dk must be"):
        cp.ring_attention_backward(q, [(q, q, 0)], q, lse32, lse32,
                                   grads=[(torch.zeros((1, 4, 2, 32)), torch.zeros((1, 4, 2, 64)))])


def test_error_text_cleared_by_success():
    assert _partial(D=96) == UNSUPPORTED and cp.last_error() != ""
    assert _partial(Sq=0) == OK and cp.last_error() == ""


FAKE7, FAKE8, FAKE9, FAKE10 = 0x7f6000000000, 0x7f7000000000, 0x7f8000000000, 0x7f9000000000


def _chunk_bwd(q=FAKE, k=FAKE2, v=FAKE3, do=FAKE4, lse=FAKE5, delta=FAKE6, dq=FAKE7, dk=FAKE8,
               dv=FAKE9, B=1, H=2, Sq=8, Skv=8, D=128, dt=BF16, scale=0.1, causal=0, qp=0, kp=0,
               flags=0):
    return cp._chunk_bwd(q, k, v, do, lse, delta, dq, dk, dv, B, H, Sq, Skv, D, dt, scale, causal,
                         qp, kp, flags, None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=96), UNSUPPORTED), (dict(dt=7), INVALID),
    (dict(B=-1), INVALID), (dict(Skv=-1), INVALID), (dict(Skv=1 << 30), UNSUPPORTED),
    (dict(Sq=1 << 30), UNSUPPORTED), (dict(causal=2), INVALID),
    (dict(scale=float("inf")), INVALID), (dict(flags=4), INVALID),
    (dict(q=None), INVALID), (dict(do=None), INVALID), (dict(lse=None), INVALID),
    (dict(delta=None), INVALID), (dict(dq=None), INVALID), (dict(k=None), INVALID),
    (dict(dk=None), INVALID), (dict(dv=None), INVALID),
    (dict(q=FAKE + 8), INVALID), (dict(dq=FAKE7 + 4), INVALID), (dict(lse=FAKE5 + 2), INVALID),
    (dict(dq=FAKE + 64), INVALID),        # dq overlaps q
    (dict(dv=FAKE8 + 64), INVALID),       # dv overlaps dk
    (dict(dk=FAKE5), INVALID),            # dk overlaps lse
])
def test_chunk_backward_rejects(kw, status):
    assert _chunk_bwd(**kw) == status
    assert cp.last_error().startswith("cp_attn_chunk_backward")


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(Sq=0, Skv=0)])
def test_chunk_backward_zero_size_is_noop(kw):
    assert _chunk_bwd(**kw) == OK and cp.last_error() == ""


def _delta(o=FAKE, do=FAKE2, delta=FAKE3, B=1, H=2, Sq=8, D=128, dt=BF16):
    return cp._bwd_delta(o, do, delta, B, H, Sq, D, dt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=32), UNSUPPORTED), (dict(dt=5), INVALID), (dict(Sq=-2), INVALID),
    (dict(o=None), INVALID), (dict(delta=None), INVALID), (dict(do=FAKE2 + 8), INVALID),
    (dict(delta=FAKE + 4), INVALID),
])
def test_backward_delta_rejects(kw, status):
    assert _delta(**kw) == status
    assert cp.last_error().startswith("cp_attn_backward_delta")


def test_backward_delta_zero_size_is_noop():
    assert _delta(Sq=0, o=None, do=None, delta=None) == OK


def _ring_bwd(P=2, lens=(8, 8), q=FAKE, do=FAKE4, lse=FAKE5, delta=FAKE6, dq=FAKE7,
              kv=None, gr=None, B=1, H=2, Sq=8, D=128, dt=BF16, scale=0.1, causal=0, qp=0,
              flags=0, null_arrays=False):
    kv = kv or [(FAKE2 + 0x100000 * c, FAKE3 + 0x100000 * c) for c in range(P)]
    gr = gr or [(FAKE8 + 0x100000 * c, FAKE9 + 0x100000 * c) for c in range(P)]
    n = max(1, P)
    arr, garr = (cp.KVChunk * n)(), (cp.KVGrad * n)()
    for c in range(min(P, len(lens))):
        arr[c] = cp.KVChunk(kv[c][0], kv[c][1], lens[c], 8 * c)
        garr[c] = cp.KVGrad(gr[c][0], gr[c][1])
    if null_arrays:
        arr, garr = None, None
    return cp._ring_bwd(q, arr, P, do, lse, delta, dq, garr, B, H, Sq, D, dt, scale, causal, qp,
                        flags, None)


@pytest.mark.parametrize("kw,status", [
    (dict(P=0), INVALID), (dict(P=65), UNSUPPORTED), (dict(null_arrays=True), INVALID),
    (dict(dt=5), INVALID), (dict(D=80), UNSUPPORTED), (dict(flags=8), INVALID),
    (dict(lens=(8, -1)), INVALID), (dict(lens=(8, 1 << 30)), UNSUPPORTED),
    (dict(q=None), INVALID), (dict(dq=FAKE7 + 8), INVALID),
    (dict(kv=[(FAKE2, FAKE3), (None, FAKE3)]), INVALID),
    (dict(gr=[(FAKE8, FAKE9), (FAKE8 + 0x100000, None)]), INVALID),
    (dict(gr=[(FAKE8, FAKE9), (FAKE8, FAKE9 + 0x100000)]), INVALID),   # dk of both chunks alias
    (dict(gr=[(FAKE2, FAKE9), (FAKE8 + 0x100000, FAKE9 + 0x100000)]), INVALID),  # dk on K
    (dict(dq=FAKE8), INVALID),                                          # dq on a chunk's dk
])
def test_ring_backward_rejects(kw, status):
    assert _ring_bwd(**kw) == status
    assert cp.last_error().startswith("cp_ring_attention_backward")


def test_ring_backward_zero_size_is_noop():
    assert _ring_bwd(B=0) == OK
    assert _ring_bwd(Sq=0, lens=(0, 0)) == OK and cp.last_error() == ""


@pytest.mark.parametrize("name", ["_seq2head_n", "_head2seq_n"])
@pytest.mark.parametrize("count,kw,status", [
    (0, {}, INVALID), (65536, {}, UNSUPPORTED), (3, dict(H=6, P=4), DIVISIBILITY),
    (3, dict(out=FAKE + 3 * 4 * 1 * 8 * 8 * 128 * 2 - 64), INVALID),   # out overlaps the 3rd tensor
])
def test_batched_relayout_rejects(name, count, kw, status):
    args = dict(inp=FAKE, out=FAKE2, P=4, B=1, S=8, H=8, D=128, dt=BF16)
    args.update(kw)
    fn = getattr(cp, name)
    assert fn(args["inp"], args["out"], count, args["P"], args["B"], args["S"], args["H"],
              args["D"], args["dt"], None) == status
    assert cp.last_error().startswith("cp_ulysses")


def _partial_vt(**kw):
    a = dict(q=FAKE, k=FAKE2, v=FAKE3, o=FAKE4, lse=FAKE5, B=1, H=2, Sq=8, Skv=8, D=128, dt=BF16,
             odt=F32, scale=0.1, causal=0, qp=0, kp=0)
    a.update(kw)
    return cp._chunk_partial_vt(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Sq"],
                                a["Skv"], a["D"], a["dt"], a["odt"], a["scale"], a["causal"],
                                a["qp"], a["kp"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=64), UNSUPPORTED),                 # key-contiguous V: D = 128 only
    (dict(dt=F32, odt=F32), UNSUPPORTED),      # bf16 inputs only
    (dict(Skv=1 << 30), UNSUPPORTED),
    (dict(D=96), UNSUPPORTED),
    (dict(v=None), INVALID),
    (dict(v=FAKE3 + 8), INVALID),
    (dict(o=FAKE3 + 64), INVALID),             # output overlaps vt
    (dict(causal=2), INVALID),
])
def test_chunk_partial_vt_rejects(kw, status):
    assert _partial_vt(**kw) == status
    assert cp.last_error().startswith("cp_attn_chunk_partial_vt")


def test_chunk_partial_vt_zero_size_is_noop():
    assert _partial_vt(Sq=0) == OK
    assert _partial_vt(B=0, q=None, o=None) == OK


@pytest.mark.parametrize("kw,status", [
    (dict(H=6), DIVISIBILITY), (dict(P=0), INVALID), (dict(B=-1), INVALID),
    (dict(inp=None), INVALID), (dict(out=FAKE + 256), INVALID), (dict(dt=F32), UNSUPPORTED),
    (dict(dt=5), INVALID), (dict(D=96), UNSUPPORTED), (dict(inp=FAKE + 8), INVALID),
])
def test_seq2head_vt_rejects(kw, status):
    assert _relayout(cp._seq2head_vt, **kw) == status
    assert cp.last_error().startswith("cp_ulysses_seq2head_vt")


def test_seq2head_vt_zero_size_is_noop():
    assert _relayout(cp._seq2head_vt, S=0) == OK
    assert _relayout(cp._seq2head_vt, B=0, inp=None, out=None) == OK


@pytest.mark.parametrize("kw,status", [
    (dict(P=0), INVALID), (dict(B=-1), INVALID), (dict(inp=None), INVALID),
    (dict(out=FAKE + 256), INVALID), (dict(dt=F32), UNSUPPORTED), (dict(D=64), UNSUPPORTED),
    (dict(inp=FAKE + 8), INVALID),
])
def test_kv_gather_vt_rejects(kw, status):
    assert _relayout(cp._kv_gather_vt, **kw) == status
    assert cp.last_error().startswith("cp_kv_gather_vt")


def test_kv_gather_vt_any_head_count_and_zero_size():
    assert _relayout(cp._kv_gather_vt, S=0) == OK
    assert _relayout(cp._kv_gather_vt, H=6, S=0) == OK     # no head divisibility rule
