"""The benchmark's accounting, checked on the CPU: the FLOP count behind every
TFLOP/s figure (4*D per visible (query, key) pair, causal pairs only) against a
brute-force count of the mask, and the cold-buffer rotation sizing."""
import itertools

import numpy as np
import pytest

import bench


def _visible_pairs(Sq, Skv, causal, q0, k0):
    qp = q0 + np.arange(Sq)[:, None]
    kp = k0 + np.arange(Skv)[None, :]
    return int((kp <= qp).sum()) if causal else Sq * Skv


@pytest.mark.parametrize("Sq,Skv,q0,k0", [
    (1, 1, 0, 0), (7, 7, 0, 0), (5, 9, 4, 0), (9, 5, 0, 4), (6, 4, 100, 0), (6, 4, 0, 100),
    (33, 65, 17, 3),
])
@pytest.mark.parametrize("causal", [False, True])
def test_attn_flops_counts_visible_pairs(Sq, Skv, q0, k0, causal):
    H, D = 3, 64
    want = 4.0 * D * H * _visible_pairs(Sq, Skv, causal, q0, k0)
    assert bench.attn_flops(Sq, Skv, H, D, causal, q0, k0) == want


def test_causal_square_pairs():
    for S in (1, 2, 3, 10, 257):
        assert bench.causal_pairs_square(S) == _visible_pairs(S, S, True, 0, 0)


def test_headline_flop_count():
    """The FLUX ring rank: 4 * H * Sq * S * D = 65.23 GFLOP per call."""
    assert bench.attn_flops(1152, 4608, 24, 128, False) == 4 * 24 * 1152 * 4608 * 128


def test_ring_anything_shares_sum_to_the_whole():
    """The ring ranks' causal shares of S = 4099 add up to the full causal count."""
    lens, S = (1025, 1025, 1025, 1024), 4099
    starts = list(itertools.accumulate((0,) + lens[:-1]))
    total = sum(bench.attn_flops(n, S, 1, 1, True, s0, 0) for s0, n in zip(starts, lens))
    assert total == 4 * bench.causal_pairs_square(S)


@pytest.mark.parametrize("nbytes", [1, 64 << 20, 116 << 20, 700 << 20, 3 << 30])
def test_rotation_spans_the_caches(nbytes):
    n = bench.buffer_sets(nbytes)
    assert n >= 2 and n * nbytes >= bench.ROTATE_BYTES
    assert (n - 1) * nbytes < bench.ROTATE_BYTES or n == 2


def test_code_digest_ignores_comments_only(tmp_path):
    """The counter records are tied to the attention kernel's code: a comment
    edit keeps the digest, a code edit changes it."""
    base = "// header\nint f(int x) {\n  return x + 1;  // one\n}\n/* block\n comment */\n"
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text(base)
    b.write_text(base.replace("// one", "// plus one, reworded").replace("// header\n", ""))
    c.write_text(base.replace("x + 1", "x + 2"))
    assert bench.code_digest(str(a)) == bench.code_digest(str(b))
    assert bench.code_digest(str(a)) != bench.code_digest(str(c))
