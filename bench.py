"""Benchmark of the context-parallel attention hot path on one MI355X.

Default workload (the headline line): one Ulysses rank of a 128K-token causal
LLM at sequence-parallel degree 8 — S=131072, H=32 (4 heads per rank), D=128,
bf16, causal from positions. One step is one pass of the rank's whole hot
path: the Ulysses regrouping of Q and K ([8][1][16384][32][128] ->
[8][1][131072][4][128], one stacked launch) and of V into each head's
key-contiguous 64-token tiles (cp_ulysses_seq2head_vt), rank 0's causal
attention over the full sequence on its 4 heads (cp_attn_chunk_partial_vt,
bf16 O, fp32 LSE), and the inverse regrouping of O. The same step with V
token-major is a detail entry. ``value`` is attention TFLOP/s over the whole step (4*D FLOP
per visible (query, key) pair, 17.59 TFLOP per step) with inputs resident in
HBM; ``roofline`` is the attention kernel alone, timed with HIP events on its
launch stream.

The same JSON line also carries, under ``detail``, every other workload:
the FLUX ring rank (with its own roofline), Ulysses seq2head/head2seq GB/s
and rank-0 attention TFLOP/s for the Qwen-Image and Wan shapes, the
ring-anything S=4099 ranks, the standalone LSE merge GB/s, the uneven
regroupings, K/V gather, unified share and backward entries; plus the fp64
CPU oracle timed on the host (``cpu_baseline``).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
ROTATE_BYTES = 1 << 30        # footprint of the buffer sets an HBM-bound kernel rotates over
WARM_MS = 30.0                # sustained GPU work before a detail entry's timed region
HEADLINE_WARM_MS = 2000.0     # before the headline's: the clock under this load settles,
                              # and a sampler of GPU activity sees the work
MIN_TIMED_MS = 20.0           # shortest timed region of a detail entry
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_llm_causal_counters.json")
FLUX_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_flux_ring_traffic.json")
ATTN_SRC = os.path.join(ROOT, "context_attention_dit_amd", "csrc", "attn_bf16.hip")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def attn_flops(Sq: int, Skv: int, H: int, D: int, causal: bool, q0: int = 0, k0: int = 0) -> float:
    """4*D FLOP per visible (query, key) pair: 2*D for Q.K, 2*D for P.V."""
    if not causal:
        pairs = Sq * Skv
    else:
        pairs = 0
        # key j visible to query i iff k0 + j <= q0 + i
        for i in range(Sq):
            pairs += max(0, min(Skv, q0 + i - k0 + 1))
    return 4.0 * D * H * pairs


def causal_pairs_square(S: int) -> int:
    return S * (S + 1) // 2


def buffer_sets(bytes_per_launch: int) -> int:
    """Buffer sets to rotate over so that a launch never finds its operands in
    the caches: together they span ROTATE_BYTES (4x the 256 MB last-level cache
    and the L2s), and there are at least two."""
    return max(2, math.ceil(ROTATE_BYTES / max(1, bytes_per_launch)))


def rotating_pairs(x, out_like, nbytes: int):
    """(input, output) buffer sets for an HBM-bound transform of `x`: copies of
    the input and fresh outputs shaped like `out_like`, enough of them that
    they span ROTATE_BYTES together."""
    return [(x.clone(), out_like.new_empty(out_like.shape)) for _ in range(buffer_sets(nbytes))]


def warm_up(torch, fn, ms: float = WARM_MS) -> float:
    """Run `fn` back to back until `ms` of GPU work has passed, so the GPU is
    at its steady clocks when the timed region starts (it takes about 20 ms of
    sustained work from idle; the detail entries follow host-side input
    generation, during which the GPU idles). Returns the mean ms per call."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        if n % 4 == 0 or n < 4:
            torch.cuda.synchronize()
            el = (time.perf_counter() - t0) * 1e3
            if el >= ms:
                return el / n


def time_rotating(torch, fns, warmup: int, rounds: int) -> float:
    """Mean ms per launch of an HBM-bound kernel, issued back to back over
    `rounds` passes (at least MIN_TIMED_MS of work) through `fns` (one closure
    per buffer set) between one pair of HIP events, after warm_up. Each launch
    reads operands last touched a full rotation earlier, so they come from HBM,
    and there is no per-launch event or cache flush in the timed region."""
    def one_round():
        for f in fns:
            f()
    for _ in range(warmup):
        one_round()
    est = warm_up(torch, one_round)
    rounds = max(rounds, math.ceil(MIN_TIMED_MS / max(est, 1e-3)))
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(rounds):
        one_round()
    b.record()
    b.synchronize()
    return a.elapsed_time(b) / (rounds * len(fns))


def time_back_to_back(torch, fn, warmup: int, iters: int) -> float:
    """Mean ms per call of at least `iters` calls (and MIN_TIMED_MS of work)
    issued back to back between one pair of HIP events on the current stream,
    after warm_up (host-side argument marshalling overlaps the GPU work of the
    previous call, as it does in a training loop)."""
    for _ in range(warmup):
        fn()
    est = warm_up(torch, fn)
    iters = max(iters, math.ceil(MIN_TIMED_MS / max(est, 1e-3)))
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        fn()
    b.record()
    b.synchronize()
    return a.elapsed_time(b) / iters


def median(xs):
    return xs[len(xs) // 2]


def code_digest(path=ATTN_SRC) -> str:
    """SHA-256 of a HIP source's code: comments removed and whitespace runs
    collapsed, so an edit to comments alone keeps the digest and any change to
    the code changes it."""
    import re
    src = open(path, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return hashlib.sha256(" ".join(src.split()).encode()).hexdigest()


def counter_record(path=TRAFFIC_FILE):
    """rocprofv3 counter record of the attention kernel (profiles/), if it was
    taken on the current kernel code; else None."""
    try:
        rec = json.load(open(path))
        if rec.get("attn_bf16_code_sha256") == code_digest():
            return rec
    except (OSError, ValueError):
        pass
    return None


def traffic_record(path=TRAFFIC_FILE):
    """HBM bytes per launch of the attention kernel, if taken on the current source."""
    rec = counter_record(path)
    return None if rec is None else rec.get("bytes_per_launch")


def cpu_baseline(qkv_cpu, budget_s: float = 15.0):
    """fp64 oracle on a bounded stratified sample of the headline's attention.

    Rank 0 of the 128K causal Ulysses workload attends heads 0..3 over the whole
    sequence. Per head the sample is the first 512 and the last 512 query rows
    plus 4096 rows drawn at random (seeded), each against every key it may see;
    heads are taken in turn until ~budget_s is spent. FLOP are counted as on
    the GPU: 4*D per visible (query, key) pair of the sampled rows."""
    import numpy as np
    import torch

    import oracle
    import synthetic
    w = synthetic.LLM_ULYSSES
    q, k, v = qkv_cpu
    f64 = lambda t: oracle.bf16_bits_to_f64(t.contiguous().view(torch.int16).numpy())
    ncores = len(os.sched_getaffinity(0))
    torch.set_num_threads(ncores)
    rng = np.random.default_rng(1005)
    S, D = w.S, w.D
    mid = rng.choice(np.arange(512, S - 512), size=4096, replace=False)
    rows = np.unique(np.concatenate([np.arange(512), mid, np.arange(S - 512, S)]))
    kpos = np.arange(S)
    done, flops, t0 = 0, 0.0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s and done < w.H_local:
        h = slice(done, done + 1)   # rank 0's heads are 0 .. H/P - 1
        qh = f64(q[:, rows, h])
        kh, vh = f64(k[:, :, h]), f64(v[:, :, h])
        oracle.attention(qh, kh, vh, 1 / math.sqrt(D), causal=True, q_pos=rows, k_pos=kpos)
        flops += 4.0 * D * float((rows + 1).sum())
        done += 1
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": ncores, "kind": "oracle",
            "sample": f"128K causal Ulysses rank 0: {done} of its {w.H_local} heads, "
                      f"{len(rows)} query rows per head (first 512, last 512, 4096 seeded "
                      f"random) against every visible key, fp64 numpy oracle.attention, "
                      f"{flops / 1e9:.0f} GFLOP (visible pairs) in {dt:.1f} s"}


def cpu_oracle_relayout(budget_s: float = 2.0):
    """The oracle's seq2head (a numpy transpose copy) on the Qwen rank's Q tensor,
    repeated for ~budget_s on the host: host GB/s (read + write per element)."""
    import torch

    import oracle
    import synthetic
    w = synthetic.QWEN_ULYSSES
    x = synthetic.make_qkv(w)[0].view(w.P, 1, w.S_local, w.H, w.D)
    bits = x.contiguous().view(torch.int16).numpy()
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        oracle.seq2head(bits, w.P)
        n += 1
    dt = time.perf_counter() - t0
    nbytes = 2 * bits.nbytes
    return {"gbs": n * nbytes / dt / 1e9, "unit": "GB/s", "kind": "oracle",
            "sample": f"seq2head of the Qwen-Image rank's Q ({bits.nbytes / 1e6:.1f} MB, "
                      f"[{w.P}][1][{w.S_local}][{w.H}][{w.D}] bf16 bits) {n} times in {dt:.1f} s "
                      f"(numpy transpose copy)"}


def copy_ceiling(torch, cp, dev) -> float:
    """GB/s (read + write) of a plain 16-byte streaming copy: the regrouping with
    one rank is the identity permutation, so cp_ulysses_seq2head with P = 1 is
    the library's own copy kernel. 512 MiB per launch, cold buffers."""
    x = torch.empty((1, 1, 1 << 18, 8, 128), dtype=torch.bfloat16, device=dev).fill_(1.0)
    nbytes = 2 * x.numel() * x.element_size()
    pairs = rotating_pairs(x, x, nbytes)
    d = time_rotating(torch, [lambda a=a, b=b: cp.ulysses_seq2head(a, 1, b) for a, b in pairs],
                      1, 5)
    del pairs, x
    torch.cuda.empty_cache()
    return nbytes / (d * 1e-3) / 1e9


def copy_same_bytes(torch, cp, dev, nbytes: int):
    """(GB/s, us) of a plain copy that moves nbytes (read plus write), timed
    like the HBM-bound launch it is compared with: the ceiling at that size,
    where launch ramp and tail weigh more than on the 512 MiB copy."""
    x = torch.ones((1, 1, max(1, nbytes // 4096), 8, 128), dtype=torch.bfloat16, device=dev)
    cbytes = 2 * x.numel() * x.element_size()
    pairs = rotating_pairs(x, x, cbytes)
    dc = time_rotating(torch, [lambda a=a, b=b: cp.ulysses_seq2head(a, 1, b) for a, b in pairs],
                       1, 10)
    del pairs, x
    return cbytes / (dc * 1e-3) / 1e9, dc * 1e3


def headline(torch, cp, synthetic, dev, steps: int, warmup: int, qkv_cpu, vt: bool = True,
             warm_ms: float = HEADLINE_WARM_MS):
    """The 128K causal Ulysses rank's step: seq2head of Q, K, V (all 8 ranks'
    regrouping), rank 0's causal attention on its 4 heads, head2seq of O
    (rank 0's output in its slot; the other slots hold stand-in outputs).
    vt: Q and K regrouped in one launch and V by cp_ulysses_seq2head_vt (each
    head's values key-contiguous), attention by cp_attn_chunk_partial_vt;
    otherwise Q, K, V in one launch and cp_attn_chunk_partial."""
    w = synthetic.LLM_ULYSSES
    P, S_l, H, D, Hl, S = w.P, w.S_local, w.H, w.D, w.H_local, w.S
    log(f"{w.name}: inputs to the GPU")
    qkv = torch.stack([x.view(P, 1, S_l, H, D) for x in qkv_cpu]).to(dev)  # [3][P][1][S_l][H][D]
    heads = torch.empty((3, P, 1, S, Hl, D), dtype=w.dtype, device=dev)
    o_all = torch.empty((P, 1, S, Hl, D), dtype=w.dtype, device=dev)
    back = torch.empty((P, 1, S_l, H, D), dtype=w.dtype, device=dev)
    lse = torch.empty((1, Hl, S), dtype=torch.float32, device=dev)
    vt_all = torch.empty((P, 1, Hl, S // 64, D, 64), dtype=w.dtype, device=dev) if vt else None
    cp.ulysses_seq2head(qkv, P, heads)
    o_all.copy_(heads[2])   # the other ranks' slots: their V head shards as stand-ins
    rq, rk, rv, ro = heads[0, 0], heads[1, 0], heads[2, 0], o_all[0]

    def regroup():
        if vt:
            cp.ulysses_seq2head(qkv[:2], P, heads[:2])
            cp.ulysses_seq2head_vt(qkv[2], P, vt_all)
        else:
            cp.ulysses_seq2head(qkv, P, heads)
    flops = 4.0 * D * Hl * causal_pairs_square(S)
    relayout_bytes = 3 * 2 * qkv[0].numel() * qkv.element_size() + \
        2 * o_all.numel() * o_all.element_size()

    def attend():
        if vt:
            cp.attn_chunk_partial_vt(rq, rk, vt_all[0], ro, lse, causal=True, out_dtype=w.dtype)
        else:
            cp.attn_chunk_partial(rq, rk, rv, ro, lse, causal=True, out_dtype=w.dtype)

    def step(ev=None):
        regroup()
        if ev is not None:
            ev[0].record()
        attend()
        if ev is not None:
            ev[1].record()
        cp.ulysses_head2seq(o_all, P, back)

    log(f"{w.name}: warmup {warmup} steps, then >= {warm_ms:.0f} ms of steps")
    for _ in range(warmup):
        step()
    warm_ms_per_step = warm_up(torch, step, warm_ms)
    # K steps back to back; an event pair around each attention launch (on the
    # launch stream: torch's current stream, which the binding passes) gives
    # the attention kernel's own duration inside the step
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(steps):
        step(evs[i])
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    ms_step_ev = ev0.elapsed_time(ev1) / steps
    attn_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    relayout_ms = ms_step_ev - attn_ms
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (attn_ms * 1e-3) / 1e12
    log(f"{w.name}: {ms_step:.2f} ms/step ({value:.0f} TFLOP/s), attention kernel "
        f"{attn_ms:.2f} ms ({achieved:.0f} TFLOP/s), regroupings {relayout_ms * 1e3:.0f} us")
    # the regroupings alone, back to back over cold buffer sets, for their GB/s
    s2h_qkv = time_rotating(torch, [regroup], 1, 5)
    h2s = time_rotating(torch, [lambda: cp.ulysses_head2seq(o_all, P, back)], 1, 5)
    s2h_bytes = 3 * 2 * qkv[0].numel() * qkv.element_size()
    h2s_bytes = 2 * o_all.numel() * o_all.element_size()
    res = {
        "value": value, "ms_per_step": ms_step, "flops": flops,
        "attn_ms": attn_ms, "achieved": achieved, "warm_ms_per_step": warm_ms_per_step,
        "step_event_ms": ms_step_ev, "relayout_in_step_us": relayout_ms * 1e3,
        "relayout_bytes_per_step": relayout_bytes,
        "seq2head_qkv_us": s2h_qkv * 1e3,
        "seq2head_qkv_gbs": s2h_bytes / (s2h_qkv * 1e-3) / 1e9,
        "head2seq_us": h2s * 1e3, "head2seq_gbs": h2s_bytes / (h2s * 1e-3) / 1e9,
    }
    res["v_layout"] = "key-contiguous per head" if vt else "token-major"
    del qkv, heads, o_all, back, lse, rq, rk, rv, ro, vt_all
    torch.cuda.empty_cache()
    return res


def flux_ring(torch, cp, synthetic, dev):
    """FLUX ring rank 0 (detail entry with its own roofline): 1152 query rows over
    4 chunks of 1152 in ring order, one cp_ring_attention call per step."""
    w = synthetic.FLUX_RING
    log(f"{w.name}: inputs")
    q, k, v = (x.to(dev) for x in synthetic.make_qkv(w))
    n = w.chunk_lens[0]
    q0 = q[:, :n].contiguous()
    starts = w.chunk_starts()
    chunks = [(k[:, s:s + ln].contiguous(), v[:, s:s + ln].contiguous(), s)
              for s, ln in zip(starts, w.chunk_lens)]
    vis = [chunks[c] for c in synthetic.ring_order(0, w.P)]
    o = torch.empty_like(q0)
    lse = torch.empty((1, w.H, n), dtype=torch.float32, device=dev)
    ws_bytes = cp.ring_attention_workspace_bytes(w.P, 1, w.H, n, w.D)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    flops = attn_flops(n, w.S, w.H, w.D, False)
    ms = time_back_to_back(torch, lambda: cp.ring_attention(q0, vis, o, lse, workspace=ws), 5, 200)
    achieved = flops / (ms * 1e-3) / 1e12
    log(f"{w.name}: kernel {ms * 1e3:.1f} us, {achieved:.1f} TFLOP/s")
    res = {"kernel_us": ms * 1e3, "tflops": achieved, "gflop": flops / 1e9,
           "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                        "traffic": traffic_record(FLUX_TRAFFIC_FILE),
                        "kernel": "attn_g2pp_kernel<128, causal=false, out_bf16=true> (two-group ping-pong)"}}
    return res, q0, vis


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # one step is ~20 ms; each timed region is preceded by >= 30 ms of warm-up
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--only", default=None,
                    help="run only this detail workload (flux, qwen, wan, overlap, ra, merge, llmring, "
                         "anything, kvgather, unified, bwd) after the headline; for profiling")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        return 2
    if args.steps < 1:
        print("--steps must be >= 1", file=sys.stderr)
        return 2

    import torch

    import context_attention_dit_amd as cp
    import synthetic

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.ones(1 << 26, dtype=torch.float32, device=dev)   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied 256 MiB x 5 (read 268435456 B, write 268435456 B per launch)")
        return 0
    # ---------------------------------------------------------------- headline
    w = synthetic.LLM_ULYSSES
    log(f"{w.name}: drawing inputs on the host")
    qkv_cpu = synthetic.make_qkv(w)
    h = headline(torch, cp, synthetic, dev, args.steps, args.warmup, qkv_cpu)
    copy_gbs = copy_ceiling(torch, cp, dev)
    log(f"copy ceiling {copy_gbs:.0f} GB/s")

    detail = {}
    if not args.quick:
        if args.only in (None, "flux", "merge", "bwd"):
            fl, q0, vis = flux_ring(torch, cp, synthetic, dev)
            detail["flux_ring_rank0"] = fl
        else:
            q0 = vis = None
        detail.update(other_workloads(torch, cp, synthetic, dev, q0, vis, synthetic.FLUX_RING,
                                      args.only))
        if args.only in (None, "llmring"):
            detail["llm-128k-causal-ring8-rank7"] = llm_ring_workload(torch, cp, dev, w, qkv_cpu)
        if args.only in (None, "layout"):
            # the same step with V token-major (Q, K, V regrouped in one launch,
            # cp_attn_chunk_partial): what the key-contiguous layout gains
            hb = headline(torch, cp, synthetic, dev, args.steps, 0, qkv_cpu, vt=False,
                          warm_ms=WARM_MS * 10)
            detail["llm-128k-causal-ulysses8-rank0-v-token-major"] = {
                "step_tflops": hb["value"], "ms_per_step": hb["ms_per_step"],
                "attn_ms": hb["attn_ms"], "attn_tflops": hb["achieved"],
                "attn_mfma_frac": hb["achieved"] / PEAK_BF16_TFLOPS,
                "seq2head_qkv_us": hb["seq2head_qkv_us"], "head2seq_us": hb["head2seq_us"],
                "kernel": "attn_pp_kernel<128, causal=true, out_bf16=true> with V token-major "
                          "(transposing LDS reads for P*V)"}

    rec = counter_record()
    traffic = None if rec is None else rec.get("bytes_per_launch")
    sclk = None if rec is None else rec.get("clock_mhz")
    line = {
        "metric": "attention TFLOP/s (bf16, 1 MI355X) + % MFMA peak; relayout GB/s",
        "value": h["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": h["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic N(0,1) inputs, seed 1005, rounded to bf16",
        "config": {"workload": "128K-token causal LLM, Ulysses SP8 rank 0: S=131072 H=32 "
                               "(4 heads per rank) D=128 bf16, causal from positions; step = "
                               "seq2head of Q and K [8][1][16384][32][128] -> "
                               "[8][1][131072][4][128] (one launch) and of V into each head's "
                               "key-contiguous 64-key tiles [8][1][4][2048][128][64] "
                               "(cp_ulysses_seq2head_vt), "
                               "rank-0 attention (cp_attn_chunk_partial_vt), head2seq of O",
                   "global_batch": 1, "seq_len": w.S, "parallelism": "one Ulysses rank (P=8)"},
        "roofline": {"bound": "mfma", "achieved": h["achieved"], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": h["achieved"] / PEAK_BF16_TFLOPS,
                     "traffic": traffic,
                     "kernel": "attn_pp_kernel<128, causal=true, out_bf16=true, chunk list=false, "
                               "split=false, key-contiguous V=true> (8-wave blocks of 256 query "
                               "rows)",
                     "flop_per_launch": h["flops"], "kernel_ms": h["attn_ms"],
                     # clock and MFMA busy of this kernel from the rocprofv3
                     # counter pass on the current source (profiles/), or null
                     "measured_sclk_mhz": sclk,
                     "sclk_source": None if rec is None else
                     "rocprofv3 counter pass of this kernel code (GRBM_GUI_ACTIVE / 8 over the "
                     "dispatch), profiles/attn_llm_causal_counters.json; boxes of the pool differ "
                     "by a few percent",
                     "mfma_busy": None if rec is None else rec.get("mfma_busy"),
                     "peak_at_measured_sclk": (PEAK_BF16_TFLOPS * sclk / 2400.0
                                               if sclk else None)},
        "relayout": {"seq2head_qkv": "Q and K in one launch, V key-contiguous in a second",
                     "seq2head_qkv_gbs": h["seq2head_qkv_gbs"],
                     "seq2head_qkv_hbm_frac": h["seq2head_qkv_gbs"] / PEAK_HBM_GBS,
                     "head2seq_gbs": h["head2seq_gbs"],
                     "head2seq_hbm_frac": h["head2seq_gbs"] / PEAK_HBM_GBS,
                     "seq2head_qkv_us": h["seq2head_qkv_us"], "head2seq_us": h["head2seq_us"],
                     "in_step_us": h["relayout_in_step_us"],
                     "copy_ceiling_gbs": copy_gbs,
                     "copy_ceiling_hbm_frac": copy_gbs / PEAK_HBM_GBS},
        "warm_ms_per_step": h["warm_ms_per_step"],
        "detail": detail,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle)")
        line["cpu_baseline"] = cpu_baseline(qkv_cpu)
        detail["cpu_oracle_relayout"] = cpu_oracle_relayout()
    print(json.dumps(line), flush=True)
    return 0


def llm_ring_workload(torch, cp, dev, w, qkv_cpu):
    """The headline's 128K causal sequence split as a ring of 8 instead:
    rank 7 holds query rows [7*16384, 8*16384) over all 32 heads and visits
    the 8 key chunks in ring order 7, 6, .., 0 (the rank that sees every
    key; its own chunk is the diagonal), one cp_ring_attention call."""
    P = w.P
    S_l = w.S // P
    q, k, v = qkv_cpu
    r = P - 1
    q7 = q[:, r * S_l:(r + 1) * S_l].contiguous().to(dev)
    kd, vd = k.to(dev), v.to(dev)
    chunks = [(kd[:, c * S_l:(c + 1) * S_l], vd[:, c * S_l:(c + 1) * S_l], c * S_l)
              for c in range(r, -1, -1)]
    chunks = [(a.contiguous(), b.contiguous(), p0) for a, b, p0 in chunks]
    del kd, vd
    o = torch.empty_like(q7)
    lse = torch.empty((1, w.H, S_l), dtype=torch.float32, device=dev)
    # visible pairs per head: every key of chunks 0..6, the diagonal of chunk 7
    flops = 4.0 * w.D * w.H * (S_l * S_l * r + causal_pairs_square(S_l))
    ms = time_back_to_back(torch, lambda: cp.ring_attention(
        q7, chunks, o, lse, causal=True, q_pos0=r * S_l), 1, 5)
    res = {"kernel_ms": ms, "tflops": flops / (ms * 1e-3) / 1e12,
           "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "gflop": flops / 1e9,
           "kernel": "attn_pp_kernel chunk-list form (8-wave blocks of 256 query rows)"}
    log(f"llm-128k-causal-ring8-rank7: {ms:.2f} ms, {res['tflops']:.0f} TFLOP/s")
    del q7, chunks, o, lse
    torch.cuda.empty_cache()
    return res


def other_workloads(torch, cp, synthetic, dev, q0, vis, wf, only=None):
    out = {}
    want = (lambda tag: only is None or only == tag)
    # standalone merge of the FLUX ring's 4 fp32 partials (HBM-bound)
    if want("merge"):
        out.update(merge_workload(torch, cp, dev, q0, vis, wf))
    # (the 128K causal Ulysses rank is the headline)
    tags = {synthetic.QWEN_ULYSSES.name: "qwen", synthetic.WAN_ULYSSES.name: "wan"}
    for w in (synthetic.QWEN_ULYSSES, synthetic.WAN_ULYSSES):
        if want(tags[w.name]):
            out[w.name] = ulysses_workload(torch, cp, synthetic, dev, w)
    if only == "overlap":   # two-stream layer pipelining: on request only
        out["qwen-image-1536-ulysses4-stream-overlap"] = stream_overlap_workload(
            torch, cp, synthetic, dev)
    if want("ra"):
        out[synthetic.LLM_RING_ANYTHING.name] = ring_anything_workload(torch, cp, synthetic, dev)
    if want("anything"):
        out[synthetic.FLUX_ANYTHING.name] = ulysses_anything_workload(torch, cp, synthetic, dev)
    if want("kvgather"):
        out[synthetic.WAN_KV_GATHER.name] = kv_gather_workload(torch, cp, synthetic, dev)
    if want("unified"):
        out[synthetic.FLUX_UNIFIED.name] = unified_workload(torch, cp, synthetic, dev)
    if want("bwd"):
        out.update(backward_workloads(torch, cp, synthetic, dev, q0, vis, wf))
    return out


def backward_workloads(torch, cp, synthetic, dev, q0, vis, wf):
    """Attention backward: the FLUX ring rank's share (Delta, then one
    cp_ring_attention_backward call: dQ over the 4 chunks, each chunk's dK/dV
    share written for its owner) and the Wan and
    128K-causal Ulysses ranks (one chunk over the whole sequence). The saved
    O and LSE come from this library's own forward. FLOP convention: 2.5x the
    forward's (five D-long products per visible pair: S, dP, dV, dK, dQ); the
    kernels recompute S and dP in both passes, so they execute 7/5 of that."""
    out = {}
    f32 = torch.float32
    n, H, D = q0.shape[1], wf.H, wf.D
    o, lse = cp.ring_attention(q0, vis)
    do = synthetic.make_tensor(tuple(q0.shape), torch.bfloat16, 1077).to(dev)
    delta = cp.attn_backward_delta(o, do)
    dq = torch.empty((1, n, H, D), dtype=f32, device=dev)
    grads = [(torch.empty(k.shape, dtype=f32, device=dev), torch.empty(k.shape, dtype=f32,
                                                                     device=dev))
             for k, _, _ in vis]

    def ring_step():
        cp.attn_backward_delta(o, do, delta)
        cp.ring_attention_backward(q0, vis, do, lse, delta, dq, grads)

    flops = 2.5 * attn_flops(n, wf.S, H, D, False)
    ms = time_back_to_back(torch, ring_step, 3, 20)
    out["flux_ring_rank0_backward"] = {
        "us": ms * 1e3, "tflops": flops / (ms * 1e-3) / 1e12,
        "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "gflop": flops / 1e9,
        "launches": 2}
    log(f"flux ring rank0 backward: {ms * 1e3:.0f} us, "
        f"{out['flux_ring_rank0_backward']['tflops']:.0f} TFLOP/s")
    del o, lse, do, delta, dq, grads
    for w in (synthetic.WAN_ULYSSES, synthetic.LLM_ULYSSES):
        S, Hl = w.S, w.H_local
        q, k, v, do = (synthetic.make_tensor((1, S, Hl, D), torch.bfloat16, 1100 + t).to(dev)
                       for t in range(4))
        o, lse = cp.attn_chunk_partial(q, k, v, causal=w.causal, out_dtype=torch.bfloat16)
        delta = cp.attn_backward_delta(o, do)
        g = [torch.empty((1, S, Hl, D), dtype=f32, device=dev) for _ in range(3)]
        step = lambda: (cp.attn_backward_delta(o, do, delta),
                        cp.attn_chunk_backward(q, k, v, do, lse, delta, *g, causal=w.causal))
        flops = 2.5 * 4.0 * D * Hl * (causal_pairs_square(S) if w.causal else S * S)
        ms = time_back_to_back(torch, step, 1, 3 if w.causal else 5)
        out[w.name + "_backward"] = {
            "us": ms * 1e3, "tflops": flops / (ms * 1e-3) / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "gflop": flops / 1e9, "causal": w.causal}
        log(f"{w.name} backward: {ms * 1e3:.0f} us, "
            f"{out[w.name + '_backward']['tflops']:.0f} TFLOP/s")
        del q, k, v, do, o, lse, delta, g
        torch.cuda.empty_cache()
    return out


def merge_workload(torch, cp, dev, q0, vis, wf):
    out = {}
    parts = [cp.attn_chunk_partial(q0, kc, vc) for kc, vc, _ in vis]
    po = torch.stack([p[0] for p in parts])
    pl = torch.stack([p[1] for p in parts])
    del parts
    mo = torch.empty_like(q0)
    ml = torch.empty((1, wf.H, q0.shape[1]), dtype=torch.float32, device=dev)
    P, B, Sq, H, D = po.shape
    mbytes = P * (Sq * H * D * 4 + Sq * H * 4) + Sq * H * D * 2 + Sq * H * 4
    sets = [(po.clone(), pl.clone(), torch.empty_like(mo), torch.empty_like(ml))
            for _ in range(buffer_sets(mbytes))]
    d = time_rotating(torch, [lambda s=s: cp.lse_merge(*s) for s in sets], 1, 10)
    del sets
    # the ceiling at this size: a plain copy moving the same bytes
    c_gbs, c_us = copy_same_bytes(torch, cp, dev, mbytes)
    out["flux_lse_merge"] = {"us": d * 1e3, "gbs": mbytes / (d * 1e-3) / 1e9, "bytes": mbytes,
                             "hbm_frac": mbytes / (d * 1e-3) / 1e9 / PEAK_HBM_GBS,
                             "copy_same_bytes_gbs": c_gbs, "copy_same_bytes_us": c_us}
    # the per-hop form of the same rank: one partial per chunk into its slot of
    # the stacked fp32 partials, then the merge (what a P2P ring does per hop)
    flops = attn_flops(q0.shape[1], wf.S, wf.H, wf.D, False)

    def hops():
        for c, (kc, vc, _) in enumerate(vis):
            cp.attn_chunk_partial(q0, kc, vc, po[c], pl[c])

    ms = time_back_to_back(torch, hops, 3, 20)
    ms_m = time_back_to_back(torch, lambda: (hops(), cp.lse_merge(po, pl, mo, ml)), 3, 20)
    out["flux_partials_x4"] = {"us": ms * 1e3, "tflops": flops / (ms * 1e-3) / 1e12,
                               "with_merge_us": ms_m * 1e3,
                               "with_merge_tflops": flops / (ms_m * 1e-3) / 1e12}
    return out


def ulysses_workload(torch, cp, synthetic, dev, w):
    log(f"{w.name}: inputs")
    P, S_l, H, D = w.P, w.S_local, w.H, w.D
    qkv = [x.view(P, 1, S_l, H, D).to(dev) for x in synthetic.make_qkv(w)]
    heads = [torch.empty((P, 1, w.S, w.H_local, D), dtype=w.dtype, device=dev) for _ in qkv]
    nbytes = qkv[0].numel() * qkv[0].element_size() * 2    # read + write, one tensor
    pairs = rotating_pairs(qkv[0], heads[0], nbytes)
    d_s2h = time_rotating(torch, [lambda x=x, y=y: cp.ulysses_seq2head(x, P, y)
                                  for x, y in pairs], 1, 5)
    # head2seq over the same sets, from head layout back into the sequence copies
    d_h2s = time_rotating(torch, [lambda x=x, y=y: cp.ulysses_head2seq(y, P, x)
                                  for x, y in pairs], 1, 5)
    del pairs
    for x, y in zip(qkv, heads):
        cp.ulysses_seq2head(x, P, y)
    rq, rk, rv = (y[0] for y in heads)
    o = torch.empty_like(rq)
    lse = torch.empty((1, w.H_local, w.S), dtype=torch.float32, device=dev)
    flops = 4.0 * D * w.H_local * (causal_pairs_square(w.S) if w.causal else w.S * w.S)
    reps = 3 if w.causal else 10
    d_cp = [time_back_to_back(torch, lambda: cp.attn_chunk_partial(
        rq, rk, rv, o, lse, causal=w.causal, out_dtype=torch.bfloat16), 1, reps)]
    # the same attention through the ring call with one chunk and the workspace
    # it reports (which lets a half-full last round of query tiles split keys)
    ws = torch.empty(max(1, cp.ring_attention_workspace_bytes(1, 1, w.H_local, w.S, D)),
                     dtype=torch.uint8, device=dev)
    d_att = [time_back_to_back(torch, lambda: cp.ring_attention(
        rq, [(rk, rv, 0)], o, lse, causal=w.causal, workspace=ws), 1, reps)]
    # V regrouped key-contiguous (cp_ulysses_seq2head_vt) and the attention that reads it
    vt = cp.ulysses_seq2head_vt(qkv[2], P)
    d_vt = [time_back_to_back(torch, lambda: cp.attn_chunk_partial_vt(
        rq, rk, vt[0], o, lse, causal=w.causal, out_dtype=torch.bfloat16), 1, reps)]
    vt_pairs = rotating_pairs(qkv[2], vt, nbytes)
    d_s2h_vt = time_rotating(torch, [lambda x=x, y=y: cp.ulysses_seq2head_vt(x, P, y)
                                     for x, y in vt_pairs], 1, 5)
    del o, lse, ws, vt, vt_pairs
    # the rank's Q, K and V regrouped together in one launch (stacked tensors)
    qkv3 = torch.stack(qkv)
    heads3 = torch.empty((3,) + tuple(heads[0].shape), dtype=w.dtype, device=dev)
    pairs = rotating_pairs(qkv3, heads3, 3 * nbytes)
    del qkv3, heads3
    d_s2h3 = time_rotating(torch, [lambda x=x, y=y: cp.ulysses_seq2head(x, P, y)
                                   for x, y in pairs], 1, 5)
    del pairs
    copy1 = copy_same_bytes(torch, cp, dev, nbytes)
    copy3 = copy_same_bytes(torch, cp, dev, 3 * nbytes)
    res = {
        "attn_call": "cp_ring_attention, one chunk, with its workspace",
        "attn_us": median(d_att) * 1e3,
        "attn_tflops": flops / (median(d_att) * 1e-3) / 1e12,
        "attn_mfma_frac": flops / (median(d_att) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "attn_us_chunk_partial_vt": median(d_vt) * 1e3,
        "attn_tflops_chunk_partial_vt": flops / (median(d_vt) * 1e-3) / 1e12,
        "seq2head_vt_us": d_s2h_vt * 1e3,
        "seq2head_vt_gbs": nbytes / (d_s2h_vt * 1e-3) / 1e9,
        "attn_us_chunk_partial": median(d_cp) * 1e3,
        "attn_tflops_chunk_partial": flops / (median(d_cp) * 1e-3) / 1e12,
        "seq2head_us": d_s2h * 1e3,
        "seq2head_gbs": nbytes / (d_s2h * 1e-3) / 1e9,
        "head2seq_us": d_h2s * 1e3,
        "head2seq_gbs": nbytes / (d_h2s * 1e-3) / 1e9,
        "relayout_bytes_per_tensor": nbytes,
        "relayout_hbm_frac": nbytes / (d_s2h * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "seq2head_qkv_us": d_s2h3 * 1e3,
        "seq2head_qkv_gbs": 3 * nbytes / (d_s2h3 * 1e-3) / 1e9,
        "seq2head_qkv_hbm_frac": 3 * nbytes / (d_s2h3 * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "copy_same_bytes_gbs": copy1[0], "copy_same_bytes_qkv_gbs": copy3[0],
        "causal": w.causal, "gflop": flops / 1e9,
    }
    log(f"{w.name}: attn {res['attn_tflops']:.0f} TFLOP/s (chunk_partial "
        f"{res['attn_tflops_chunk_partial']:.0f}), seq2head "
        f"{res['seq2head_gbs']:.0f} GB/s, head2seq {res['head2seq_gbs']:.0f}, "
        f"Q+K+V in one launch {res['seq2head_qkv_gbs']:.0f}; same-size copies "
        f"{res['copy_same_bytes_gbs']:.0f} / {res['copy_same_bytes_qkv_gbs']:.0f}")
    del qkv, heads, rq, rk, rv
    torch.cuda.empty_cache()
    return res


def ulysses_anything_workload(torch, cp, synthetic, dev):
    """FLUX 1008x1008 over a Ulysses degree of 4 with uneven shards (Ulysses Anything)."""
    w = synthetic.FLUX_ANYTHING
    log(f"{w.name}: inputs")
    s_lens, h_counts, S, D = list(w.chunk_lens), list(w.head_counts), w.S, w.D
    qkv = [x.to(dev).reshape(-1) for x in synthetic.make_qkv(w)]
    groups = [torch.empty_like(x) for x in qkv]
    nbytes = qkv[0].numel() * qkv[0].element_size() * 2
    pairs = rotating_pairs(qkv[0], groups[0], nbytes)
    d_s2h = time_rotating(torch, [lambda x=x, y=y: cp.ulysses_anything_seq2head(
        x, s_lens, h_counts, 1, D, y) for x, y in pairs], 1, 5)
    d_h2s = time_rotating(torch, [lambda x=x, y=y: cp.ulysses_anything_head2seq(
        y, s_lens, h_counts, 1, D, x) for x, y in pairs], 1, 5)
    del pairs
    # the rank's Q, K and V regrouped in one launch (stacked tensors)
    qkv3 = torch.stack(qkv)
    pairs = rotating_pairs(qkv3, qkv3, 3 * nbytes)
    del qkv3
    d_s2h3 = time_rotating(torch, [lambda x=x, y=y: cp.ulysses_anything_seq2head(
        x, s_lens, h_counts, 1, D, y) for x, y in pairs], 1, 5)
    del pairs
    copy1 = copy_same_bytes(torch, cp, dev, nbytes)
    copy3 = copy_same_bytes(torch, cp, dev, 3 * nbytes)
    for x, y in zip(qkv, groups):
        cp.ulysses_anything_seq2head(x, s_lens, h_counts, 1, D, y)
    h0 = h_counts[0]
    rq, rk, rv = (y[:S * h0 * D].view(1, S, h0, D) for y in groups)
    o = torch.empty_like(rq)
    lse = torch.empty((1, h0, S), dtype=torch.float32, device=dev)
    flops = 4.0 * D * h0 * S * S
    d_att = [time_back_to_back(torch, lambda: cp.attn_chunk_partial(
        rq, rk, rv, o, lse, out_dtype=torch.bfloat16), 5, 50)]
    res = {
        "seq_split": s_lens, "head_split": h_counts,
        "attn_us": median(d_att) * 1e3,
        "attn_tflops": flops / (median(d_att) * 1e-3) / 1e12,
        "attn_mfma_frac": flops / (median(d_att) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "seq2head_us": d_s2h * 1e3,
        "seq2head_gbs": nbytes / (d_s2h * 1e-3) / 1e9,
        "head2seq_us": d_h2s * 1e3,
        "head2seq_gbs": nbytes / (d_h2s * 1e-3) / 1e9,
        "relayout_bytes_per_tensor": nbytes,
        "relayout_hbm_frac": nbytes / (d_s2h * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "seq2head_qkv_us": d_s2h3 * 1e3,
        "seq2head_qkv_gbs": 3 * nbytes / (d_s2h3 * 1e-3) / 1e9,
        "seq2head_qkv_hbm_frac": 3 * nbytes / (d_s2h3 * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "copy_same_bytes_gbs": copy1[0], "copy_same_bytes_qkv_gbs": copy3[0],
        "gflop": flops / 1e9,
    }
    log(f"{w.name}: attn {res['attn_tflops']:.0f} TFLOP/s, seq2head "
        f"{res['seq2head_gbs']:.0f} GB/s, head2seq {res['head2seq_gbs']:.0f}, "
        f"Q+K+V in one launch {res['seq2head_qkv_gbs']:.0f}; same-size copies "
        f"{res['copy_same_bytes_gbs']:.0f} / {res['copy_same_bytes_qkv_gbs']:.0f}")
    return res


def kv_gather_workload(torch, cp, synthetic, dev):
    """Wan over a K/V-gather degree of 4: rank 0's query shard over the gathered K/V."""
    w = synthetic.WAN_KV_GATHER
    log(f"{w.name}: inputs")
    S, H, D, lens = w.S, w.H, w.D, list(w.chunk_lens)
    q, k, v = (x.to(dev) for x in synthetic.make_qkv(w))
    kg = torch.empty_like(k)
    nbytes = k.numel() * k.element_size() * 2
    pairs = rotating_pairs(k.reshape(-1), kg, nbytes)
    d_g = time_rotating(torch, [lambda x=x, y=y: cp.kv_gather(x, lens, 1, H, D, y)
                                for x, y in pairs], 1, 5)
    # K and V gathered in one launch (stacked)
    kv2 = torch.stack([k.reshape(-1), v.reshape(-1)])
    pairs = rotating_pairs(kv2, torch.stack([kg, kg]), 2 * nbytes)
    del kv2
    d_g2 = time_rotating(torch, [lambda x=x, y=y: cp.kv_gather(x, lens, 1, H, D, y)
                                 for x, y in pairs], 1, 5)
    del pairs
    cp.kv_gather(k.reshape(-1), lens, 1, H, D, kg)
    vg = cp.kv_gather(v.reshape(-1), lens, 1, H, D)
    n0 = lens[0]
    q0 = q[:, :n0].contiguous()
    o = torch.empty_like(q0)
    lse = torch.empty((1, H, n0), dtype=torch.float32, device=dev)
    flops = 4.0 * D * H * n0 * S
    d_att = [time_back_to_back(torch, lambda: cp.attn_chunk_partial(
        q0, kg, vg, o, lse, out_dtype=torch.bfloat16), 1, 5)]
    # V gathered key-contiguous (cp_kv_gather_vt, equal shards) and the attention on it
    P = len(lens)
    assert lens == [lens[0]] * P
    vsh = v.view(P, 1, lens[0], H, D)
    vt = cp.kv_gather_vt(vsh)
    d_att_vt = [time_back_to_back(torch, lambda: cp.attn_chunk_partial_vt(
        q0, kg, vt, o, lse, out_dtype=torch.bfloat16), 1, 5)]
    pairs = rotating_pairs(vsh, vt, nbytes)
    d_gvt = time_rotating(torch, [lambda x=x, y=y: cp.kv_gather_vt(x, y) for x, y in pairs], 1, 5)
    del pairs, vt, vsh
    res = {
        "rank_rows": n0,
        "attn_us_vt": median(d_att_vt) * 1e3,
        "attn_tflops_vt": flops / (median(d_att_vt) * 1e-3) / 1e12,
        "attn_mfma_frac_vt": flops / (median(d_att_vt) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "gather_vt_gbs": nbytes / (d_gvt * 1e-3) / 1e9,
        "attn_us": median(d_att) * 1e3,
        "attn_tflops": flops / (median(d_att) * 1e-3) / 1e12,
        "attn_mfma_frac": flops / (median(d_att) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "gather_us": d_g * 1e3,
        "gather_gbs": nbytes / (d_g * 1e-3) / 1e9,
        "gather_hbm_frac": nbytes / (d_g * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "gather_kv_us": d_g2 * 1e3,
        "gather_kv_gbs": 2 * nbytes / (d_g2 * 1e-3) / 1e9,
        "gather_kv_hbm_frac": 2 * nbytes / (d_g2 * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "gather_bytes_per_tensor": nbytes, "gflop": flops / 1e9,
    }
    log(f"{w.name}: attn {res['attn_tflops']:.0f} TFLOP/s (key-contiguous V "
        f"{res['attn_tflops_vt']:.0f}), gather {res['gather_gbs']:.0f} GB/s, "
        f"K+V in one launch {res['gather_kv_gbs']:.0f}")
    del q, k, v, kg, vg, q0, o, lse
    torch.cuda.empty_cache()
    return res


def unified_workload(torch, cp, synthetic, dev):
    """FLUX 1024x1024 as Ulysses 2 x ring 2: one rank's whole step (Ulysses regrouping of
    Q, K, V inside both segments, ring attention, inverse regrouping of O).

    The rank's projected Q, K and V of both ring segments sit in one stacked buffer
    ([segment][q, k, v][U][1][S/(R U)][H][D]), so the six regroupings are one
    cp_ulysses_seq2head_n launch; the step is three launches, timed back to back."""
    w = synthetic.FLUX_UNIFIED
    log(f"{w.name}: inputs")
    R = len(w.chunk_lens)
    U = w.P // R
    S, H, D, seg = w.S, w.H, w.D, w.chunk_lens[0]
    sub = seg // U
    q, k, v = (x.to(dev) for x in synthetic.make_qkv(w))
    # stacked input: tensor 3 r + t is tensor t (q, k, v) of segment r, as U sequence shards
    stack = torch.stack([x[:, r * seg:(r + 1) * seg].reshape(U, 1, sub, H, D)
                         for r in range(R) for x in (q, k, v)])
    grp = torch.empty((3 * R, U, 1, seg, H // U, D), dtype=w.dtype, device=dev)
    o_all = torch.empty((U, 1, seg, H // U, D), dtype=w.dtype, device=dev)
    back = torch.empty((U, 1, sub, H, D), dtype=w.dtype, device=dev)
    lse = torch.empty((1, H // U, seg), dtype=torch.float32, device=dev)
    ws = torch.empty(max(cp.ring_attention_workspace_bytes(R, 1, H // U, seg, D), 16),
                     dtype=torch.uint8, device=dev)
    r, u = 0, 0
    chunks = [(grp[3 * c + 1][u], grp[3 * c + 2][u], c * seg) for c in range(R)]
    visit = [chunks[c] for c in synthetic.ring_order(r, R)]

    def attend():
        cp.ring_attention(grp[3 * r][u], visit, o_all[u], lse, workspace=ws)

    def step():
        cp.ulysses_seq2head(stack, U, grp)
        attend()
        cp.ulysses_head2seq(o_all, U, back)

    flops = 4.0 * D * (H // U) * seg * S
    att_ms = time_back_to_back(torch, attend, 3, 20)
    step_ms = time_back_to_back(torch, step, 3, 20)
    res = {"ulysses": U, "ring": R, "attn_us": att_ms * 1e3,
           "attn_tflops": flops / (att_ms * 1e-3) / 1e12,
           "attn_mfma_frac": flops / (att_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
           "step_us": step_ms * 1e3,
           "step_tflops": flops / (step_ms * 1e-3) / 1e12, "gflop": flops / 1e9,
           "note": "step = one launch regrouping Q, K, V of both ring segments (stacked), "
                   "ring attention, inverse regrouping of O; back-to-back steps"}
    log(f"{w.name}: attn {res['attn_tflops']:.0f} TFLOP/s, whole step {res['step_tflops']:.0f}")
    return res


def stream_overlap_workload(torch, cp, synthetic, dev, layers: int = 4):
    """Qwen-Image Ulysses layers, sequential against pipelined on two streams: the
    stacked Q, K, V regrouping of layer l+1 (all P ranks' pack and unpack, on
    stream B) runs beside layer l's rank-0 attention (stream A), ordered by
    events. Both orders compute the same bytes."""
    w = synthetic.QWEN_ULYSSES
    log(f"{w.name}: stream overlap, {layers} layers")
    P, S_l, H, D, Hl, S = w.P, w.S_local, w.H, w.D, w.H_local, w.S
    base = torch.stack([x.view(P, 1, S_l, H, D) for x in synthetic.make_qkv(w)]).to(dev)
    qkv = [base.clone() for _ in range(layers)]
    del base
    heads = [torch.empty((3, P, 1, S, Hl, D), dtype=w.dtype, device=dev) for _ in range(layers)]
    o = torch.empty((1, S, Hl, D), dtype=w.dtype, device=dev)
    lse = torch.empty((1, Hl, S), dtype=torch.float32, device=dev)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    ready = [torch.cuda.Event() for _ in range(layers)]

    def attend(l, stream):
        cp.attn_chunk_partial(heads[l][0, 0], heads[l][1, 0], heads[l][2, 0], o, lse,
                              out_dtype=w.dtype, stream=stream)

    def sequential():
        for l in range(layers):
            cp.ulysses_seq2head(qkv[l], P, heads[l])
            attend(l, None)

    def pipelined():
        sb.wait_stream(torch.cuda.current_stream())
        cp.ulysses_seq2head(qkv[0], P, heads[0], stream=sb)
        ready[0].record(sb)
        for l in range(layers):
            sa.wait_event(ready[l])
            attend(l, sa)
            if l + 1 < layers:
                cp.ulysses_seq2head(qkv[l + 1], P, heads[l + 1], stream=sb)
                ready[l + 1].record(sb)
        torch.cuda.current_stream().wait_stream(sa)

    seq_ms = time_back_to_back(torch, sequential, 2, 10) / layers
    pipe_ms = time_back_to_back(torch, pipelined, 2, 10) / layers
    res = {"layers": layers, "sequential_us_per_layer": seq_ms * 1e3,
           "pipelined_us_per_layer": pipe_ms * 1e3,
           "note": "per layer: stacked Q, K, V seq2head of all 4 ranks (349 MB moved) and "
                   "rank-0 attention (6 heads x 9472); pipelined = next layer's regrouping on "
                   "a second stream beside this layer's attention"}
    log(f"{w.name}: sequential {res['sequential_us_per_layer']:.0f} us/layer, pipelined "
        f"{res['pipelined_us_per_layer']:.0f} us/layer")
    del qkv, heads
    torch.cuda.empty_cache()
    return res


def ring_anything_workload(torch, cp, synthetic, dev):
    w = synthetic.LLM_RING_ANYTHING
    log(f"{w.name}: ranks")
    q, k, v = (x.to(dev) for x in synthetic.make_qkv(w))
    starts = w.chunk_starts()
    chunks = [(k[:, s:s + n].contiguous(), v[:, s:s + n].contiguous(), s)
              for s, n in zip(starts, w.chunk_lens)]
    res = {}
    for causal in (False, True):
        tot_us, tot_flops = 0.0, 0.0
        for r in range(w.P):
            s0, n = starts[r], w.chunk_lens[r]
            qr = q[:, s0:s0 + n].contiguous()
            vis = [chunks[c] for c in synthetic.ring_order(r, w.P)]
            # outputs and workspace allocated once, as a training step would
            o = torch.empty_like(qr)
            lse = torch.empty((1, w.H, n), dtype=torch.float32, device=dev)
            ws = torch.empty(max(1, cp.ring_attention_workspace_bytes(w.P, 1, w.H, n, w.D)),
                             dtype=torch.uint8, device=dev)
            d = [time_back_to_back(
                torch, lambda: cp.ring_attention(qr, vis, o, lse, causal=causal, q_pos0=s0,
                                                 workspace=ws), 5, 50)]
            tot_us += median(d) * 1e3
            tot_flops += attn_flops(n, w.S, w.H, w.D, causal, s0, 0)
        res["causal" if causal else "noncausal"] = {
            "us_all_ranks": tot_us, "tflops": tot_flops / (tot_us * 1e-6) / 1e12,
            "gflop": tot_flops / 1e9}
    return res


if __name__ == "__main__":
    sys.exit(main())
