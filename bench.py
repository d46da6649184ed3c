"""Benchmark of the attention forward pass (libfa355) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one call of fa_fwd (one kernel launch) over one batch of seeded
synthetic inputs already resident in HBM.  The default workload is the
LLM-prefill shape B=4 H=32 N=4096 d=128, bf16, causal.  Prints ONE JSON line
on stdout (human-readable detail goes to stderr):

  value      attention TFLOP/s = 4 B H N^2 d (halved for causal) / time per step
  roofline   the kernel against the bf16 dense matrix-core peak, with its
             average launch duration measured by HIP events on the launch
             stream, and (when a counter summary of the current kernel source
             is committed under profiles/) its HBM traffic per launch
  cpu_baseline  the fp64 oracle timed on the host cores on a bounded sample
             of the same workload (whole heads), scaled to TFLOP/s
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

import numpy as np  # noqa: E402

import fa_inputs  # noqa: E402

METRIC = "attention fwd TFLOP/s + % bf16 MFMA peak, B4 H32 N4096 d128 causal, 1 GPU"
# MI355X dense bf16 matrix-core peak: 256 CUs x 2.4 GHz x 4096 flop/clk/CU.
PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12   # 2516.6
PEAK_F32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
# Vector-ALU work of the method per (query, allowed key) pair, in wave64
# instruction slots of one SIMD: one exp2 (v_exp_f32), and 2.5 plain fp32 ops
# (the scale-and-subtract FMA, the row-sum add, half of a two-value bf16
# pack).  Issue cost per wave64 instruction on one SIMD, measured on MI355X
# with two waves per SIMD issuing independent streams (see the design notes):
VALU_CYC_EXP = 8.0
VALU_CYC_OP = 4.0
VALU_OPS_PER_PAIR = 2.5
SIMDS = 256 * 4
CLOCK_HZ = 2.4e9
KERNEL_SOURCES = ["flashattention_forward_07_amd/csrc/fa_fwd_kernel.hip",
                  "flashattention_forward_07_amd/csrc/fa_fwd_pipe.hip",
                  "flashattention_forward_07_amd/csrc/fa_bf16_tile.h",
                  "flashattention_forward_07_amd/csrc/fa_common.h",
                  "flashattention_forward_07_amd/csrc/fa_fwd_launch.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attention_flops(lengths, H, d, causal):
    """4 N^2 d per head (Q K^T and P V, 2 flops per multiply-add), halved when
    causal -- the metric's convention."""
    n2 = float(np.sum(np.asarray(lengths, dtype=np.float64) ** 2))
    f = 4.0 * H * n2 * d
    return f / 2.0 if causal else f


def attention_pairs(lengths, H, causal):
    """(query, allowed key) pairs: N^2 per head, N (N + 1) / 2 when causal."""
    n = np.asarray(lengths, dtype=np.float64)
    return float(H * np.sum(n * (n + 1) / 2 if causal else n * n))


def roofline_terms(flops, pairs, nbytes, kern_s, mfma_peak_tflops):
    """Lower bounds on the launch time from each unit, and the fraction of
    the measured launch time each one accounts for:
      mfma  the metric's flops at the dense matrix-core peak;
      valu  the softmax's vector work (one exp2 and VALU_OPS_PER_PAIR plain
            ops per pair, 64 lanes per instruction) at the measured issue
            costs, on all SIMDs at the 2.4 GHz peak clock;
      hbm   the compulsory bytes at 8 TB/s.
    The binding term is the largest bound."""
    t_mfma = flops / (mfma_peak_tflops * 1e12)
    t_valu = pairs / 64.0 * (VALU_CYC_EXP + VALU_OPS_PER_PAIR * VALU_CYC_OP) / (SIMDS * CLOCK_HZ)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    terms = {"mfma_us": t_mfma * 1e6, "valu_us": t_valu * 1e6, "hbm_us": t_hbm * 1e6}
    out = {k: round(v, 3) for k, v in terms.items()}
    out.update({"mfma_frac": round(t_mfma / kern_s, 4), "valu_frac": round(t_valu / kern_s, 4),
                "hbm_frac": round(t_hbm / kern_s, 4)})
    out["binding"] = max(("mfma", t_mfma), ("valu", t_valu), ("hbm", t_hbm), key=lambda x: x[1])[0]
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def prewarm(torch, step, seconds):
    """Untimed launches for a fixed wall time, so the timed steps start from
    the clock and power state the GPU holds under sustained load (a fresh
    GPU's first tens of milliseconds of launches run slower)."""
    if seconds <= 0:
        return 0, 0.0
    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(8):
            step()
        n += 8
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        if el >= seconds:
            return n, el


def cold_cache_us(torch, step, reps, flush_bytes=1 << 30):
    """Median launch time with the caches flushed before every launch: a
    1 GiB buffer (larger than the L2s and the Infinity Cache together) is
    overwritten between launches, outside the timed events."""
    st = torch.cuda.current_stream()
    junk = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")
    times = []
    for i in range(reps):
        junk.fill_(float(i))
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(st)
        step()
        b.record(st)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) * 1e3)
    del junk
    return float(np.median(times))


def algorithmic_bytes(total_tokens, H, d, elem):
    """Compulsory HBM bytes: read Q, K, V once, write O once, write lse."""
    return total_tokens * H * (4 * d * elem + 4)


def naive_bytes(N, B, H, d, elem, causal):
    """HBM bytes the unfused three-step method cannot avoid per launch: Q, K,
    V read and O, lse written once, and every allowed score written as fp32,
    read back, its probability written in the input dtype and read again
    (N^2 scores per head, about half of them when causal)."""
    scores = N * (N + 1) / 2 if causal else float(N) * N
    return B * H * (N * (4 * d * elem + 4) + scores * (4 + 4 + 2 * elem))


DECODE_SOURCES = ["flashattention_forward_07_amd/csrc/fa_decode.hip",
                  "flashattention_forward_07_amd/csrc/fa_decode_launch.h",
                  "flashattention_forward_07_amd/csrc/fa355_api.hip"]


def kernel_source_hash(sources=None):
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES if sources is None else sources):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(workload_name, prefix="fa_fwd", sources=None):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{prefix}_{workload_name}_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != kernel_source_hash(sources):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, inp, budget_s):
    """Time the oracle on whole heads of the workload until ~budget_s."""
    import oracle
    # the host share of this GPU: OMP_NUM_THREADS when set, else the affinity mask
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    flops = 0.0
    heads = 0
    t0 = time.perf_counter()
    if w.varlen:
        cu = inp.cu_seqlens
        order = np.argsort(np.diff(cu))[::-1]  # long sequences first
        for s in order:
            a, b = int(cu[s]), int(cu[s + 1])
            for h in range(w.H):
                oracle.attention(inp.q[a:b, h], inp.k[a:b, h], inp.v[a:b, h], w.scale, w.causal)
                flops += attention_flops([b - a], 1, w.d, w.causal)
                heads += 1
                if time.perf_counter() - t0 > budget_s:
                    break
            if time.perf_counter() - t0 > budget_s:
                break
        sample = f"{heads} whole (sequence, head) slices, longest sequences first"
    else:
        # whole (batch, head) slices in order; a workload that finishes in
        # under two seconds is repeated so the rate is not timer noise
        B, H = w.B, w.H
        i = 0
        while True:
            b, h = divmod(i % (B * H), H)
            oracle.attention(inp.q[b, h], inp.k[b, h], inp.v[b, h], w.scale, w.causal)
            flops += attention_flops([w.N], 1, w.d, w.causal)
            heads += 1
            i += 1
            el = time.perf_counter() - t0
            if el > budget_s or (i >= B * H and el > 2.0):
                break
        sample = (f"{heads} of {B * H} whole (batch, head) slices" if heads <= B * H else
                  f"the whole workload ({B * H} (batch, head) slices) {heads / (B * H):.0f} times")
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{sample}; {flops / 1e9:.1f} GFLOP in {dt:.1f} s, fp64"}


def decode_flops(w):
    """4 d flops per visible (query, key) pair."""
    if w.causal:
        vis = sum(min(w.Nk, max(0, w.Nk - w.Nq + i + 1)) for i in range(w.Nq))
    else:
        vis = w.Nq * w.Nk
    return 4.0 * w.B * w.H * vis * w.d


def decode_bytes(w, elem):
    """Compulsory HBM bytes of a decode step: K and V read once, Q read, O
    and lse written."""
    return w.B * w.H * (2 * w.Nk * w.d * elem + w.Nq * (2 * w.d * elem + 4))


def bench_decode(args, torch, fa):
    """One step = one fa_decode_fwd call (split kernel + merge kernel) over a
    decode workload resident in HBM; reported in GB/s of compulsory bytes."""
    w = fa_inputs.decode_by_name(args.workload)
    log(f"[bench] decode workload {w.name}: generating seeded inputs")
    inp = fa_inputs.make_decode_workload(w)
    elem = 2 if w.dtype == "bf16" else 4
    code = fa.FA_DTYPE_BF16 if w.dtype == "bf16" else fa.FA_DTYPE_F32

    def dev(x):
        if w.dtype == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda")
        return torch.from_numpy(x).to("cuda")

    q, k, v = (dev(x) for x in inp.device_arrays())
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    splits = fa.fa_decode_num_splits(w.B, w.H, w.Nq, w.Nk, 0)
    wsb = fa.fa_decode_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d, 0)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    log(f"[bench] {splits} key ranges per (b, h), workspace {wsb / 2**20:.2f} MiB")

    def step():
        fa.fa_decode_fwd(q, k, v, o, lse, ws, wsb, w.B, w.H, w.Nq, w.Nk, w.d, w.scale, w.causal,
                         code, 0)

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [s_.elapsed_time(e_) for s_, e_ in zip(starts, ends)]
    kern_ms = float(np.mean(per))
    ms_per_step = wall * 1e3 / args.steps
    nbytes = decode_bytes(w, elem)
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    log(f"[bench] step mean {kern_ms:.4f} ms (median {np.median(per):.4f}, min {np.min(per):.4f}); "
        f"wall {ms_per_step:.4f} ms/step; {achieved:.0f} GB/s = "
        f"{100 * achieved / PEAK_HBM_GBS:.1f}% of {PEAK_HBM_GBS:.0f}")
    result = {
        "metric": f"attention decode GB/s (compulsory bytes), {w.name}",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "method": "split-kv decode", "via": "fa_decode_fwd",
                   "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d, "causal": w.causal,
                   "splits": splits, "bytes_per_step": nbytes,
                   "flops_per_step": decode_flops(w)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": committed_traffic(w.name, "fa_decode", DECODE_SOURCES)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
        oracle.set_threads(threads)
        t0 = time.perf_counter()
        n = 0
        while True:  # whole batches of heads until the budget is spent
            b = n % w.B
            oracle.attention_decode(inp.q[b:b + 1], inp.k[b:b + 1], inp.v[b:b + 1], w.scale,
                                    w.causal)
            n += 1
            if time.perf_counter() - t0 > args.cpu_budget:
                break
        dt = time.perf_counter() - t0
        cb = n * nbytes / w.B
        result["cpu_baseline"] = {"value": round(cb / dt / 1e9, 3), "unit": "GB/s",
                                  "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
                                  "sample": f"{n} of {w.B} batch entries (all {w.H} heads each) "
                                            f"in {dt:.1f} s, fp64"}
        log(f"[bench] cpu baseline {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)


def _timed(torch, fn, reps, warmup):
    for _ in range(warmup):
        fn()
    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(st)
        fn()
        b.record(st)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]))


def _timed_back_to_back(torch, fn, reps, warmup):
    """Mean launch time of reps launches issued back to back between two
    events (as the workload bench times its steps)."""
    for _ in range(warmup):
        fn()
    st = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(st)
    for _ in range(reps):
        fn()
    b.record(st)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def compare_short(torch, fa, reps=50, warmup=10):
    """Many short sequences (one head each, causal, bf16 and fp32): fa_fwd,
    which takes the one-tile kernels for N <= 128 (fp32 only while
    latency-bound), against the general streaming kernel on the same data
    (fa_fwd_varlen with equal lengths and max_seqlen 129: with one head the
    packed and the fixed layouts coincide) and the naive method.  Median
    launch times, each launch between its own pair of events; for fa_fwd also
    the mean over launches issued back to back (where one launch's last
    workgroups overlap the next one's first), and the compulsory bytes per
    second of both."""
    print("| dtype | d | sequences | N | fa_fwd path | fa_fwd us | general kernel us | naive us | "
          "fa_fwd GB/s | general / fa_fwd | fa_fwd us, back to back | GB/s, back to back |")
    print("|---|---|---:|---:|---|---:|---:|---:|---:|---:|---:|---:|")
    for dtype, d, B, N in [(dt, d, B, N) for dt in ("bf16", "f32") for d in (64, 128)
                           for B in (1, 1024, 8192) for N in (16, 64, 128)]:
                inp = fa_inputs.make_fixed(B, 1, N, d, dtype, seed=9500 + N + d)
                if dtype == "bf16":
                    q, k, v = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda")
                               for x in inp.device_arrays())
                else:
                    q, k, v = (torch.from_numpy(x).to("cuda") for x in inp.device_arrays())
                scale = float(np.float32(1.0 / math.sqrt(d)))
                o1, o2, o3 = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
                l1 = torch.empty((B, 1, N), dtype=torch.float32, device="cuda")
                l2, l3 = torch.empty_like(l1), torch.empty_like(l1)
                cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device="cuda")
                wsb = fa.fa_naive_workspace_bytes(B, 1, N)
                ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
                code = fa.FA_DTYPE_BF16 if dtype == "bf16" else fa.FA_DTYPE_F32
                elem = 2 if dtype == "bf16" else 4
                t1 = _timed(torch, lambda: fa.fa_fwd(q, k, v, o1, l1, B, 1, N, d, scale, True,
                                                     code), reps, warmup)
                # max_seqlen 129 (an upper bound, so still valid) keeps fa_fwd_varlen
                # on the streaming kernel: with every sequence at most 128 tokens it
                # would take the one-tile kernel too
                t2 = _timed(torch, lambda: fa.fa_fwd_varlen(q, k, v, o2, l2, cu, B, 129, 1, d,
                                                            scale, True, code), reps, warmup)
                t3 = _timed(torch, lambda: fa.fa_naive_fwd(q, k, v, o3, l3, ws, wsb, B, 1, N, d,
                                                           scale, True, code), reps, warmup)
                t4 = _timed_back_to_back(torch, lambda: fa.fa_fwd(q, k, v, o1, l1, B, 1, N, d, scale,
                                                                  True, code), reps, warmup)
                diff = (o1.float() - o2.float()).abs().max().item()
                if diff > (2e-2 if dtype == "bf16" else 2e-5):
                    raise SystemExit(f"one-tile and general kernel disagree by {diff}")
                gbs = algorithmic_bytes(B * N, 1, d, elem) / (t1 * 1e-3) / 1e9
                gbs4 = algorithmic_bytes(B * N, 1, d, elem) / (t4 * 1e-3) / 1e9
                # the library's rule: bf16 always one-tile; fp32 while latency-bound
                path = ("one-tile" if dtype == "bf16" or N <= 32 or 4.0 * B * N * N * d <= 2 ** 28
                        else "general")
                print(f"| {dtype} | {d} | {B} | {N} | {path} | {t1 * 1e3:.1f} | {t2 * 1e3:.1f} | "
                      f"{t3 * 1e3:.1f} | {gbs:.0f} | {t2 / t1:.2f} | {t4 * 1e3:.1f} | {gbs4:.0f} |",
                      flush=True)


def compare_naive(torch, fa, reps=20, warmup=5):
    """Fused kernel against the unfused three-step method on the same inputs:
    one head of d=64 (the single-head shape of the pages' naive-versus-tiled
    timing) in fp32 and bf16, and 32 heads in bf16, over N = 128 .. 16384,
    non-causal.  Per point: mean launch time of each method (HIP events on the
    launch stream), the speedup, and the largest |O_fused - O_naive|."""
    def timed(fn):
        for _ in range(warmup):
            fn()
        st = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record(st)
            fn()
            b.record(st)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev]))

    print("| dtype | B x H | N | fused ms | naive ms | naive / fused | max abs O diff |")
    print("|---|---|---:|---:|---:|---:|---:|")
    for dtype, H, ns in (("f32", 1, [128, 256, 512, 1024, 2048, 4096, 8192, 16384]),
                         ("bf16", 1, [128, 256, 512, 1024, 2048, 4096, 8192, 16384]),
                         ("bf16", 32, [128, 512, 1024, 2048, 4096, 8192])):
        for N in ns:
            B, d = 1, 64
            inp = fa_inputs.make_fixed(B, H, N, d, dtype, seed=9000 + N + H)
            if dtype == "bf16":
                q, k, v = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda")
                           for x in inp.device_arrays())
                code = fa.FA_DTYPE_BF16
            else:
                q, k, v = (torch.from_numpy(x).to("cuda") for x in inp.device_arrays())
                code = fa.FA_DTYPE_F32
            scale = float(np.float32(1.0 / math.sqrt(d)))
            o1, o2 = torch.empty_like(q), torch.empty_like(q)
            l1 = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
            l2 = torch.empty_like(l1)
            wsb = fa.fa_naive_workspace_bytes(B, H, N)
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            tf = timed(lambda: fa.fa_fwd(q, k, v, o1, l1, B, H, N, d, scale, False, code))
            tn = timed(lambda: fa.fa_naive_fwd(q, k, v, o2, l2, ws, wsb, B, H, N, d, scale,
                                               False, code))
            diff = (o1.float() - o2.float()).abs().max().item()
            print(f"| {dtype} | {B} x {H} | {N} | {tf:.4f} | {tn:.4f} | {tn / tf:.2f} | "
                  f"{diff:.2e} |", flush=True)
            del ws


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=fa_inputs.HEADLINE.name,
                    choices=[w.name for w in fa_inputs.WORKLOADS] +
                    [w.name for w in fa_inputs.DECODE_WORKLOADS],
                    help="a prefill workload (fa_fwd), or a decode_* workload (fa_decode_fwd, "
                         "split-KV, measured in GB/s against the HBM peak)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prewarm-s", type=float, default=2.0,
                    help="seconds of untimed launches before the warm-up steps (reported as "
                         "prewarm_s; 0 disables)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time")
    ap.add_argument("--method", choices=["fused", "naive"], default="fused",
                    help="fused: fa_fwd (the library's kernel); naive: fa_naive_fwd, the "
                         "unfused three-step baseline (fixed-length workloads)")
    ap.add_argument("--via-op", action="store_true",
                    help="time the step through the PyTorch operator torch.ops.fa355.fwd "
                         "(fixed-length workloads; outputs allocated per call)")
    ap.add_argument("--compare-naive", action="store_true",
                    help="instead of the bench line, time the fused kernel against the naive "
                         "three-step method over a range of N (one head and 32 heads, d=64, "
                         "non-causal) and print a markdown table")
    ap.add_argument("--compare-short", action="store_true",
                    help="instead of the bench line, time the one-tile path fa_fwd takes for "
                         "bf16 N <= 128 against the general streaming kernel and the naive "
                         "method on many short sequences, and print a markdown table")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, run a plain 1 GiB device copy (for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU; --gpus {args.gpus} is not "
              "supported (every (batch, head) is independent, so several GPUs would each run "
              "this kernel on their own heads).", file=sys.stderr)
        sys.exit(2)

    import torch
    import flashattention_forward_07_amd as fa
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    if args.compare_naive:
        compare_naive(torch, fa)
        return
    if args.compare_short:
        compare_short(torch, fa)
        return
    if args.workload.startswith("decode_"):
        bench_decode(args, torch, fa)
        return

    w = fa_inputs.by_name(args.workload)
    log(f"[bench] workload {w.name}: generating seeded inputs")
    inp = fa_inputs.make(w)
    elem = 2 if w.dtype == "bf16" else 4
    code = fa.FA_DTYPE_BF16 if w.dtype == "bf16" else fa.FA_DTYPE_F32

    def dev(x):
        if w.dtype == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda")
        return torch.from_numpy(x).to("cuda")

    q, k, v = (dev(x) for x in inp.device_arrays())
    o = torch.empty_like(q)
    if w.varlen:
        T = inp.q.shape[0]
        lse = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
        cu = torch.from_numpy(inp.cu_seqlens).to("cuda")
        lengths = np.diff(inp.cu_seqlens)
        nseq = lengths.size

        def step():
            fa.fa_fwd_varlen(q, k, v, o, lse, cu, nseq, w.max_len, w.H, w.d, w.scale, w.causal,
                             code)
        total_tokens = int(inp.cu_seqlens[-1])
    else:
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
        lengths = [w.N] * w.B

        if args.method == "naive":
            ws_bytes = fa.fa_naive_workspace_bytes(w.B, w.H, w.N)
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
            log(f"[bench] naive three-step method, {ws_bytes / 2**30:.2f} GiB scores workspace")

            def step():
                fa.fa_naive_fwd(q, k, v, o, lse, ws, ws_bytes, w.B, w.H, w.N, w.d, w.scale,
                                w.causal, code)
        elif args.via_op:
            import flashattention_forward_07_amd.torch_ops  # noqa: F401  (registers the op)

            def step():
                torch.ops.fa355.fwd(q, k, v, w.causal, w.scale)
        else:
            def step():
                fa.fa_fwd(q, k, v, o, lse, w.B, w.H, w.N, w.d, w.scale, w.causal, code)
        total_tokens = w.B * w.N

    if w.varlen and args.method != "fused":
        raise SystemExit("bench.py: --method naive takes fixed-length workloads")
    flops = attention_flops(lengths, w.H, w.d, w.causal)
    alg_bytes = algorithmic_bytes(total_tokens, w.H, w.d, elem)
    if args.method == "naive":
        alg_bytes = naive_bytes(w.N, w.B, w.H, w.d, elem, w.causal)

    stream = torch.cuda.current_stream()  # fa_fwd launches on this stream
    n_pre, t_pre = prewarm(torch, step, args.prewarm_s)
    log(f"[bench] prewarm: {n_pre} untimed launches in {t_pre:.2f} s")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps")

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    kern_ms = float(np.mean(per_launch_ms))
    ms_per_step = wall * 1e3 / args.steps
    qn = max(1, len(per_launch_ms) // 4)
    q1_ms = float(np.mean(per_launch_ms[:qn]))
    q4_ms = float(np.mean(per_launch_ms[-qn:]))
    log(f"[bench] kernel mean {kern_ms:.4f} ms, median {np.median(per_launch_ms):.4f} ms, "
        f"min {np.min(per_launch_ms):.4f} ms; first quarter {q1_ms:.4f} ms, last quarter "
        f"{q4_ms:.4f} ms; wall {ms_per_step:.4f} ms/step")

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 3 x 1 GiB device copies done")

    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS
    traffic = committed_traffic(w.name) if args.method == "fused" else None
    pairs = attention_pairs(lengths, w.H, w.causal)
    terms = roofline_terms(flops, pairs, alg_bytes, kern_ms * 1e-3, peak)
    log(f"[bench] roofline terms {terms}")
    log(f"[bench] {value:.1f} TFLOP/s per step, kernel {achieved:.1f} TFLOP/s = "
        f"{100 * achieved / peak:.1f}% of {peak:.1f}; algorithmic bytes {alg_bytes / 1e6:.1f} MB "
        f"-> {alg_bytes / (kern_ms * 1e-3) / 1e9:.0f} GB/s")

    result = {
        "metric": (METRIC if w is fa_inputs.HEADLINE and args.method == "fused" else
                   f"attention fwd TFLOP/s, {w.name}" + ("" if args.method == "fused" else
                                                       f", {args.method} method")),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "method": args.method,
                   "via": ("fa_naive_fwd" if args.method == "naive" else
                           "torch.ops.fa355.fwd" if args.via_op else "fa_fwd"),
                   "B": w.B if not w.varlen else int(len(lengths)),
                   "H": w.H, "N": w.N if not w.varlen else int(max(lengths)), "d": w.d,
                   "causal": w.causal, "varlen": w.varlen, "tokens": total_tokens,
                   "flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": round(peak, 1),
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic, "terms": terms},
        "launch_ms": {"mean": round(kern_ms, 5), "median": round(float(np.median(per_launch_ms)), 5),
                      "min": round(float(np.min(per_launch_ms)), 5),
                      "first_quarter": round(q1_ms, 5), "last_quarter": round(q4_ms, 5)},
        "prewarm_s": round(t_pre, 3),
        "prewarm_launches": n_pre,
    }
    if terms["binding"] == "valu" and args.method == "fused":
        # the softmax's vector work bounds this workload (d = 64: half the
        # matrix work per exp2); report the fraction against that unit, in
        # (query, key) pairs per second, and keep the matrix-core fraction
        vpeak = pairs / (terms["valu_us"] * 1e-6) / 1e9
        vach = pairs / (kern_ms * 1e-3) / 1e9
        result["roofline"].update({"bound": "alu", "achieved": round(vach, 1),
                                   "peak": round(vpeak, 1), "unit": "Gpair/s",
                                   "frac": round(vach / vpeak, 4),
                                   "mfma_achieved_tflops": round(achieved, 3),
                                   "mfma_frac": round(achieved / peak, 4)})
    elif terms["binding"] == "hbm" and args.method == "fused":
        gbs = alg_bytes / (kern_ms * 1e-3) / 1e9
        result["roofline"].update({"bound": "hbm", "achieved": round(gbs, 1),
                                   "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": round(gbs / PEAK_HBM_GBS, 4),
                                   "mfma_achieved_tflops": round(achieved, 3),
                                   "mfma_frac": round(achieved / peak, 4)})
    if alg_bytes <= (64 << 20) and args.method == "fused":
        # small workloads: also the launch with cold caches
        cc = cold_cache_us(torch, step, reps=max(10, min(args.steps, 50)))
        result["cold_cache_us"] = round(cc, 2)
        log(f"[bench] cold caches: median {cc:.2f} us per launch")
    if args.method == "naive":
        # three launches per step, bound by the N x N round trips through HBM
        gbs = alg_bytes / (kern_ms * 1e-3) / 1e9
        result["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                              "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                              "traffic": None, "algorithmic_bytes": alg_bytes}
    if not args.no_cpu_baseline:
        log(f"[bench] timing the fp64 oracle on the host (~{args.cpu_budget:.0f} s)")
        result["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_budget)
        result["cpu_baseline"]["cpu_model"] = cpu_model()
        log(f"[bench] cpu baseline {result['cpu_baseline']}")
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
