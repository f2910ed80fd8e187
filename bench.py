#!/usr/bin/env python3
"""Benchmark of the fused LM-head projection + full-vocabulary reverse KL on one GPU.

A step is one pass of the whole path over one batch that is already resident in
device memory: loss-mask compaction, row gather, fused forward (both
projections + online log-sum-exp / KL), scatter of the per-token loss,
recomputing backward (dz, dW, dh) and scatter of dh.  The compaction runs one
batch ahead, as a trainer prefetching its next batch would run it (NextRows):
each step enqueues its kernels, then compacts the next batch's mask on a side
stream; every step still runs one compaction.

Workload: Qwen3-1.7B-shaped hidden-state path, B=4 sequences of S=1025 tokens,
every one of the T = B(S-1) = 4096 positions trainable (N = 4096), Hs = Ht =
2048, V = 151936, bf16 inputs (synthetic, seeded), fp32 accumulation.

--payload logits times the same step with the teacher given as fp32 logits
[T, V] (formed once from the same tensors) instead of hidden states; the
kernels read the compacted rows through the row index (no [N, V] copy).

--workload logprob_entropy times the compact actor path instead: per row the
log-probability of a sampled token and the entropy of softmax(h_s W_s^T)
(forward), and the gradients dh, dW of g_lp logp + g_H H (backward), on the
same student tensors.

--workload teachers times the reverse-KL step with --teachers K teacher
weights and a teacher chosen per row (--teacher-order grouped: K contiguous
runs of rows; interleaved: i.i.d. ids, so every tile holds several teachers).

--workload topk times the top-k estimator of the reverse KL on the same
student tensors: the teacher's payload is its log-probabilities at its --topk
K largest logits and at a sampled token per row.

--dp-ranks G times one rank's share of a G-way data-parallel group: the
first T/G positions of the same workload with the weights replicated (the
rows are independent: no exchange but the trainer's dW all-reduce).

--workload vocab_shard times one rank's share of a --shards G-way
vocabulary-parallel step on the same tensors: the shard forward over its
V/G vocabulary rows, the merge of all G shards' partials (the other shards'
already resident, as an all-gather would leave them), the loss scatter, the
shard backward with the merged stats and the scatter of its dh term.  The
exchanges between ranks (all-gather of the partials, all-reduce of dh) are
not part of it.

Prints one JSON line:
  value      = masked tokens/s for forward + backward (wall clock over the
               timed steps, synchronised on both sides);
  per_kernel = every kernel of the path with its device time per step and
               per launch, measured in the timed steps with hipEvents that
               each launch stamps with its kernel's begin and end, and for
               the MFMA kernels their algorithmic FLOPs against the dense
               bf16/fp16 MFMA peak (the side-stream compaction is left out:
               it waits for a free compute unit while the step's kernels
               hold them all, so its event span is not its run time);
  roofline   = the kernel with the most device time per step, with the HBM
               traffic per launch from the committed counter record while
               the kernel sources are unchanged;
  cpu_baseline = the fp64 oracle on a bounded row sample on the host cores
               (reverse-KL, log-probability / entropy and top-k workloads).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "masked tokens/sec fwd+bwd full-vocab reverse KL (H2048,V152k); MFMA % peak"
# MI355X dense bf16/fp16 MFMA peak: 256 CUs x 4096 FLOP/clk x 2.4 GHz.
PEAK_BF16 = 256 * 4096 * 2.4e9
HBM_PEAK = 8.0e12
DTYPE = "bf16 projections; fp16 dz/dh/dW GEMM operands (power-of-two scaled); fp32 accumulation"

FWD_KERNELS = ("fwd_tiles", "fwd_combine", "fwd_rows_logits", "topk_terms")
BWD_KERNELS = ("grad_scale", "absmax_bf16", "convert_h", "bwd_dz_tiles", "w_rescale", "dw_gemm", "dh_gemm", "dh_reduce",
               "bwd_rows_logits", "topk_dz_add")
MFMA_KERNELS = ("fwd_tiles", "bwd_dz_tiles", "dw_gemm", "dh_gemm")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU work for the oracle sample")
    ap.add_argument("--profile-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (counter calibration)")
    ap.add_argument("--payload", choices=("hidden", "logits"), default="hidden",
                    help="teacher payload: hidden states (default, the headline) or fp32 logits [N, V]")
    ap.add_argument("--workload", choices=("reverse_kl", "logprob_entropy", "teachers", "vocab_shard", "topk"),
                    default="reverse_kl",
                    help="reverse KL distillation step (default, the headline), log-probability + entropy, "
                         "reverse KL with a teacher chosen per row, one rank's share of a vocabulary-parallel "
                         "step, or the top-k estimator")
    ap.add_argument("--topk", type=int, default=64, help="support size K for --workload topk")
    ap.add_argument("--shards", type=int, default=8, help="vocabulary shards for --workload vocab_shard")
    ap.add_argument("--dp-ranks", type=int, default=1,
                    help="reverse_kl workload: time one rank's share of a data-parallel group of this many "
                         "ranks (the first T/ranks positions, weights replicated)")
    ap.add_argument("--teachers", type=int, default=4, help="teachers for --workload teachers")
    ap.add_argument("--teacher-order", choices=("grouped", "interleaved"), default="grouped",
                    help="row order for --workload teachers")
    ap.add_argument("--report-c5", action="store_true",
                    help="time compact vs full-row on the long-prompt workload (T=32768, N=4096, Ht=4096)")
    return ap.parse_args()


# ---------------------------------------------------------------- traffic record

def kernel_source_hash() -> str:
    """Hash of the HIP sources with comments and blank space removed: a
    recorded traffic measurement is only reused while the code it was taken
    on is unchanged."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "lm_head_reverse_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        src = "\n".join(line.strip() for line in src.splitlines() if line.strip())
        h.update(name.encode() + b"\0" + src.encode())
    return h.hexdigest()[:16]


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "headline_kernels_hbm_traffic.txt")


def recorded_traffic() -> dict:
    """{kernel: record} of HBM bytes per launch on the headline workload from
    the committed counter summary (FETCH_SIZE + WRITE_SIZE scaled by the
    copy-kernel factors), for the records taken on the current sources."""
    out = {}
    try:
        with open(TRAFFIC_FILE) as f:
            for line in f:
                line = line.strip()
                if line.startswith("{"):
                    rec = json.loads(line)
                    if rec.get("kernel_source_hash") == kernel_source_hash():
                        out[rec["kernel"]] = rec
    except OSError:
        pass
    return out


def profile_copy():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)


def report_c5():
    """Warm timing and peak extra memory of compact vs full-row."""
    import numpy as np
    import torch
    import lm_head_reverse_amd as R
    import synth
    dev = torch.device("cuda:0")
    case = synth.config("c5")

    def bf(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    h_s, h_t, W_s, W_t = bf(case.h_s), bf(case.h_t), bf(case.W_s), bf(case.W_t)
    mask = torch.from_numpy(case.mask).to(dev)
    dW = torch.empty(W_s.shape, dtype=torch.float32, device=dev)

    def compact():
        idx, N = R.compact_rows(mask)
        hs, ht = R.gather_rows(h_s, idx), R.gather_rows(h_t, idx)
        loss, st = R.forward_hidden(hs, W_s, ht, W_t)
        dh, _ = R.backward_hidden(hs, W_s, ht, W_t, st, dW=dW)
        return R.scatter_rows(loss, idx, case.T), R.scatter_rows(dh, idx, case.T)

    def full():
        loss, st = R.forward_hidden(h_s, W_s, h_t, W_t, row_mask=mask)
        dh, _ = R.backward_hidden(h_s, W_s, h_t, W_t, st, row_mask=mask, dW=dW)
        return loss, dh

    out = {"workload": "long masked prompts: B=2, S=16385 (T=32768), last 2048 of each sequence trainable "
                       "(N=4096), Hs=2048, Ht=4096, V=151936"}
    for name, fn in (("compact", compact), ("full_row", full)):
        fn()
        torch.cuda.synchronize()
        R._ws_cache.clear()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        reps = 3
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        out[name + "_ms"] = round((time.perf_counter() - t0) * 1e3 / reps, 3)
        out[name + "_extra_peak_GiB"] = round((torch.cuda.max_memory_allocated() - base) / 2 ** 30, 3)
    out["full_over_compact_time"] = round(out["full_row_ms"] / out["compact_ms"], 2)
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------- CPU baseline

def host_info() -> dict:
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "host_logical_cpus": os.cpu_count(), "usable_cpus": usable}


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def grow_sample(run, target_s: float, cap: int, step: int = 32):
    """Grow the row sample until one run takes about target_s (the per-row
    cost of a small probe overstates the steady cost)."""
    n = step
    t = run(n)
    while t < target_s / 2 and n < cap:
        n = int(min(cap, max(n + step, n * target_s / max(t, 1e-3))) // step * step)
        t = run(n)
    return n, t


def single_core_small() -> dict:
    """The fp64 oracle on one thread: forward + backward of the tiny logits
    workload (T=64, V=1024) and of the small hidden-state workload (N=256,
    Hs=Ht=256, V=8192), in masked tokens/s."""
    import numpy as np
    import synth
    from oracle import rkl_oracle as O
    from threadpoolctl import threadpool_limits
    out = {}
    with threadpool_limits(limits=1):
        for name in ("c1", "c2"):
            case = synth.config(name)
            inp = O.Inputs.from_case(case)
            rows = O.compact_rows(case.mask)
            best = float("inf")
            for _ in range(3):
                t0 = time.perf_counter()
                O.forward(inp, rows)
                O.backward(inp, rows)
                best = min(best, time.perf_counter() - t0)
            out[name] = {"masked_tokens": int(rows.shape[0]), "seconds": round(best, 4),
                         "tokens_per_s": round(rows.shape[0] / best, 1)}
    out["c1"]["workload"] = "logits both sides, T=64, V=1024"
    out["c2"]["workload"] = "hidden states, B=2 S=129 (T=256), Hs=Ht=256, V=8192"
    return out


def cpu_baseline(case, target_s: float):
    """Time the fp64 oracle (forward + backward) on a bounded row sample."""
    import numpy as np
    from oracle import rkl_oracle as O

    def run(nrows):
        inp = O.Inputs(h_s=case.h_s[:nrows], W_s=case.W_s, h_t=case.h_t[:nrows], W_t=case.W_t)
        rows = np.arange(nrows)
        t0 = time.perf_counter()
        O.forward(inp, rows)
        O.backward(inp, rows)
        return time.perf_counter() - t0

    n, t = grow_sample(run, target_s, min(4096, case.T))
    out = {"value": n / t, "unit": "masked tokens/s", "cores": int(blas_threads()), "kind": "oracle",
           "sample": f"fp64 numpy oracle, forward+backward (L, dh, dW) over the first {n} of the {case.T} "
                     f"positions of this workload, full V={case.V}; {t:.1f} s wall; bf16->fp64 widening "
                     f"of the weights done once outside the timed region"}
    out.update(host_info())
    out["single_core"] = single_core_small()
    return out


def cpu_baseline_lpe(case, y, target_s: float):
    """Time the fp64 log-probability / entropy oracle (forward + backward) on a
    bounded row sample."""
    from oracle import logprob_entropy_oracle as E
    from oracle import rkl_oracle as O
    W = O.widen_bf16(case.W_s)

    def run(nrows):
        h = O.widen_bf16(case.h_s[:nrows])
        t0 = time.perf_counter()
        E.forward(h, W, y[:nrows])
        E.backward(h, W, y[:nrows])
        return time.perf_counter() - t0

    n, t = grow_sample(run, target_s, min(4096, case.T))
    out = {"value": n / t, "unit": "masked tokens/s", "cores": int(blas_threads()), "kind": "oracle",
           "sample": f"fp64 numpy oracle, log-probability + entropy forward+backward (logp, H, dh, dW) over the "
                     f"first {n} of the {case.T} positions of this workload, full V={case.V}; {t:.1f} s wall; "
                     f"bf16->fp64 widening of the weights done once outside the timed region"}
    out.update(host_info())
    return out


# ---------------------------------------------------------------- timing harness

class NextRows:
    """Loss-mask compaction one batch ahead.

    compact_rows waits for its kernel: the row count N sizes every later
    launch.  Issued at a step's start, that wait would drain the device (it
    finishes the previous step, then idles through the round trip and the
    host's first launches).  So each step takes the rows compacted during the
    previous one and, after enqueueing its own kernels, calls advance(): the
    next batch's mask is compacted on a side stream (default priority) while
    the device works through the queued step, and the host waits for that
    one small kernel only.  Per-kernel timing is paused around it (see the
    module docstring).  The inputs are the same every step here, so every
    batch has the same rows."""

    def __init__(self, mask):
        import torch
        self.mask = mask
        self.main = torch.cuda.current_stream(mask.device)
        self.side = torch.cuda.Stream(mask.device)
        self.timed = False
        self.rows = self._compact()

    def _compact(self):
        import torch
        import lm_head_reverse_amd as R
        if self.timed:
            R.kernel_timing(False)
        with torch.cuda.stream(self.side):
            idx, N = R.compact_rows(self.mask)   # returns once the side stream has run it
        if self.timed:
            R.kernel_timing(True)
        idx.record_stream(self.main)   # used by the main stream's kernels
        return idx, N

    def advance(self):
        self.rows = self._compact()


def run_timed(step, args, rows=None):
    """W untimed warm-up steps, then exactly K timed steps bracketed by
    device synchronisation, with the library's per-kernel event timing on.
    Returns (N, wall seconds, {kernel: (total ms, launches)})."""
    import numpy as np
    import torch
    import lm_head_reverse_amd as R
    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        N, out = step()
    torch.cuda.synchronize()
    assert np.all(np.isfinite(out.cpu().numpy())), "non-finite output"
    print("[bench] timing", file=sys.stderr, flush=True)
    R.kernel_timing(True)
    R.kernel_times()   # forget the warm-up's records
    if rows is not None:
        rows.timed = True
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        N, _ = step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = R.kernel_times()
    R.kernel_timing(False)
    if rows is not None:
        rows.timed = False
    return N, wall, times


def kernel_report(times, steps, work):
    """Per-kernel entries and the dominant kernel.  work: {kernel: (FLOPs
    per step, algorithmic bytes per step)} for the MFMA kernels."""
    per = []
    for k, (ms, n) in sorted(times.items(), key=lambda kv: -kv[1][0]):
        e = {"kernel": k, "launches_per_step": round(n / steps, 3), "ms_per_step": round(ms / steps, 4),
             "us_per_launch": round(ms * 1e3 / n, 1)}
        if k in work:
            flop, nbytes = work[k]
            launches = n / steps
            sec = ms * 1e-3 / n
            e["tflop_per_launch"] = round(flop / launches / 1e12, 4)
            e["algorithmic_gb_per_launch"] = round(nbytes / launches / 1e9, 4)
            e["tflops"] = round(flop / launches / sec / 1e12, 2)
            e["frac"] = round(flop / launches / sec / PEAK_BF16, 4)
        per.append(e)
    mfma = [e for e in per if e["kernel"] in work]
    dom = max(mfma, key=lambda e: e["ms_per_step"]) if mfma else None
    return per, dom


def group_ms(times, steps, names):
    return sum(ms for k, (ms, _) in times.items() if k in names) / steps


def emit(args, metric, N, wall, times, work, flop_fwd, flop_step, config, extra=None, traffic=None):
    """The JSON line common to every workload."""
    per, dom = kernel_report(times, args.steps, work)
    ms_step = wall * 1e3 / args.steps
    fwd_ms = group_ms(times, args.steps, FWD_KERNELS)
    bwd_ms = group_ms(times, args.steps, BWD_KERNELS)
    out = {
        "metric": metric,
        "value": round(N * args.steps / wall, 1),
        "unit": "masked tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "data": "synthetic",
        "config": config,
        "mfma_peak_frac_fwd_bwd": round(flop_step / (ms_step * 1e-3) / PEAK_BF16, 4),
        "fwd_tokens_per_s": round(N / (fwd_ms * 1e-3), 1),
        "fwd_kernel_ms": round(fwd_ms, 4),
        "bwd_kernel_ms": round(bwd_ms, 4),
        "mfma_peak_frac_fwd": round(flop_fwd / (fwd_ms * 1e-3) / PEAK_BF16, 4),
        "mfma_peak_frac_bwd": round((flop_step - flop_fwd) / (bwd_ms * 1e-3) / PEAK_BF16, 4),
        "per_kernel": per,
    }
    if dom is not None:
        rec = (traffic or {}).get(dom["kernel"])
        out["roofline"] = {
            "kernel": dom["kernel"] + " (the kernel with the most device time per step; algorithmic FLOPs per "
                                      "launch over the mean event-timed launch in the timed steps)",
            "bound": "mfma",
            "achieved": dom["tflops"],
            "peak": round(PEAK_BF16 / 1e12, 1),
            "unit": "TFLOP/s",
            "frac": dom["frac"],
            "traffic": None if rec is None else rec["hbm_bytes_per_launch"],
        }
        if rec is not None:
            out["roofline"]["traffic_note"] = ("FETCH_SIZE (L2 misses served by the last-level cache or HBM) + "
                                               "WRITE_SIZE per launch, copy-calibrated, from " +
                                               os.path.relpath(TRAFFIC_FILE, ROOT))
    if extra:
        out.update(extra)
    return out


def bf16_dev(bits, dev):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


# ---------------------------------------------------------------- workloads

def rkl_work(N, V, Hs, Ht, logits=False, K=1):
    """Algorithmic FLOPs and bytes per step of the MFMA kernels of one
    reverse-KL step (Ht = 0 and logits: the teacher as fp32 logits; K
    teacher weights read)."""
    t_flop = 0 if logits else 2.0 * N * V * Ht
    t_read = 4.0 * N * V if logits else 2.0 * K * V * Ht + 2.0 * N * Ht
    proj = 2.0 * N * V * Hs + t_flop
    read = 2.0 * V * Hs + 2.0 * N * Hs + t_read
    return {
        "fwd_tiles": (proj, read),
        "bwd_dz_tiles": (proj, read + 2.0 * N * V + 2.0 * V * Hs),   # + fp16 dz, fp16 copy of W_s
        "dw_gemm": (2.0 * N * V * Hs, 2.0 * N * V + 2.0 * N * Hs + 4.0 * V * Hs),
        "dh_gemm": (2.0 * N * V * Hs, 2.0 * N * V + 2.0 * V * Hs + 4.0 * N * Hs),
    }


def bench_reverse_kl(args):
    import numpy as np
    import torch
    import lm_head_reverse_amd as R
    import synth

    R.lib()
    dev = torch.device("cuda:0")
    print("[bench] generating inputs", file=sys.stderr, flush=True)
    case = synth.config("headline")
    G = args.dp_ranks
    if G < 1 or case.T % G:
        raise SystemExit(f"bench.py: --dp-ranks must divide T={case.T}")
    T, V, Hs, Ht = case.T, case.V, case.Hs, case.Ht
    if G > 1:   # one data-parallel rank: its T/G positions, the weights replicated
        T = case.T // G
        case.h_s, case.h_t, case.mask = case.h_s[:T], case.h_t[:T], case.mask[:T]
    h_s_all, h_t_all = bf16_dev(case.h_s, dev), bf16_dev(case.h_t, dev)
    W_s, W_t = bf16_dev(case.W_s, dev), bf16_dev(case.W_t, dev)
    logits = args.payload == "logits"
    if logits:
        # teacher logits payload: z_t = h_t W_t^T formed once in fp32 (input
        # preparation, outside the timed region); the library streams it
        z_t_all = h_t_all.float() @ W_t.float().t()
        del h_t_all, W_t
    mask = torch.from_numpy(case.mask).to(dev)
    N_expected = int(case.mask.sum())
    grad_pos = torch.full((T,), 1.0 / N_expected, dtype=torch.float32, device=dev)   # token-mean upstream
    dW = torch.empty((V, Hs), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    rows = NextRows(mask)

    def step():
        idx, N = rows.rows
        h_s = R.gather_rows(h_s_all, idx)
        g = R.gather_rows(grad_pos, idx)
        if logits:
            # the kernels read the teacher's logits rows through idx: no copy
            loss, stats = R.forward_logits(z_t_all, h_s=h_s, W_s=W_s, z_rows=idx)
        else:
            h_t = R.gather_rows(h_t_all, idx)
            loss, stats = R.forward_hidden(h_s, W_s, h_t, W_t)
        loss_pos = R.scatter_rows(loss, idx, T)
        if logits:
            dh, _ = R.backward_logits(z_t_all, stats, h_s=h_s, W_s=W_s, grad_loss=g, dW=dW, z_rows=idx)
        else:
            dh, _ = R.backward_hidden(h_s, W_s, h_t, W_t, stats, grad_loss=g, dW=dW)
        R.scatter_rows(dh, idx, T)
        rows.advance()
        return N, loss_pos

    N, wall, times = run_timed(step, args, rows)
    assert N == N_expected
    Ht_eff = 0 if logits else Ht
    work = rkl_work(N, V, Hs, Ht_eff, logits=logits)
    flop_fwd = 2.0 * N * V * (Hs + Ht_eff)
    flop_step = 4.0 * N * V * (Hs + Ht_eff) + 4.0 * N * V * Hs
    config = {"workload": ("Qwen3-1.7B-shaped fp32 teacher logits [T, V] read through the row index, " if logits else
                           "Qwen3-1.7B-shaped hidden-state teacher, ") +
                          "B=4 S=1025 (T=N=4096 trainable), Hs=Ht=2048, V=151936",
              "B": case.B, "S": case.S, "N": int(N), "Hs": Hs, "Ht": Ht_eff, "V": V,
              "payload": "logits" if logits else "hidden_states", "parallelism": "single GPU"}
    if G > 1:
        config["workload"] += f"; one rank of {G}-way data parallelism: its {T} positions"
        config["parallelism"] = f"one rank's share of dp{G}"
    if os.environ.get("RKL_VOCAB_CHUNK"):
        config["backward_vocab_chunk"] = int(os.environ["RKL_VOCAB_CHUNK"])
    headline = not logits and G == 1 and not os.environ.get("RKL_VOCAB_CHUNK")
    out = emit(args, METRIC, N, wall, times, work, flop_fwd, flop_step, config,
               traffic=recorded_traffic() if headline else None)
    if not args.no_cpu_baseline and headline:
        print("[bench] oracle cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def bench_logprob_entropy(args):
    """The compact actor log-probability / entropy step on the headline tensors."""
    import torch
    import lm_head_reverse_amd as R
    import synth

    R.lib()
    dev = torch.device("cuda:0")
    print("[bench] generating inputs", file=sys.stderr, flush=True)
    case = synth.config("headline")
    T, V, H = case.T, case.V, case.Hs
    y_np = synth.sampled_tokens(3, T, V)
    h_all, W = bf16_dev(case.h_s, dev), bf16_dev(case.W_s, dev)
    y_all = torch.from_numpy(y_np).to(dev)
    mask = torch.from_numpy(case.mask).to(dev)
    N_expected = int(case.mask.sum())
    # token-mean upstream gradients: policy term and a small entropy bonus
    g_lp_all = torch.full((T,), 1.0 / N_expected, dtype=torch.float32, device=dev)
    g_h_all = torch.full((T,), -0.01 / N_expected, dtype=torch.float32, device=dev)
    dW = torch.empty((V, H), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    rows = NextRows(mask)

    def step():
        idx, N = rows.rows
        h = R.gather_rows(h_all, idx)
        y = R.gather_rows(y_all, idx)
        gl, gh = R.gather_rows(g_lp_all, idx), R.gather_rows(g_h_all, idx)
        logp, ent, stats = R.forward_logprob_entropy(h, W, y)
        lp_pos = R.scatter_rows(logp, idx, T)
        R.scatter_rows(ent, idx, T)
        dh, _ = R.backward_logprob_entropy(h, W, y, stats, grad_logp=gl, grad_entropy=gh, dW=dW)
        R.scatter_rows(dh, idx, T)
        rows.advance()
        return N, lp_pos

    N, wall, times = run_timed(step, args, rows)
    assert N == N_expected
    work = rkl_work(N, V, H, 0)
    config = {"workload": "Qwen3-1.7B-shaped actor log-probability + entropy, B=4 S=1025 (T=N=4096 "
                          "trainable), H=2048, V=151936, uniform sampled tokens",
              "B": case.B, "S": case.S, "N": int(N), "H": H, "V": V, "parallelism": "single GPU"}
    out = emit(args, "masked tokens/sec fwd+bwd log-prob + entropy (H2048,V152k); MFMA % peak", N, wall, times,
               work, 2.0 * N * V * H, 8.0 * N * V * H, config)
    if not args.no_cpu_baseline:
        print("[bench] oracle cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_lpe(case, y_np, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_baseline_topk(case, y, S, lpt_S, lpt_y, target_s: float):
    """Time the fp64 top-k estimator oracle (forward + backward) on a bounded row sample."""
    from oracle import rkl_oracle as O
    from oracle import topk_oracle as TK
    W = O.widen_bf16(case.W_s)

    def run(nrows):
        h = O.widen_bf16(case.h_s[:nrows])
        t0 = time.perf_counter()
        TK.forward_backward(h, W, y[:nrows], S[:nrows], lpt_S[:nrows], lpt_y[:nrows])
        return time.perf_counter() - t0

    n, t = grow_sample(run, target_s, min(4096, case.T), step=16)
    out = {"value": n / t, "unit": "masked tokens/s", "cores": int(blas_threads()), "kind": "oracle",
           "sample": f"fp64 numpy oracle, top-k estimator forward+backward (L, dz, dh, dW) over the first {n} of "
                     f"the {case.T} positions of this workload, K={S.shape[1]}, full V={case.V}; {t:.1f} s wall; "
                     f"bf16->fp64 widening of the weight done once outside the timed region"}
    out.update(host_info())
    return out


def bench_topk(args):
    """The top-k estimator on the headline student tensors: the teacher's
    log-probabilities on its top K logits and at the sampled token."""
    import numpy as np
    import torch
    import lm_head_reverse_amd as R
    import synth

    R.lib()
    dev = torch.device("cuda:0")
    K = args.topk
    print(f"[bench] generating inputs (K = {K})", file=sys.stderr, flush=True)
    case = synth.config("headline")
    T, V, H = case.T, case.V, case.Hs
    h_all, W = bf16_dev(case.h_s, dev), bf16_dev(case.W_s, dev)
    # teacher payload (input preparation, outside the timed region): log-probabilities of the
    # teacher logits h_t W_t^T at its K largest logits and at the sampled token
    with torch.no_grad():
        z_t = bf16_dev(case.h_t, dev).float() @ bf16_dev(case.W_t, dev).float().t()
        lpt = torch.log_softmax(z_t, dim=1)
        del z_t
        S_all = torch.topk(lpt, K, dim=1).indices.to(torch.int32).contiguous()
        lptS_all = torch.gather(lpt, 1, S_all.long()).contiguous()
        y_np = synth.sampled_tokens(3, T, V)
        y_all = torch.from_numpy(y_np).to(dev)
        lpty_all = torch.gather(lpt, 1, y_all.long()[:, None])[:, 0].contiguous()
        del lpt
    mask = torch.from_numpy(case.mask).to(dev)
    N_expected = int(case.mask.sum())
    g_all = torch.full((T,), 1.0 / N_expected, dtype=torch.float32, device=dev)
    dW = torch.empty((V, H), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    rows = NextRows(mask)

    def step():
        idx, N = rows.rows
        h, y = R.gather_rows(h_all, idx), R.gather_rows(y_all, idx)
        S, lS, ly = R.gather_rows(S_all, idx), R.gather_rows(lptS_all, idx), R.gather_rows(lpty_all, idx)
        g = R.gather_rows(g_all, idx)
        # the student's log-probabilities on the support, kept from the
        # forward for the backward
        lps = torch.empty((N, S.shape[1]), dtype=torch.float32, device=dev)
        loss, stats = R.forward_topk(h, W, y, S, lS, ly, logps_support=lps)
        loss_pos = R.scatter_rows(loss, idx, T)
        dh, _ = R.backward_topk(h, W, y, S, lS, stats, grad_loss=g, dW=dW, logps_support=lps)
        R.scatter_rows(dh, idx, T)
        rows.advance()
        return N, loss_pos

    N, wall, times = run_timed(step, args, rows)
    assert N == N_expected
    work = rkl_work(N, V, H, 0)
    config = {"workload": f"Qwen3-1.7B-shaped student, top-k estimator with the teacher's top {K} log-probabilities "
                          f"and uniform sampled tokens, B=4 S=1025 (T=N=4096 trainable), H=2048, V=151936",
              "B": case.B, "S": case.S, "N": int(N), "H": H, "V": V, "K": K, "parallelism": "single GPU"}
    out = emit(args, "masked tokens/sec fwd+bwd top-k estimator of the reverse KL (H2048,V152k); MFMA % peak", N,
               wall, times, work, 2.0 * N * V * H, 8.0 * N * V * H, config)
    if not args.no_cpu_baseline:
        print("[bench] oracle cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_topk(case, y_np, S_all.cpu().numpy().astype(np.int64),
                                                lptS_all.cpu().numpy().astype(np.float64),
                                                lpty_all.cpu().numpy().astype(np.float64), args.cpu_seconds)
    print(json.dumps(out), flush=True)


def bench_teachers(args):
    """Reverse KL on the headline tensors with K teachers chosen per row."""
    import torch
    import lm_head_reverse_amd as R
    import synth

    R.lib()
    dev = torch.device("cuda:0")
    K = args.teachers
    print(f"[bench] generating inputs ({K} teachers)", file=sys.stderr, flush=True)
    case = synth.config("headline")
    T, V, Hs, Ht = case.T, case.V, case.Hs, case.Ht
    h_s_all, h_t_all, W_s = bf16_dev(case.h_s, dev), bf16_dev(case.h_t, dev), bf16_dev(case.W_s, dev)
    W_t = bf16_dev(synth.teacher_weights(3, K, V, Ht), dev)
    tid_all = torch.from_numpy(synth.teacher_ids(3, T, K, args.teacher_order)).to(dev)
    mask = torch.from_numpy(case.mask).to(dev)
    N_expected = int(case.mask.sum())
    grad_pos = torch.full((T,), 1.0 / N_expected, dtype=torch.float32, device=dev)
    dW = torch.empty((V, Hs), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    rows = NextRows(mask)

    def step():
        idx, N = rows.rows
        h_s, h_t = R.gather_rows(h_s_all, idx), R.gather_rows(h_t_all, idx)
        tk, g = R.gather_rows(tid_all, idx), R.gather_rows(grad_pos, idx)
        loss, stats = R.forward_hidden_teachers(h_s, W_s, h_t, W_t, tk)
        loss_pos = R.scatter_rows(loss, idx, T)
        dh, _ = R.backward_hidden_teachers(h_s, W_s, h_t, W_t, tk, stats, grad_loss=g, dW=dW)
        R.scatter_rows(dh, idx, T)
        rows.advance()
        return N, loss_pos

    N, wall, times = run_timed(step, args, rows)
    assert N == N_expected
    config = {"workload": f"Qwen3-1.7B-shaped hidden-state teachers, {K} teachers chosen per row "
                          f"({args.teacher_order}), B=4 S=1025 (T=N=4096 trainable), Hs=Ht=2048, V=151936",
              "B": case.B, "S": case.S, "N": int(N), "Hs": Hs, "Ht": Ht, "V": V, "K": K,
              "teacher_order": args.teacher_order, "parallelism": "single GPU"}
    out = emit(args, "masked tokens/sec fwd+bwd full-vocab reverse KL, teacher per row (H2048,V152k); MFMA % peak",
               N, wall, times, rkl_work(N, V, Hs, Ht, K=K), 2.0 * N * V * (Hs + Ht),
               4.0 * N * V * (Hs + Ht) + 4.0 * N * V * Hs, config)
    print(json.dumps(out), flush=True)


def bench_vocab_shard(args):
    """One rank's share of a G-way vocabulary-parallel reverse-KL step."""
    import torch
    import lm_head_reverse_amd as R
    import synth

    R.lib()
    dev = torch.device("cuda:0")
    G = args.shards
    print(f"[bench] generating inputs ({G} vocabulary shards)", file=sys.stderr, flush=True)
    case = synth.config("headline")
    T, V, Hs, Ht = case.T, case.V, case.Hs, case.Ht
    if not 1 <= G <= V:
        raise SystemExit(f"bench.py: --shards must be in [1, {V}]")
    q, r = divmod(V, G)
    bounds = []
    for k in range(G):
        a = bounds[-1][1] if bounds else 0
        bounds.append((a, a + q + (1 if k < r else 0)))
    v0, v1 = bounds[0]   # this rank's vocabulary rows
    h_s_all, h_t_all = bf16_dev(case.h_s, dev), bf16_dev(case.h_t, dev)
    W_s_full, W_t_full = bf16_dev(case.W_s, dev), bf16_dev(case.W_t, dev)
    mask = torch.from_numpy(case.mask).to(dev)
    N_expected = int(case.mask.sum())
    grad_pos = torch.full((T,), 1.0 / N_expected, dtype=torch.float32, device=dev)
    # the other ranks' partials, as the all-gather would deliver them
    idx, N = R.compact_rows(mask)
    h_s, h_t = R.gather_rows(h_s_all, idx), R.gather_rows(h_t_all, idx)
    partials = torch.stack([R.forward_hidden_shard(h_s, W_s_full[a:b], h_t, W_t_full[a:b])
                            for a, b in bounds]).contiguous()
    W_s, W_t = W_s_full[v0:v1], W_t_full[v0:v1]
    dW = torch.empty((v1 - v0, Hs), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    rows = NextRows(mask)

    def step():
        idx, N = rows.rows
        h_s, h_t = R.gather_rows(h_s_all, idx), R.gather_rows(h_t_all, idx)
        g = R.gather_rows(grad_pos, idx)
        partials[0] = R.forward_hidden_shard(h_s, W_s, h_t, W_t)
        loss, stats = R.combine_shards(partials)
        loss_pos = R.scatter_rows(loss, idx, T)
        dh, _ = R.backward_hidden(h_s, W_s, h_t, W_t, stats, grad_loss=g, dW=dW)
        R.scatter_rows(dh, idx, T)
        rows.advance()
        return N, loss_pos

    N, wall, times = run_timed(step, args, rows)
    assert N == N_expected
    Vs = v1 - v0
    config = {"workload": f"Qwen3-1.7B-shaped hidden-state teacher, one rank's share of a {G}-way "
                          f"vocabulary split ({Vs} of 151936 vocabulary rows), B=4 S=1025 (T=N=4096 "
                          f"trainable), Hs=Ht=2048; inter-rank exchanges excluded",
              "B": case.B, "S": case.S, "N": int(N), "Hs": Hs, "Ht": Ht, "V": V, "shards": G,
              "V_shard": Vs, "parallelism": "single GPU (one rank's share)"}
    out = emit(args, "masked tokens/sec fwd+bwd full-vocab reverse KL, one rank of a vocabulary-parallel group "
                     "(H2048,V152k); MFMA % peak", N, wall, times, rkl_work(N, Vs, Hs, Ht),
               2.0 * N * Vs * (Hs + Ht), 4.0 * N * Vs * (Hs + Ht) + 4.0 * N * Vs * Hs, config)
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.profile_copy:
        return profile_copy()
    if args.report_c5:
        return report_c5()
    if args.gpus != 1:
        print(f"bench.py measures one GPU (asked for --gpus {args.gpus}): the library has no collectives; "
              f"a vocabulary-parallel rank's share is the vocab_shard workload", file=sys.stderr)
        sys.exit(2)
    {"reverse_kl": bench_reverse_kl, "logprob_entropy": bench_logprob_entropy, "teachers": bench_teachers,
     "vocab_shard": bench_vocab_shard, "topk": bench_topk}[args.workload](args)


if __name__ == "__main__":
    main()
