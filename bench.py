#!/usr/bin/env python3
"""Benchmark of the MTP verify + end-to-end TV-loss hot path on one MI355X.

Primary number (`value`): draft positions verified per second on the rollout
workload (64 sequences x gamma = 3 draft positions + 1 bonus row, V = 151936,
bfloat16 logits), inputs resident in HBM, four input sets rotated (545 MB, more
than the 256 MB Infinity Cache).  One step = one mtp_verify call: softmax of both
rows, acceptance tests, overlap / TV / entropy, inverse-CDF samples of every row,
accepted lengths and next tokens.

Also reported (`tv_loss`): end-to-end TV loss forward + backward on T = 8192
positions x 3 heads, V = 151936 (bf16 in, bf16 gradient out), as algorithmic GB/s
against the 8 TB/s HBM peak, by the forward and backward calls and (`tv_fused`) by
the one call that does both in one sweep; (`long_tail`) verify on 512 x 4 positions at V = 2^18
with Zipf-like logits; (`entropy_sweep`) verify on the 15 temperature x noise cells
(128 sequences each), with each cell's acceptance rate, mean accepted length and
mean target entropy; (`target_only`) target-only verify of the rollout workload;
(`gumbel`) verify at temperature 0.7 with Gumbel-max row samples, and the
Gumbel-max draft sampler on the rollout's draft rows; (`tv_topk`) the TV loss
forward + backward with top-K targets (K = 256) on the TV workload.

`roofline` uses per-launch HIP events recorded on the stream the kernels run on;
`cpu_baseline` times the float64 oracle on a bounded sample of the same workload
(and of the TV, long-tail and entropy-sweep workloads in their lines); each
entropy-sweep cell also reports the oracle's acceptance rate, mean accepted length
and mean entropy on a seeded sample of its sequences beside the GPU's.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft positions verified/sec at V=151936, γ=3; TV fwd+bwd GB/s vs HBM peak"
HBM_PEAK_GBS = 8000.0
C3_SAMPLE = 16   # sequences per entropy-sweep cell run through the oracle beside the GPU
EXTRAS = ("tv_topk", "target_only", "gumbel", "long_tail", "entropy_sweep", "stream_context")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def profiled_traffic(summary, sources):
    """HBM bytes per call from a committed rocprofv3 summary (FETCH_SIZE and
    WRITE_SIZE passes, scaled by a plain copy's reading), or None when the kernel
    sources have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", " ")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip().split()[0] if v.strip() else ""
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if fields.get("source_sha256") != h.hexdigest()[:16] or "traffic_bytes_per_call" not in fields:
        return None
    return float(fields["traffic_bytes_per_call"])


def profiled_valu_busy(kernels, weights=None):
    """rocprofv3's VALUBusy (%) for the named kernels from the committed summary,
    averaged with the given time weights, or None when the kernel sources have
    changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "valu_busy_bench_kernels.md")
    if not os.path.exists(path):
        return None
    sha, busy = None, {}
    for line in open(path):
        if line.startswith("source_sha256:"):
            sha = line.split(":", 1)[1].split()[0]
        elif line.startswith("| `"):
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            busy[cells[0].strip("`")] = float(cells[3])
    h = hashlib.sha256()
    for f in VALU_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    vals = [busy[k] for k in kernels if k in busy]
    if sha != h.hexdigest()[:16] or len(vals) != len(kernels):
        return None
    weights = weights or [1.0] * len(vals)
    return sum(v * w for v, w in zip(vals, weights)) / sum(weights)


VERIFY_SOURCES = ["tv_loss_amd/csrc/verify.hip", "tv_loss_amd/csrc/device_common.hpp", "tv_loss_amd/csrc/kernels.hpp"]
TV_SOURCES = ["tv_loss_amd/csrc/tv_loss.hip", "tv_loss_amd/csrc/device_common.hpp", "tv_loss_amd/csrc/kernels.hpp"]
VALU_SOURCES = ["tv_loss_amd/csrc/verify.hip", "tv_loss_amd/csrc/tv_loss.hip", "tv_loss_amd/csrc/device_common.hpp",
                "tv_loss_amd/csrc/kernels.hpp"]


def verify_bytes(B, G, V, elem):
    """Algorithmic bytes of one verify call: every logit read once (target B*(G+1)
    rows, draft B*G rows), tokens read, per-row outputs written."""
    logits = B * (2 * G + 1) * V * elem
    small = B * G * 4 + B * G * 1 + 2 * B * 4 + B * (G + 1) * (4 + 4 + 4) + B * G * 8
    return logits, logits + small


def check_waits(mtp, ws):
    """Stop if a bounded cluster wait timed out (the kernels set the workspace's
    error word): the timings of such a run would mean nothing."""
    word = mtp.workspace_error(ws)
    if word:
        sys.exit(f"bench: a cluster wait timed out (workspace error word {word:#x})")


def time_verify(mtp, torch, w, steps, warmup, nsets, target_only=False, temperature=None):
    import synthetic
    dev = "cuda:0"
    B, G, V = w["B"], w["G"], w["V"]
    plans = []
    for i in range(nsets):
        t, d, y = synthetic.verify_inputs(w, dev, seed=w["seed"] + i)
        if target_only:
            plans.append(mtp.VerifyPlan(t, d, None, target_only=True))
        else:
            plans.append(mtp.VerifyPlan(t, d, y, temperature=temperature))
    torch.cuda.synchronize()
    rows = B * (G + 1)
    plans[0].run(seed=w["seed"], offset=0)
    check_waits(mtp, plans[0].ws)
    for i in range(warmup):
        plans[i % nsets].run(seed=w["seed"], offset=i * rows)
    torch.cuda.synchronize()
    check_waits(mtp, plans[0].ws)
    # per-call GPU times: events around every call
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        plans[i % nsets].run(seed=w["seed"], offset=(warmup + i) * rows)
        evs[i][1].record()
    torch.cuda.synchronize()
    kernel_ms = [a.elapsed_time(b) for a, b in evs]
    # throughput: the same calls back to back, without the event records in between
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        plans[i % nsets].run(seed=w["seed"], offset=(warmup + steps + i) * rows)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, kernel_ms, plans


def time_tv_fused(mtp, torch, w, steps, warmup):
    """mtp_tv_loss_fwd_bwd on the TV workload: per-call HIP events and the wall time
    of the same calls back to back."""
    import synthetic
    t, d = synthetic.tv_inputs(w, "cuda:0")
    plan = mtp.TVPlan(t, d, grad_dtype=torch.bfloat16)
    for _ in range(warmup):
        plan.fused()
    torch.cuda.synchronize()
    check_waits(mtp, plan.ws_fused)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        plan.fused()
        ev[i][1].record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        plan.fused()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    check_waits(mtp, plan.ws_fused)
    ms = [a.elapsed_time(b) for a, b in ev]
    loss = plan.loss.item()
    del plan, t, d
    torch.cuda.empty_cache()
    return wall, ms, loss


def time_tv(mtp, torch, w, steps, warmup, topk=None):
    import synthetic
    dev = "cuda:0"
    if topk:
        i, v, d = synthetic.topk_inputs(w, topk, dev)
        plan = mtp.TVTopKPlan(i, v, d, grad_dtype=torch.bfloat16)
        t = (i, v)
    else:
        t, d = synthetic.tv_inputs(w, dev)
        plan = mtp.TVPlan(t, d, grad_dtype=torch.bfloat16)
    check_waits(mtp, plan.ws)
    for _ in range(warmup):
        plan.forward()
        plan.backward()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record()
        plan.forward()
        ev[i][1].record()
        plan.backward()
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd = [a.elapsed_time(b) for a, b, _ in ev]
    bwd = [b.elapsed_time(c) for _, b, c in ev]
    loss = plan.loss.item()
    del plan, t, d
    torch.cuda.empty_cache()
    return wall, fwd, bwd, loss


def _f64(torch, x):
    """bf16 tensor on the GPU -> float64 NumPy array (exact)."""
    import numpy as np

    from oracle.bf16 import bf16_bits_to_f64
    return bf16_bits_to_f64(x.cpu().view(torch.int16).numpy().view(np.uint16))


class _one_core:
    """Pin this thread to a single CPU for a timed oracle loop."""

    def __enter__(self):
        self.old = os.sched_getaffinity(0) if hasattr(os, "sched_getaffinity") else None
        if self.old:
            os.sched_setaffinity(0, {min(self.old)})
        return self

    def __exit__(self, *exc):
        if self.old:
            os.sched_setaffinity(0, self.old)


def cpu_baseline(torch, w, seconds, nseq=16):
    """The float64 oracle, untuned, on whole sequences of a verify workload (the
    first `nseq` sequences, cycled) until about `seconds` of CPU time: returns
    (sequences done, wall seconds)."""
    import synthetic
    from oracle import mtp as omtp
    t, d, y = synthetic.verify_inputs(w, "cuda:0", B=nseq)
    tb, db, yb = _f64(torch, t), _f64(torch, d), y.cpu().numpy()
    G1 = w["G"] + 1
    n = 0
    with _one_core():
        t0 = time.process_time()
        w0 = time.perf_counter()
        while True:
            b = n % tb.shape[0]
            omtp.verify(tb[b:b + 1], db[b:b + 1], yb[b:b + 1], w["seed"], b * G1)
            n += 1
            if time.process_time() - t0 >= seconds:
                break
        wall = time.perf_counter() - w0
    return n, wall


def cpu_tv_baseline(torch, w, seconds):
    """The float64 oracle, untuned, on the first positions of the TV workload, one
    position at a time (statistics, position loss and gradient, with the gradient
    scale of the full mean), until about `seconds` of CPU time: returns (positions
    done, wall seconds)."""
    import synthetic
    from oracle import mtp as omtp
    P = 64
    t, d = synthetic.tv_inputs(w, "cuda:0", T=P)
    tb, db = _f64(torch, t), _f64(torch, d)
    scale = 1.0 / w["T"]
    n = 0
    with _one_core():
        t0 = time.process_time()
        w0 = time.perf_counter()
        while True:
            i = n % P
            omtp.tv_loss(tb[i:i + 1], db[i:i + 1])
            omtp.tv_loss_grad(tb[i:i + 1], db[i:i + 1], scale)
            n += 1
            if time.process_time() - t0 >= seconds:
                break
        wall = time.perf_counter() - w0
    return n, wall


def oracle_cell(torch, w, seqs):
    """The oracle's acceptance rate, mean accepted length and mean target entropy
    on the given sequences of a verify workload (its own seed, offsets b (gamma+1)),
    and the wall seconds it took on one core."""
    import numpy as np

    import synthetic
    from oracle import mtp as omtp
    t, d, y = synthetic.verify_inputs(w, "cuda:0")
    G1 = w["G"] + 1
    acc, n, H = [], [], []
    with _one_core():
        w0 = time.perf_counter()
        for b in seqs:
            r = omtp.verify(_f64(torch, t[b:b + 1]), _f64(torch, d[b:b + 1]), y[b:b + 1].cpu().numpy(),
                            w["seed"], b * G1)
            acc.append(np.asarray(r["accept"], dtype=np.float64).ravel())
            n.append(float(np.asarray(r["accepted_len"]).ravel()[0]))
            H.append(np.asarray(r["entropy"], dtype=np.float64).ravel())
        wall = time.perf_counter() - w0
    del t, d, y
    return {"accept_rate": float(np.concatenate(acc).mean()), "mean_accepted_len": float(np.mean(n)),
            "mean_entropy": float(np.concatenate(H).mean())}, wall


def stream_context(torch, nbytes=1 << 31, reps=10):
    """Achievable-bandwidth context from plain torch kernels on the same GPU: a
    device-to-device copy (bytes read + written) and a float32 sum (bytes read)."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    out = {}
    for name, fn, moved in (("copy_gbs", lambda: dst.copy_(src), 2 * nbytes),
                            ("read_sum_gbs", lambda: src.sum(), nbytes)):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        out[name] = moved * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return out


def pct(xs, q):
    s = sorted(xs)
    return s[min(len(s) - 1, int(round(q * (len(s) - 1))))]


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--tv-steps", type=int, default=None, help="TV-loss steps (default: max(3, steps // 20))")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tv", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="only the headline lines (rollout verify, TV loss)")
    ap.add_argument("--extra", default=",".join(EXTRAS),
                    help=f"comma-separated extra lines to run (default: all of {','.join(EXTRAS)})")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="after the bench, copy BYTES of device memory three times with torch (a plain copy "
                         "kernel of known size, to calibrate HBM byte counters)")
    args = ap.parse_args()
    extras = set() if args.no_extra else {e for e in args.extra.split(",") if e}
    if extras - set(EXTRAS):
        ap.error(f"unknown extra lines: {sorted(extras - set(EXTRAS))}")

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this hot path is data-parallel and every run here uses a "
              "single MI355X; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import numpy as np

    import synthetic
    import tv_loss_amd as mtp
    mtp.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    w = synthetic.VERIFY_WORKLOADS["rollout"]
    B, G, V = w["B"], w["G"], w["V"]
    nsets = 4
    log(f"verify: rollout workload B={B} gamma={G} V={V} bf16, {nsets} input sets")
    wall, kms, _ = time_verify(mtp, torch, w, args.steps, args.warmup, nsets)
    positions = B * G * args.steps
    value = positions / wall
    logit_bytes, alg_bytes = verify_bytes(B, G, V, 2)
    kmean = sum(kms) / len(kms)
    ksorted = sorted(kms)
    achieved = alg_bytes / (kmean * 1e-3) / 1e9
    log(f"verify: {value / 1e6:.3f} M positions/s wall, kernel mean {kmean * 1e3:.2f} us "
        f"(median {ksorted[len(ksorted) // 2] * 1e3:.2f} us), {achieved:.0f} GB/s")

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "draft positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "rollout verify: 64 sequences x gamma=3 draft positions (+1 bonus row), "
                               "V=151936, bf16 logits, target N(0,1)/0.7, draft = target + N(0,0.3^2)",
                   "batch": B, "gamma": G, "vocab": V, "storage": "bf16", "input_sets": nsets},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": profiled_traffic("verify_rollout_64x3_V151936_bf16.md", VERIFY_SOURCES),
                     "kernel": "verify_main (one mtp_verify call: layers and finish in one launch)", "bytes_per_launch": alg_bytes,
                     "kernel_us_mean": kmean * 1e3, "kernel_us_median": ksorted[len(ksorted) // 2] * 1e3,
                     "kernel_us_p10": pct(kms, 0.1) * 1e3, "kernel_us_p90": pct(kms, 0.9) * 1e3,
                     "valu_busy_pct": profiled_valu_busy(["void mtp::verify_main<1, 2, 0>(mtp::VerifyArgs)"])},
    }

    if not args.no_tv:
        tw = synthetic.TV_WORKLOADS["tv_loss"]
        T, TG, TV = tw["T"], tw["G"], tw["V"]
        tv_steps = args.tv_steps or max(3, args.steps // 20)
        log(f"tv loss: T={T} gamma={TG} V={TV} bf16, {tv_steps} steps")
        twall, fwd, bwd, loss = time_tv(mtp, torch, tw, tv_steps, max(1, min(3, args.warmup)))
        fwd_bytes = T * (1 + TG) * TV * 2
        bwd_bytes = T * (1 + TG) * TV * 2 + T * TG * TV * 2
        fm, bm = sum(fwd) / len(fwd), sum(bwd) / len(bwd)
        gbs = (fwd_bytes + bwd_bytes) / ((fm + bm) * 1e-3) / 1e9
        result["tv_loss"] = {
            "workload": "e2e TV loss fwd+bwd: T=8192 positions x gamma=3 heads, V=151936, bf16 in, bf16 grad "
                        "out, target N(0,1)/0.8 shared by heads, head k = target + N(0,(0.2k)^2)",
            "value": gbs, "unit": "GB/s", "frac_of_hbm_peak": gbs / HBM_PEAK_GBS,
            "fwd_ms": fm, "bwd_ms": bm, "fwd_gbs": fwd_bytes / (fm * 1e-3) / 1e9,
            "bwd_gbs": bwd_bytes / (bm * 1e-3) / 1e9, "bytes_fwd": fwd_bytes, "bytes_bwd": bwd_bytes,
            "steps": tv_steps, "wall_ms_per_step": twall / tv_steps * 1e3, "loss": loss,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "traffic": profiled_traffic("tv_loss_T8192x3_V151936_bf16.md", TV_SOURCES),
                         "kernel": "tv_pipe_main + tv_pipe_finish + tv_fwd_mean + tv_bwd_kernel",
                         "valu_busy_pct": profiled_valu_busy(["void mtp::tv_pipe_main<1, 3, true>(mtp::TvArgs)",
                                                              "void mtp::tv_bwd_kernel<1, 1, 3, true>(mtp::TvArgs)"],
                                                             [fm, bm]),
                         "bytes_per_launch": fwd_bytes + bwd_bytes},
        }
        log(f"tv loss: fwd {fm:.3f} ms ({fwd_bytes / fm / 1e6:.0f} GB/s), bwd {bm:.3f} ms "
            f"({bwd_bytes / bm / 1e6:.0f} GB/s), total {gbs:.0f} GB/s")

        # forward and backward in one sweep (mtp_tv_loss_fwd_bwd): every logit read
        # once, the gradient written once
        fwall, fms, floss = time_tv_fused(mtp, torch, tw, tv_steps, max(1, min(3, args.warmup)))
        fused_bytes = T * (1 + TG) * TV * 2 + T * TG * TV * 2
        fmean = sum(fms) / len(fms)
        fgbs = fused_bytes / (fmean * 1e-3) / 1e9
        result["tv_fused"] = {
            "workload": "e2e TV loss forward + backward in one call (mtp_tv_loss_fwd_bwd) on the tv_loss workload: "
                        "T=8192 x gamma=3, V=151936, bf16 in, bf16 grad out",
            "value": fgbs, "unit": "GB/s", "ms": fmean, "ms_two_calls": fm + bm,
            "wall_ms_per_step": fwall / tv_steps * 1e3, "steps": tv_steps, "loss": floss,
            "roofline": {"bound": "hbm", "achieved": fgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": fgbs / HBM_PEAK_GBS,
                         "traffic": profiled_traffic("tv_fused_T8192x3_V151936_bf16.md", TV_SOURCES),
                         "kernel": "tv_fused_main + tv_fused_finish + tv_fwd_mean",
                         "valu_busy_pct": profiled_valu_busy(["void mtp::tv_fused_main<1, 1, 3, true>(mtp::TvArgs)"]),
                         "bytes_per_launch": fused_bytes},
        }
        log(f"tv loss fused: {fmean:.3f} ms ({fgbs:.0f} GB/s of {fused_bytes / 1e9:.2f} GB) against "
            f"{fm + bm:.3f} ms for the two calls")

        if not args.no_cpu_baseline:
            n, cwall = cpu_tv_baseline(torch, tw, args.cpu_seconds)
            per_pos = (fwd_bytes + bwd_bytes) / T
            est = cwall / n * T
            result["tv_loss"]["cpu_baseline"] = {
                "value": n * per_pos / cwall / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"the first {min(n, 64)} positions of the workload, cycled: {n} positions (forward "
                          f"statistics, position loss and gradient) through the float64 NumPy oracle on one CPU "
                          f"in {cwall:.1f} s; GB/s counts the two calls' bytes per position; extrapolated to "
                          f"all {T} positions: {est:.0f} s per step",
                "extrapolated_s_per_step": est}
            result["tv_fused"]["cpu_baseline"] = dict(
                result["tv_loss"]["cpu_baseline"], value=n * (fused_bytes / T) / cwall / 1e9,
                sample=result["tv_loss"]["cpu_baseline"]["sample"].replace("the two calls' bytes",
                                                                          "the one call's bytes"))
            log(f"cpu oracle tv: {n} positions in {cwall:.1f} s, {est:.0f} s per full step extrapolated")

    if "tv_topk" in extras:
        # the top-K path on the same workload: each position's target reduced to its
        # 256 largest logits (indices + float32 values, shared by the heads)
        tw = synthetic.TV_WORKLOADS["tv_loss"]
        T, TG, TV, TK = tw["T"], tw["G"], tw["V"], 256
        tv_steps = args.tv_steps or max(3, args.steps // 20)
        log(f"tv loss top-K: T={T} gamma={TG} V={TV} K={TK} bf16, {tv_steps} steps")
        kwall, kf, kb, kloss = time_tv(mtp, torch, tw, tv_steps, 2, topk=TK)
        kfm, kbm = sum(kf) / len(kf), sum(kb) / len(kb)
        kfb = T * TG * TV * 2 + T * TK * 8
        kbb = 2 * T * TG * TV * 2 + T * TK * 8
        kgbs = (kfb + kbb) / ((kfm + kbm) * 1e-3) / 1e9
        result["tv_topk"] = {
            "workload": "e2e TV loss fwd+bwd with top-K targets: T=8192 x gamma=3 heads, V=151936, K=256 target "
                        "entries per position (the tv_loss workload's target reduced to its 256 largest logits), "
                        "bf16 draft in, bf16 grad out",
            "value": kgbs, "unit": "GB/s", "fwd_ms": kfm, "bwd_ms": kbm, "bytes_fwd": kfb, "bytes_bwd": kbb,
            "fwd_gbs": kfb / (kfm * 1e-3) / 1e9, "bwd_gbs": kbb / (kbm * 1e-3) / 1e9, "loss": kloss,
            "roofline": {"bound": "hbm", "achieved": kgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": kgbs / HBM_PEAK_GBS, "bytes_per_launch": kfb + kbb},
        }
        log(f"tv loss top-K: fwd {kfm:.3f} ms ({kfb / kfm / 1e6:.0f} GB/s), bwd {kbm:.3f} ms "
            f"({kbb / kbm / 1e6:.0f} GB/s), total {kgbs:.0f} GB/s")

    if "target_only" in extras:
        # target-only verify of the rollout workload (greedy draft tokens, the RS/TO flag)
        log("verify: target-only on the rollout workload")
        owall, okms, plans = time_verify(mtp, torch, w, args.steps, args.warmup, nsets, target_only=True)
        out = plans[0].run(seed=w["seed"], offset=0)
        to_acc = out["accept"].float().mean().item()
        rs_share = out["rs_better"].float().mean().item()
        del plans, out
        omean = sum(okms) / len(okms)
        result["target_only"] = {
            "workload": "target-only verify of the rollout workload (greedy draft tokens argmax q, accept with "
                        "p(yhat), RS/TO boundary TV < 1 - p(yhat))",
            "value": positions / owall, "unit": "draft positions/s", "kernel_us_mean": omean * 1e3,
            "accept_rate": to_acc, "rs_better_share": rs_share,
            "roofline": {"bound": "hbm", "achieved": alg_bytes / (omean * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": alg_bytes / (omean * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "bytes_per_launch": alg_bytes},
        }
        # a low-temperature cell (tau = 0.25, sigma = 1), where p(yhat) is large and the
        # draft far from the target: positions on both sides of the RS/TO boundary
        lw = synthetic.sweep_cell(0, 2)
        lwall, lkms, plans = time_verify(mtp, torch, lw, max(5, args.steps // 10), 2, 1, target_only=True)
        out = plans[0].run(seed=lw["seed"], offset=0)
        result["target_only"]["low_tau_cell"] = {
            "workload": "target-only verify of the entropy-sweep cell tau=0.25, sigma=1.0 (128 sequences x "
                        "gamma=3, V=151936, bf16)",
            "accept_rate": out["accept"].float().mean().item(),
            "rs_better_share": out["rs_better"].float().mean().item(),
            "kernel_us_mean": sum(lkms) / len(lkms) * 1e3}
        del plans, out
        log(f"verify target-only at tau=0.25: accept rate {result['target_only']['low_tau_cell']['accept_rate']:.3f}, "
            f"RS better on {result['target_only']['low_tau_cell']['rs_better_share']:.3f} of positions")
    if "gumbel" in extras:
        # rejection sampling at temperature 0.7 with Gumbel-max row samples, and the
        # Gumbel-max draft sampler on the rollout's draft rows
        log("verify: Gumbel-max at T=0.7 on the rollout workload")
        gwall, gkms, plans = time_verify(mtp, torch, w, args.steps, args.warmup, nsets, temperature=0.7)
        out = plans[0].run(seed=w["seed"], offset=0)
        g_acc = out["accept"].float().mean().item()
        drafts = [p.inputs[1] for p in plans]
        del out
        gmean = sum(gkms) / len(gkms)
        sevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)]
        for i in range(args.warmup):
            mtp.gumbel_sample(drafts[i % nsets], 0.7, seed=1, offset=i * B * G)
        for i in range(args.steps):
            sevs[i][0].record()
            mtp.gumbel_sample(drafts[i % nsets], 0.7, seed=1, offset=i * B * G)
            sevs[i][1].record()
        torch.cuda.synchronize()
        smean = sum(a.elapsed_time(b) for a, b in sevs) / args.steps
        sbytes = B * G * V * 2 + B * G * 4
        del plans, drafts
        result["gumbel"] = {
            "workload": "rejection-sampling verify of the rollout workload at temperature 0.7 (p, q tempered), "
                        "row tokens by the Gumbel-max trick with per-element Philox noise; draft sampler on "
                        "its 192 draft rows",
            "value": positions / gwall, "unit": "draft positions/s", "kernel_us_mean": gmean * 1e3,
            "accept_rate": g_acc,
            "roofline": {"bound": "hbm", "achieved": alg_bytes / (gmean * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": alg_bytes / (gmean * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "bytes_per_launch": alg_bytes},
            "sampler_us_mean": smean * 1e3, "sampler_gbs": sbytes / (smean * 1e-3) / 1e9,
        }
        log(f"verify Gumbel-max: {gmean * 1e3:.2f} us per call, accept rate {g_acc:.3f}; sampler "
            f"{smean * 1e3:.2f} us per call ({sbytes / smean / 1e6:.0f} GB/s)")

    if "long_tail" in extras:
        # the long-tail workload (Zipf-like logits, V = 2^18, gamma = 4), timed like
        # the rollout workload
        lw = synthetic.VERIFY_WORKLOADS["long_tail"]
        lsteps = max(5, args.steps // 10)
        log(f"verify: long-tail workload B={lw['B']} gamma={lw['G']} V={lw['V']} bf16, {lsteps} steps")
        lwall, lkms, plans = time_verify(mtp, torch, lw, lsteps, 2, 1)
        del plans
        torch.cuda.empty_cache()
        lmean = sum(lkms) / len(lkms)
        _, lbytes = verify_bytes(lw["B"], lw["G"], lw["V"], 2)
        lpos = lw["B"] * lw["G"]
        result["long_tail"] = {
            "workload": "long-tail verify: 512 sequences x gamma=4 (+1 bonus row), V=262144, bf16, Zipf-like "
                        "logits -1.1 ln(rank) + N(0,0.5^2), draft = target + N(0,0.4^2)",
            "value": lpos / (lmean * 1e-3), "unit": "draft positions/s", "kernel_us_mean": lmean * 1e3,
            "roofline": {"bound": "hbm", "achieved": lbytes / (lmean * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": lbytes / (lmean * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "bytes_per_launch": lbytes},
        }
        log(f"verify long tail: {lpos / lmean / 1e3:.3f} M positions/s, {lmean * 1e3:.1f} us per call, "
            f"{lbytes / lmean / 1e6:.0f} GB/s")
        if not args.no_cpu_baseline:
            n, cwall = cpu_baseline(torch, lw, args.cpu_seconds / 2, nseq=8)
            result["long_tail"]["cpu_baseline"] = {
                "value": n * lw["G"] / cwall, "unit": "draft positions/s", "cores": 1, "kind": "oracle",
                "sample": f"the first 8 sequences of the workload, cycled: {n} sequences ({n * lw['G']} draft "
                          f"positions) through the float64 NumPy oracle on one CPU in {cwall:.1f} s"}
            log(f"cpu oracle long tail: {n * lw['G'] / cwall:.1f} positions/s")

    if "entropy_sweep" in extras:
        # the 15 cells of the entropy sweep
        cells = []
        oracle_seqs, oracle_wall = 0, 0.0
        for it in range(len(synthetic.SWEEP_TAUS)):
            for isg in range(len(synthetic.SWEEP_SIGMAS)):
                cw = synthetic.sweep_cell(it, isg)
                cwall_, ckms, plans = time_verify(mtp, torch, cw, max(5, args.steps // 10), 2, 3)
                out = plans[0].run(seed=cw["seed"], offset=0)
                acc = out["accept"].float().mean().item()
                mean_n = out["accepted_len"].float().mean().item()
                ent = out["entropy"].float().mean().item()
                cm = sum(ckms) / len(ckms)
                cell = {"tau": synthetic.SWEEP_TAUS[it], "sigma": synthetic.SWEEP_SIGMAS[isg],
                        "us_per_call": cm * 1e3, "positions_per_s": cw["B"] * cw["G"] / (cm * 1e-3),
                        "accept_rate": acc, "mean_accepted_len": mean_n, "mean_entropy": ent}
                if not args.no_cpu_baseline:
                    # the same statistics on a seeded sample of sequences, from the GPU
                    # call above and from the oracle
                    seqs = sorted(np.random.default_rng(1000 + 10 * it + isg).choice(cw["B"], C3_SAMPLE,
                                                                                    replace=False).tolist())
                    ref, owall = oracle_cell(torch, cw, seqs)
                    cell["sample"] = {
                        "sequences": seqs,
                        "gpu": {"accept_rate": out["accept"][seqs].float().mean().item(),
                                "mean_accepted_len": out["accepted_len"][seqs].float().mean().item(),
                                "mean_entropy": out["entropy"][seqs].float().mean().item()},
                        "oracle": ref}
                    oracle_seqs += len(seqs)
                    oracle_wall += owall
                del plans, out
                cells.append(cell)
        torch.cuda.empty_cache()
        _, cbytes = verify_bytes(128, 3, 151936, 2)
        cmean = sum(c["us_per_call"] for c in cells) / len(cells)
        result["entropy_sweep"] = {
            "workload": "entropy sweep: 15 cells tau x sigma, 128 sequences x gamma=3 (+1 bonus row), V=151936, "
                        "bf16, target N(0,1)/tau, draft = target + N(0,sigma^2), 3 input sets per cell",
            "value": 128 * 3 / (cmean * 1e-6), "unit": "draft positions/s", "kernel_us_mean": cmean,
            "roofline": {"bound": "hbm", "achieved": cbytes / (cmean * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": cbytes / (cmean * 1e-6) / 1e9 / HBM_PEAK_GBS,
                         "bytes_per_launch": cbytes},
            "cells": cells,
        }
        if oracle_seqs:
            result["entropy_sweep"]["cpu_baseline"] = {
                "value": oracle_seqs * 3 / oracle_wall, "unit": "draft positions/s", "cores": 1, "kind": "oracle",
                "sample": f"{C3_SAMPLE} seeded sequences of each cell ({oracle_seqs} sequences, "
                          f"{oracle_seqs * 3} draft positions) through the float64 NumPy oracle on one CPU in "
                          f"{oracle_wall:.1f} s; each cell's 'sample' holds the oracle's and the GPU's acceptance "
                          f"rate, mean accepted length and mean entropy on them"}
        log(f"verify entropy sweep: {cmean:.1f} us per call on average over 15 cells")

    if not args.no_cpu_baseline:
        n, cwall = cpu_baseline(torch, w, args.cpu_seconds)
        cores = 1
        result["cpu_baseline"] = {
            "value": n * G / cwall, "unit": "draft positions/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} rollout sequences ({n * G} draft positions, {n * (2 * G + 1)} rows of V={V}) "
                      f"through the float64 NumPy oracle, pinned to one CPU, {cwall:.1f} s; host has "
                      f"{os.cpu_count()} CPUs",
        }
        log(f"cpu oracle: {n * G / cwall:.1f} positions/s on one core")

    if "stream_context" in extras:
        ctx = stream_context(torch)
        result["roofline"]["stream_context"] = ctx
        log(f"stream context: torch copy {ctx['copy_gbs']:.0f} GB/s, torch float32 sum {ctx['read_sum_gbs']:.0f} GB/s")

    if args.copy_probe > 0:
        src = torch.ones(args.copy_probe, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
