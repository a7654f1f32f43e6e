"""DropKV eviction-scoring benchmark on one MI355X.

One step = one full scoring call (pass 1, merge, fix-up, pass 2, fold,
pool/protect/select) over one Llama-3.1-8B-shaped layer: 32 query heads,
8 KV heads, d = 128, n = 131072 tokens, window 64, bf16, MaxPool1D kernel 7,
5% of the tokens kept per KV head. Inputs are seeded synthetic Gaussian Q/K/V
with a planted attention sink and 64 needle keys, already resident in HBM
when the timed region starts.

Prints one JSON line: scored tokens/s for the layer (K steps back to back
with nothing else on the stream), the median and minimum per-step time (the
same K steps again, each bracketed by events), the dominant kernel's achieved
HBM bandwidth against MI355X's 8 TB/s (K more steps with the library's
per-kernel stage log), and the fp64 CPU oracle timed on a bounded sample of
the same workload (one KV head) as a reported baseline. After the timed
steps it also times, apart from `value`: the 4K and 32K Llama-shaped layers
(both 32K budgets), scoring from given row statistics, the Qwen2.5-7B-shaped
28-layer sweep (with its layers (0, 0) and (1, 27) scored on their own
seeds, checked against the oracle on one head each, and the oracle's time
extrapolated to the whole sweep), cache compaction and decode-time
rescoring (first window, per appended token in the two-pass and the
single-pass form, the flush of pending terms, re-eviction).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU needs ~60 back-to-back steps (~25 ms) before its clocks settle; the
    # default warm-up covers that, so the timed steps measure the steady state.
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="llama_128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the headline step: skip the scoring-from-statistics, "
                         "Qwen2.5-7B sweep, cache-compaction and decode-rescoring timings that "
                         "follow it")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 512 MiB (3 times): the reference kernel "
                         "that scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    ap.add_argument("--out", default=None, help="also write the JSON line to this new file")
    ap.add_argument("--qwen-seeded-sweep", action="store_true",
                    help="also run the Qwen2.5-7B-shaped sweep with every (sequence, layer) on its own "
                         "seeds: all 56 layers generated on the host (a few seconds each) and held in "
                         "HBM, then the 56 calls timed back to back, each on its own layer")
    return ap.parse_args()


def git_sha():
    try:
        return subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT, capture_output=True,
                              text=True, timeout=5).stdout.strip() or None
    except Exception:
        return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or None


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_llama_128k.txt")


def source_sha(rel):
    import hashlib
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def counted_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None.

    The summary records FETCH_SIZE + WRITE_SIZE per dispatch scaled by the same
    counters on a plain copy of known size, and the SHA-256 of the kernel
    source they were taken on; a changed source makes the figure stale (None).
    """
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    vals, shas = {}, {}
    for ln in lines:
        parts = ln.split()
        if len(parts) == 3 and parts[0] == "bytes_per_launch":
            vals[parts[1]] = float(parts[2])
        if len(parts) == 3 and parts[0] == "source_sha256":
            shas[parts[1]] = parts[2]
    if kernel not in vals or not shas:
        return None
    for rel, sha in shas.items():
        if not os.path.exists(os.path.join(ROOT, rel)) or source_sha(rel) != sha:
            return None
    return int(vals[kernel])


def step_times(torch, fn, reps):
    """Median and minimum of `reps` calls of fn, each bracketed by events on the current stream."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    return {"median": float(np.median(ms)), "min": float(ms[0]), "mean": float(np.mean(ms))}


def time_layer(torch, K, synth, name, dev, warmup, steps, n_evict=None):
    """Whole-path steps on one more synthetic workload: ms per step (mean of
    `steps` back-to-back steps after `warmup`), per-step median/min, the
    per-kernel means from the stage log, and the HBM fractions."""
    cfg = synth.CONFIGS[name]
    case = synth.make_case(cfg)
    ne = cfg.n_evicts()[0] if n_evict is None else n_evict
    q, k, v = (torch.from_numpy(t.view(np.int16)).view(torch.bfloat16).to(dev).contiguous()
               for t in (case.q, case.k, case.v))
    ws = torch.empty(K.workspace_bytes(K.BF16, case.n, case.window, case.Hq, case.Hkv, case.d),
                     dtype=torch.uint8, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    sc = torch.empty((case.Hkv, case.n), dtype=torch.float32, device=dev)
    ix = torch.empty((case.Hkv, ne), dtype=torch.int64, device=dev)

    def step(flags=0):
        K.score_ex(q, k, v, pool_kernel=cfg.pool_kernel, n_evict=ne, workspace=ws, status=st, scores=sc,
                   evict_idx=ix, flags=flags)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    per = step_times(torch, step, steps)
    K.stage_log()
    for _ in range(steps):
        step(K.FLAG_STAGE_LOG)
    torch.cuda.synchronize()
    _, stages = K.stage_log()
    if int(st.item()) != 0:
        raise SystemExit(f"device status {int(st.item())} on {name}")
    stage_ms = {a: b for a, b in stages}
    pass_bytes = case.Hkv * case.n * case.d * 2 * 2
    dom = max((x for x in ("pass1", "pass2") if x in stage_ms), key=lambda x: stage_ms[x])
    out = {
        "workload": f"{name}: Hq {case.Hq}, Hkv {case.Hkv}, d {case.d}, n {case.n}, window {case.window}, "
                    f"pool {cfg.pool_kernel}, evict {ne} per head",
        "ms_per_step": round(ms, 4), "ms_per_step_median": round(per["median"], 4),
        "ms_per_step_min": round(per["min"], 4),
        "tokens_per_s": round(case.n / (ms * 1e-3), 1),
        "step_hbm_frac": round(2 * pass_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "dominant_kernel": dom,
        "dominant_kernel_hbm_frac": round(pass_bytes / (stage_ms[dom] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "stages_ms": {a: round(b, 4) for a, b in stage_ms.items()},
    }
    del q, k, v, ws
    return out


def copy_calibration():
    import torch
    dev = torch.device("cuda:0")
    nbytes = 512 << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": 3}), flush=True)


def qwen_seeded_sweep(torch, K, synth, qcfg, to_dev, qws, qst, qsc, qix, qne, warmup):
    """The 28-layer, 2-sequence sweep with every call on its own (sequence, layer)
    seeds: the layers are generated one by one on the host and kept in HBM
    (56 x 256 MiB of K/V), then the 56 calls run back to back on one stream.
    Each call's status and own-bottom-k property are checked afterwards."""
    layers = []
    t0 = time.time()
    for b_ in range(qcfg.batch):
        for l_ in range(qcfg.layers):
            lc = synth.make_case(qcfg, layer=l_, b=b_)
            layers.append(tuple(to_dev(t).contiguous() for t in (lc.q, lc.k, lc.v)))
            print(f"[qwen seeded sweep] generated (b={b_}, l={l_}) {time.time() - t0:.0f} s", file=sys.stderr,
                  flush=True)
    calls = len(layers)
    outs = [(torch.empty_like(qsc), torch.empty_like(qix)) for _ in range(calls)]
    sts = torch.zeros(calls, dtype=torch.int32, device=qsc.device)

    def call(i):
        lq, lk, lv = layers[i]
        K.score_ex(lq, lk, lv, pool_kernel=qcfg.pool_kernel, n_evict=qne, workspace=qws, status=sts[i:i + 1],
                   scores=outs[i][0], evict_idx=outs[i][1])
    for i in range(min(warmup, calls)):
        call(i)
    torch.cuda.synchronize()
    sts.zero_()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(calls):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    bad = int((sts != 0).sum().item())
    own_ok = True
    for sc_, ix_ in outs:
        P = sc_.cpu().numpy()
        ix = ix_.cpu().numpy()
        for g in range(P.shape[0]):
            own_ok &= bool(np.array_equal(ix[g], np.sort(np.argsort(P[g], kind="stable")[:qne])))
    n = layers[0][1].shape[1]
    Hkv, d = layers[0][1].shape[0], layers[0][1].shape[2]
    G = layers[0][0].shape[0] // Hkv
    w = layers[0][0].shape[1]
    flop = calls * 8 * d * G * w * Hkv * n
    return {"calls": calls, "ms": round(ms, 3), "ms_per_call": round(ms / calls, 4),
            "tokens_per_s": round(calls * n / (ms * 1e-3), 1),
            "mfma_TFLOPs": round(flop / (ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(flop / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "calls_with_nonzero_status": bad, "evicted_sets_are_own_bottom_k": own_ok,
            "generation_s": round(time.time() - t0 - ms * 1e-3, 1)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the DropKV scoring path here runs on a single "
              "MI355X (no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import kv_cache_eviction_pass1_amd as K
    from kv_cache_eviction_pass1_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    cfg = synth.CONFIGS[args.workload]
    n_evict = cfg.n_evicts()[0]
    t_gen = time.perf_counter()
    case = synth.make_case(cfg)
    t_gen = time.perf_counter() - t_gen

    def to_dev(a):
        if case.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q, k, v = (to_dev(t).contiguous() for t in (case.q, case.k, case.v))
    dcode = K.BF16 if case.dtype == "bf16" else K.F32
    ws = torch.empty(K.workspace_bytes(dcode, case.n, case.window, case.Hq, case.Hkv, case.d),
                     dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    scores = torch.empty((case.Hkv, case.n), dtype=torch.float32, device=dev)
    evict = torch.empty((case.Hkv, n_evict), dtype=torch.int64, device=dev)

    def step(flags=0):
        K.score_ex(q, k, v, pool_kernel=cfg.pool_kernel, n_evict=n_evict, workspace=ws,
                   status=status, scores=scores, evict_idx=evict, flags=flags)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise SystemExit(f"device status {int(status.item())} after warm-up")

    # timed region: K whole-path steps back to back, synchronised on both
    # sides, nothing else on the stream (value and ms_per_step come from here)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    st_word = int(status.item())
    if st_word != 0:
        raise SystemExit(f"device status {st_word} in the timed region")
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    tokens_per_s = case.n / (ms_per_step * 1e-3)

    # per-step distribution: the same K steps again, each bracketed by events
    # on the stream the library launches on (the current torch stream)
    per_step = step_times(torch, step, args.steps)

    # per-kernel mean durations: K more steps with the library's stage log (a
    # stage's begin and end from its kernels' own dispatch timestamps)
    K.stage_log()  # empty the log
    for _ in range(args.steps):
        step(K.FLAG_STAGE_LOG)
    torch.cuda.synchronize()
    logged, stages = K.stage_log()
    stage_ms = {name: ms for name, ms in stages}
    kv_bytes_per_pass = case.Hkv * case.n * case.d * 2 * 2  # K and V read once
    passes = [s for s in ("pass1", "pass2") if s in stage_ms]
    if passes:
        dom = max(passes, key=lambda s: stage_ms[s])
        dom_ms = stage_ms[dom]
        achieved = kv_bytes_per_pass / (dom_ms * 1e-3) / 1e9
    else:
        dom = max(stage_ms, key=stage_ms.get)
        dom_ms = stage_ms[dom]
        achieved = 2 * kv_bytes_per_pass / (dom_ms * 1e-3) / 1e9
    roofline = {
        "bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": counted_traffic(dom) if args.workload == "llama_128k" else None,
        "bytes_per_launch": kv_bytes_per_pass, "avg_ms": round(dom_ms, 4), "timed_launches": logged,
    }
    step_bytes = 2 * kv_bytes_per_pass
    flops = 8 * case.d * case.group * case.window * case.Hkv * case.n

    rec = {
        "metric": "DropKV scored KV tokens/s per layer at n=128K; achieved HBM GB/s vs peak",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: Llama-3.1-8B-shaped layer" if cfg.name.startswith("llama")
            else cfg.name,
            "query_heads": case.Hq, "kv_heads": case.Hkv, "head_dim": case.d, "n": case.n,
            "window": case.window, "pool_kernel": cfg.pool_kernel, "n_evict_per_head": n_evict,
            "batch": 1, "sink": cfg.sink, "needles": cfg.needles,
        },
        "roofline": roofline,
        "step_hbm": {"alg_bytes": step_bytes,
                     "achieved_GBs": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                     "frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "mfma": {"alg_flop": flops,
                 "achieved_TFLOPs": round(flops / (ms_per_step * 1e-3) / 1e12, 1),
                 "frac": round(flops / (ms_per_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        "ms_per_step_median": round(per_step["median"], 4),
        "ms_per_step_min": round(per_step["min"], 4),
        "stages_ms": {k_: round(v_, 4) for k_, v_ in stage_ms.items()},
        "workspace_bytes": int(ws.numel()),
        "path": "mfma" if K.uses_mfma(dcode, case.d) else "generic",
        "git": git_sha(),
        "device": torch.cuda.get_device_name(dev),
    }

    # The shorter Llama-3.1-8B-shaped layers (4K; 32K at both budgets), timed
    # the same way, apart from `value`.
    if args.workload == "llama_128k" and not args.no_extras:
        c3 = synth.CONFIGS["llama_32k"]
        rec["workloads"] = {
            "llama_4k": time_layer(torch, K, synth, "llama_4k", dev, args.warmup, args.steps),
            "llama_32k_keep5": time_layer(torch, K, synth, "llama_32k", dev, args.warmup, args.steps,
                                          c3.n_evicts()[0]),
            "llama_32k_keep20": time_layer(torch, K, synth, "llama_32k", dev, args.warmup, args.steps,
                                           c3.n_evicts()[1]),
        }

    # Scoring from given row statistics (no pass 1; the step a prefill kernel's
    # statistics would allow), timed apart from the scoring steps above.
    if K.uses_mfma(dcode, case.d) and not args.no_extras:
        m_, rest_, arg_, a_ = (t.contiguous() for t in K.row_stats(q, k, v))
        fs_sc = torch.empty_like(scores)
        fs_ix = torch.empty_like(evict)

        def fs_step():
            K.score_from_stats(q, k, v, m_, rest_, arg_, a_, pool_kernel=cfg.pool_kernel,
                               n_evict=n_evict, workspace=ws, status=status, scores=fs_sc,
                               evict_idx=fs_ix)
        for _ in range(args.warmup):
            fs_step()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fs_step()
        e1.record()
        torch.cuda.synchronize()
        if int(status.item()) != 0:
            raise SystemExit(f"device status {int(status.item())} scoring from statistics")
        fs_ms = e0.elapsed_time(e1) / args.steps
        rec["from_stats"] = {
            "ms_per_step": round(fs_ms, 4), "tokens_per_s": round(case.n / (fs_ms * 1e-3), 1),
            "speedup_vs_step": round(ms_per_step / fs_ms, 3),
            "evict_equal": bool(torch.equal(fs_ix, evict)),
        }

    # Prefill attention at this layer's shape, handing the window rows'
    # statistics to scoring (the producer of scoring from statistics): its
    # kernel time and MFMA rate (causal: 4 d sum_pos (pos + 1) flops per query
    # head), and prefill + scoring from its statistics against prefill + the
    # two-pass scoring step.
    if args.workload == "llama_128k" and K.uses_mfma(dcode, case.d) and not args.no_extras:
        qa_np = synth.prefill_queries(case, seed=cfg.seeds[0] + 7)
        q_all = torch.from_numpy(qa_np.view(np.int16)).view(torch.bfloat16).to(dev).contiguous()
        del qa_np
        o_buf = torch.empty((case.Hq, case.n, case.d), dtype=torch.bfloat16, device=dev)
        pst = torch.zeros(1, dtype=torch.int32, device=dev)
        outs = K.prefill_attention(q_all, k, v, window=case.window, status=pst, out_o=o_buf)
        torch.cuda.synchronize()
        reps = 3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            outs = K.prefill_attention(q_all, k, v, window=case.window, status=pst, out_o=o_buf)
        e1.record()
        torch.cuda.synchronize()
        if int(pst.item()) != 0:
            raise SystemExit(f"prefill status {int(pst.item())}")
        p_ms = e0.elapsed_time(e1) / reps
        _, pm, prest, parg, pa = outs
        pf_sc = torch.empty_like(scores)
        pf_ix = torch.empty_like(evict)
        K.score_from_stats(q, k, v, pm, prest, parg, pa, pool_kernel=cfg.pool_kernel, n_evict=n_evict,
                           workspace=ws, status=status, scores=pf_sc, evict_idx=pf_ix)
        torch.cuda.synchronize()
        p_flop = 4 * case.d * case.Hq * case.n * (case.n + 1) // 2
        rec["prefill"] = {
            "workload": "causal prefill attention of the same layer (all 131072 positions, 32 query heads), "
                        "window statistics handed to scoring",
            "ms": round(p_ms, 3), "flop": p_flop,
            "mfma_TFLOPs": round(p_flop / (p_ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(p_flop / (p_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "scores_from_prefill_stats_max_rel_diff": float(
                (pf_sc - scores).abs().div(scores.abs().clamp_min(1e-30)).nan_to_num(0.0).max().item()),
            "evict_equal_to_step": bool(torch.equal(pf_ix, evict)),
        }
        del q_all, o_buf, outs

    # The Qwen2.5-7B-shaped sweep (28 layers x 2 sequences of one 128K layer
    # shape, G = 7), back to back on one stream; MFMA-bound by its arithmetic
    # intensity. One generated layer's tensors serve every call (the throughput
    # does not depend on the values; parity of this shape is a test's job).
    if args.workload == "llama_128k" and not args.no_extras:
        qcfg = synth.CONFIGS["qwen_128k_sweep"]
        qc = synth.make_case(qcfg)
        qq, qk, qv = (to_dev(t).contiguous() for t in (qc.q, qc.k, qc.v))
        qne = qcfg.n_evicts()[0]
        qws = torch.empty(K.workspace_bytes(K.BF16, qc.n, qc.window, qc.Hq, qc.Hkv, qc.d),
                          dtype=torch.uint8, device=dev)
        qst = torch.zeros(1, dtype=torch.int32, device=dev)
        qsc = torch.empty((qc.Hkv, qc.n), dtype=torch.float32, device=dev)
        qix = torch.empty((qc.Hkv, qne), dtype=torch.int64, device=dev)
        calls = qcfg.layers * qcfg.batch

        def q_step():
            K.score_ex(qq, qk, qv, pool_kernel=qcfg.pool_kernel, n_evict=qne, workspace=qws,
                       status=qst, scores=qsc, evict_idx=qix)
        for _ in range(args.warmup):
            q_step()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(calls):
            q_step()
        e1.record()
        torch.cuda.synchronize()
        if int(qst.item()) != 0:
            raise SystemExit(f"device status {int(qst.item())} in the Qwen sweep")
        q_ms = e0.elapsed_time(e1)
        q_flop = calls * 8 * qc.d * qc.group * qc.window * qc.Hkv * qc.n
        rec["qwen_sweep"] = {
            "workload": "Qwen2.5-7B-shaped layer (Hq 28, Hkv 4, d 128, n 131072, w 64), 28 layers x 2 sequences",
            "calls": calls, "ms": round(q_ms, 3), "ms_per_call": round(q_ms / calls, 4),
            "tokens_per_s": round(calls * qc.n / (q_ms * 1e-3), 1),
            "mfma_TFLOPs": round(q_flop / (q_ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(q_flop / (q_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        }
        if args.qwen_seeded_sweep:
            rec["qwen_sweep"]["seeded"] = qwen_seeded_sweep(torch, K, synth, qcfg, to_dev, qws, qst, qsc, qix, qne,
                                                            args.warmup)
        # the sweep's sampled layers with their own seeds, (sequence, layer) = (0, 0)
        # and (1, 27): scored once each here, checked against the oracle below
        qwen_layers = {}
        for b_, l_ in ((0, 0), (1, 27)):
            lc = synth.make_case(qcfg, layer=l_, b=b_)
            lq, lk, lv = (to_dev(t).contiguous() for t in (lc.q, lc.k, lc.v))
            K.score_ex(lq, lk, lv, pool_kernel=qcfg.pool_kernel, n_evict=qne, workspace=qws, status=qst,
                       scores=qsc, evict_idx=qix)
            torch.cuda.synchronize()
            if int(qst.item()) != 0:
                raise SystemExit(f"device status {int(qst.item())} on Qwen layer {(b_, l_)}")
            qwen_layers[(b_, l_)] = (lc, qsc.cpu().numpy(), qix.cpu().numpy())
            del lq, lk, lv
        del qq, qk, qv, qws

    if "prefill" in rec and "from_stats" in rec:
        rec["prefill"]["prefill_plus_scoring_from_stats_ms"] = round(
            rec["prefill"]["ms"] + rec["from_stats"]["ms_per_step"], 3)
        rec["prefill"]["prefill_plus_scoring_step_ms"] = round(rec["prefill"]["ms"] + ms_per_step, 3)

    # Cache compaction (the step after scoring), timed apart from `value`:
    # copies each head's kept rows of K and V into a compact cache. Each
    # compaction is timed with events right after a scoring step (the order a
    # pipeline runs them in: pass 2 has just streamed K and V, so part of them
    # sits in the memory-side cache); back-to-back compactions of the same
    # rows, whose inputs then stay cache-resident, are reported apart.
    if n_evict < case.n and not args.no_extras:
        n_keep = case.n - n_evict
        out_k = torch.empty((case.Hkv, n_keep, case.d), dtype=k.dtype, device=dev)
        out_v = torch.empty_like(out_k)
        cst = torch.zeros(1, dtype=torch.int32, device=dev)
        keep = torch.empty((case.Hkv, n_keep), dtype=torch.int64, device=dev)
        kev = torch.empty_like(evict)
        elem = 2 if case.dtype == "bf16" else 4
        rows_bytes = 2 * 2 * case.Hkv * n_keep * case.d * elem

        def score_keep():
            K.score_keep_ex(q, k, v, pool_kernel=cfg.pool_kernel, n_evict=n_evict, workspace=ws,
                            status=status, scores=scores, evict_idx=kev, keep_idx=keep)

        def after_scoring(compact_fn, score_fn):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
            for _ in range(3):
                score_fn()
                compact_fn()
            for a_, b_ in evs:
                score_fn()
                a_.record()
                compact_fn()
                b_.record()
            torch.cuda.synchronize()
            return float(np.median([a_.elapsed_time(b_) for a_, b_ in evs]))

        def repeated(compact_fn):
            for _ in range(10):
                compact_fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                compact_fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.steps

        by_evict = lambda: K.compact(k, v, evict, status=cst, out_k=out_k, out_v=out_v)
        by_keep = lambda: K.compact_kept(k, v, keep, status=cst, out_k=out_k, out_v=out_v)
        c_ms = after_scoring(by_evict, step)
        c_rep = repeated(by_evict)
        ok0, ov0 = out_k.clone(), out_v.clone()
        kc_ms = after_scoring(by_keep, score_keep)
        kc_rep = repeated(by_keep)
        if int(cst.item()) != 0 or int(status.item()) != 0:
            raise SystemExit(f"compaction status {int(cst.item())} / {int(status.item())}")
        if not (torch.equal(kev, evict) and torch.equal(ok0, out_k) and torch.equal(ov0, out_v)):
            raise SystemExit("kept-list compaction differs from compaction by the eviction list")
        # the scoring step with the kept list written (one more list output in select)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            score_keep()
        e1.record()
        torch.cuda.synchronize()
        sk_ms = e0.elapsed_time(e1) / args.steps
        c_bytes = rows_bytes + case.Hkv * n_evict * 8
        kc_bytes = rows_bytes + case.Hkv * n_keep * 8
        gbs = lambda by, ms: round(by / (ms * 1e-3) / 1e9, 1)
        rec["compact"] = {
            "ms": round(c_ms, 4), "alg_bytes": c_bytes, "achieved_GBs": gbs(c_bytes, c_ms),
            "frac": round(gbs(c_bytes, c_ms) / HBM_PEAK_GBS, 4),
            "ms_repeated_cache_resident": round(c_rep, 4),
            "score_plus_compact_ms": round(ms_per_step + c_ms, 4),
            "from_keep_list": {
                "ms": round(kc_ms, 4), "alg_bytes": kc_bytes, "achieved_GBs": gbs(kc_bytes, kc_ms),
                "frac": round(gbs(kc_bytes, kc_ms) / HBM_PEAK_GBS, 4),
                "ms_repeated_cache_resident": round(kc_rep, 4),
                "score_keep_step_ms": round(sk_ms, 4),
                "score_keep_plus_compact_ms": round(sk_ms + kc_ms, 4),
            },
        }

    # Decode-time rescoring on the same layer: the prefix scored once (init),
    # then one step per appended token (the new position's rows added, the
    # leaving rows subtracted), then a re-eviction on the kept score. The
    # layer's tensors stand in for the grown cache (head stride = n); the query
    # rows of the appended positions are the layer's window rows in turn.
    if args.workload == "llama_128k" and K.uses_mfma(dcode, case.d) and not args.no_extras:
        dsteps = 64
        n0 = case.n - dsteps
        dec = K.DecodeScorer(n_max=case.n, window=case.window, Hq=case.Hq, Hkv=case.Hkv, d=case.d, device=dev)
        qrows = [q[:, i % case.window].contiguous() for i in range(dsteps)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(3):
            dec.init(q, k, v, n0)
        e0.record()
        dec.init(q, k, v, n0)
        e1.record()
        torch.cuda.synchronize()
        init_ms = e0.elapsed_time(e1)
        for i in range(dsteps // 2):  # warm-up steps, then the state is scored again
            dec.step(qrows[i], k, v)
        dec.init(q, k, v, n0)
        torch.cuda.synchronize()
        e0.record()
        for i in range(dsteps):
            dec.step(qrows[i], k, v)
        e1.record()
        torch.cuda.synchronize()
        step_ms = e0.elapsed_time(e1) / dsteps
        # the same 64 appended tokens with single-pass steps (one read of the
        # cache per token; the newest position's terms wait for the next step),
        # then the flush that adds the last step's pending terms
        dec.init(q, k, v, n0)
        for i in range(dsteps // 2):
            dec.step(qrows[i], k, v, deferred=True)
        dec.init(q, k, v, n0)
        torch.cuda.synchronize()
        e0.record()
        for i in range(dsteps):
            dec.step(qrows[i], k, v, deferred=True)
        e1.record()
        torch.cuda.synchronize()
        step1_ms = e0.elapsed_time(e1) / dsteps
        e0.record()
        dec.flush()
        e1.record()
        torch.cuda.synchronize()
        flush_ms = e0.elapsed_time(e1)
        for _ in range(3):
            dec.select(pool_kernel=cfg.pool_kernel, n_evict=n_evict)
        e0.record()
        for _ in range(10):
            dec.select(pool_kernel=cfg.pool_kernel, n_evict=n_evict)
        e1.record()
        torch.cuda.synchronize()
        sel_ms = e0.elapsed_time(e1) / 10
        dec.check()
        step_bytes = 4 * case.Hkv * case.n * case.d * 2  # K and V read by the statistics and the terms kernels
        step1_bytes = step_bytes // 2  # K and V read once
        rec["decode"] = {
            "workload": "same layer grown by 64 tokens from n - 64, window 64",
            "init_ms": round(init_ms, 4), "step_ms": round(step_ms, 4), "select_ms": round(sel_ms, 4),
            "step_alg_bytes": step_bytes,
            "step_achieved_GBs": round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
            "step_frac": round(step_bytes / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "single_pass_step_ms": round(step1_ms, 4),
            "single_pass_alg_bytes": step1_bytes,
            "single_pass_achieved_GBs": round(step1_bytes / (step1_ms * 1e-3) / 1e9, 1),
            "single_pass_frac": round(step1_bytes / (step1_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "flush_ms": round(flush_ms, 4),
            "full_rescore_ms": round(ms_per_step, 4),
        }
        del dec

    if not args.no_cpu_baseline:
        import oracle
        ncores = len(os.sched_getaffinity(0))
        if os.environ.get("OMP_NUM_THREADS", "").isdigit():
            ncores = min(ncores, int(os.environ["OMP_NUM_THREADS"]))
        blas_threads = None
        try:
            from threadpoolctl import threadpool_info, threadpool_limits
            threadpool_limits(limits=ncores)
            blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=None)
        except Exception:
            pass
        head = 0
        sc = scores.cpu().numpy()
        ev = evict.cpu().numpy()
        t_c = time.perf_counter()
        ref = oracle.dropkv_oracle(case.q, case.k, case.v, n=case.n, window=case.window,
                                   Hq=case.Hq, Hkv=case.Hkv, d=case.d, pool_kernel=cfg.pool_kernel,
                                   n_evict=n_evict, dtype=case.dtype, heads=[head])
        t_c = time.perf_counter() - t_c
        P = ref["P"][0]
        fin = np.isfinite(P)
        gpu = sc[head].astype(np.float64)
        rel = float(np.max(np.abs(gpu[fin] - P[fin]) / np.maximum(np.abs(P[fin]), 1e-300)))
        same_set = bool(np.array_equal(np.sort(ev[head]), ref["evict"][0]))
        inter = np.intersect1d(ev[head], ref["evict"][0]).size
        jac = inter / np.union1d(ev[head], ref["evict"][0]).size
        cpu_tps = case.n / (t_c * case.Hkv)
        rec["cpu_baseline"] = {
            "value": round(cpu_tps, 2), "unit": "tokens/s", "cores": blas_threads or ncores,
            "kind": "oracle",
            "sample": (f"fp64 numpy oracle on KV head {head} of {case.Hkv} of the same layer "
                       f"(all {case.group * case.window} window rows x {case.n} tokens, pool and "
                       f"select), {t_c:.1f} s, scaled to the layer by x{case.Hkv}; BLAS threads "
                       f"{blas_threads or ncores}, elementwise numpy single-threaded; CPU "
                       f"{cpu_model()}"),
        }
        rec["parity_sample"] = {"head": head, "max_rel_err": rel, "evict_set_equal": same_set,
                                "jaccard": round(float(jac), 6)}
        if args.workload == "llama_128k" and not args.no_extras:
            # the Qwen2.5-7B-shaped sweep: the oracle on KV head 0 of the two
            # sampled layers, extrapolated to all heads and all 56 calls
            qcfg = synth.CONFIGS["qwen_128k_sweep"]
            qne = qcfg.n_evicts()[0]
            times, checks = [], []
            for (b_, l_), (lc, qsc_np, qix_np) in qwen_layers.items():
                t_q = time.perf_counter()
                qref = oracle.dropkv_oracle(lc.q, lc.k, lc.v, n=lc.n, window=lc.window, Hq=lc.Hq,
                                            Hkv=lc.Hkv, d=lc.d, pool_kernel=qcfg.pool_kernel, n_evict=qne,
                                            dtype=lc.dtype, heads=[0])
                times.append(time.perf_counter() - t_q)
                Pq = qref["P"][0]
                fq = np.isfinite(Pq)
                rq = float(np.max(np.abs(qsc_np[0][fq].astype(np.float64) - Pq[fq]) / np.abs(Pq[fq])))
                jq = (np.intersect1d(qix_np[0], qref["evict"][0]).size
                      / np.union1d(qix_np[0], qref["evict"][0]).size)
                checks.append({"seq": b_, "layer": l_, "head": 0, "max_rel_err": rq,
                               "jaccard": round(float(jq), 6)})
            t_head = float(np.mean(times))
            calls = qcfg.layers * qcfg.batch
            rec["qwen_sweep"]["cpu_baseline_extrapolated"] = {
                "value": round(qcfg.n / (t_head * qcfg.Hkv), 2), "unit": "tokens/s",
                "cores": blas_threads or ncores, "kind": "oracle",
                "sweep_s": round(t_head * qcfg.Hkv * calls, 1),
                "sample": (f"fp64 numpy oracle on KV head 0 of {qcfg.Hkv} of (sequence, layer) = (0, 0) and "
                           f"(1, 27), {t_head:.1f} s per head, extrapolated x{qcfg.Hkv} heads x{calls} calls "
                           f"(EXTRAPOLATED, not run in full)"),
            }
            rec["qwen_sweep"]["parity_sample"] = checks
    line = json.dumps(rec)
    print(line, flush=True)
    if args.out:
        if os.path.exists(args.out):
            raise SystemExit(f"{args.out} exists; refusing to overwrite")
        with open(args.out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
