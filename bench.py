"""Benchmark of the block-diffusion denoising hot path on one MI355X.

Default workload: one bf16 MoE layer (D 2048, 16 q / 8 kv heads x 128, 128
experts top-8, expert FFN 768, vocabulary 32768), a 1024-token cached prefix
and a 256-token canvas denoised in 8 passes.  One step is one whole canvas:
noise initialisation, 8 x (denoising pass, expert coverage, re-noise between
passes; the last two run inside the pass's final kernel), then the causal
append-prefill of the committed canvas; the cache length is reset afterwards
so every step sees the same prefix.  For the 8-layer chained workload a step
is one whole request: the prompt prefill and four chained canvases.

Prints one JSON line: value = canvas-token passes per second (B*N*S per
canvas), the roofline of the dominant kernel (timed with HIP events on the
compute stream inside the timed region), the whole-pass roofline, warm and
cold pass times, per-stage times, and the CPU oracle timed on a bounded
sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def _source_hash(files):
    """Hash of the kernel sources a counter summary was taken on."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "block_diffusion_lm_denoise_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# dominant kernel per workload: (stage, bound, kernel name, sources it is built from)
DOMINANT = {
    "bf16": ("gateup", "hbm", "dg::wstream_k<bf16, bf16, 4, 4, 2, 4> (grouped gate/up + SwiGLU)",
             ("kern_stream.hip", "common.h", "launch.h")),
    "fp8": ("head", "mfma", "dg::lmhead_wide_k (LM head + argmax/confidence partials, 2048 rows)",
            ("kern_gemm.hip", "common.h", "launch.h")),
}


def _traffic(workload, stage, files):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary, if it was taken on this workload and the current kernel
    source; else None."""
    path = os.path.join(ROOT, "profiles", f"{stage}_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("source_hash") != _source_hash(files) or not str(d.get("workload", "")).startswith(workload):
        return None
    return d.get("hbm_bytes_per_launch")


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sampler", choices=("uniform", "masked"), default="uniform",
                    help="update between passes: uniform-state noise, or masked (absorbing) diffusion")
    ap.add_argument("--early-exit", action="store_true",
                    help="stop a canvas once it has converged (reads two counts per pass to the host)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 4 GiB device copy (counter calibration)")
    ap.add_argument("--no-ar-baseline", action="store_true",
                    help="skip the autoregressive-step comparison (keeps kernel traces to the pass)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the pass runs on a single MI355X (no multi-GPU path is "
              "built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_diffusion_lm_denoise_amd import dgpass, roofline, synth
    from block_diffusion_lm_denoise_amd.configs import BENCH_WORKLOAD, WORKLOADS

    wl = WORKLOADS[args.workload or BENCH_WORKLOAD]
    cfg = wl.model
    dev = "cuda:0"
    torch.cuda.set_device(0)
    B, N, P, S, C = wl.B, wl.N, wl.P, wl.S, wl.canvases
    chained = C > 1
    print(f"bench: workload {wl.name}", file=sys.stderr, flush=True)
    w = synth.make_weights(cfg, wl.seed, device=dev)
    model = dgpass.Model(cfg, w)
    cap = P + C * N
    kv = model.kv_cache(B, cap, device=dev)
    ws = model.workspace(max(B * P, B * N), cap, device=dev)
    prompt = synth.tokens(cfg.V, (B, P), wl.seed, device=dev)
    if not chained:
        model.kv_prefill(kv, prompt, ws)
    torch.cuda.synchronize()
    base_lens = kv.lens.copy()

    canvas = torch.empty(B, N, dtype=torch.int32, device=dev)
    argmax = torch.empty(B, N, dtype=torch.int32, device=dev)
    conf = torch.empty(B, N, dtype=torch.float32, device=dev)
    touched = torch.zeros(C, S, cfg.L, dtype=torch.int32, device=dev)
    dom_stage, dom_bound, dom_kernel, dom_files = DOMINANT[cfg.expert if cfg.expert == "fp8" else "bf16"]
    if cfg.expert == "mxfp4":
        dom_kernel = "dg::wstream_k<bf16, mxfp4, 4, 4, 2, 2> (grouped gate/up + SwiGLU, 4-bit experts)"
    stage_id = {"gateup": dgpass.STAGE_GATEUP, "head": dgpass.STAGE_HEAD}[dom_stage]
    ev_layer = cfg.L - 1 if dom_stage == "head" else 0

    def stage_list(ev_pair, stage, layer):
        """flat [L][NSTAGES][2] event list with one stage of one layer set"""
        lst = [None] * (cfg.L * dgpass.NSTAGES * 2)
        i = (layer * dgpass.NSTAGES + stage) * 2
        lst[i], lst[i + 1] = ev_pair
        return lst

    masked = args.sampler == "masked"
    counts = torch.zeros(2, B, dtype=torch.int32, device=dev)
    passes_run = []

    def canvas_loop(c, events=None, marks=None):
        pos0 = kv.lens.copy()
        base = dict(sampler=args.sampler, mask_id=cfg.V - 1, tau=wl.tau, seed=wl.seed, pos0=pos0,
                    changed=counts[0] if args.early_exit else None,
                    masked_left=counts[1] if args.early_exit else None)
        dgpass.canvas_update(canvas, None, None, dict(base, pass_tag=0), cfg.V)
        ran = S
        carry = False   # the workspace holds the first layer's input of `canvas`
        for p in range(S):
            # one mid-canvas pass of each timed step carries the stage events of
            # the dominant kernel (an event record costs a few us of GPU time)
            se = None if events is None or p != S // 2 else stage_list(events, stage_id, ev_layer)
            # coverage and the update for the next pass run in the pass's last
            # kernel (uniform: none after the last pass; masked: the last update
            # fills every masked slot)
            # (and the embedding of the updated canvas, when the next pass
            # takes an update: that pass then skips its own embedding)
            last = p == S - 1
            ahead = p + 1 < S and (masked or p + 1 < S - 1)
            nxt = None if (last and not masked) else dict(base, pass_tag=p + 1, final_pass=last,
                                                          embed_next=ahead, input_embedded=carry)
            model.denoise_pass_next(kv, canvas, argmax, conf, ws, touched=touched[c, p], renoise=nxt,
                                    stage_events=se)
            carry = nxt is not None and nxt["embed_next"]
            if args.early_exit and not last:
                torch.cuda.synchronize()
                if int(counts[1 if masked else 0].max()) == 0:
                    ran = p + 1
                    break
        passes_run.append(ran)
        if marks is not None:
            marks[0].record()
        model.kv_prefill(kv, canvas if masked else argmax, ws)   # append the committed canvas
        if marks is not None:
            marks[1].record()

    def step(events=None):
        kv.lens[:] = base_lens
        if chained:
            model.kv_prefill(kv, prompt, ws)
        for c in range(C):
            canvas_loop(c, events if c == 0 else None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps, the dominant kernel's launches of one pass
    # per step bracketed by HIP events recorded on the same stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for e in evs:          # torch creates the HIP event on its first record
        e[0].record()
        e[1].record()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(evs[i])
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    dom_us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
    cov = touched.cpu().numpy()                                  # [C][S][L]
    cov_layer = cov.reshape(-1, cfg.L).mean(axis=0)              # mean per layer
    mean_touched = float(cov.mean())

    def ev_pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # ---- outside the timed region: pass-only timings on the benchmark's prefix ----
    kv.lens[:] = base_lens
    if chained:   # the pass-only figures use a cache holding the prompt
        model.kv_prefill(kv, prompt, ws)
    pass_lens = kv.lens.copy()
    # a pass as it runs inside a canvas: the fused tail (coverage, update,
    # embedding of the updated canvas) included, its own embedding skipped
    inner = dict(sampler=args.sampler, mask_id=cfg.V - 1, tau=wl.tau, seed=wl.seed,
                 pos0=pass_lens.copy(), pass_tag=1, embed_next=True, input_embedded=False)
    cov_scratch = torch.zeros(cfg.L, dtype=torch.int32, device=dev)

    def inner_pass():
        model.denoise_pass_next(kv, canvas, argmax, conf, ws, touched=cov_scratch, renoise=inner)
        inner["input_embedded"] = True

    inner_pass()
    torch.cuda.synchronize()
    npass = max(8, args.steps)
    p0, p1 = ev_pair()
    p0.record()
    for _ in range(npass):
        inner_pass()
    p1.record()
    torch.cuda.synchronize()
    pass_us = p0.elapsed_time(p1) / npass * 1e3
    # cold passes: a 512 MB write between passes evicts the last-level cache
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(5):
        scratch.fill_(1)
        a, b = ev_pair()
        a.record()
        inner_pass()
        b.record()
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b) * 1e3)
    del scratch
    # per-stage times of one warm pass (stage events of every layer)
    stage_names = ("attention", "gateup", "down", "head")
    pairs = {(l, s): ev_pair() for l in range(cfg.L) for s in range(dgpass.NSTAGES)}
    lst = [None] * (cfg.L * dgpass.NSTAGES * 2)
    for (l, s), (a, b) in pairs.items():
        lst[(l * dgpass.NSTAGES + s) * 2], lst[(l * dgpass.NSTAGES + s) * 2 + 1] = a, b
    for _ in range(2):
        for e in lst:
            e.record()
        model.denoise_pass(kv, canvas, argmax, conf, ws, stage_events=lst)
        torch.cuda.synchronize()
    stages = {n: 0.0 for n in stage_names}
    for (l, s), (a, b) in pairs.items():
        if s == dgpass.STAGE_HEAD and l != cfg.L - 1:
            continue
        stages[stage_names[s]] += a.elapsed_time(b) * 1e3
    # chained workload: time to first token (prompt prefill), one canvas, the request
    c3 = None
    if chained:
        m = [ev_pair() for _ in range(3)]
        kv.lens[:] = base_lens
        m[0][0].record()
        model.kv_prefill(kv, prompt, ws)
        m[0][1].record()
        canvas_loop(0, marks=m[1])
        m[2][0].record()
        for c in range(1, C):
            canvas_loop(c)
        m[2][1].record()
        torch.cuda.synchronize()
        prefill_ms = m[0][0].elapsed_time(m[0][1])
        request_ms = m[0][0].elapsed_time(m[2][1])
        c3 = {"prompt_prefill_ms": prefill_ms,
              "first_canvas_ms": m[0][1].elapsed_time(m[1][1]),
              "append_prefill_ms": m[1][0].elapsed_time(m[1][1]),
              "time_to_first_canvas_ms": m[0][0].elapsed_time(m[1][1]),
              "request_ms": request_ms,
              "steady_state_pass_us": pass_us,
              "output_tokens_per_s": B * N * C / (request_ms / 1e3)}

    ar_us = ar_roof = nar = None
    if not args.no_ar_baseline:
        # autoregressive baseline (course page, break-even solution): decoding
        # steps over the same prefix, one new token per request per step
        ar_tok = torch.zeros(B, dtype=torch.int32, device=dev)
        ar_am = torch.empty(B, dtype=torch.int32, device=dev)
        ar_cf = torch.empty(B, dtype=torch.float32, device=dev)
        kv.lens[:] = pass_lens
        nar = 16 if cap - int(kv.lens.max()) >= 20 else max(1, cap - int(kv.lens.max()) - 4)
        model.decode_step(kv, ar_tok, ar_am, ar_cf, ws)
        kv.lens[:] = pass_lens
        torch.cuda.synchronize()
        a0, a1 = ev_pair()
        a0.record()
        for _ in range(nar):
            model.decode_step(kv, ar_am, ar_am, ar_cf, ws)   # greedy: each step feeds its own output
        a1.record()
        torch.cuda.synchronize()
        ar_us = a0.elapsed_time(a1) / nar * 1e3
        kv.lens[:] = pass_lens
        ar_work = roofline.decode_step_work(cfg, B, list(pass_lens), [min(cfg.E, B * cfg.k)] * cfg.L)
        ar_roof = roofline.roof_time(ar_work.total_bytes, ar_work.total_flops, roofline.HBM_BYTES_PER_S,
                                     roofline.MFMA_PEAK["bf16"])

    passes_per_step = S * C
    if args.early_exit:   # the passes the timed steps actually ran
        passes_per_step = float(np.mean(passes_run[-args.steps * C:])) * C
    value = B * N * passes_per_step / (ms_step / 1e3)
    if dom_stage == "gateup":
        dom_work, _ = roofline.gateup_work(cfg, mean_touched, B * N * cfg.k)
        achieved = dom_work / (dom_us / 1e6)
        peak = roofline.HBM_BYTES_PER_S
        dom_obj = {"bound": "hbm", "achieved": achieved / 1e9, "peak": peak / 1e9, "unit": "GB/s"}
    else:
        dom_work = 2.0 * B * N * cfg.V * cfg.D
        achieved = dom_work / (dom_us / 1e6)
        peak = roofline.MFMA_PEAK["bf16"]
        dom_obj = {"bound": "mfma", "achieved": achieved / 1e12, "peak": peak / 1e12, "unit": "TFLOP/s"}
    dom_obj.update({"frac": achieved / peak, "traffic": _traffic(wl.name, dom_stage, dom_files),
                    "kernel": dom_kernel, "alg_work_per_launch": dom_work, "avg_launch_us": dom_us})
    work = roofline.denoise_pass_work(cfg, B, N, list(pass_lens), cov_layer)
    t_roof = roofline.roof_time(work.total_bytes, work.total_flops, roofline.HBM_BYTES_PER_S,
                                roofline.MFMA_PEAK["bf16"])

    out = {
        "metric": "canvas-token passes/sec (256-tok canvas MoE layer) + % HBM/MFMA roofline",
        "value": value,
        "unit": "canvas-token passes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.act,
        "data": "synthetic (seeded N(0,0.02) weights, uniform tokens)",
        "config": {"workload": wl.name, "B": B, "canvas": N, "prefix": P, "passes": S,
                   "canvases": C, "layers": cfg.L, "d_model": cfg.D, "experts": cfg.E,
                   "top_k": cfg.k, "expert_ffn": cfg.F, "vocab": cfg.V, "expert_dtype": cfg.expert,
                   "sampler": args.sampler, "early_exit": bool(args.early_exit),
                   "step": ("prompt prefill + " if chained else "") +
                           f"{C} x (init noise + {S} x (pass + coverage + re-noise, fused tail) + "
                           "append prefill)"},
        "roofline": dom_obj,
        "pass_roofline": {"pass_us": pass_us, "roof_us": t_roof * 1e6, "frac": t_roof * 1e6 / pass_us,
                          "alg_bytes": work.total_bytes, "alg_flops": work.total_flops,
                          "prefix_lens": [int(x) for x in pass_lens]},
        "pass_us_cold": float(np.median(cold)),
        "stage_us": stages,
        "experts_touched_per_pass": mean_touched,
        "experts_touched_per_layer": [float(x) for x in cov_layer],
    }
    if ar_us is not None:
        out["ar_baseline"] = {
            "step_us": ar_us, "tok_s": B / (ar_us / 1e6), "roof_us": ar_roof * 1e6,
            "frac": ar_roof * 1e6 / ar_us, "steps_timed": nar,
            "breakeven_passes": N * ar_us / pass_us,
            "breakeven_passes_at_roofline": N * ar_roof / t_roof,
            "note": "a canvas of N tokens in S passes beats N decoding steps iff S < N * step / pass"}
    if c3 is not None:
        out["request"] = c3

    if args.copy_probe:
        # counter calibration: a device copy of 4 GiB (16x the last-level
        # cache, so its reads come from HBM) with known read and write bytes
        n = 4 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        dst.fill_(2)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_probe_bytes"] = n
        del src, dst

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, w, prompt, canvas, B, N, P, cap)
    print(json.dumps(out), flush=True)


def cpu_baseline(wl, w, prompt, canvas, B, N, P, cap):
    """The oracle as it stands, on the host's cores: whole passes of the
    workload until about 10 s (at most 16), then on one core a pass over the
    first 32 canvas rows of one request (same prefix)."""
    import numpy as np

    import oracle
    from block_diffusion_lm_denoise_amd import synth

    cfg = wl.model
    cpu_w = synth.weights_to(w, "cpu")
    om = oracle.Model(cfg, cpu_w)
    ks, vs = om.new_cache(B, cap)
    ln = np.zeros(B, np.int32)
    om.kv_prefill(ks, vs, ln, prompt.cpu().numpy())
    cv = canvas.cpu().numpy()
    npass, t = 0, time.perf_counter()
    while npass < 16:
        om.denoise_pass(ks, vs, ln, cv)
        npass += 1
        if time.perf_counter() - t >= 10.0:
            break
    dt = time.perf_counter() - t
    om1 = oracle.Model(cfg, cpu_w, nthreads=1)
    n1 = min(32, N)
    t1 = time.perf_counter()
    om1.denoise_pass([k[:1] for k in ks], [v[:1] for v in vs], ln[:1], cv[:1, :n1])
    dt1 = time.perf_counter() - t1
    return {
        "value": npass * B * N / dt, "unit": "canvas-token passes/s", "cores": om.nthreads,
        "kind": "oracle", "cpu_model": _cpu_model(),
        "sample": f"{npass} full denoising passes ({B}x{N} canvas tokens, {P}-token prefix) of the "
                  f"fp64 CPU oracle on {om.nthreads} threads, {dt:.2f} s; its prefix prefill is not "
                  "timed",
        "one_core": {"value": n1 / dt1, "unit": "canvas-token passes/s",
                     "sample": f"one pass over {n1} canvas rows of one request ({P}-token prefix) on "
                               f"1 thread, {dt1:.2f} s"},
    }


if __name__ == "__main__":
    main()
