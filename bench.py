"""Benchmark of the block-diffusion denoising hot path on one MI355X.

Workload: one bf16 MoE layer (D 2048, 16 q / 8 kv heads x 128, 128 experts
top-8, expert FFN 768, vocabulary 32768), a 1024-token cached prefix and a
256-token canvas denoised in 8 passes.  One step is one whole canvas: noise
initialisation, 8 x (denoising pass, expert coverage, re-noise between
passes; the last two run inside the pass's final kernel), then the causal
append-prefill of the committed canvas; the cache
length is reset afterwards so every step sees the same 1024-token prefix.

Prints one JSON line:  value = canvas-token passes per second (B*N*S per
step), with the roofline of the dominant kernel (the gate/up grouped expert
GEMM, timed with HIP events on the compute stream) and the CPU oracle timed
on a bounded sample.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


GATEUP_KERNEL = "dg::wstream_k<bf16, bf16, 4, 4, 2, 4>"   # SG_GATEUP, 4 waves split K, 2 buffers, 64-row tiles


def _gateup_source_hash():
    """Hash of the sources the gate/up kernel is built from (the counter
    summary is only used if it was taken on this code)."""
    h = hashlib.sha256()
    for f in ("kern_stream.hip", "common.h", "launch.h"):
        with open(os.path.join(ROOT, "block_diffusion_lm_denoise_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(workload):
    """HBM bytes per gate/up launch from the committed rocprofv3 counter summary,
    if it was taken on this workload and the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"gateup_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("source_hash") != _gateup_source_hash() or not str(d.get("workload", "")).startswith(workload):
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the pass runs on a single MI355X (no multi-GPU path); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_diffusion_lm_denoise_amd import dgpass, roofline, synth
    from block_diffusion_lm_denoise_amd.configs import BENCH_WORKLOAD, WORKLOADS

    wl = WORKLOADS[args.workload or BENCH_WORKLOAD]
    cfg = wl.model
    dev = "cuda:0"
    torch.cuda.set_device(0)
    B, N, P, S = wl.B, wl.N, wl.P, wl.S
    w = synth.make_weights(cfg, wl.seed, device=dev)
    model = dgpass.Model(cfg, w)
    cap = P + N
    kv = model.kv_cache(B, cap, device=dev)
    ws = model.workspace(max(B * P, B * N), cap, device=dev)
    prompt = synth.tokens(cfg.V, (B, P), wl.seed, device=dev)
    model.kv_prefill(kv, prompt, ws)
    torch.cuda.synchronize()
    base_lens = kv.lens.copy()

    canvas = torch.empty(B, N, dtype=torch.int32, device=dev)
    argmax = torch.empty(B, N, dtype=torch.int32, device=dev)
    conf = torch.empty(B, N, dtype=torch.float32, device=dev)
    touched = torch.zeros(S, cfg.L, dtype=torch.int32, device=dev)

    def step(events=None):
        kv.lens[:] = base_lens
        pos0 = base_lens
        dgpass.renoise(canvas, None, None, wl.tau, wl.seed, 0, pos0, cfg.V)
        for p in range(S):
            # the gate/up launches of one mid-canvas pass of each timed step carry
            # the HIP events (an event record itself costs a few us of GPU time)
            ev = None if events is None or p != S // 2 else events[p]
            # coverage and the re-noise for the next pass run in the pass's last kernel
            nxt = dict(tau=wl.tau, seed=wl.seed, pass_tag=p + 1, pos0=pos0) if p < S - 1 else None
            model.denoise_pass_next(kv, canvas, argmax, conf, ws, touched=touched[p], renoise=nxt,
                                    events=ev)
        model.kv_prefill(kv, argmax, ws)   # append the committed canvas

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps; the gate/up expert launches of one pass per
    # step (pass S/2) are bracketed by HIP events recorded on the same stream
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(2 * cfg.L)] for _ in range(S)]
           for _ in range(args.steps)]
    for st in evs:          # torch creates the HIP event on its first record
        for e in st:
            for x in e:
                x.record()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(evs[i])
    t1.record()
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps
    gateup_ms = [st[S // 2][2 * l].elapsed_time(st[S // 2][2 * l + 1]) for st in evs for l in range(cfg.L)]
    gateup_avg_s = float(np.mean(gateup_ms)) / 1e3
    cov = touched.cpu().numpy()

    # pass-only timing (no append), for the per-pass figure
    for _ in range(3):
        model.denoise_pass(kv, canvas, argmax, conf, ws)
    torch.cuda.synchronize()
    p0 = torch.cuda.Event(enable_timing=True)
    p1 = torch.cuda.Event(enable_timing=True)
    npass = max(8, args.steps)
    p0.record()
    for _ in range(npass):
        model.denoise_pass(kv, canvas, argmax, conf, ws)
    p1.record()
    torch.cuda.synchronize()
    pass_us = p0.elapsed_time(p1) / npass * 1e3

    value = B * N * S / (ms_step / 1e3)
    mean_touched = float(cov.mean())
    gu_bytes, gu_flops = roofline.gateup_work(cfg, mean_touched, B * N * cfg.k)
    achieved = gu_bytes / gateup_avg_s
    traffic = _traffic(wl.name)
    work = roofline.denoise_pass_work(cfg, B, N, [P] * B, cov.mean(axis=0))
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
                   "layers": cfg.L, "d_model": cfg.D, "experts": cfg.E, "top_k": cfg.k,
                   "expert_ffn": cfg.F, "vocab": cfg.V, "expert_dtype": cfg.expert,
                   "step": "init noise + 8 x (pass + coverage + re-noise, fused tail) + append prefill"},
        "roofline": {"kernel": "moe gate/up grouped GEMM (" + GATEUP_KERNEL + ")", "bound": "hbm",
                     "achieved": achieved / 1e9, "peak": roofline.HBM_BYTES_PER_S / 1e9,
                     "unit": "GB/s", "frac": achieved / roofline.HBM_BYTES_PER_S,
                     "traffic": traffic, "alg_bytes_per_launch": gu_bytes,
                     "avg_launch_us": gateup_avg_s * 1e6},
        "pass_us": pass_us,
        "pass_roofline_us": t_roof * 1e6,
        "pass_roofline_frac": t_roof * 1e6 / pass_us,
        "experts_touched_per_pass": mean_touched,
    }

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
        import oracle
        cpu_w = synth.weights_to(w, "cpu")
        om = oracle.Model(cfg, cpu_w)
        ks, vs = om.new_cache(B, cap)
        ln = np.zeros(B, np.int32)
        om.kv_prefill(ks, vs, ln, prompt.cpu().numpy())
        cv = canvas.cpu().numpy()
        # a bounded sample: whole passes until about 10 s of CPU time (at most 16)
        npass_cpu, t = 0, time.perf_counter()
        while npass_cpu < 16:
            om.denoise_pass(ks, vs, ln, cv)
            npass_cpu += 1
            if time.perf_counter() - t >= 10.0:
                break
        dt = time.perf_counter() - t
        out["cpu_baseline"] = {
            "value": npass_cpu * B * N / dt, "unit": "canvas-token passes/s", "cores": om.nthreads,
            "kind": "oracle",
            "sample": f"{npass_cpu} full denoising passes ({B}x{N} canvas tokens, {P}-token prefix) of "
                      f"the fp64 CPU oracle, {dt:.2f} s; its prefix prefill is not timed"}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
