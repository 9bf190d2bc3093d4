"""Roofline calculator pinned to the values the course page "Module 12.
Diffusion Language Models" prints in its break-even and dense-8B exercises."""
import os

import pytest

from block_diffusion_lm_denoise_amd import roofline as R
from block_diffusion_lm_denoise_amd.configs import WORKLOADS

GOLD = os.path.join(os.path.dirname(__file__), "golden", "roofline_worked_example.txt")


def _gold():
    out = {}
    for line in open(GOLD):
        if line.startswith("#") or "=" not in line:
            continue
        k, v = line.split("=")
        out[k.strip()] = float(v)
    return out


def test_dense_8b_worked_example():
    g = _gold()
    bw, pk, n = g["hbm_bytes_per_s"], g["peak_flops"], g["params"]
    assert n * g["bytes_bf16"] == g["weights_bf16_bytes"]
    assert n * g["bytes_4bit"] == g["weights_4bit_bytes"]
    assert R.dense_weight_read_time(n, g["bytes_bf16"], bw) == pytest.approx(g["read_bf16_s"], abs=5e-7)
    assert R.dense_weight_read_time(n, g["bytes_4bit"], bw) == pytest.approx(g["read_4bit_s"], abs=5e-7)
    # 256-position pass: the arithmetic floor, and which floor binds
    assert 2 * n * 256 / pk == pytest.approx(g["canvas256_flop_floor_s"], abs=5e-7)
    assert R.dense_pass_time(n, g["bytes_bf16"], 256, bw, pk) == pytest.approx(g["read_bf16_s"], abs=5e-7)
    assert R.dense_pass_time(n, g["bytes_4bit"], 256, bw, pk) == pytest.approx(
        g["canvas256_flop_floor_s"], abs=5e-7)


def test_breakeven_worked_example():
    g = _gold()
    bw, pk, n = g["hbm_bytes_per_s"], g["peak_flops"], g["params"]
    ar = R.dense_weight_read_time(n, g["bytes_bf16"], bw)
    assert ar == pytest.approx(g["ar_step_s"], rel=1e-7)
    assert R.ar_ceiling_tok_s(ar) == pytest.approx(g["ar_ceiling_tok_s"], rel=1e-9)
    p1024 = R.dense_pass_time(n, g["bytes_bf16"], 1024, bw, pk)
    assert p1024 == pytest.approx(g["canvas1024_pass_s"], rel=1e-7)
    s = R.breakeven_passes(1024, p1024, ar)
    assert s == pytest.approx(g["breakeven_passes"], abs=5e-3)
    assert int(s) == g["breakeven_largest_integer"]
    assert R.diffusion_rate_tok_s(1024, 295, p1024) > R.ar_ceiling_tok_s(ar)
    assert R.diffusion_rate_tok_s(1024, 296, p1024) < R.ar_ceiling_tok_s(ar)
    # break-even equals the machine balance for a compute-bound dense canvas
    assert s == pytest.approx(pk / bw / g["bytes_bf16"] * 2, rel=1e-6)


def test_moe_layer_pass_work_is_expert_dominated():
    wl = WORKLOADS["layer_p1024"]
    work = R.denoise_pass_work(wl.model, wl.B, wl.N, [wl.P], [128])
    assert work.bytes["experts"] == 128 * 3 * 2048 * 768 * 2
    assert 0.85 < work.bytes["experts"] / work.total_bytes < 0.9
    t = R.roof_time(work.total_bytes, work.total_flops, R.HBM_BYTES_PER_S, R.MFMA_PEAK["bf16"])
    assert t == pytest.approx(work.total_bytes / R.HBM_BYTES_PER_S)
    assert 165e-6 < t < 180e-6


def test_decode_step_work_is_a_one_slot_canvas_pass():
    """One autoregressive step of a token over prefix P does the work of a
    denoising pass over a one-slot canvas (its query sees the prefix and
    itself); both read the touched experts, the attention weights and the
    head once."""
    cfg = WORKLOADS["layer_p1024"].model
    for P, touched in ((1024, 8), (0, 8), (4096, 3)):
        a = R.decode_step_work(cfg, 1, [P], [touched])
        b = R.denoise_pass_work(cfg, 1, 1, [P], [touched])
        assert a.total_bytes == b.total_bytes
        assert a.total_flops == b.total_flops
    # weights dominate the step: at the 1024 prefix it reads ~0.24 GB
    w = R.decode_step_work(cfg, 1, [1024], [8])
    assert 0.2e9 < w.total_bytes < 0.3e9
