"""Denoising pass on the GPU (through the C ABI) against the CPU oracle."""
import numpy as np
import pytest
import torch

from block_diffusion_lm_denoise_amd import synth
from block_diffusion_lm_denoise_amd.configs import WORKLOADS, ModelConfig
from gpu_helpers import ALL_TAPS, DEV, Pair, compare_pass, host

pytestmark = pytest.mark.gpu


def _cfg(**kw):
    base = dict(L=1, D=256, Hq=4, Hkv=2, hd=128, E=16, k=4, F=128, V=640, act="bf16", expert="bf16")
    base.update(kw)
    return ModelConfig(**base)


def _run(pair, B, lens, N, seed, synthetic=False, inject=True, scale_note=""):
    """One pass on both sides.  Injected run: the GPU routes on the oracle's
    router logits, starts every layer from the oracle's layer input and feeds
    the oracle's final-norm rows to its LM head, so every stage is compared on
    inputs identical to the oracle's (argmax bar asserted).  Free run: the GPU
    computes everything itself (end-to-end drift reported)."""
    cap = max(lens) + N + 3
    oks, ovs, oln, kv = pair.caches(B, cap, lens, seed, synthetic=synthetic)
    if not synthetic:
        for l in range(pair.cfg.L):
            assert np.array_equal(oln, kv.lens)
            # prefilled caches agree within the storage tolerance
            from gpu_helpers import f64, max_rel, TOL
            for b in range(B):
                n = lens[b]
                if n:
                    assert max_rel(f64(host(kv.k[l][b, :, :n]), pair.cfg.act),
                                   f64(oks[l][b, :, :n], pair.cfg.act)) < TOL[pair.cfg.act]
                    assert max_rel(f64(host(kv.v[l][b, :, :n]), pair.cfg.act),
                                   f64(ovs[l][b, :, :n], pair.cfg.act)) < TOL[pair.cfg.act]
    canvas = synth.tokens(pair.cfg.V, (B, N), seed, "canvas").numpy()
    o = pair.om.denoise_pass(oks, ovs, oln, canvas, taps=ALL_TAPS)
    reps = {}
    if inject:
        g = pair.gpu_pass(kv, canvas, inject=o[2]["router"], inject_x=pair.layer_inputs(canvas, o[2]),
                          inject_uf=o[2]["uf"])
        reps["inject"] = compare_pass(pair.cfg, o, g[:3], True, "inject", head_injected=True)
    g = pair.gpu_pass(kv, canvas)
    reps["free"] = compare_pass(pair.cfg, o, g[:3], False, "free")
    # the pass never writes the cache
    if synthetic:
        for l in range(pair.cfg.L):
            np.testing.assert_array_equal(host(kv.k[l]), oks[l])
            np.testing.assert_array_equal(host(kv.v[l]), ovs[l])
    print(scale_note, reps, flush=True)
    return reps, g


def test_tiny_fp32_workload():
    wl = WORKLOADS["tiny_fp32"]
    pair = Pair(wl.model, wl.seed, gain="ones")
    _run(pair, 1, [wl.P], wl.N, wl.seed)


@pytest.mark.parametrize("act,hd,G", [("f32", 64, 1), ("f32", 128, 2), ("bf16", 128, 2), ("bf16", 64, 4)])
def test_small_layers_ragged_batch(act, hd, G):
    cfg = _cfg(L=2, act=act, expert=act, hd=hd, Hkv=8 // G, Hq=8)
    pair = Pair(cfg, 11, scale_lm=10.0)
    _run(pair, 3, [50, 0, 13], 37, 11)


def test_single_slot_canvas_and_empty_prefix():
    pair = Pair(_cfg(), 12)
    _run(pair, 1, [0], 1, 12)
    _run(pair, 2, [1, 0], 1, 13)


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_rows_longer_than_2048(act):
    # D 2560: the row kernels' loop over elements past the 2048 held in
    # registers (embedding, the RMSNorm folded into top-k, combine), with the
    # streamed projections at 40 (bf16) or 80 (fp32) pieces per weight row
    cfg = _cfg(L=2, D=2560, Hq=4, Hkv=2, hd=128, E=8, k=2, F=128, V=512, act=act, expert=act)
    # head scale 3: logits grow with sqrt(D), so this keeps the spread of the
    # D 256 tests' scale 10
    pair = Pair(cfg, 18, scale_lm=3.0)
    _run(pair, 2, [20, 7], 19, 18)


def test_fp8_experts_small():
    pair = Pair(_cfg(expert="fp8", L=2), 14, scale_lm=10.0)
    _run(pair, 2, [20, 9], 33, 14)


@pytest.mark.parametrize("act,expert", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "fp8")])
def test_many_rows_per_expert_uses_tiled_expert_path(act, expert):
    # 4 experts, top-2, 200 tokens: ~100 rows per expert (LDS-tiled grouped GEMM)
    cfg = _cfg(E=4, k=2, act=act, expert=expert, V=384)
    pair = Pair(cfg, 15)
    _run(pair, 2, [30, 5], 100, 15)


@pytest.mark.parametrize("expert,D,F", [("bf16", 384, 192), ("fp8", 384, 384)])
def test_tiled_expert_path_narrow_column_blocks(expert, D, F):
    # ~100 rows per expert take the LDS-tiled grouped GEMMs; D % 256 != 0 (and
    # for bf16 F % 128 != 0) selects their 128-column blocks, with 3 column
    # blocks and ragged 64-row expert tiles
    cfg = _cfg(E=4, k=2, expert=expert, V=384, D=D, F=F)
    pair = Pair(cfg, 17)
    _run(pair, 2, [30, 5], 100, 17)


def test_wide_lm_head_many_rows_ragged_vocab():
    """Over 1024 rows the bf16 LM head takes 512-column vocabulary tiles of
    64 columns per wave.  Five requests of 230 canvas tokens (1150 rows: the
    last 128-row tile holds 126) and a vocabulary of 1000 (a second tile of 488
    columns) reach its masked epilogue and its rows past the end; with the
    oracle's final-norm rows injected the argmax bar is asserted."""
    cfg = _cfg(V=1000)
    pair = Pair(cfg, 19, scale_lm=10.0)
    _run(pair, 5, [30, 5, 0, 12, 7], 230, 19)


def test_ragged_prefixes_with_key_splits_full_width():
    """Two requests at the 1024-prefix layer's width, one with a 2048-token
    prefix and one with none: the attention splits the keys four ways, so the
    second request's blocks of splits 1-3 have no keys at all (their staged
    slots must still read keys of that request; the host replay of the
    addresses is tests/test_attn_plan.py)."""
    wl = WORKLOADS["layer_p1024"]
    pair = Pair(wl.model, 31, gain="ones")
    _run(pair, 2, [2048, 0], wl.N, 31, synthetic=True, scale_note="ragged [2048, 0]")


@pytest.mark.parametrize("E,k,N", [(16, 4, 33), (4, 2, 100)])
def test_mxfp4_experts(E, k, N):
    """4-bit (MXFP4) expert weights decoded in registers by the streamed
    grouped GEMMs (few rows per expert, and ~100 rows per expert over several
    32-row tiles); ragged requests, two layers."""
    cfg = _cfg(L=2, E=E, k=k, D=256, F=256, expert="mxfp4", V=384)
    pair = Pair(cfg, 18, scale_lm=10.0)
    _run(pair, 2, [30, 5], N, 18, scale_note=f"mxfp4 E{E} k{k}")


def test_mxfp4_layer_prefix1024_full_size():
    """The 1024-prefix layer with MXFP4 experts at its full size (synthetic
    cache given to both sides)."""
    wl = WORKLOADS["layer_p1024_mxfp4"]
    pair = Pair(wl.model, wl.seed, gain="ones")
    _run(pair, 1, [wl.P], wl.N, wl.seed, synthetic=True, scale_note="layer_p1024_mxfp4")


def test_injected_router_ties_are_bit_exact():
    cfg = _cfg(E=8, k=3)
    pair = Pair(cfg, 16)
    N = 4
    oks, ovs, oln, kv = pair.caches(1, 8, [3], 16)
    inj = np.zeros((1, N, 8), np.float32)
    inj[0, 0] = [1, 2, 2, 0, 2, -1, 5, 0]
    inj[0, 1] = 0
    inj[0, 2] = [3, 1, 3, 1, 3, 9, 3, 1]
    inj[0, 3] = [-1, -1, -2, -1, 7, -1, 7, 7]
    canvas = synth.tokens(cfg.V, (1, N), 16, "canvas").numpy()
    g = pair.gpu_pass(kv, canvas, inject=inj)
    np.testing.assert_array_equal(g[2]["ids"][0], [[6, 1, 2], [0, 1, 2], [5, 0, 2], [4, 6, 7]])
    o = pair.om.denoise_pass(oks, ovs, oln, canvas, taps=ALL_TAPS, inject_router=inj)
    compare_pass(cfg, o, g[:3], True, "ties")


def test_moe_layer_prefix1024_full_size():
    """One bf16 MoE layer, 1024-token prefix prefilled on both sides, 256-token canvas."""
    wl = WORKLOADS["layer_p1024"]
    pair = Pair(wl.model, wl.seed, gain="ones")
    reps, g = _run(pair, 1, [wl.P], wl.N, wl.seed, scale_note="layer_p1024")
    # expert coverage of the pass (union of the selected experts)
    touched = torch.zeros(1, dtype=torch.int32, device=DEV)
    pair.gm.expert_coverage(g[3], touched)
    assert int(touched.item()) == int((g[2]["counts"][0] > 0).sum())
    assert int(touched.item()) >= 96   # most of the 128 experts are touched by one pass


def test_moe_layer_prefix8192_full_size_synthetic_cache():
    wl = WORKLOADS["layer_p8192"]
    pair = Pair(wl.model, wl.seed, gain="ones")
    _run(pair, 1, [wl.P], wl.N, wl.seed, synthetic=True, inject=False, scale_note="layer_p8192")


def test_batch8_fp8_full_size_all_requests():
    """Eight requests with fp8 experts in one pass at the full size (2048
    canvas rows: the fused routing kernel and the LDS-tiled fp8 grouped GEMMs
    at ~128 rows per expert).  The oracle computes the same batch (block
    diagonal); with its router logits injected every tap of all eight
    requests is compared, and the head reads the oracle's final-norm rows."""
    wl = WORKLOADS["batch8_fp8"]
    cfg = wl.model
    pair = Pair(cfg, wl.seed, gain="ones")
    B, N, P = wl.B, wl.N, wl.P
    cap = P + N
    ks, vs = synth.kv_cache_values(cfg, B, cap, P, wl.seed)
    kv = pair.gm.kv_cache(B, cap, device=DEV)
    for l in range(cfg.L):
        kv.k[l].copy_(ks[l])
        kv.v[l].copy_(vs[l])
    kv.lens[:] = P
    canvas = synth.tokens(cfg.V, (B, N), wl.seed, "canvas").numpy()
    oks, ovs = [host(k) for k in ks], [host(v) for v in vs]
    o = pair.om.denoise_pass(oks, ovs, np.full(B, P, np.int32), canvas, taps=ALL_TAPS)
    g = pair.gpu_pass(kv, canvas, inject=o[2]["router"], inject_uf=o[2]["uf"])
    rep = compare_pass(cfg, o, g[:3], True, "batch8_fp8 inject", head_injected=True)
    print("batch8_fp8 injected", rep, flush=True)
    touched = torch.zeros(1, dtype=torch.int32, device=DEV)
    pair.gm.expert_coverage(g[3], touched)
    assert int(touched.item()) == int((g[2]["counts"][0] > 0).sum()) >= 120
    # free routing over the same batch: the GPU's own router logits and routing
    gf = pair.gpu_pass(kv, canvas)
    rep = compare_pass(cfg, o, gf[:3], False, "batch8_fp8 free")
    print("batch8_fp8 free", rep, flush=True)


def test_pass_is_deterministic_and_reads_cache_only():
    wl = WORKLOADS["layer_p1024"]
    cfg = wl.model
    w = synth.make_weights(cfg, 5, device=DEV)
    from block_diffusion_lm_denoise_amd import dgpass
    gm = dgpass.Model(cfg, w)
    kv = gm.kv_cache(1, 1280, device=DEV)
    ws = gm.workspace(1024, 1280, device=DEV)
    gm.kv_prefill(kv, synth.tokens(cfg.V, (1, 1024), 5, device=DEV), ws)
    k0, v0 = kv.k[0].clone(), kv.v[0].clone()
    canvas = synth.tokens(cfg.V, (1, 256), 5, "canvas", device=DEV)
    outs = []
    for _ in range(2):
        am = torch.empty(1, 256, dtype=torch.int32, device=DEV)
        cf = torch.empty(1, 256, dtype=torch.float32, device=DEV)
        gm.denoise_pass(kv, canvas, am, cf, ws)
        outs.append((am, cf))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(kv.k[0], k0) and torch.equal(kv.v[0], v0)
