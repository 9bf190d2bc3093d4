"""Causal prefill on the GPU against the oracle: cache contents, ragged
lengths, chaining, capacity errors."""
import numpy as np
import pytest
import torch

from block_diffusion_lm_denoise_amd import dgpass, synth
from block_diffusion_lm_denoise_amd.configs import ModelConfig
from gpu_helpers import DEV, TOL, Pair, f64, host, max_rel

pytestmark = pytest.mark.gpu


def _cfg(**kw):
    base = dict(L=3, D=256, Hq=4, Hkv=2, hd=64, E=8, k=2, F=128, V=512, act="bf16", expert="bf16")
    base.update(kw)
    return ModelConfig(**base)


def _compare_caches(cfg, kv, oks, ovs, lens, label):
    out = []
    for l in range(cfg.L):
        for b in range(kv.B):
            n = int(lens[b])
            a = f64(host(kv.k[l][b, :, :n]), cfg.act)
            o = f64(oks[l][b, :, :n], cfg.act)
            out.append(max_rel(a, o))
            assert out[-1] < TOL[cfg.act], (label, l, b, "k", out[-1])
            a = f64(host(kv.v[l][b, :, :n]), cfg.act)
            o = f64(ovs[l][b, :, :n], cfg.act)
            out.append(max_rel(a, o))
            assert out[-1] < TOL[cfg.act], (label, l, b, "v", out[-1])
    return max(out)


@pytest.mark.parametrize("act,T1,T2", [("f32", 37, 29), ("bf16", 64, 1), ("bf16", 130, 70)])
def test_prefill_matches_oracle_and_chains(act, T1, T2):
    cfg = _cfg(act=act, expert=act)
    pair = Pair(cfg, 21)
    B, cap = 2, T1 + T2 + 5
    a = synth.tokens(cfg.V, (B, T1), 21, "a")
    b = synth.tokens(cfg.V, (B, T2), 21, "b")
    oks, ovs = pair.om.new_cache(B, cap)
    oln = np.zeros(B, np.int32)
    ra = pair.om.kv_prefill(oks, ovs, oln, a.numpy(), taps=("router",))["router"]
    rb = pair.om.kv_prefill(oks, ovs, oln, b.numpy(), taps=("router",))["router"]
    # the GPU routes on the oracle's logits: a near-tie flip in an early layer
    # would change that token's later K/V entirely (checked separately below)
    kv = pair.gm.kv_cache(B, cap, device=DEV)
    ws = pair.gm.workspace(B * max(T1, T2), cap, device=DEV)
    pair.gm.kv_prefill(kv, a.to(DEV), ws, inject_router=torch.from_numpy(ra).to(DEV))
    pair.gm.kv_prefill(kv, b.to(DEV), ws, inject_router=torch.from_numpy(rb).to(DEV))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kv.lens, oln)
    print(act, T1, T2, "cache max-rel", _compare_caches(cfg, kv, oks, ovs, oln, "chained"))
    # one prefill of the concatenation gives the same cache (within rounding)
    kv2 = pair.gm.kv_cache(B, cap, device=DEV)
    ws2 = pair.gm.workspace(B * (T1 + T2), cap, device=DEV)
    rab = np.concatenate([ra.reshape(cfg.L, B, T1, cfg.E), rb.reshape(cfg.L, B, T2, cfg.E)], 2)
    pair.gm.kv_prefill(kv2, torch.cat([a, b], 1).to(DEV), ws2,
                       inject_router=torch.from_numpy(np.ascontiguousarray(rab)).to(DEV))
    torch.cuda.synchronize()
    _compare_caches(cfg, kv2, oks, ovs, oln, "joint")
    # free routing: the GPU's own router logits agree with the oracle's and
    # routing differs only at near-ties
    kv3 = pair.gm.kv_cache(B, cap, device=DEV)
    tp = dgpass.make_taps(cfg, B * T1, ("router", "ids"), device=DEV)
    pair.gm.kv_prefill(kv3, a.to(DEV), ws, taps=tp)
    oks3, ovs3 = pair.om.new_cache(B, cap)
    ot = pair.om.kv_prefill(oks3, ovs3, np.zeros(B, np.int32), a.numpy(), taps=("router", "ids"))
    torch.cuda.synchronize()
    from gpu_helpers import kth_gap
    gids, oids = host(tp["ids"])[0], ot["ids"][0]
    gap = kth_gap(ot["router"][0], cfg.k)
    flips = int(((gap > 1e-2) & np.any(np.sort(gids, -1) != np.sort(oids, -1), -1)).sum())
    print(act, "first-layer routing flips at k-th gaps > 1e-2:", flips)
    if act == "f32":
        assert flips == 0
    assert max_rel(host(tp["router"])[0], ot["router"][0]) < TOL[act]


def test_prefill_ragged_request_lengths():
    cfg = _cfg(L=2)
    pair = Pair(cfg, 22)
    cap = 90
    # request 0 already holds 40 tokens, request 1 holds 3
    pre = [synth.tokens(cfg.V, (1, n), 22, f"pre{b}") for b, n in enumerate((40, 3))]
    oks, ovs = pair.om.new_cache(2, cap)
    kv = pair.gm.kv_cache(2, cap, device=DEV)
    ws = pair.gm.workspace(2 * 40, cap, device=DEV)
    for b in range(2):
        kb = [k[b:b + 1].copy() for k in oks]
        vb = [v[b:b + 1].copy() for v in ovs]
        l1 = np.zeros(1, np.int32)
        pair.om.kv_prefill(kb, vb, l1, pre[b].numpy())
        for l in range(cfg.L):
            oks[l][b], ovs[l][b] = kb[l][0], vb[l][0]
        sub = dgpass.KVCache(cfg, 1, cap, device=DEV, k=[k[b:b + 1] for k in kv.k], v=[v[b:b + 1] for v in kv.v])
        pair.gm.kv_prefill(sub, pre[b].to(DEV), ws)
        kv.lens[b] = sub.lens[0]
    oln = np.array([40, 3], np.int32)
    nxt = synth.tokens(cfg.V, (2, 33), 22, "next")
    pair.om.kv_prefill(oks, ovs, oln, nxt.numpy())
    pair.gm.kv_prefill(kv, nxt.to(DEV), ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kv.lens, [73, 36])
    _compare_caches(cfg, kv, oks, ovs, oln, "ragged")


def test_prefill_capacity_error_changes_nothing():
    cfg = _cfg(L=1)
    pair = Pair(cfg, 23)
    kv = pair.gm.kv_cache(1, 10, device=DEV)
    ws = pair.gm.workspace(16, 10, device=DEV)
    pair.gm.kv_prefill(kv, synth.tokens(cfg.V, (1, 8), 23).to(DEV), ws)
    k0 = kv.k[0].clone()
    with pytest.raises(dgpass.DgError) as e:
        pair.gm.kv_prefill(kv, synth.tokens(cfg.V, (1, 3), 24).to(DEV), ws)
    assert e.value.status == -2
    torch.cuda.synchronize()
    assert kv.lens[0] == 8 and torch.equal(kv.k[0], k0)


@pytest.mark.parametrize("act,expert", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "fp8")])
def test_large_prefill_uses_tiled_dense_gemm(act, expert):
    # 3 x 400 = 1200 rows: above the weight-streaming row limit, so the dense
    # projections take the LDS-tiled GEMM, and ~300 rows per expert the tiled
    # grouped expert GEMMs; a ragged 1200 = 9 x 128 + 48 row tail
    cfg = _cfg(L=2, act=act, expert=expert)
    pair = Pair(cfg, 25)
    B, T = 3, 400
    toks = synth.tokens(cfg.V, (B, T), 25, "big")
    oks, ovs = pair.om.new_cache(B, T)
    oln = np.zeros(B, np.int32)
    ro = pair.om.kv_prefill(oks, ovs, oln, toks.numpy(), taps=("router",))["router"]
    kv = pair.gm.kv_cache(B, T, device=DEV)
    ws = pair.gm.workspace(B * T, T, device=DEV)
    pair.gm.kv_prefill(kv, toks.to(DEV), ws, inject_router=torch.from_numpy(ro).to(DEV))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kv.lens, oln)
    print(act, expert, "cache max-rel", _compare_caches(cfg, kv, oks, ovs, oln, "large"))


def test_prefill_ragged_lengths_with_key_splits_full_width():
    """Append 256 tokens to two requests holding 2048 and 0 keys at the
    1024-prefix layer's width (two layers): the causal attention splits the
    keys, and the short request's late splits are empty.  Routing on the
    oracle's logits; caches compared with the oracle."""
    from block_diffusion_lm_denoise_amd.configs import WORKLOADS, scaled
    wl = scaled(WORKLOADS["layer_p1024"], L=2)
    cfg = wl.model
    pair = Pair(cfg, 32)
    cap, T = 2048 + 256, 256
    ks, vs = synth.kv_cache_values(cfg, 2, cap, 2048, 32)
    for l in range(cfg.L):
        ks[l][1] = 0
        vs[l][1] = 0
    kv = pair.gm.kv_cache(2, cap, device=DEV)
    for l in range(cfg.L):
        kv.k[l].copy_(ks[l])
        kv.v[l].copy_(vs[l])
    kv.lens[:] = [2048, 0]
    oks, ovs = [host(k) for k in ks], [host(v) for v in vs]
    oln = np.array([2048, 0], np.int32)
    toks = synth.tokens(cfg.V, (2, T), 32, "append")
    ro = pair.om.kv_prefill(oks, ovs, oln, toks.numpy(), taps=("router",))["router"]
    ws = pair.gm.workspace(2 * T, cap, device=DEV)
    pair.gm.kv_prefill(kv, toks.to(DEV), ws, inject_router=torch.from_numpy(ro).to(DEV))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kv.lens, oln)
    print("ragged split prefill cache max-rel", _compare_caches(cfg, kv, oks, ovs, oln, "ragged-split"))
