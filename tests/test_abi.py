"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, sizes workspaces, and rejects bad arguments before any launch."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from block_diffusion_lm_denoise_amd import dgpass
from block_diffusion_lm_denoise_amd.configs import WORKLOADS, ModelConfig

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]

pytestmark = pytest.mark.skipif(not os.path.exists(dgpass.LIB_PATH),
                                reason="libdgpass.so not built (run __graft_entry__.build())")


def _declared():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(dg_\w+)\s*\(", src, flags=re.M))
    return sorted(names)


def test_header_declares_the_boundary():
    names = _declared()
    assert set(names) == set(dgpass.EXPORTS), names


def test_library_exports_every_declared_symbol():
    L = dgpass.lib()
    for n in _declared():
        assert hasattr(L, n), n


def test_status_strings():
    L = dgpass.lib()
    for st, msg in dgpass.STATUS.items():
        assert L.dg_status_str(st).decode() == msg


def _cfg(**kw):
    base = dict(L=2, D=256, Hq=4, Hkv=2, hd=64, E=8, k=2, F=128, V=512, act="bf16", expert="bf16")
    base.update(kw)
    return ModelConfig(**base)


def test_workspace_bytes_grows_with_rows_and_rejects_bad_config():
    c = _cfg()
    a = dgpass.workspace_bytes(c, 16)
    b = dgpass.workspace_bytes(c, 256)
    assert 0 < a < b
    assert dgpass.workspace_bytes(c, 0) == 0
    bad = dgpass.make_config(c)
    bad.L = 0
    assert dgpass.lib().dg_workspace_bytes(C.byref(bad), 16, 0) == 0
    wl = WORKLOADS["layer_p1024"]
    assert dgpass.workspace_bytes(wl.model, 256) < 64 << 20


def _fake_weights(cfg, escale=False):
    w = dgpass.dg_weights()
    w.emb = w.gf = w.lm = 0x1000
    for l in range(cfg.L):
        L = w.layers[l]
        for n in ("g1", "wq", "wk", "wv", "wo", "g2", "wr", "wg", "wu", "wd"):
            setattr(L, n, 0x2000)
        L.escale = 0x3000 if escale else None
    return w


def _init(cfg, w):
    m = dgpass.dg_model()
    c = dgpass.make_config(cfg)
    return dgpass.lib().dg_model_init(C.byref(m), C.byref(c), C.byref(w)), m


def test_model_init_validation():
    c = _cfg()
    st, _ = _init(c, _fake_weights(c))
    assert st == 0
    w = _fake_weights(c)
    w.layers[1].wd = None
    assert _init(c, w)[0] == -1
    assert _init(_cfg(expert="fp8"), _fake_weights(c))[0] == -1          # fp8 needs scales
    assert _init(_cfg(expert="fp8"), _fake_weights(c, escale=True))[0] == 0
    assert _init(_cfg(act="f32", expert="bf16"), _fake_weights(c))[0] == -3
    assert _init(_cfg(hd=96), _fake_weights(c))[0] == -3
    assert _init(_cfg(k=9, E=16), _fake_weights(c))[0] == -3
    assert _init(_cfg(D=192), _fake_weights(c))[0] == -3


def test_calls_reject_bad_arguments_before_launching():
    c = _cfg()
    st, m = _init(c, _fake_weights(c))
    assert st == 0
    L = dgpass.lib()
    lens = np.array([5, 7], np.int32)
    kv = dgpass.dg_kv()
    for l in range(c.L):
        kv.k[l] = kv.v[l] = 0x4000
    kv.cap = 8
    kv.len = lens.ctypes.data_as(C.POINTER(C.c_int32))
    need = dgpass.workspace_bytes(c, 2 * 4)
    dev = C.c_void_p(0x5000)
    # prefill that would overflow the cache: CAPACITY, and len untouched
    assert L.dg_kv_prefill(C.byref(m), C.byref(kv), dev, 2, 4, None, dev, need, None) == -2
    assert list(lens) == [5, 7]
    # too small a workspace
    assert L.dg_kv_prefill(C.byref(m), C.byref(kv), dev, 2, 1, None, dev, 16, None) == -4
    assert L.dg_denoise_pass(C.byref(m), C.byref(kv), dev, 2, 4, dev, dev, None, dev, 16, None) == -4
    # bad shapes / null pointers
    assert L.dg_denoise_pass(C.byref(m), C.byref(kv), dev, 0, 4, dev, dev, None, dev, need, None) == -1
    assert L.dg_denoise_pass(C.byref(m), C.byref(kv), dev, 65, 4, dev, dev, None, dev, need, None) == -1
    assert L.dg_denoise_pass(C.byref(m), C.byref(kv), None, 2, 4, dev, dev, None, dev, need, None) == -1
    assert L.dg_denoise_pass(None, C.byref(kv), dev, 2, 4, dev, dev, None, dev, need, None) == -1
    bogus = dgpass.dg_model()   # never initialised
    assert L.dg_denoise_pass(C.byref(bogus), C.byref(kv), dev, 2, 4, dev, dev, None, dev, need, None) == -1
    pos0 = np.zeros(2, np.int32)
    p0 = pos0.ctypes.data_as(C.c_void_p)
    assert L.dg_renoise(dev, None, dev, 0.5, 1, 0, p0, None, 2, 4, 512, None) == -1  # conf w/o argmax
    assert L.dg_renoise(dev, None, None, 0.5, 1, 0, None, None, 2, 4, 512, None) == -1
    assert L.dg_renoise(dev, None, None, 0.5, 1, 0, p0, None, 65, 4, 512, None) == -1
    assert L.dg_expert_coverage(C.byref(m), dev, 4, dev, None, None) == -4
    assert L.dg_expert_coverage(C.byref(m), dev, 1 << 20, None, None, None) == -1
    # the pass with the between-pass work: same checks as the pass, plus its
    # re-noise arguments
    nxt = dgpass.dg_renoise_args(0.5, 1, 1, p0, None)
    d2, d3 = C.c_void_p(0x6000), C.c_void_p(0x7000)
    args = lambda cv, am, nx, wsb: (C.byref(m), C.byref(kv), cv, 2, 4, am, d3, dev, nx, None, dev, wsb,
                                    None)
    assert L.dg_denoise_pass_next(*args(dev, d2, C.byref(nxt), 16)) == -4
    assert L.dg_denoise_pass_next(*args(dev, d2, None, 16)) == -4
    assert L.dg_denoise_pass_next(*args(dev, dev, C.byref(nxt), need)) == -1   # canvas is argmax
    assert L.dg_denoise_pass_next(*args(d3, d2, C.byref(nxt), need)) == -1     # canvas is conf
    assert L.dg_denoise_pass_next(*args(None, d2, C.byref(nxt), need)) == -1
    no_pos = dgpass.dg_renoise_args(0.5, 1, 1, None, None)
    assert L.dg_denoise_pass_next(*args(dev, d2, C.byref(no_pos), need)) == -1
    neg = np.array([0, -1], np.int32)
    bad_pos = dgpass.dg_renoise_args(0.5, 1, 1, neg.ctypes.data_as(C.c_void_p), None)
    assert L.dg_denoise_pass_next(*args(dev, d2, C.byref(bad_pos), need)) == -1


def test_packed_bytes_pads_rows_and_requires_128_byte_rows():
    L = dgpass.lib()
    F32, BF16, FP8 = 0, 1, 2
    assert L.dg_packed_bytes(32, 64, BF16) == 32 * 128
    assert L.dg_packed_bytes(8, 64, BF16) == 16 * 128           # rows padded to 16
    assert L.dg_packed_bytes(17, 2048, BF16) == 32 * 4096
    assert L.dg_packed_bytes(16, 128, FP8) == 16 * 128
    assert L.dg_packed_bytes(16, 32, F32) == 16 * 128
    assert L.dg_packed_bytes(16, 96, BF16) == 0                 # 192-byte rows
    assert L.dg_packed_bytes(16, 64, FP8) == 0                  # 64-byte rows
    assert L.dg_packed_bytes(0, 64, BF16) == 0
    assert L.dg_packed_bytes(16, 64, 7) == 0


def test_pack_weight_rejects_bad_arguments_before_launch():
    L = dgpass.lib()
    a = C.c_void_p(0x1000)
    b = C.c_void_p(0x2000)
    assert L.dg_pack_weight(None, b, 16, 64, 1, None) == -1
    assert L.dg_pack_weight(a, None, 16, 64, 1, None) == -1
    assert L.dg_pack_weight(a, a, 16, 64, 1, None) == -1
    assert L.dg_pack_weight(a, b, 16, 96, 1, None) == -1
    assert L.dg_pack_weight(a, b, 0, 64, 1, None) == -1
