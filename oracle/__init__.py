"""ctypes front end of the CPU oracle.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark; the product path never imports it.

Arrays cross as numpy views of torch CPU tensors: bf16 as uint16 bit
patterns, fp8 e4m3 as uint8 codes, int32 ids, fp32.
"""
import ctypes as C
import os

import numpy as np
import torch

from .build import LIB, build

OR_F32, OR_BF16, OR_FP8, OR_MXFP4 = 0, 1, 2, 3
_DT = {"f32": OR_F32, "bf16": OR_BF16, "fp8": OR_FP8, "mxfp4": OR_MXFP4}
_NP = {OR_F32: np.float32, OR_BF16: np.uint16}


class _Config(C.Structure):
    _fields_ = [(n, C.c_int) for n in ("L", "D", "Hq", "Hkv", "hd", "E", "k", "F", "V")] + [
        ("eps", C.c_double), ("act_dt", C.c_int), ("exp_dt", C.c_int)]


class _Layer(C.Structure):
    _fields_ = [("g1", C.c_void_p), ("wq", C.c_void_p), ("wk", C.c_void_p), ("wv", C.c_void_p),
                ("wo", C.c_void_p), ("g2", C.c_void_p), ("wr", C.c_void_p), ("wg", C.c_void_p),
                ("wu", C.c_void_p), ("wd", C.c_void_p), ("escale", C.c_void_p),
                ("wg_mx", C.c_void_p), ("wu_mx", C.c_void_p), ("wd_mx", C.c_void_p)]


class _Weights(C.Structure):
    _fields_ = [("emb", C.c_void_p), ("layers", C.POINTER(_Layer)), ("gf", C.c_void_p),
                ("lm", C.c_void_p)]


_TAP_FIELDS = ("qkv", "attn", "x1", "u2", "router", "ids", "gates", "counts", "offsets", "perm",
               "hmid", "yexp", "xout", "uf", "logits", "inject_router")


class _Taps(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in _TAP_FIELDS]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = C.CDLL(LIB)
        vp, i32 = C.c_void_p, C.c_int
        L.or_kv_prefill.argtypes = [vp, vp, vp, vp, i32, vp, vp, i32, i32, vp, i32]
        L.or_denoise_pass.argtypes = [vp, vp, vp, vp, i32, vp, vp, i32, i32, vp, vp, vp, i32]
        L.or_renoise.argtypes = [vp, vp, vp, C.c_float, C.c_uint64, C.c_uint32, vp, vp, i32, i32, i32]
        L.or_unmask.argtypes = [vp, vp, vp, C.c_float, C.c_int32, i32, i32, i32, vp, vp]
        L.or_philox4x64_10.argtypes = [vp, vp, vp]
        L.or_round_to.argtypes = [i32, C.c_double]
        L.or_round_to.restype = C.c_double
        L.or_fp8e4m3_decode.argtypes = [C.c_uint8]
        L.or_fp8e4m3_decode.restype = C.c_double
        L.or_fp4e2m1_decode.argtypes = [C.c_uint8]
        L.or_fp4e2m1_decode.restype = C.c_double
        L.or_e8m0_decode.argtypes = [C.c_uint8]
        L.or_e8m0_decode.restype = C.c_double
        L.or_bf16_bits.argtypes = [C.c_double]
        L.or_bf16_bits.restype = C.c_uint16
        _lib = L
    return _lib


def _np(t):
    """numpy view (bit pattern for bf16 / fp8) of a CPU tensor, kept contiguous."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def nthreads_default():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


class Model:
    """Oracle view of a model: config + weights (torch CPU tensors from synth)."""

    def __init__(self, cfg, weights, nthreads=None):
        self.cfg = cfg
        self.nthreads = nthreads or nthreads_default()
        self._keep = []
        self.c = _Config(cfg.L, cfg.D, cfg.Hq, cfg.Hkv, cfg.hd, cfg.E, cfg.k, cfg.F, cfg.V,
                         float(cfg.eps), _DT[cfg.act], _DT[cfg.expert])
        layers = (_Layer * cfg.L)()
        for l, lw in enumerate(weights["layers"]):
            arrs = {}
            for n in ("g1", "wq", "wk", "wv", "wo", "g2", "wr", "wg", "wu", "wd", "escale", "wg_mx",
                      "wu_mx", "wd_mx"):
                a = _np(lw.get(n))
                arrs[n] = a
                self._keep.append(a)
            for n, a in arrs.items():
                setattr(layers[l], n, None if a is None else a.ctypes.data)
        self._layers = layers
        top = {n: _np(weights[n]) for n in ("emb", "gf", "lm")}
        self._keep += list(top.values())
        self.w = _Weights(top["emb"].ctypes.data, layers, top["gf"].ctypes.data, top["lm"].ctypes.data)

    @property
    def act_np(self):
        return _NP[_DT[self.cfg.act]]

    def new_cache(self, B, cap):
        c = self.cfg
        ks = [np.zeros((B, c.Hkv, cap, c.hd), dtype=self.act_np) for _ in range(c.L)]
        vs = [np.zeros((B, c.Hkv, cap, c.hd), dtype=self.act_np) for _ in range(c.L)]
        return ks, vs

    @staticmethod
    def _ptr_array(arrs):
        a = (C.c_void_p * len(arrs))(*[x.ctypes.data for x in arrs])
        return a

    def kv_prefill(self, ks, vs, lens, tokens, taps=()):
        """Append tokens [B, T] to caches ks/vs (numpy, modified in place); lens (np.int32)
        advanced in place.  Returns the requested taps (rows = B*T)."""
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        B, T = tokens.shape
        cap = ks[0].shape[2]
        tp, out = self._taps(B * T, taps, None)
        rc = lib().or_kv_prefill(C.byref(self.c), C.byref(self.w), self._ptr_array(ks),
                                 self._ptr_array(vs), cap, _ptr(lens), _ptr(tokens), B, T,
                                 C.byref(tp), self.nthreads)
        if rc != 0:
            raise ValueError(f"or_kv_prefill failed: {rc}")
        return out

    def _taps(self, BN, taps, inject_router):
        c = self.cfg
        act = self.act_np
        shapes = {
            "qkv": ((c.L, BN, c.qkv_dim), act), "attn": ((c.L, BN, c.Hq * c.hd), act),
            "x1": ((c.L, BN, c.D), act), "u2": ((c.L, BN, c.D), act),
            "router": ((c.L, BN, c.E), np.float32), "ids": ((c.L, BN, c.k), np.int32),
            "gates": ((c.L, BN, c.k), np.float32), "counts": ((c.L, c.E), np.int32),
            "offsets": ((c.L, c.E + 1), np.int32), "perm": ((c.L, BN * c.k), np.int32),
            "hmid": ((c.L, BN, c.k, c.F), act), "yexp": ((c.L, BN, c.k, c.D), act),
            "xout": ((c.L, BN, c.D), act), "uf": ((BN, c.D), act), "logits": ((BN, c.V), np.float32),
        }
        out = {}
        tp = _Taps()
        for n in taps:
            shp, dt = shapes[n]
            out[n] = np.zeros(shp, dtype=dt)
            setattr(tp, n, out[n].ctypes.data)
        if inject_router is not None:
            inj = np.ascontiguousarray(inject_router, dtype=np.float32).reshape(c.L, BN, c.E)
            out["_inject"] = inj
            tp.inject_router = inj.ctypes.data
        return tp, out

    def denoise_pass(self, ks, vs, lens, canvas, taps=(), inject_router=None):
        """One pass over canvas [B, N].  Returns (argmax, conf, taps dict)."""
        c = self.cfg
        canvas = np.ascontiguousarray(canvas, dtype=np.int32)
        B, N = canvas.shape
        BN = B * N
        cap = ks[0].shape[2] if ks else 0
        lens = np.ascontiguousarray(lens, dtype=np.int32)
        am = np.zeros((B, N), np.int32)
        cf = np.zeros((B, N), np.float32)
        tp, out = self._taps(BN, taps, inject_router)
        kp = self._ptr_array(ks) if ks else None
        vp = self._ptr_array(vs) if vs else None
        rc = lib().or_denoise_pass(C.byref(self.c), C.byref(self.w), kp, vp, cap, _ptr(lens),
                                   _ptr(canvas), B, N, _ptr(am), _ptr(cf), C.byref(tp),
                                   self.nthreads)
        if rc != 0:
            raise ValueError(f"or_denoise_pass failed: {rc}")
        out.pop("_inject", None)
        return am, cf, out


def renoise(canvas, argmax, conf, tau, seed, pass_tag, pos0, V, req_id=None):
    """Returns the re-noised copy of canvas [B, N] (conf None: noise every slot)."""
    cv = np.array(canvas, dtype=np.int32, copy=True, order="C")
    B, N = cv.shape
    am = None if argmax is None else np.ascontiguousarray(argmax, dtype=np.int32)
    cf = None if conf is None else np.ascontiguousarray(conf, dtype=np.float32)
    p0 = np.ascontiguousarray(pos0, dtype=np.int32)
    rq = None if req_id is None else np.ascontiguousarray(req_id, dtype=np.uint32)
    rc = lib().or_renoise(_ptr(cv), _ptr(am), _ptr(cf), float(tau), int(seed) & (2**64 - 1),
                          int(pass_tag) & 0xFFFFFFFF, _ptr(p0), _ptr(rq), B, N, V)
    if rc != 0:
        raise ValueError(f"or_renoise failed: {rc}")
    return cv


def unmask(canvas, argmax, conf, tau, mask_id, final_pass=False):
    """Masked-diffusion update of a copy of canvas [B, N]: returns (canvas,
    changed [B], masked_left [B])."""
    cv = np.array(canvas, dtype=np.int32, copy=True, order="C")
    B, N = cv.shape
    am = np.ascontiguousarray(argmax, dtype=np.int32)
    cf = np.ascontiguousarray(conf, dtype=np.float32)
    ch = np.zeros(B, np.int32)
    ml = np.zeros(B, np.int32)
    rc = lib().or_unmask(_ptr(cv), _ptr(am), _ptr(cf), float(tau), int(mask_id), int(bool(final_pass)),
                         B, N, _ptr(ch), _ptr(ml))
    if rc != 0:
        raise ValueError(f"or_unmask failed: {rc}")
    return cv, ch, ml


def philox4x64_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    o = np.zeros(4, np.uint64)
    lib().or_philox4x64_10(_ptr(c), _ptr(k), _ptr(o))
    return o


def round_to(dt: str, x: float) -> float:
    return lib().or_round_to(_DT[dt], float(x))


def fp8_decode(code: int) -> float:
    return lib().or_fp8e4m3_decode(code)


def fp4_decode(code: int) -> float:
    return lib().or_fp4e2m1_decode(code)


def e8m0_decode(code: int) -> float:
    return lib().or_e8m0_decode(code)


def bf16_bits(x: float) -> int:
    return lib().or_bf16_bits(float(x))
