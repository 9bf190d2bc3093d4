"""ctypes binding of libdgpass (include/dgpass.h), same names as the C ABI.

Argument marshalling only: every step of the pass runs in the HIP kernels of
libdgpass.so.  PyTorch provides device memory and the current stream.  There
is no fallback: if the library is not built the import of `lib()` raises.
"""
import ctypes as C
import os

import numpy as np
import torch

from .configs import ModelConfig

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdgpass.so")
MAX_LAYERS = 64
MAX_BATCH = 64

DG_F32, DG_BF16, DG_FP8E4M3, DG_MXFP4 = 0, 1, 2, 3
_DT = {"f32": DG_F32, "bf16": DG_BF16, "fp8": DG_FP8E4M3, "mxfp4": DG_MXFP4}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}

TAP_FIELDS = ("qkv", "attn", "x1", "u2", "router", "ids", "gates", "counts", "offsets", "perm",
              "hmid", "yexp", "xout", "uf", "logits")
STATUS = {0: "ok", -1: "invalid argument", -2: "KV cache capacity exceeded",
          -3: "unsupported shape or dtype", -4: "workspace too small", -5: "HIP launch error"}


class DgError(RuntimeError):
    def __init__(self, status, where):
        super().__init__(f"{where}: {STATUS.get(status, 'unknown')} ({status})")
        self.status = status


class dg_config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("L", "D", "Hq", "Hkv", "hd", "E", "k", "F", "V")] + [
        ("eps", C.c_float), ("act_dtype", C.c_int32), ("expert_dtype", C.c_int32)]


class dg_layer_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("g1", "wq", "wk", "wv", "wo", "g2", "wr", "wg", "wu",
                                          "wd", "escale", "wg_mx", "wu_mx", "wd_mx")]


class dg_weights(C.Structure):
    _fields_ = [("emb", C.c_void_p), ("gf", C.c_void_p), ("lm", C.c_void_p),
                ("layers", dg_layer_weights * MAX_LAYERS)]


class dg_model(C.Structure):
    _fields_ = [("cfg", dg_config), ("w", dg_weights), ("magic", C.c_uint32)]


class dg_kv(C.Structure):
    _fields_ = [("k", C.c_void_p * MAX_LAYERS), ("v", C.c_void_p * MAX_LAYERS), ("cap", C.c_int32),
                ("len", C.POINTER(C.c_int32))]


class dg_taps(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in TAP_FIELDS] + [
        ("inject_router", C.c_void_p), ("inject_x", C.c_void_p), ("inject_uf", C.c_void_p),
        ("stage_events", C.c_void_p)]


# stages a call can bracket with HIP events (dg_taps.stage_events)
STAGE_ATTN, STAGE_GATEUP, STAGE_DOWN, STAGE_HEAD = 0, 1, 2, 3
NSTAGES = 4


class dg_renoise_args(C.Structure):
    _fields_ = [("tau", C.c_float), ("seed", C.c_uint64), ("pass_tag", C.c_uint32),
                ("pos0", C.c_void_p), ("req_id", C.c_void_p), ("mode", C.c_int32),
                ("mask_id", C.c_int32), ("final_pass", C.c_int32), ("changed", C.c_void_p),
                ("masked_left", C.c_void_p), ("embed_next", C.c_int32),
                ("input_embedded", C.c_int32)]


SAMPLER_UNIFORM, SAMPLER_MASKED = 0, 1
_SAMPLER = {"uniform": SAMPLER_UNIFORM, "masked": SAMPLER_MASKED}


EXPORTS = ("dg_model_init", "dg_workspace_bytes", "dg_kv_prefill", "dg_denoise_pass",
           "dg_denoise_pass_next", "dg_renoise", "dg_expert_coverage", "dg_packed_bytes",
           "dg_pack_weight", "dg_status_str", "dg_check_attention_addresses",
           "dg_denoise_pass_next_noalloc", "dg_decode_step", "dg_canvas_update",
           "dg_packed_mx_scale_bytes", "dg_pack_mx_scales")
NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


def lib():
    """Load libdgpass.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() (hipcc, gfx950)")
        L = C.CDLL(LIB_PATH)
        vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
        L.dg_model_init.argtypes = [vp, vp, vp]
        L.dg_model_init.restype = i32
        L.dg_workspace_bytes.argtypes = [vp, i32, i32]
        L.dg_workspace_bytes.restype = sz
        L.dg_kv_prefill.argtypes = [vp, vp, vp, i32, i32, vp, vp, sz, vp]
        L.dg_kv_prefill.restype = i32
        L.dg_canvas_update.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp]
        L.dg_canvas_update.restype = i32
        L.dg_decode_step.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]
        L.dg_decode_step.restype = i32
        L.dg_denoise_pass.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, vp, sz, vp]
        L.dg_denoise_pass.restype = i32
        L.dg_denoise_pass_next.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.dg_denoise_pass_next.restype = i32
        L.dg_denoise_pass_next_noalloc.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp]
        L.dg_denoise_pass_next_noalloc.restype = i32
        L.dg_renoise.argtypes = [vp, vp, vp, C.c_float, C.c_uint64, C.c_uint32, vp, vp, i32, i32, i32,
                                 vp]
        L.dg_renoise.restype = i32
        L.dg_expert_coverage.argtypes = [vp, vp, sz, vp, vp, vp]
        L.dg_expert_coverage.restype = i32
        L.dg_packed_bytes.argtypes = [i32, i32, i32]
        L.dg_packed_bytes.restype = sz
        L.dg_pack_weight.argtypes = [vp, vp, i32, i32, i32, vp]
        L.dg_pack_weight.restype = i32
        L.dg_packed_mx_scale_bytes.argtypes = [i32, i32]
        L.dg_packed_mx_scale_bytes.restype = sz
        L.dg_pack_mx_scales.argtypes = [vp, vp, i32, i32, vp]
        L.dg_pack_mx_scales.restype = i32
        L.dg_status_str.argtypes = [i32]
        L.dg_status_str.restype = C.c_char_p
        L.dg_check_attention_addresses.argtypes = [i32, i32, i32, vp, i32, i32, i32, C.c_long,
                                                   C.POINTER(C.c_long)]
        L.dg_check_attention_addresses.restype = C.c_long
        _lib = L
    return _lib


def _check(st, where):
    if st != 0:
        raise DgError(st, where)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def make_config(cfg: ModelConfig) -> dg_config:
    return dg_config(cfg.L, cfg.D, cfg.Hq, cfg.Hkv, cfg.hd, cfg.E, cfg.k, cfg.F, cfg.V, float(cfg.eps),
                     _DT[cfg.act], _DT[cfg.expert])


def workspace_bytes(cfg: ModelConfig, max_rows: int, max_keys: int = 0) -> int:
    c = make_config(cfg)
    return lib().dg_workspace_bytes(C.byref(c), int(max_rows), int(max_keys))


class KVCache:
    """Per-layer K/V device tensors [B][Hkv][cap][hd] plus host lengths."""

    def __init__(self, cfg: ModelConfig, B: int, cap: int, device="cuda", k=None, v=None):
        self.cfg, self.B, self.cap = cfg, B, cap
        dt = TORCH_DT[cfg.act]
        self.k = k if k is not None else [torch.zeros(B, cfg.Hkv, cap, cfg.hd, dtype=dt, device=device)
                                          for _ in range(cfg.L)]
        self.v = v if v is not None else [torch.zeros(B, cfg.Hkv, cap, cfg.hd, dtype=dt, device=device)
                                          for _ in range(cfg.L)]
        self.lens = np.zeros(B, dtype=np.int32)

    def struct(self) -> dg_kv:
        s = dg_kv()
        for l in range(self.cfg.L):
            s.k[l] = self.k[l].data_ptr()
            s.v[l] = self.v[l].data_ptr()
        s.cap = self.cap
        s.len = self.lens.ctypes.data_as(C.POINTER(C.c_int32))
        return s


def make_taps(cfg: ModelConfig, rows: int, names, device="cuda") -> dict:
    """Device tensors for the requested taps of a call over `rows` token rows."""
    a = TORCH_DT[cfg.act]
    shapes = {
        "qkv": ((cfg.L, rows, cfg.qkv_dim), a), "attn": ((cfg.L, rows, cfg.Hq * cfg.hd), a),
        "x1": ((cfg.L, rows, cfg.D), a), "u2": ((cfg.L, rows, cfg.D), a),
        "router": ((cfg.L, rows, cfg.E), torch.float32), "ids": ((cfg.L, rows, cfg.k), torch.int32),
        "gates": ((cfg.L, rows, cfg.k), torch.float32), "counts": ((cfg.L, cfg.E), torch.int32),
        "offsets": ((cfg.L, cfg.E + 1), torch.int32), "perm": ((cfg.L, rows * cfg.k), torch.int32),
        "hmid": ((cfg.L, rows, cfg.k, cfg.F), a), "yexp": ((cfg.L, rows, cfg.k, cfg.D), a),
        "xout": ((cfg.L, rows, cfg.D), a), "uf": ((rows, cfg.D), a),
        "logits": ((rows, cfg.V), torch.float32),
    }
    return {n: torch.zeros(*shapes[n][0], dtype=shapes[n][1], device=device) for n in names}


def _taps_struct(taps, inject_router=None, inject_x=None, inject_uf=None, stage_events=None):
    """dg_taps for the given device tensors; stage_events: flat list of
    torch.cuda.Event (or None) indexed [l][stage][0/1]."""
    if not taps and inject_router is None and inject_x is None and inject_uf is None \
            and stage_events is None:
        return None, None
    t = dg_taps()
    for n, v in (taps or {}).items():
        setattr(t, n, v.data_ptr())
    t.inject_router = _ptr(inject_router)
    t.inject_x = _ptr(inject_x)
    t.inject_uf = _ptr(inject_uf)
    keep = None
    if stage_events is not None:
        keep = (C.c_void_p * len(stage_events))(
            *[None if e is None else e.cuda_event for e in stage_events])
        t.stage_events = C.cast(keep, C.c_void_p)
    return t, keep


def _renoise_struct(renoise):
    """dg_renoise_args for dict(tau, seed, pass_tag, pos0[, req_id, sampler,
    mask_id, final_pass, changed, masked_left, embed_next, input_embedded])
    (or None), with the host arrays it points to (kept alive by the caller).
    sampler: "uniform" or "masked"; changed / masked_left: device int32
    tensors [B] or None; embed_next / input_embedded: booleans (the carry of
    the first layer's input between consecutive passes, see dgpass.h)."""
    if renoise is None:
        return None, None
    p0 = renoise.get("pos0")
    p0 = None if p0 is None else np.ascontiguousarray(p0, dtype=np.int32)
    rq = renoise.get("req_id")
    rq = None if rq is None else np.ascontiguousarray(rq, dtype=np.uint32)
    nx = dg_renoise_args(float(renoise.get("tau", 0.0)), int(renoise.get("seed", 0)) & (2**64 - 1),
                         int(renoise.get("pass_tag", 0)) & 0xFFFFFFFF,
                         None if p0 is None else p0.ctypes.data_as(C.c_void_p),
                         None if rq is None else rq.ctypes.data_as(C.c_void_p),
                         _SAMPLER[renoise.get("sampler", "uniform")], int(renoise.get("mask_id", 0)),
                         int(bool(renoise.get("final_pass", False))), _ptr(renoise.get("changed")),
                         _ptr(renoise.get("masked_left")),
                         int(bool(renoise.get("embed_next", False))),
                         int(bool(renoise.get("input_embedded", False))))
    return nx, (p0, rq)


def canvas_update(canvas: torch.Tensor, argmax, conf, args: dict, V: int, stream=None):
    """The between-pass update of device canvases [B][N] in place
    (dg_canvas_update); args as for denoise_pass_next's renoise; conf None:
    initialise the canvas."""
    B, N = canvas.shape
    nx, keep = _renoise_struct(args)
    st = lib().dg_canvas_update(canvas.data_ptr(), _ptr(argmax), _ptr(conf), C.byref(nx), B, N, V,
                                _stream(stream))
    del keep
    _check(st, "dg_canvas_update")


def check_attention_addresses(act, B, T, lens, Hq, Hkv, mode, part_cap):
    """Host replay of the attention's K/V addresses (dg_check_attention_addresses):
    (slots addressing a key outside the block's request, slots checked)."""
    ln = np.ascontiguousarray(lens, dtype=np.int32)
    n = C.c_long(0)
    bad = lib().dg_check_attention_addresses(_DT[act], int(B), int(T), ln.ctypes.data_as(C.c_void_p),
                                             int(Hq), int(Hkv), int(mode), int(part_cap), C.byref(n))
    return int(bad), int(n.value)


def packed_bytes(rows: int, cols: int, dtype: str) -> int:
    return lib().dg_packed_bytes(int(rows), int(cols), _DT[dtype])


def pack_weight(src: torch.Tensor, rows: int, cols: int, dtype: str, stream=None) -> torch.Tensor:
    """Packed copy (a new uint8 device tensor) of the row-major device matrix src [rows][cols]."""
    n = packed_bytes(rows, cols, dtype)
    if n == 0:
        raise DgError(-1, "dg_packed_bytes")
    dst = torch.empty(n, dtype=torch.uint8, device=src.device)
    _check(lib().dg_pack_weight(src.data_ptr(), dst.data_ptr(), int(rows), int(cols), _DT[dtype],
                                _stream(stream)), "dg_pack_weight")
    return dst


def pack_mx_scales(src: torch.Tensor, rows: int, cols: int, stream=None) -> torch.Tensor:
    """Packed copy (a new uint8 device tensor) of the E8M0 scales src
    [rows][cols/32] of an MXFP4 matrix [rows][cols]."""
    n = lib().dg_packed_mx_scale_bytes(int(rows), int(cols))
    if n == 0:
        raise DgError(-1, "dg_packed_mx_scale_bytes")
    dst = torch.empty(n, dtype=torch.uint8, device=src.device)
    _check(lib().dg_pack_mx_scales(src.data_ptr(), dst.data_ptr(), int(rows), int(cols), _stream(stream)),
           "dg_pack_mx_scales")
    return dst


# streamed weight matrices: name -> (rows, cols, dtype field of the config)
def _packed_shapes(cfg: ModelConfig):
    QD, KD = cfg.Hq * cfg.hd, cfg.Hkv * cfg.hd
    return {"wq": (QD, cfg.D, cfg.act), "wk": (KD, cfg.D, cfg.act), "wv": (KD, cfg.D, cfg.act),
            "wo": (cfg.D, QD, cfg.act), "wr": (cfg.E, cfg.D, cfg.act),
            "wg": (cfg.E * cfg.F, cfg.D, cfg.expert), "wu": (cfg.E * cfg.F, cfg.D, cfg.expert),
            "wd": (cfg.E * cfg.D, cfg.F, cfg.expert)}


class Model:
    """A model on the device: config + weight tensors.  The streamed weight
    matrices are packed once here (new device tensors, kept alive with the
    caller's row-major weights)."""

    def __init__(self, cfg: ModelConfig, weights: dict):
        if cfg.L > MAX_LAYERS:
            raise ValueError("too many layers")
        self.cfg = cfg
        self.weights = weights
        shapes = _packed_shapes(cfg)
        self.packed = {"lm": pack_weight(weights["lm"], cfg.V, cfg.D, cfg.act), "layers": []}
        w = dg_weights()
        w.emb = weights["emb"].data_ptr()
        w.gf = weights["gf"].data_ptr()
        w.lm = self.packed["lm"].data_ptr()
        for l, lw in enumerate(weights["layers"]):
            L = w.layers[l]
            pk = {n: pack_weight(lw[n], *shapes[n]) for n in shapes}
            if cfg.expert == "mxfp4":
                for n in ("wg", "wu", "wd"):
                    pk[n + "_mx"] = pack_mx_scales(lw[n + "_mx"], shapes[n][0], shapes[n][1])
            self.packed["layers"].append(pk)
            for n in ("g1", "g2"):
                setattr(L, n, lw[n].data_ptr())
            for n in shapes:
                setattr(L, n, pk[n].data_ptr())
            L.escale = _ptr(lw.get("escale"))
            for n in ("wg_mx", "wu_mx", "wd_mx"):
                setattr(L, n, _ptr(pk.get(n)))
        self._c = make_config(cfg)
        self._m = dg_model()
        _check(lib().dg_model_init(C.byref(self._m), C.byref(self._c), C.byref(w)), "dg_model_init")

    def workspace(self, max_rows: int, max_keys: int = 0, device="cuda") -> torch.Tensor:
        n = lib().dg_workspace_bytes(C.byref(self._c), int(max_rows), int(max_keys))
        if n == 0:
            raise DgError(-1, "dg_workspace_bytes")
        return torch.empty(n, dtype=torch.uint8, device=device)

    def kv_cache(self, B: int, cap: int, device="cuda") -> KVCache:
        return KVCache(self.cfg, B, cap, device)

    def kv_prefill(self, kv: KVCache, tokens: torch.Tensor, ws: torch.Tensor, taps=None,
                   inject_router=None, inject_x=None, stage_events=None, stream=None):
        B, T = tokens.shape
        s = kv.struct()
        ts, keep = _taps_struct(taps, inject_router, inject_x, None, stage_events)
        st = lib().dg_kv_prefill(C.byref(self._m), C.byref(s), tokens.data_ptr(), B, T,
                                 None if ts is None else C.byref(ts), ws.data_ptr(), ws.numel(),
                                 _stream(stream))
        del keep
        _check(st, "dg_kv_prefill")

    def decode_step(self, kv: KVCache, tokens: torch.Tensor, argmax: torch.Tensor, conf: torch.Tensor,
                    ws: torch.Tensor, taps=None, inject_uf=None, stage_events=None, stream=None):
        """One autoregressive step: append tokens [B] and write the next token
        and its confidence per request."""
        B = tokens.shape[0]
        s = kv.struct()
        ts, keep = _taps_struct(taps, None, None, inject_uf, stage_events)
        st = lib().dg_decode_step(C.byref(self._m), C.byref(s), tokens.data_ptr(), B, argmax.data_ptr(),
                                  conf.data_ptr(), None if ts is None else C.byref(ts), ws.data_ptr(),
                                  ws.numel(), _stream(stream))
        del keep
        _check(st, "dg_decode_step")

    def denoise_pass(self, kv: KVCache, canvas: torch.Tensor, argmax: torch.Tensor, conf: torch.Tensor,
                     ws: torch.Tensor, taps=None, inject_router=None, inject_x=None, inject_uf=None,
                     stage_events=None, stream=None):
        B, N = canvas.shape
        s = kv.struct()
        ts, keep = _taps_struct(taps, inject_router, inject_x, inject_uf, stage_events)
        st = lib().dg_denoise_pass(C.byref(self._m), C.byref(s), canvas.data_ptr(), B, N,
                                   argmax.data_ptr(), conf.data_ptr(),
                                   None if ts is None else C.byref(ts), ws.data_ptr(), ws.numel(),
                                   _stream(stream))
        del keep
        _check(st, "dg_denoise_pass")

    def denoise_pass_next(self, kv: KVCache, canvas: torch.Tensor, argmax: torch.Tensor,
                          conf: torch.Tensor, ws: torch.Tensor, touched=None, renoise=None, taps=None,
                          inject_router=None, inject_x=None, inject_uf=None, stage_events=None,
                          stream=None):
        """A pass whose last kernel also writes the expert coverage (touched:
        device [L] int32, or None) and, with renoise = dict(tau, seed,
        pass_tag, pos0[, req_id]), re-noises canvas in place for the next pass."""
        B, N = canvas.shape
        s = kv.struct()
        ts, keep = _taps_struct(taps, inject_router, inject_x, inject_uf, stage_events)
        nx, arrs = _renoise_struct(renoise)
        st = lib().dg_denoise_pass_next(C.byref(self._m), C.byref(s), canvas.data_ptr(), B, N,
                                        argmax.data_ptr(), conf.data_ptr(), _ptr(touched),
                                        None if nx is None else C.byref(nx),
                                        None if ts is None else C.byref(ts), ws.data_ptr(), ws.numel(),
                                        _stream(stream))
        del keep, arrs
        _check(st, "dg_denoise_pass_next")

    def denoise_pass_next_noalloc(self, kv: KVCache, canvas: torch.Tensor, argmax: torch.Tensor,
                                  conf: torch.Tensor, touched=None, renoise=None, taps=None,
                                  inject_router=None, inject_x=None, inject_uf=None, stream=None):
        """denoise_pass_next on the library's static per-GPU scratch (no workspace)."""
        B, N = canvas.shape
        s = kv.struct()
        ts, keep = _taps_struct(taps, inject_router, inject_x, inject_uf, None)
        nx, arrs = _renoise_struct(renoise)
        st = lib().dg_denoise_pass_next_noalloc(C.byref(self._m), C.byref(s), canvas.data_ptr(), B, N,
                                                argmax.data_ptr(), conf.data_ptr(), _ptr(touched),
                                                None if nx is None else C.byref(nx),
                                                None if ts is None else C.byref(ts), _stream(stream))
        del keep, arrs
        _check(st, "dg_denoise_pass_next_noalloc")

    def expert_coverage(self, ws: torch.Tensor, touched: torch.Tensor, counts=None, stream=None):
        st = lib().dg_expert_coverage(C.byref(self._m), ws.data_ptr(), ws.numel(), touched.data_ptr(),
                                      _ptr(counts), _stream(stream))
        _check(st, "dg_expert_coverage")


def renoise(canvas: torch.Tensor, argmax, conf, tau: float, seed: int, pass_tag: int, pos0, V: int,
            req_id=None, stream=None):
    """Re-noise device canvases [B][N] in place (conf None: noise every slot)."""
    B, N = canvas.shape
    p0 = np.ascontiguousarray(pos0, dtype=np.int32)
    rq = None if req_id is None else np.ascontiguousarray(req_id, dtype=np.uint32)
    st = lib().dg_renoise(canvas.data_ptr(), _ptr(argmax), _ptr(conf), float(tau),
                          int(seed) & (2**64 - 1), int(pass_tag) & 0xFFFFFFFF,
                          p0.ctypes.data_as(C.c_void_p),
                          None if rq is None else rq.ctypes.data_as(C.c_void_p), B, N, V,
                          _stream(stream))
    _check(st, "dg_renoise")
