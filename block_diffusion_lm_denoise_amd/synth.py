"""Seeded synthetic inputs shared by the GPU path and the CPU oracle.

Holds none of the method's arithmetic: weights are N(0, 0.02) draws rounded
to their storage type, prompt tokens are uniform vocabulary ids, and fp8
expert weights are quantised once with one scale per expert and matrix
(amax / 448, round-to-nearest-even, the e4m3 range).  Every tensor has its
own generator seeded from (seed, tensor name), so a tensor does not depend
on the order tensors are made in.
"""
import zlib

import torch

from .configs import ModelConfig

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
FP8_MAX = 448.0


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1000003 + zlib.crc32(name.encode())) & 0x7FFFFFFFFFFFFFFF)
    return g


def normal(shape, seed: int, name: str, std: float = 0.02, device="cpu") -> torch.Tensor:
    """fp32 N(0, std^2) draws of the given shape."""
    return torch.randn(*shape, generator=_gen(seed, name, device), device=device,
                       dtype=torch.float32) * std


def quantize_fp8(w: torch.Tensor):
    """Per-expert e4m3 quantisation of w [E, R, C]: returns (codes uint8 view, scales f32 [E])."""
    amax = w.abs().amax(dim=(1, 2)).clamp_min(1e-30)
    s = amax / FP8_MAX
    q = (w / s[:, None, None]).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return q, s.to(torch.float32)


# E2M1 magnitudes and the midpoints between neighbours, with the neighbour a
# tie rounds to (the one with an even code)
_FP4_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
_FP4_MIDS = ((0.25, False), (0.75, True), (1.25, False), (1.75, True), (2.5, False), (3.5, True),
             (5.0, False))   # (midpoint, a tie goes up)


def quantize_mxfp4(w: torch.Tensor):
    """OCP microscaling FP4 of w [..., cols] (cols a multiple of 32): per block
    of 32 consecutive elements of a row an E8M0 scale 2^(floor(log2 amax) - 2)
    (2 is E2M1's largest exponent) and E2M1 codes of w / scale, rounded to
    nearest (ties to even), saturating at 6.  Returns (codes packed two per
    byte, element 2i in the low nibble: uint8 [..., cols/2]; scales uint8
    [..., cols/32])."""
    shp = w.shape
    blocks = w.reshape(*shp[:-1], shp[-1] // 32, 32).to(torch.float64)
    amax = blocks.abs().amax(-1).clamp_min(2.0 ** -126)
    e = torch.floor(torch.log2(amax)) - 2
    y = (blocks / torch.pow(2.0, e)[..., None]).clamp(-6.0, 6.0)
    a = y.abs()
    idx = torch.zeros_like(a, dtype=torch.int64)
    for mid, up in _FP4_MIDS:
        idx += (a >= mid if up else a > mid).to(torch.int64)
    codes = (idx | ((y < 0).to(torch.int64) << 3)).reshape(*shp[:-1], shp[-1])
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).to(torch.uint8)
    scales = (e + 127).to(torch.uint8)
    return packed.contiguous(), scales.contiguous()


def make_weights(cfg: ModelConfig, seed: int, device="cpu", gain: str = "ones") -> dict:
    """All weights of a model.

    gain: "ones" (RMSNorm gains 1) or "random" (1 + 0.1 N(0,1), used by tests so
    that a dropped gain shows).
    """
    adt = _TORCH_DT[cfg.act]

    def act(shape, name):
        return normal(shape, seed, name, device=device).to(adt)

    def gvec(name):
        if gain == "ones":
            return torch.ones(cfg.D, dtype=torch.float32, device=device)
        return 1.0 + normal((cfg.D,), seed, name, std=0.1, device=device)

    w = {"emb": act((cfg.V, cfg.D), "emb"), "gf": gvec("gf"), "lm": act((cfg.V, cfg.D), "lm"),
         "layers": []}
    for l in range(cfg.L):
        p = f"l{l}."
        lw = {
            "g1": gvec(p + "g1"),
            "wq": act((cfg.Hq * cfg.hd, cfg.D), p + "wq"),
            "wk": act((cfg.Hkv * cfg.hd, cfg.D), p + "wk"),
            "wv": act((cfg.Hkv * cfg.hd, cfg.D), p + "wv"),
            "wo": act((cfg.D, cfg.Hq * cfg.hd), p + "wo"),
            "g2": gvec(p + "g2"),
            "wr": act((cfg.E, cfg.D), p + "wr"),
            "escale": None,
        }
        mats = {"wg": (cfg.E, cfg.F, cfg.D), "wu": (cfg.E, cfg.F, cfg.D), "wd": (cfg.E, cfg.D, cfg.F)}
        scales = []
        for name, shape in mats.items():
            if cfg.expert == "mxfp4":
                codes, mx = [], []
                for e in range(cfg.E):
                    q, sc = quantize_mxfp4(normal(shape[1:], seed, f"{p}{name}.{e}", device=device))
                    codes.append(q)
                    mx.append(sc)
                lw[name] = torch.stack(codes)          # [E, rows, cols/2] uint8
                lw[name + "_mx"] = torch.stack(mx)     # [E, rows, cols/32] uint8
            elif cfg.expert == "fp8":
                # one expert at a time keeps the fp32 staging small
                codes, sc = [], []
                for e in range(cfg.E):
                    x = normal(shape[1:], seed, f"{p}{name}.{e}", device=device)
                    q, s = quantize_fp8(x[None])
                    codes.append(q[0])
                    sc.append(s[0])
                lw[name] = torch.stack(codes)
                scales.append(torch.stack(sc))
            else:
                lw[name] = normal(shape, seed, p + name, device=device).to(_TORCH_DT[cfg.expert])
        if cfg.expert == "fp8":
            lw["escale"] = torch.stack(scales, dim=1).contiguous()   # [E, 3] gate, up, down
        w["layers"].append(lw)
    return w


def tokens(V: int, shape, seed: int, name: str = "prompt", device="cpu") -> torch.Tensor:
    """Uniform vocabulary ids, int32."""
    return torch.randint(0, V, tuple(shape), generator=_gen(seed, name, device), device=device,
                         dtype=torch.int64).to(torch.int32)


def kv_cache_values(cfg: ModelConfig, B: int, cap: int, P: int, seed: int, device="cpu"):
    """Synthetic prefix K/V, [B][Hkv][cap][hd] per layer, N(0, 0.9^2) in the first P slots.

    Stands in for a prefilled cache when a test exercises the denoising pass
    alone (0.9 is the spread of a projection of a unit-RMS row by N(0, 0.02)
    weights at width 2048).
    """
    adt = _TORCH_DT[cfg.act]
    ks, vs = [], []
    for l in range(cfg.L):
        k = torch.zeros(B, cfg.Hkv, cap, cfg.hd, dtype=adt, device=device)
        v = torch.zeros_like(k)
        if P:
            k[:, :, :P] = normal((B, cfg.Hkv, P, cfg.hd), seed, f"kc{l}", std=0.9, device=device).to(adt)
            v[:, :, :P] = normal((B, cfg.Hkv, P, cfg.hd), seed, f"vc{l}", std=0.9, device=device).to(adt)
        ks.append(k)
        vs.append(v)
    return ks, vs


def weights_to(w: dict, device) -> dict:
    """Copy a weight dict to another device."""
    out = {k: (v.to(device) if torch.is_tensor(v) else v) for k, v in w.items() if k != "layers"}
    out["layers"] = [{k: (v.to(device) if torch.is_tensor(v) else v) for k, v in lw.items()}
                     for lw in w["layers"]]
    return out
