"""Roofline arithmetic for the denoising pass.

The rule is the one the course page "Module 12. Diffusion Language Models"
uses in its dense-8B exercise: the weight-read time and the arithmetic time
are both lower bounds on a pass, and the binding one is their maximum, not
their sum.  The same page's break-even exercise turns a per-pass time into a
canvas generation rate and compares it with the autoregressive ceiling.

Algorithmic bytes count what the method must move (weights of touched
experts only, the cached prefix, one read of each input and one write of
each output), not intermediates; algorithmic flops count the dense
contractions (2 per multiply-add), not exponentials or norms.
"""
from dataclasses import dataclass

# MI355X nominal ceilings
HBM_BYTES_PER_S = 8.0e12
MFMA_PEAK = {"bf16": 2.5e15, "fp16": 2.5e15, "fp8": 5.0e15, "f32": 157.3e12, "f64": 78.6e12}

# bytes per element; MXFP4 adds one E8M0 scale byte per 32 elements
_BYTES = {"f32": 4, "bf16": 2, "fp8": 1, "mxfp4": 0.5 + 1 / 32}


def roof_time(bytes_moved: float, flops: float, bw: float, peak: float) -> float:
    """Binding floor: max(bytes / bandwidth, flops / peak)."""
    return max(bytes_moved / bw, flops / peak)


def dense_weight_read_time(params: float, bytes_per_param: float, bw: float) -> float:
    return params * bytes_per_param / bw


def dense_pass_time(params: float, bytes_per_param: float, tokens: int, bw: float, peak: float) -> float:
    """One forward over `tokens` positions of a dense model: 2*params flops per token."""
    return roof_time(params * bytes_per_param, 2.0 * params * tokens, bw, peak)


def ar_ceiling_tok_s(step_s: float) -> float:
    """Autoregressive decoding emits one token per weight read."""
    return 1.0 / step_s


def diffusion_rate_tok_s(canvas: int, passes: int, pass_s: float) -> float:
    """A canvas of `canvas` tokens revealed after `passes` full passes."""
    return canvas / (passes * pass_s)


def breakeven_passes(canvas: int, pass_s: float, ar_step_s: float) -> float:
    """Largest real S with canvas / (S * pass_s) > 1 / ar_step_s."""
    return canvas * ar_step_s / pass_s


@dataclass
class PassWork:
    bytes: dict
    flops: dict

    @property
    def total_bytes(self) -> float:
        return float(sum(self.bytes.values()))

    @property
    def total_flops(self) -> float:
        return float(sum(self.flops.values()))


def denoise_pass_work(cfg, B: int, N: int, prefix_lens, touched_per_layer) -> PassWork:
    """Algorithmic bytes and flops of one denoising pass, split by kernel family."""
    w = _BYTES[cfg.act]
    we = _BYTES[cfg.expert]
    BN = B * N
    D, F, E = cfg.D, cfg.F, cfg.E
    attn_w = (cfg.Hq * cfg.hd * D * 2 + cfg.Hkv * cfg.hd * D * 2)   # Wq, Wo, Wk, Wv elements
    by = {"embed": BN * D * w + BN * 4, "attn_proj": 0.0, "attention": 0.0, "router": 0.0,
          "experts": 0.0, "head": V_bytes(cfg) + BN * 8}
    fl = {"attn_proj": 0.0, "attention": 0.0, "router": 0.0, "experts": 0.0,
          "head": 2.0 * BN * cfg.V * D}
    for l in range(cfg.L):
        by["attn_proj"] += attn_w * w + 2 * D * 4
        by["attention"] += sum(int(p) for p in prefix_lens) * cfg.Hkv * cfg.hd * 2 * w
        by["router"] += E * D * w
        scales = 12 if cfg.expert == "fp8" else 0
        by["experts"] += int(touched_per_layer[l]) * (3 * D * F * we + scales)
        fl["attn_proj"] += 2.0 * BN * attn_w
        fl["attention"] += sum(4.0 * N * (int(p) + N) * cfg.Hq * cfg.hd for p in prefix_lens)
        fl["router"] += 2.0 * BN * E * D
        fl["experts"] += 2.0 * BN * cfg.k * 3 * D * F
    by["head"] += D * 4
    return PassWork(by, fl)


def V_bytes(cfg) -> int:
    return cfg.V * cfg.D * _BYTES[cfg.act]


def gateup_work(cfg, touched: int, rows: int):
    """Gate+up grouped GEMM: (bytes, flops) per launch.  Per touched expert
    2*F*D expert weights; per routed row one D-wide input read and one F-wide
    SwiGLU output written."""
    we = _BYTES[cfg.expert]
    w = _BYTES[cfg.act]
    b = touched * 2 * cfg.F * cfg.D * we + rows * (cfg.D + cfg.F) * w
    f = 2.0 * rows * 2 * cfg.F * cfg.D
    return b, f


def down_work(cfg, touched: int, rows: int):
    we = _BYTES[cfg.expert]
    w = _BYTES[cfg.act]
    b = touched * cfg.F * cfg.D * we + rows * (cfg.D + cfg.F) * w
    f = 2.0 * rows * cfg.F * cfg.D
    return b, f


def decode_step_work(cfg, B: int, prefix_lens, experts_per_layer) -> PassWork:
    """Algorithmic bytes and flops of one autoregressive decoding step of B
    requests (one new token each, attending its prefix and itself):
    experts_per_layer distinct experts read per layer (at most B*k)."""
    w = _BYTES[cfg.act]
    we = _BYTES[cfg.expert]
    D, F = cfg.D, cfg.F
    attn_w = (cfg.Hq * cfg.hd * D * 2 + cfg.Hkv * cfg.hd * D * 2)
    by = {"embed": B * D * w + B * 4, "attn_proj": 0.0, "attention": 0.0, "router": 0.0,
          "experts": 0.0, "head": V_bytes(cfg) + D * 4 + B * 8}
    fl = {"attn_proj": 0.0, "attention": 0.0, "router": 0.0, "experts": 0.0,
          "head": 2.0 * B * cfg.V * D}
    for l in range(cfg.L):
        by["attn_proj"] += attn_w * w + 2 * D * 4
        by["attention"] += sum(int(p) for p in prefix_lens) * cfg.Hkv * cfg.hd * 2 * w
        by["router"] += cfg.E * D * w
        scales = 12 if cfg.expert == "fp8" else 0
        by["experts"] += int(experts_per_layer[l]) * (3 * D * F * we + scales)
        fl["attn_proj"] += 2.0 * B * attn_w
        fl["attention"] += sum(4.0 * (int(p) + 1) * cfg.Hq * cfg.hd for p in prefix_lens)
        fl["router"] += 2.0 * B * cfg.E * D
        fl["experts"] += 2.0 * B * cfg.k * 3 * D * F
    return PassWork(by, fl)
