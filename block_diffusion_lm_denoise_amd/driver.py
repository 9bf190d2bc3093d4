"""Block-diffusion generation loop on the device (host control only).

Explainer "DiffusionGemma": the prompt is prefilled causally into the KV
cache ("Two modes, one model"); each canvas starts as uniform noise, is
denoised in several passes with low-confidence slots re-noised between
passes ("Uniform State Diffusion"), and once finished is appended to the
cache by a prefill before a fresh canvas opens ("Long-form text: chaining
canvases").  Plain readings where the pages are silent: the committed
canvas is the last pass's argmax (no re-noise after the last pass); RNG
pass tags are 0 for the initial noise and p+1 for the re-noise after pass
p; positions are absolute, so chained canvases draw different noise.
"""
from dataclasses import dataclass, field

import torch

from . import dgpass


@dataclass
class GenerateResult:
    canvases: list                       # committed canvases, [B][N] int32 each
    touched: torch.Tensor                # [canvases][S][L] experts touched per pass
    lens: list = field(default_factory=list)


def generate(model: dgpass.Model, kv: dgpass.KVCache, prompt: torch.Tensor, n_canvases: int, N: int,
             S: int, tau: float, seed: int, ws: torch.Tensor, prefill_prompt: bool = True,
             stream=None) -> GenerateResult:
    cfg = model.cfg
    B = kv.B
    dev = prompt.device if prompt is not None else kv.k[0].device
    if prefill_prompt and prompt is not None:
        model.kv_prefill(kv, prompt, ws, stream=stream)
    canvas = torch.empty(B, N, dtype=torch.int32, device=dev)
    argmax = torch.empty(B, N, dtype=torch.int32, device=dev)
    conf = torch.empty(B, N, dtype=torch.float32, device=dev)
    touched = torch.zeros(n_canvases, S, cfg.L, dtype=torch.int32, device=dev)
    out = []
    for c in range(n_canvases):
        pos0 = kv.lens.copy()
        dgpass.renoise(canvas, None, None, tau, seed, 0, pos0, cfg.V, stream=stream)
        for p in range(S):
            # the pass's last kernel writes the coverage and, before every pass
            # but the last, re-noises the canvas for the next one
            nxt = dict(tau=tau, seed=seed, pass_tag=p + 1, pos0=pos0) if p < S - 1 else None
            model.denoise_pass_next(kv, canvas, argmax, conf, ws, touched=touched[c, p], renoise=nxt,
                                    stream=stream)
        committed = argmax.clone()
        model.kv_prefill(kv, committed, ws, stream=stream)
        out.append(committed)
    return GenerateResult(out, touched, [int(x) for x in kv.lens])
