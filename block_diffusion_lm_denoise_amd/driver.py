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

Stop and resume: the whole state between two passes is the KV cache (with
its lengths), the canvas, the canvas and pass indices and the seed (the
noise is a function of position, pass tag and seed alone).  stop=(c, p)
returns before pass p of canvas c with that state in `state`; start=state
continues from it (on the same cache, or on a copy of it) and produces what
the uninterrupted loop would have.

Two variants of the same loop (the kernels are the same; only the update
between passes changes):
  - sampler="masked": masked ("absorbing") diffusion, the earlier scheme the
    explainer contrasts with ("First attempt: masked diffusion"): the canvas
    starts as the [MASK] token, a masked slot takes the prediction once its
    confidence reaches tau and is then locked in; after the last pass every
    slot still masked takes its prediction, and the canvas is committed;
  - early_exit: stop a canvas once it has converged ("Uniform State
    Diffusion": after several passes the canvas converges) -- under uniform
    noise when a pass's update changed no slot (every slot kept, each equal to
    its prediction: the next pass would see the same canvas), under masked
    diffusion when no slot is masked any more.  Each check reads two counts
    per request back to the host after the pass.
"""
from dataclasses import dataclass, field

import torch

from . import dgpass


@dataclass
class GenerateResult:
    canvases: list                       # committed canvases, [B][N] int32 each
    touched: torch.Tensor                # [canvases][S][L] experts touched per pass
    lens: list = field(default_factory=list)
    passes: list = field(default_factory=list)   # passes run per canvas
    state: dict = None                   # set when stopped: where to resume


def generate(model: dgpass.Model, kv: dgpass.KVCache, prompt: torch.Tensor, n_canvases: int, N: int,
             S: int, tau: float, seed: int, ws: torch.Tensor, prefill_prompt: bool = True,
             stream=None, sampler: str = "uniform", mask_id: int = None,
             early_exit: bool = False, stop=None, start=None) -> GenerateResult:
    cfg = model.cfg
    B = kv.B
    if sampler not in ("uniform", "masked"):
        raise ValueError(f"unknown sampler {sampler}")
    if sampler == "masked":
        mask_id = cfg.V - 1 if mask_id is None else int(mask_id)
        if not 0 <= mask_id < cfg.V:
            raise ValueError("mask_id must be a vocabulary id")
    dev = prompt.device if prompt is not None else kv.k[0].device
    c_first, p_first = 0, 0
    if start is not None:
        c_first, p_first = int(start["canvas_index"]), int(start["pass_index"])
        if not (0 <= c_first < n_canvases and 0 <= p_first < S) or prefill_prompt:
            raise ValueError("start needs a canvas and pass inside the run, and no prompt prefill")
    if prefill_prompt and prompt is not None:
        model.kv_prefill(kv, prompt, ws, stream=stream)
    canvas = torch.empty(B, N, dtype=torch.int32, device=dev)
    argmax = torch.empty(B, N, dtype=torch.int32, device=dev)
    conf = torch.empty(B, N, dtype=torch.float32, device=dev)
    changed = torch.zeros(B, dtype=torch.int32, device=dev)
    masked_left = torch.zeros(B, dtype=torch.int32, device=dev)
    touched = torch.zeros(n_canvases, S, cfg.L, dtype=torch.int32, device=dev)
    out, used = [], []
    for c in range(c_first, n_canvases):
        pos0 = kv.lens.copy()
        base = dict(sampler=sampler, mask_id=mask_id or 0, tau=tau, seed=seed, pos0=pos0)
        p0 = 0
        if start is not None and c == c_first:
            canvas.copy_(start["canvas"])
            p0 = p_first
        else:
            dgpass.canvas_update(canvas, None, None, dict(base, pass_tag=0), cfg.V, stream=stream)
        ran = S
        carry = False   # the workspace holds the first layer's input of `canvas`
        for p in range(p0, S):
            if stop is not None and (c, p) == tuple(stop):
                state = dict(canvas_index=c, pass_index=p, canvas=canvas.clone())
                return GenerateResult(out, touched, [int(x) for x in kv.lens], used, state)
            last = p == S - 1
            # the pass's last kernel writes the coverage and the update for the
            # next pass (uniform: none after the last pass; masked: the last
            # update fills every masked slot)
            if sampler == "uniform" and last:
                nxt = None
            else:
                # the pass's last kernel also embeds the updated canvas when the
                # next pass takes an update (it then skips its own embedding)
                ahead = p + 1 < S and not (sampler == "uniform" and p + 1 == S - 1)
                nxt = dict(base, pass_tag=p + 1, final_pass=last, changed=changed,
                           masked_left=masked_left, embed_next=ahead, input_embedded=carry)
            model.denoise_pass_next(kv, canvas, argmax, conf, ws, touched=touched[c, p], renoise=nxt,
                                    stream=stream)
            carry = nxt is not None and nxt["embed_next"]
            if early_exit and not last:
                left = masked_left if sampler == "masked" else changed
                if stream is not None:
                    stream.synchronize()
                else:
                    torch.cuda.synchronize(dev)
                if int(left.cpu().max()) == 0:
                    ran = p + 1
                    break
        committed = (argmax if sampler == "uniform" else canvas).clone()
        model.kv_prefill(kv, committed, ws, stream=stream)
        out.append(committed)
        used.append(ran)
    return GenerateResult(out, touched, [int(x) for x in kv.lens], used)
