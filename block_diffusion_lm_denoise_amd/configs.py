"""Model shapes and synthetic workloads of the denoising pass.

Shapes only -- no arithmetic of the method lives here.  The five workloads are
the ones the pass is measured and parity-checked on: a tiny fp32 layer, one
bf16 MoE layer with a 1024- or 8192-token cached prefix, an 8-layer stack that
chains four 256-token canvases after a 4096-token prompt, and a batch of eight
requests with fp8 expert weights.
"""
from dataclasses import dataclass, field, replace

ACT_DTYPES = ("f32", "bf16")
EXPERT_DTYPES = ("f32", "bf16", "fp8", "mxfp4")


@dataclass(frozen=True)
class ModelConfig:
    L: int          # layers
    D: int          # model width
    Hq: int         # query heads
    Hkv: int        # key/value heads (grouped-query attention)
    hd: int         # head dim
    E: int          # experts
    k: int          # experts per token
    F: int          # expert FFN width
    V: int          # vocabulary
    act: str = "bf16"      # activations, attention/router/head weights, KV cache
    expert: str = "bf16"   # expert weights
    eps: float = 1e-6      # RMSNorm epsilon

    def __post_init__(self):
        if self.act not in ACT_DTYPES or self.expert not in EXPERT_DTYPES:
            raise ValueError(f"unsupported dtypes act={self.act} expert={self.expert}")
        if self.Hq % self.Hkv:
            raise ValueError("Hq must be a multiple of Hkv")
        if self.expert == "mxfp4" and self.act != "bf16":
            raise ValueError("MXFP4 expert weights go with bf16 activations")

    @property
    def qkv_dim(self) -> int:
        return (self.Hq + 2 * self.Hkv) * self.hd


@dataclass(frozen=True)
class Workload:
    name: str
    model: ModelConfig
    B: int              # independent requests
    P: int              # cached prefix length per request (or prompt length)
    N: int              # canvas length
    S: int              # denoising passes per canvas
    tau: float          # re-noise threshold: keep iff conf >= tau
    seed: int
    canvases: int = 1   # canvases chained by append-prefill


_LAYER = dict(D=2048, Hq=16, Hkv=8, hd=128, E=128, k=8, F=768, V=32768)

WORKLOADS = {
    # one fp32 layer at oracle scale
    "tiny_fp32": Workload("tiny_fp32",
                          ModelConfig(L=1, D=256, Hq=4, Hkv=4, hd=64, E=8, k=2, F=512, V=1024,
                                      act="f32", expert="f32"),
                          B=1, P=32, N=16, S=4, tau=0.5, seed=0),
    # one bf16 MoE layer, 1024-token cached prefix, 256-token canvas, 8 passes
    "layer_p1024": Workload("layer_p1024", ModelConfig(L=1, **_LAYER), B=1, P=1024, N=256, S=8,
                            tau=0.5, seed=1),
    # the same layer with an 8192-token prefix (attention-heavy pass)
    "layer_p8192": Workload("layer_p8192", ModelConfig(L=1, **_LAYER), B=1, P=8192, N=256, S=8,
                            tau=0.5, seed=2),
    # eight layers, 4096-token prompt, four chained canvases of 16 passes
    "stack8_chain4": Workload("stack8_chain4", ModelConfig(L=8, **_LAYER), B=1, P=4096, N=256,
                              S=16, tau=0.7, seed=3, canvases=4),
    # eight independent requests, fp8 e4m3 expert weights with per-expert scales
    "batch8_fp8": Workload("batch8_fp8", ModelConfig(L=1, expert="fp8", **_LAYER), B=8, P=2048,
                           N=256, S=8, tau=0.5, seed=4),
}

# The 1024-prefix layer with 4-bit (MXFP4) expert weights: the same pass with
# a quarter of the expert bytes (course page, dense-8B solution: four-bit
# packing).
WORKLOADS["layer_p1024_mxfp4"] = Workload("layer_p1024_mxfp4", ModelConfig(L=1, expert="mxfp4", **_LAYER),
                                          B=1, P=1024, N=256, S=8, tau=0.5, seed=1)

# The workload the benchmark times on one GPU.
BENCH_WORKLOAD = "layer_p1024"


def scaled(w: Workload, **kw) -> Workload:
    """A copy of a workload with some fields (or model fields) replaced."""
    model_kw = {k: v for k, v in kw.items() if k in ModelConfig.__dataclass_fields__}
    wl_kw = {k: v for k, v in kw.items() if k not in model_kw}
    m = replace(w.model, **model_kw) if model_kw else w.model
    return replace(w, model=m, **wl_kw)
