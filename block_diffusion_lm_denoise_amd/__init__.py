"""MI355X-native block-diffusion denoising pass (libdgpass) and its Python binding.

The compute runs in hand-written gfx950 HIP kernels behind a C ABI
(include/dgpass.h); this package only marshals arguments, owns device memory
through PyTorch, and drives the block-chaining loop.
"""
from .configs import BENCH_WORKLOAD, WORKLOADS, ModelConfig, Workload, scaled  # noqa: F401
