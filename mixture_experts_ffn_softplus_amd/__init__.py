"""MI355X-native mixture-of-experts FFN block: router, permutation, grouped SwiGLU experts and
weighted combine with shared experts, as hand-written HIP kernels for gfx950 behind a C ABI.

``configs`` and ``synth`` (workload shapes and seeded inputs) import without the GPU library;
``api`` loads the compiled library and fails loudly when it is missing.
"""
from .configs import MoEConfig, PRESETS  # noqa: F401
