"""MI355X-native GPT-2 training step: HIP kernels for gfx950 behind a C-ABI.

`binding` loads the in-tree `libgpt_hip.so` (built by `build.py`) and exposes
the C entry points with the same names; `synth` draws seeded inputs.
"""
