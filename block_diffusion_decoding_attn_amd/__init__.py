"""MI355X-native cached block-diffusion denoising step (Fast-dLLM / Fast-dLLM v2).

The step runs as hand-written HIP kernels for gfx950 behind the C ABI declared
in include/fdl.h (libfdl.so); `fdl` is the thin ctypes binding over it and
`synth` draws the seeded synthetic inputs.
"""
