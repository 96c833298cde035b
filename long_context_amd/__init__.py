"""Kascade cross-layer top-k sparse attention for AMD MI355X (gfx950).

The compute path is libkascade.so (HIP kernels behind the C ABI in
include/kascade.h); `long_context_amd.kascade` is its Python binding and
`long_context_amd.synth` draws seeded synthetic inputs.
"""
