"""MI355X-native MoE verify-pass layer: per-slot and deduplicating engines.

The compute path is the HIP library built from ``csrc/`` (gfx950 kernels
behind the C ABI declared in ``include/moe_verify.h``); ``binding`` marshals
torch tensors into it and ``synth`` draws the seeded synthetic inputs.
Submodules are imported on demand so that loading ``synth`` never loads the
GPU library.
"""
__all__ = ["binding", "synth", "build"]
