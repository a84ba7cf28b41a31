"""Fused MoE expert stage for MI355X (gfx950): router softmax/top-k, stable
sort of (token, expert) pairs, bf16 MFMA grouped GEMMs with a SwiGLU epilogue,
weighted combine, forward and backward.

The product is the C-ABI library ``libmoe.so`` (include/moe.h) built from
``csrc/``; ``binding`` is its ctypes binding and ``synth`` the seeded synthetic
inputs. Importing the package loads nothing; ``from mixture_experts_expert_amd
import binding`` loads the library and fails if it is not built.
"""
