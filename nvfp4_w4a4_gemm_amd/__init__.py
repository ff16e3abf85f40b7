"""NVFP4 W4A4 prefill linear layer for MI355X (gfx950).

The layer's work runs in the HIP library ``libnvfp4_w4a4.so`` (built from
``csrc/``) behind a C ABI; ``nvfp4_w4a4_gemm_amd.binding`` marshals torch
tensors into it.  Importing this package does not load the library; the
binding does, and raises if it is missing.
"""
__all__ = ["binding", "workloads"]
