"""MLA (multi-head latent attention) query path, absorbed decode and causal prefill on AMD MI355X.

The computation runs in hand-written HIP kernels for gfx950 behind the C ABI of include/mla.h
(libmla.so); `binding` marshals torch tensors to it. Build with
`python -m head_latent_attention_fp32_amd.build`.
"""
__all__ = ["binding", "build"]
__version__ = "0.1.0"
