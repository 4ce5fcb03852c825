"""Chunked exact causal attention on MI355X (gfx950).

The C ABI is in include/chunk_attn.h and the HIP kernels in csrc/. The ctypes
binding is ``sequence_chunked_exact_amd.binding``; import it explicitly (the
workload generator does not need the built library).
"""
