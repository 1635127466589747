"""MI355X-native hybrid-tier decode attention (ActiveKV's 8-bit page tier).

The compute path is the C-ABI library ``libakv.so`` (hand-written HIP for
gfx950); ``binding`` marshals torch tensors into it.  Importing this package
does not load the library; ``from quantized_paged_kv_akv_amd import binding``
does, and raises if it is not built.
"""
__all__ = ["binding", "configs", "inputs"]
