"""MI355X-native DSA token selection and selected-token attention.

The compute path is the C-ABI library ``libdsa.so`` (hand-written HIP kernels
for gfx950) declared in ``include/dsa.h``; ``dsa_decode_amd.ops`` is a thin
binding with the same names.  Importing this package loads nothing; the first
call into ``ops`` loads the library and fails loudly if it is not built.
"""
__all__ = ["ops", "synth"]
