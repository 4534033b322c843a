"""Mixed-fidelity paged-KV attention for MI355X (gfx950).

The compute path is the HIP library ``libekv.so`` (C ABI in ``include/ekv.h``);
``mixed_precision_paged_amd.ekv`` is its thin Python binding.  Importing this
package does not load the library; importing ``.ekv`` does, and fails loudly
if the library has not been built.
"""
__all__ = ["synth", "bytemodel"]
