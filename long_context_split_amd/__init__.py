"""MI355X-native DFlash2 verification attention (paged E4M3 KV, 80 logical splits).

The compute path is the HIP library ``libdfv.so`` built from ``csrc/`` for gfx950
and reached through the C ABI declared in ``include/dfv.h``.  :mod:`.dfv` is the
thin ctypes binding; :mod:`.synth` draws seeded synthetic inputs.  Importing the
package does not load the library: :func:`long_context_split_amd.dfv.lib` does,
and raises if it has not been built.
"""
__all__ = ["dfv", "synth"]
