"""invariant_attention_amd: batch-invariant paged attention for MI355X (gfx950).

The compute path is libinvattn.so (hand-written HIP + a host page table, C ABI
declared in include/invattn.h); `binding` is a ctypes layer over it with the
same entry-point names.  Importing the package does not load the library;
`binding.load()` does, and raises if it has not been built.
"""
__all__ = ["binding"]
