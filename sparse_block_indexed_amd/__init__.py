"""Block-indexed sparse GQA decode for MI355X (gfx950).

The compute path is the C-ABI library ``libsa.so`` (hand-written HIP kernels),
reached through the thin ctypes binding in ``sparse_block_indexed_amd.ops``.
Importing this package loads nothing; the library is loaded on first use and
raises if it has not been built.
"""
__all__ = ["inputs", "bytes_model"]
