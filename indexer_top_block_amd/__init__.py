"""Indexer-selected block-sparse attention for MI355X (gfx950).

The compute path lives in ``libsparse_attn.so`` (hand-written HIP); ``sparse_attn``
is its ctypes binding.  Importing the package loads nothing: call
``indexer_top_block_amd.sparse_attn.load()`` (or any entry point) to load the library.
"""
