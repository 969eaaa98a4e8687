"""Source projection of a vocab-sharded output head on MI355X (gfx950).

The GPU work lives in the C-ABI library ``libsb.so`` (hand-written HIP); the
Python side only marshals arguments (``logit_source_projection_amd.sb``).
Importing this package loads nothing; ``sb`` loads the library on first use
and fails loudly when it is missing.
"""
