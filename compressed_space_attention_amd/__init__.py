"""IsoQuant compressed-space attention on MI355X (gfx950).

The compute path is the C-ABI library ``libisoquant.so`` (hand-written HIP
kernels); ``compressed_space_attention_amd.isoquant`` is its thin Python
binding.  Importing this package does not load the library; importing
``.isoquant`` does, and fails loudly if it has not been built.
"""
