"""libkda: Kimi Delta Attention forward pass for AMD MI355X (gfx950).

The compute path is the C-ABI shared library ``libkda.so`` (hand-written HIP
kernels, see ``include/kda.h``); ``libkda`` is its thin Python binding.
"""
