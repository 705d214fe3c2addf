"""MI355X-native Depth Exploration Decoding (DEX) lattice step.

The compute path is the HIP library ``libdex.so`` (sources in ``csrc/``, C ABI
in ``include/dex.h``); ``dex`` is its ctypes binding and ``build`` compiles it
for gfx950.
"""
