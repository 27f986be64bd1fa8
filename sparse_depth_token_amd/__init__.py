"""X-MoD sparse-depth layer forward on AMD MI355X (gfx950).

The C ABI (include/xmod.h) lives in libxmod.so, built from csrc/ by
`python -m sparse_depth_token_amd.build`. The ctypes binding is `sparse_depth_token_amd.xmod`;
importing it loads the library and fails if it is missing.
"""
