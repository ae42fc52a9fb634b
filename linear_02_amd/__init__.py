"""Fused reconstruct-and-project linear for AMD MI355X (gfx950).

    y = s (.) (W0 x) + U (V^T x)

The library libwl.so (HIP kernels behind the C ABI of include/wl.h) is bound in
``linear_02_amd.wl``; ``linear_02_amd.inputs`` draws seeded synthetic inputs;
``linear_02_amd.build`` compiles the library. Importing this package loads
nothing: import ``linear_02_amd.wl`` to load the library.
"""
