"""MI355X-native fused edge tensor-product convolution (libetp).

The product is the C ABI in include/etp.h, implemented by HIP kernels for
gfx950 in ``csrc/`` and built in-tree into ``libetp.so``
(``python -m equivariant_interatomic_potentials_amd.build``). The Python
binding with the same names lives in ``equivariant_interatomic_potentials_amd.etp``;
it is not imported here so that the build module can run before the library
exists.
"""
__all__ = ["etp"]
