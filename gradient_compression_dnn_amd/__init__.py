"""gradient_compression_dnn_amd: per-step gradient compression (AdaComp,
DGC, run-length packing, decompress-aggregate, DCD random quantization) as
hand-written HIP kernels for MI355X (gfx950) behind the libgradcomp C ABI.

Submodules:
  binding    ctypes binding of the C ABI (same names as include/gradcomp.h)
  workloads  seeded synthetic segment tables and inputs
  build      hipcc build of libgradcomp.so
Nothing is imported eagerly, so ``workloads`` works without torch or the
built library.
"""
