"""MI355X (gfx950) trellis dequantize-and-multiply.

``dequant_gemm_trellis_amd.trellis`` is the binding over the C-ABI library
``libtrellis.so`` (HIP kernels); importing it raises if the library is not
built. ``dequant_gemm_trellis_amd.synth`` holds the seeded input generators.
"""
