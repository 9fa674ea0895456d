"""MI355X (gfx950) implementation of the hot path of 6Bit-Diffusion's dynamic
mixed-precision quantization: block-Hadamard rotation fused with INT8 / NVFP4
quantization, the quantized linear layers, and the per-layer precision
selection.  The compute lives in libhdq.so (HIP, C ABI in include/hdq.h);
`bit_quantized_video_amd.hdq` is its thin Python binding.

Importing the package loads nothing; `from bit_quantized_video_amd import hdq`
loads the library and fails loudly if it has not been built.
"""
__all__ = ["hdq", "synth"]
