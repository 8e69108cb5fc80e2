"""CPU oracle for the quantized KV cache and decode attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
baseline may import this package.  The product (the HIP library and its Python
binding) never calls it, and the two share no code: the oracle is written from
the method's definitions, in float64 numpy, slowly and plainly.

Modules
  numerics   fp16 / OCP E4M3 / E2M1 rounding and decoding
  quant      affine group quantizer and NVFP4 block quantizer
  layout     byte layout of a 128-token cache block and of the fp16 residual
  cache      residual + tier schedule and the packed arenas it produces
  attention  single-token softmax attention in float64
  sizes      KV-cache size formula
"""
from . import numerics, quant, layout, cache, attention, sizes  # noqa: F401
