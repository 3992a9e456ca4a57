"""Seeded synthetic inputs for the compressed sparse KV attention hot path.

This module is shared by the GPU library's tests/benchmark and by the CPU
oracle.  It draws random tensors and encodes them into the storage formats
the kernels consume (fp32, bf16, fp8 e4m3 with a per-tensor scale, MXFP4
with a scale per 32-element block).  It holds
none of the method's arithmetic: no compression, scoring, selection or
attention happens here.

Every tensor gets its own random stream,
``numpy.random.default_rng(SeedSequence([config_id, seed, tensor_id]))``,
drawn in fp32.  Large tensors are drawn in fixed-size chunks, chunk ``c``
from ``SeedSequence([config_id, seed, tensor_id, c])``, so that they can be
generated in parallel and any row range can be regenerated on its own.
"""
from .formats import (bf16_bits, bf16_bits_to_f32, e4m3_encode, e4m3_scale, mxfp4_encode, mxfp8_encode,
                      DT_F32, DT_BF16, DT_E4M3, dtype_name)
from .gen import normal, Tensor, encode
from .configs import CONFIGS, Config, make_inputs

__all__ = [
    "bf16_bits", "bf16_bits_to_f32", "e4m3_encode", "e4m3_scale", "mxfp4_encode", "mxfp8_encode",
    "DT_F32", "DT_BF16", "DT_E4M3", "dtype_name",
    "normal", "Tensor", "encode", "CONFIGS", "Config", "make_inputs",
]
