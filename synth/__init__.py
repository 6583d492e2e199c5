"""Seeded synthetic workloads for the hybrid compressed-attention hot path.

This package only draws random numbers and stores them in the storage formats
the kernels read (OCP FP8 E4M3FN codes, BF16 bit patterns, packed MXFP4 codes
with E8M0 scales, or plain f32).  It holds none of the method's arithmetic: no
pooling, no RoPE, no scoring, no selection, no attention and no quantizer of its
own.  FP8 and BF16 codes come from PyTorch's dtype casts of drawn values;
MXFP4 codes and E8M0 scales are drawn directly as integers.

Both the CPU oracle (through the tests) and the HIP library consume the same
arrays produced here.
"""
from .configs import (CONFIGS, Geometry, TINY_GEOMETRY, FULL_GEOMETRY,  # noqa: F401
                      config_by_name)
from .gen import (tiny, csa_decode, hca_decode, csa_prefill, ragged_pair,  # noqa: F401
                  swa_layer, make, fp8_codes, bf16_bits, mxfp4_draw)
