"""CPU oracle of the H-BitLinear forward pass (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package.  The product path (``bit_quantized_gemm_bitlinear_amd``) never
imports it and shares no code with it.

The arithmetic lives in ``hbl_oracle.c`` (plain scalar C11, OpenMP over rows); this module
only builds that file with gcc and marshals numpy arrays through ctypes.
"""
from .oracle import (  # noqa: F401
    BF16,
    F32,
    build,
    dense_reference,
    dequant,
    forward,
    ffn_forward,
    fwht_f32,
    fwht_f64,
    gemm_s32,
    lib_path,
    num_threads,
    pack_bits,
    pack_codes,
    pack_codes_fp6,
    pack_weights_fp4,
    unpack_codes_fp6,
    pack_weights,
    quantize_activations,
    quantize_qkv,
    quantize_weights,
    round_bf16,
    set_num_threads,
    swiglu,
    unpack_bits,
    unpack_codes,
    dequantize_qkv,
    unpack_weights,
)
