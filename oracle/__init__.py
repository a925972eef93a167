"""fp64 CPU oracle of the KV/activation transform-and-quantize path.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the benchmark's CPU
baseline leg, never by the library.  It shares no code with the HIP path.
"""
from .kvq_oracle import (MODES, NSN_MODE, NsnQuantized, Quantized, Spec, StreamState, attention_decode, attention_decode_stream, dequantize, expand_scales, hadamard_matrix,  # noqa: F401
                         inverse_rotate, pack_nibbles, qmax, quantize, reconstruction_errors,
                         nsn_dequantize, nsn_quantize, rotate, score_decode, stream_state, unpack_nibbles,
                         RRS_GROUP, RrsActivations, rrs_gemm, rrs_quantize_act, rrs_quantize_weights,
                         rrs_smooth_scales)
