"""CPU oracle (fp64) for group-wise affine low-bit QMV.

TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import it.  It shares no code with the HIP
library.
"""
from .qmv_oracle import *  # noqa: F401,F403
from .qmv_oracle import (T5_MAX_BYTE, abs_mass, algorithmic_bytes, bits_of, check_close,
                         codes_of, dequant_f16, dequant_f64, effective_biases, pack_words,
                         qmv_brute, qmv_f64, qmv_reference, sym_ratio, t5_group_bytes,
                         t5_pack, t5_unpack, t5_unpack_scalar, tolerance, unpack_words,
                         unpack_words_scalar, weights_f64)
from .spec_oracle import spec_verify, spec_verify_scalar, target_tokens
