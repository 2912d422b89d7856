"""fp64 CPU oracle for TARA attention. Test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may
import this package; the product library never does.
"""
from .tara_oracle import (TARGET, GUIDE, PICTURE, OTHER, penalty, saturation_gap,  # noqa: F401
                          bias_block, attention_head, attention, merge_partitions,
                          attention_bruteforce, three_term_parts, fp8_e4m3_round, pow2_scale,
                          qk8_dequantize)
