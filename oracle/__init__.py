"""Oracle: plain, slow CPU reference implementations (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The library (``exact_attention_48_amd``)
never imports it and shares no code with it; the only module both sides use
is the seeded input generator ``exact_attention_48_amd.inputs``, which holds
no attention arithmetic.

  attention.py   float64 NumPy attention forward/backward (the definition), split-KV
                 partial results and their merge, FP8 (E4M3) Q/K forward
  bruteforce.py  pure-Python loops with math.fsum, tiny inputs only
"""
from .attention import (attention_forward, attention_backward, backward_rowdot,  # noqa: F401
                        head_forward, head_backward, head_backward_dq_rows, head_scores,
                        attention_forward_split, head_forward_keys, merge_partials, split_chunk,
                        attention_forward_fp8, e4m3_to_float)
