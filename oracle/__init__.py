"""CPU oracle for the attention forward with online softmax.

TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's CPU
baseline import this package; the product path (the HIP library and its
Python binding) never does, and the two share no code.

- `attention(...)`: float64 three-pass safe-softmax attention (plain C).
- `softmax_rows(x)`: float64 three-pass safe softmax of every row of a matrix
  (the standalone row-softmax operation).
- `fp8.attention_fp8(...)`: float64 attention of FP8 (E4M3) inputs with
  per-tensor descales; `fp8.e4m3_decode` / `fp8.e4m3_round` (the format by
  its definition); `fp8.online_attention_e4m3` (the Max_offset recurrence
  with E4M3-rounded probabilities, a model of the rounding).
- `attention_bwd(...)`: float64 gradients dQ, dK, dV of the attention forward
  (numpy, one head at a time).
- `softmax_ref.safe_softmax`, `softmax_ref.online_softmax`,
  `softmax_ref.online_two_pass`, `softmax_ref.online_attention`,
  `softmax_ref.merge_states`: score-level and blocked references used to pin
  the three-pass oracles (and vice versa).
"""
from .attention import attention, build, fully_masked_rows, load, max_threads  # noqa: F401
from .softmax_rows import softmax_rows  # noqa: F401
from .attention_bwd import attention_bwd  # noqa: F401
from . import softmax_ref  # noqa: F401
from . import fp8  # noqa: F401
