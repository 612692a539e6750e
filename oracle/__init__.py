"""fp64 CPU oracle for exact softmax attention.

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
It never imports the HIP library package (``exact_io_aware_27_amd``) and the
library never imports it; the two share no code.

- ``attention``: the plain definition, O = softmax(scale*QK^T)V and
  LSE = m + ln(l), in C (``attn_oracle.c``), fp64, threaded over row blocks.
- ``attention_bwd``: the gradients dQ, dK, dV of that definition for an
  upstream gradient dO, in C (``attn_bwd_oracle.c``), fp64, one thread per
  head.
- ``fp8_oracle``: FP8 (E4M3) block quantization with incoherent processing
  (random-sign Hadamard rotation of Q and K) and the FP8 attention method
  emulated in NumPy, for the FP8 path.
- ``online``: the pages' tiled recurrence (running max m and running sum l)
  and the two-block merge identity, in NumPy fp64, used to pin the reading
  of the recurrence against the definition.
"""

from .oracle import attention, attention_bwd, attention_bwd_dq_rows, build, library_path  # noqa: F401
from .online import merge_partials, online_attention  # noqa: F401
