"""Reference oracle for batched lossless draft verification and the prefix scheduler.

TEST INFRASTRUCTURE ONLY.  Plain, slow, float64 CPU code written from the
pages' statement of the method.  It shares no code with the HIP library and
imports nothing from it.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path never
does.

Modules
-------
verify    speculative-sampling verification (temperature softmax, accept test,
          first-reject scan, residual / bonus inverse-CDF draw) and its greedy
          (temperature 0) limit.
schedule  confidence-scheduled verification depth (CumProd survival, greedy
          throughput-improving prefix extension under a token budget).
acceptance  per-position acceptance overlap alpha = sum min(p, q) = 1 - TV,
          and verification with the draft distribution given as logits.
calibration  Sequential Temperature Scaling (apply c^(1/T_k); the left-to-right
          grid fit on the cumulative survival's 15-bin ECE) and the static
          scheduler's fixed-length and threshold modes.
tree      greedy verification of a candidate tree (the acceptance walk after
          the target's ancestor-masked pass).
dcut      ratio-budgeted depth (top-K scores for each ratio budget, the ratio
          that maximises estimated progress over profiled cost) and
          verification over densely packed target rows.

Every function is pinned by a ``-m "not gpu"`` test (tests/test_oracle_pins.py,
tests/test_oracle_dcut.py, tests/test_oracle_acceptance.py,
tests/test_oracle_calibration.py, tests/test_oracle_tree.py) against what the pages and the mathematics fix;
none is "parity unpinned".
"""

from .verify import (  # noqa: F401
    bf16_bits_to_f64,
    target_probs,
    accept_draft,
    residual,
    inverse_cdf,
    verify,
    verify_greedy,
    row_is_bad,
)
from .schedule import survival, schedule, schedule_value, brute_force  # noqa: F401
from . import dcut  # noqa: F401  (module: oracle.dcut.dcut, oracle.dcut.verify_packed, ...)
from . import acceptance  # noqa: F401,E402
from . import calibration  # noqa: F401,E402
from . import tree  # noqa: F401,E402
