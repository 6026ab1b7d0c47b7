"""CPU oracle for the KDA forward pass -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg import this package.  The GPU library never calls it and shares no code,
header, table or helper with it.

Contents:
  * ``recurrence``   -- float64 token-by-token gated delta rule (C, OpenMP),
                        the definition of what the forward pass computes;
  * ``recurrence_np``-- the same recurrence in plain numpy, for small inputs;
  * ``backward``     -- float64 gradients of the recurrence by reverse-mode through its token steps
                        (C, OpenMP), the definition of what a backward pass computes;
  * ``chunkwise``    -- float64 chunkwise-parallel form (numpy), an independent
                        algorithm that must reach the same result;
  * ``chunkwise_backward`` -- float64 reverse mode through that chunkwise form (numpy), the
                        algorithm the GPU backward implements, checked against ``backward``;
  * ``layer``        -- float64 fused-layer forward (projections, short conv,
                        gates, norms) around the recurrence.

Parity status of every function here: pinned (see tests/test_oracle_pins.py);
no function is "parity unpinned".
"""
from .core import backward, build, recurrence, recurrence_np, decay_gate, lib_path  # noqa: F401
from .chunkwise import chunkwise  # noqa: F401
from .chunkwise_bwd import chunkwise_backward  # noqa: F401
from . import layer  # noqa: F401
