"""CPU oracle for the event-tensor MoE layer, the split-K GEMM and split-KV decode
attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The HIP library and its Python binding never import it, and it imports nothing
from them: the two sides share no kernels, headers, helpers, tables or constants.
The only module both sides use is the seeded input generator
(``moe_layer_scheduling_amd.synth``), which holds none of the method's arithmetic.

Everything here is plain NumPy in float64, written from the definitions so that a
reader can check each step by eye.  Where the layer rounds to bfloat16 the oracle
rounds too, at the same points, with its own round-to-nearest-even routine
(``oracle.numerics``).

Sources.  The pages this follows are
  * the podcast episode page "Prompt Boundary-Aware Scheduling with Event Tensors for
    Dynamic Kernels" (AI Post Transformers): its summary paragraph names the split-K
    summation example, the symbolic batch-size template, MoE routing handled through
    event counters computed from router outputs, and static versus dynamic scheduling;
  * the OpenAlex record of "Event Tensor: A Unified Abstraction for Compiling Dynamic
    Megakernel" (abstract: event tensors encode dependencies between tiled tasks);
  * the tutorial chapter "5 · Event Tensor et le dynamisme", §5.1 (variable context
    length as a source of shape dynamism), §5.3 (parameterised dependency structure,
    one compilation) and §5.5 (counter targets computed at run time on the GPU before
    waiting; online load balancing with atomics).
The pages give no formula for RMSNorm, the router, top-k, SwiGLU or the combine.
Each function states the plain reading it takes ("reading: ...").

Parity pins: every function here is pinned by ``tests/test_oracle_*.py`` against
closed forms, hand-worked cases (``tests/golden/``), invariants, library routines
and brute force.  No function is "parity unpinned".
"""

from . import numerics, moe, splitk, sched_model, attention  # noqa: F401
