"""CPU oracle for SageBwd trainable INT8 attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the
HIP library and its Python binding) never calls it, and the two share no code:
the oracle is plain NumPy in float64, with IEEE float32 steps emulated through
``np.float32`` where the method's quantizers fix float32 arithmetic.

Sources (the SageBwd pages):
  * "SageBwd: A Trainable Low-bit Attention" (arXiv 2603.02170), abstract:
    INT8 attention that quantizes six of the seven attention matmuls;
    quantization error is dominated by the score gradient dS; K-smoothing is
    essential, Q-smoothing optional.
  * "SageAttention3: Microscaling FP4 Attention for Inference and An
    Exploration of 8-Bit Training" summary, sections "Approach", "Measured
    effects" (the ablation on the precision of dO.V^T) and "Surprising
    findings": the one matmul left in 16-bit float is dO.V^T.
  * The FlashAttention / FlashAttention-2 papers listed under "Builds on" give
    the forward/backward structure (online softmax, LSE, Delta = rowsum(dO*O)).

Modules:
  exact     -- textbook attention forward/backward in float64 (mode "exact").
  faithful  -- the quantized algorithm step by step (mode "faithful"): the same
               INT8 codes, block scales and integer tile products as the method
               defines them; a ``rounding=False`` switch removes every rounding
               step so the result must collapse to ``exact``.
  mxfp8     -- the FP8 variant for MI355X's scaled matrix instructions: OCP
               E4M3 codes with one power-of-two (E8M0) scale per 32 x 32 block,
               step by step, with the same ``rounding=False`` switch.
  fp4       -- the FP4 inference forward (SageAttention3 summary, "Approach")
               in the MXFP4 form of MI355X's scaled matrix instructions: E2M1
               codes with one E8M0 scale per 32 values of the contraction
               index, step by step, with the same ``rounding=False`` switch.
  metrics   -- cosine similarity, relative L2, L1, RMSE.

Every function here is pinned by ``tests/test_oracle_*.py`` against something
other than itself: finite differences, closed forms, invariants, brute-force
integer products, an exact-rational quantizer and the rounding-free reduction.
"""
from . import exact, faithful, fp4, metrics, mxfp8  # noqa: F401
