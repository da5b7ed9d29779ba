"""The oracle: a plain, slow, float64 CPU statement of what the hot path computes.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
CPU-baseline leg may import or run anything under oracle/.  The product path
(rl_lora_linear_amd and its HIP library) never imports it and shares no code,
header, constant or helper with it; the two meet only at the seeded inputs in
workloads/, which hold none of the method's arithmetic.

Each function writes out the plain definition of its result in NumPy float64,
citing the passage it follows.  Library primitives (matmul, argsort, exp, log)
serve as steps; there is no tiling, fusion or reordering beyond the definition.
Every function is pinned in tests/test_oracle_*.py against something other than
itself: worked values the pages print, closed forms, invariants, finite
differences, brute force, or an independent library routine.

Modules
  segments  -- per-token adapter ids -> stable order and segment offsets
  lora      -- mixed-adapter LoRA linear layer, forward and backward
  logprob   -- target-token logprob via logsumexp, and its backward
  loss      -- cross_entropy / importance_sampling / ppo / custom dLoss/dlogprob
  adam      -- per-adapter AdamW step
  mlp       -- dense SwiGLU MLP with LoRA on gate, up and down
  moe       -- top-k routed expert layer with per-(expert, adapter) LoRA
"""
from . import adam, logprob, lora, loss, mlp, moe, segments  # noqa: F401
