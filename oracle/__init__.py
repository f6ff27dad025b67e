"""CPU oracle for jagged exact-softmax attention (test infrastructure only).

Plain, slow, fp64 numpy code that states what the GPU path must compute. Only
the tests, the smoke check and the benchmark's CPU-baseline leg may import it;
the product path (the C-ABI library and its Python binding) never does, and
shares no code with it.

Modules:
  attention  forward / backward of exact softmax attention per sequence, and
             the gradient of the relative-position bias table
  plan       the longest-first work list and the offsets scan, as integers
"""
from .attention import forward, backward, bias_grad, valid_pairs  # noqa: F401
from .plan import (build_plan, build_plan_queues, q_tile_cost, kv_tile_cost, sq_chunk_cost, exclusive_scan,  # noqa: F401
                   snake, short_query, N_QUEUES, SHORT_Q_MAX, SHORT_KV_MIN)
