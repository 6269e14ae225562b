"""Plain fp64 CPU oracle for fused attention over packed segments.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, calls or links anything in this package; only
the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the GPU path.

What it computes is the textbook definition of masked scaled-dot-product
attention and its analytic gradient, written out with dense matrices, one
(batch row, query head) at a time.  The sources it follows:

* "[JAX] Align fused attn backward output gradient sharding and other test
  strengthening" (TransformerEngine PR 3516): the forward output is saved for
  the backward, which returns Q/K/V gradients (Diagram); THD metadata for Q
  and KV, a fast path when they match and a general path when they differ
  (Changes 3 and 4).
* "[JAX] Fix batcher in FusedAttn primitive for when seg ids bdims != seg
  pos bdims" (TransformerEngine PR 2692): metadata are (segment_ids,
  segment_pos) pairs of shape [batch, seqlen], pos derivable from ids
  (Description).
* maxdiffusion PR 485 (custom splash / ring attention backward): GQA with
  dK/dV accumulated over the query heads of a group (Code Review, Key
  Features), gradient isolation of padding (Testing).
* "[JAX] Make all jax attention calls use non-packed common calls"
  (TransformerEngine PR 2358): separate qk and v head dims (review of the
  KV-packed stride); zeroed gradients for ragged layouts (Greptile Overview).

``variants.py`` adds the attention variants the TransformerEngine pages
name without defining (additive bias and its gradient, score modification
by soft-capping, a sink logit and its gradient, the per-head maximum logit);
its readings are stated in its docstring.

Every function here has a pin in ``tests/test_oracle_pins.py`` or
``tests/test_oracle_variant_pins.py`` that ties it to something other than
itself (finite differences, closed forms, a library routine for the special
cases it reduces to, brute force on tiny inputs).
"""

from .attention import (  # noqa: F401
    allowed_mask,
    backward,
    derive_pos,
    fast_route_eligible,
    forward,
    kv_head_of,
    resolve_segments,
)
from .variants import backward_ex, forward_ex  # noqa: F401,E402
