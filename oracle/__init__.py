"""fp64 CPU oracle for causal softmax attention: forward, backward, GProj and
backward-over-backward.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import, call or execute anything in this
package.  It shares no code with the HIP library and never imports it; the HIP
path never imports this package.

Modules:
  attention   dense definitions (fwd, bwd, bob, hvp, rows, last_columns, gproj_project;
              grouped-query forms fwd_gqa, bwd_gqa, bob_gqa)
  online      the tiled online-softmax forward recurrence, as a model
  rounding    bf16 round-to-nearest-even and a rounding model of the bf16
              backward with and without GProj
  fp8         E4M3 codes, the Hadamard rotation, block quantisation and the
              FP8 forward model (import as oracle.fp8)
"""
from .attention import (probs, fwd, bwd, bob, hvp, rows, last_columns,  # noqa: F401
                        gproj_project, max_prob, expand_kv, reduce_kv, fwd_gqa, bwd_gqa,
                        bob_gqa)
from .online import online_fwd  # noqa: F401
