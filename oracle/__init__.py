"""fp64 CPU oracle of the gated delta rule forward pass (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product library never imports, links or calls it, and the
two share no code.

* :mod:`oracle.gdr_oracle` -- ctypes front end of ``gdr_oracle.c`` (token-by-token
  fp64 recurrence, threads over independent (b,h) pairs).
  It also holds the channel-wise write-rate variant (FG2): ``fg2_chunk_fwd`` /
  ``fg2_decode_step``, and the decoupled erase / write gates (Gated DeltaNet-2):
  ``gdn2_chunk_fwd``.
* :mod:`oracle.exact` -- exact rational brute force that multiplies out the
  explicit per-token transition matrices; used to pin the fp64 oracle on tiny
  shapes.
"""
from .gdr_oracle import (build, chunk_fwd, chunk_fwd_prologue, decode_multi,  # noqa: F401
                         decode_step, decode_tree, decode_tree_commit, decode_step_prologue, fg2_chunk_fwd, fg2_decode_step,
                         gdn2_chunk_fwd, library_path, load, prologue_decay,
                         prologue_inputs)
