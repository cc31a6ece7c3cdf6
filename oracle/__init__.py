"""fp64 CPU oracle for block-sparse attention with mean-pooled block selection.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import anything from this package.
It shares no code with the GPU path (no kernels, headers, helpers, tables or
pre/post-processing) and imports nothing from it.

What it computes, and where the pages say so:

* SLA post ("what the idea is", page 1): attention is split into critical,
  negligible and intermediate parts; critical blocks get softmax attention,
  negligible ones are skipped, intermediate ones get linear attention; a mean
  pooling step marks the blocks beforehand.
* NABLA post (page 3, points 2-4): Q and K are compressed, blocks are ranked
  by the cumulative distribution of the softmax of the compressed scores, and
  the blocks whose summed mass reaches the threshold 1 - thr are computed.
* Veda article (page 5, "what happened"): attention is computed only on the
  128-token key tiles selected for each query.

* SLA post ("results"): the method is trainable with a short fine-tuning;
  ``grad.py`` holds the gradients of the forward with the class map fixed.
* Veda article ("context"): heads get their own tile shapes; ``tiles.py``
  orders the tokens of a latent grid into per-head 3D boxes.

Every function is the plain definition, in fp64, with numpy BLAS matmuls as
the only library step.  Readings of points the pages leave open are listed in
``sla.py``'s header.

Parity status: every function here is pinned by the CPU tests (closed forms,
brute-force enumeration, special cases that reduce to library routines,
invariants, hand-derived fixtures under tests/golden; the gradients by central
finite differences and by torch autograd of dense attention).  The end-to-end values
on the structured workloads have no published number to hit; they are pinned
only through those parts.
"""

from . import grad, sla, tiles  # noqa: F401
