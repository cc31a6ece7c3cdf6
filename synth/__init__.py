"""Seeded synthetic inputs for block-sparse attention with mean-pooled block selection.

This package builds Q, K and V as bf16 bit patterns (numpy ``uint16``) and
describes the five workloads.  It holds none of the method's arithmetic: no
pooling, no scores, no selection.  Both the fp64 oracle and the GPU path read
their inputs from here, and nothing here imports either of them.

Workloads (token counts and tile sizes follow the pages' settings):

* the SLA post (page 1, "what the idea is") fixes mean pooling over blocks;
* the Veda article (page 5, "what happened") fixes 128-token key tiles and
  95% / 90% sparsity at a 245k-token layer;
* the NABLA post (page 3, points 2-3) fixes the softmax-CDF cut with a
  threshold parameter.
"""

from .configs import CONFIGS, Spec, spec_for
from .generate import generate, generate_head, load_repairs

__all__ = ["CONFIGS", "Spec", "spec_for", "generate", "generate_head", "load_repairs"]
