"""Seeded synthetic inputs for the tree-verification pass.

This package draws random numbers and nothing else.  It holds none of the
method's arithmetic (no W12 coding, no forward pass, no acceptance rule), so
both the CPU oracle and the HIP path may take their inputs from it without
sharing any computation.

Recipes (sizes and distributions follow the workloads described on the
SpecPilot summary page, section "how it differs", and the configurations this
repository measures):

* linear weights: bf16 bit patterns drawn as fp32 ``sigma_c * N(0, 1)`` per
  output channel, a fixed fraction of exact ``+0.0`` and a disjoint fraction
  of outliers (the Gaussian draw times a multiplier), rounded to bf16 by
  torch's round-to-nearest-even conversion;
* activations and KV contexts: ``N(0, 1)`` rounded to bf16;
* draft trees: best-first growth with random proposal scores (``trees``).

Every generator takes an explicit seed or ``torch.Generator`` so that a
(recipe, seed, device) triple names one input exactly.  The CPU and CUDA
torch generators produce different streams; a workload always states which
one it used.
"""

from .weights import (  # noqa: F401
    LinearRecipe,
    bf16_from_f32,
    gen_linear_bf16,
    gen_normal_bf16,
    gen_sigmas_loguniform,
    make_generator,
)
from .trees import (  # noqa: F401
    best_first_topology,
    batch_sizes,
    assign_tokens_by_depth,
    chain_topology,
)
from .configs import CONFIGS, ModelConfig  # noqa: F401
