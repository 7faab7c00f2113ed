"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the
benchmark.

This package holds the workload shapes and random-number recipes only; it
contains none of the reduce-scatter or copy-out arithmetic.  Real training
gradients are replaced by seeded normal samples rounded to bf16, at the layer
shapes the workloads name.

Recipes
-------
Host (numpy; small workloads and CPU tests):
  * rank u of workload c draws from ``numpy.random.SeedSequence([BASE_SEED, c]).spawn(W)[u]``
    (PCG64), parameters in list order;
  * a value is ``standard_normal() * sigma`` in float64, rounded to float32
    (round to nearest even), then to bf16 (round to nearest even);
  * with ``outliers``, each element independently (probability 0.01, a
    uniform draw from the same stream after the normals of that parameter)
    is multiplied by 100 before the roundings.
Device (torch on the GPU; full-size workloads):
  * rank u uses a ``torch.Generator`` on the device seeded with
    ``device_seed(c, u)``; values are float32 ``randn * sigma`` (times 100
    where ``rand < 0.01`` with ``outliers``), rounded once to bf16 by torch's
    float32 -> bfloat16 conversion (round to nearest even); fp32 gradients
    are the same float32 values, not rounded.
Both recipes give N(0, sigma^2) bf16 values; the GPU path and the oracle
always receive the same bytes, whichever recipe made them.
"""
from .workloads import CONTEXT_WORKLOADS, WORKLOADS, Workload, workload  # noqa: F401
from .gen import (  # noqa: F401
    BASE_SEED,
    bf16_bits_from_f32,
    device_seed,
    grads_host,
    grads_device,
    params_host,
    rank_major_device,
)
