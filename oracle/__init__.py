"""CPU oracle for the fused attention + Ulysses post-attention all-to-all path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or execute
anything under ``oracle/``; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header, table or helper
with the HIP library, and it never reads anything the HIP library produced.

What it computes (sources: the four-language gist.science explainer of arXiv 2607.23264,
"X-Stage: An Overlooked Pipeline Stage for Communication-Computation Overlap in DiT
Inference", technical summary):

* ``attention``: the fused FlashAttention-A2A kernel reaches exactly the result of plain
  attention followed by the post-attention all-to-all ("Contributions", FlashAttention-A2A
  piggybacking item: fusion only changes who issues the stores and when).  So the oracle is
  the textbook definition, softmax(scale * Q K^T) V, in float64 on the bf16 inputs, then an
  explicit Ulysses slab permutation.
* ``ulysses``: the pre-attention (sequence -> heads) and post-attention (heads -> sequence)
  all-to-alls of one rank of a Ulysses group, with full-head shards and receive buffers,
  as plain loops, and one rank's attention layer built from them.
* ``moe``: the mixture-of-experts layer of the expert-wave stand-in (Linear-1, bf16
  intermediate, Linear-2, then the combine all-to-all's row placement) in float64.
* ``burst_gap``: the Burst-Gap issue-time model of the "Methodology" section,
  T_iss(G; K, V) = max(T0_iss(K, V), V / R - G), its two regimes, a labelled fluid-queue
  reading that gives the capacity Q a role (with its isolated-burst limit, from which Q is
  read), and the parameter fits used on microbenchmark sweeps ("Contributions",
  characterisation item).

Pins (tests under ``tests/test_oracle_*.py``): brute force with exact summation on tiny
inputs, torch's float64 scaled_dot_product_attention, closed-form invariants, hand-computed
slab destinations, and hand-evaluated Burst-Gap values from the one drain rate the pages
print.  No function here is "parity unpinned" except where its docstring says so.
"""

from .attention import (  # noqa: F401
    attention_fp64,
    attention_weights_fp64,
    bf16_bits_to_f64,
    round_to_bf16_bits,
    slab_destination,
    ulysses_gather,
    ulysses_scatter,
)
from .ulysses import pre_gather, scatter_heads, ulysses_attention  # noqa: F401
from .moe import moe_layer  # noqa: F401
from .burst_gap import (  # noqa: F401
    fit_burst_gap,
    fit_isolated,
    regime,
    t0_linear,
    t_iss,
    t_iss_fluid,
    t_iss_isolated,
)
