"""CPU oracle for MTP rejection-sampling verification and the end-to-end TV loss.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header,
constant table or helper with the HIP library in ``tv_loss_amd/`` and imports
nothing from it.

Everything here is deliberately plain and slow: NumPy in float64, one row at a
time, every quantity computed from its textbook definition.  The sources are the
pages on "Breaking Entropy Bounds: Accelerating RL Training via MTP with
Rejection Sampling" (Bebop; arXiv 2606.12370), cited by page and section:

* paperlayer.ai summary (English): Sec. 2 "Preliminaries" (acceptance methods),
  Sec. 3 "Rejection Sampling", Sec. 4 "End-to-end TV loss", Sec. 8 "Total
  Variation Distance in Machine Learning", App. A "Derivation of TV Loss
  Gradient", App. F "Fused TV Loss Kernel", App. G.1 "Multinomial Draft
  Sampling (SGLang)".
* paper.rainbus.top summary (Chinese): prerequisites "Rejection Sampling",
  "Total Variation Distance", "Entropy"; "Method steps"; "Technical novelty".
* arxiv.myfastools.com page (a different paper, EntMTP): Related Work,
  "Speculative Decoding" -- the textbook speculative-sampling rule.

Modules
  philox   Philox4x32-10 counter-based generator (Salmon et al., SC'11).
  bf16     exact bfloat16 <-> float64 conversion (round to nearest even).
  mtp      verification (rejection sampling and target-only), overlap / TV /
           entropy, residual sampling, the
           end-to-end TV loss, its gradient.

Parity status: every function is pinned by a ``-m "not gpu"`` test against a
library routine, a closed form, an invariant or brute force.  The 32-bit Philox
constants are pinned against rocRAND's Philox4x32-10 engine (compiled at test
time from its header); the round structure is also pinned against NumPy's
Philox4x64-10.
"""
from . import bf16, philox, mtp  # noqa: F401
