"""fp64 CPU oracle for the head-wise compressed KV cache path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
and never imports it; the only module both sides use is the seeded input
generator ``kvsynth``, which holds none of the method's arithmetic.

Everything is computed in float64 on the bf16/fp32-rounded inputs widened to
float64, so input quantisation is not counted as error.

Sources (page title, then section / equation):

* "DensityKV: Density-Guided KV Cache Compression for Long Video Generation"
  (paper summary page): Method ("Soft-Riesz Density", "Online
  Density-Constrained Bank Update"), appendix A.1, appendix B.1 ("From Riesz
  Energy to a Smooth Crowding Score", "Online Bank Update"), appendix D
  (default constants), appendix E (ablation definitions).
* "Forcing-KV: Hybrid KV Cache Compression for Efficient Autoregressive Video
  Diffusion Models" (paper-notes page): section 3.3 (static structural
  retention formula), section 3.4 (segment similarity and BottomK), section
  3.5 (implementation sketch).
* DensityKV card page, Figure 2 (sink + bank + local window attended together
  through native attention).
* DensityKV paper summary, supplementary "Post-RoPE Attention Geometry"
  (memory keys carry temporal rotary coordinate 0): the memory-key
  re-rotation in ``rope``.

Parity status per function is listed in each module header.
"""
from . import density, attention, forcing, rope  # noqa: F401
