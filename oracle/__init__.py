"""CPU oracle for the INT4 weight-only hot path -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference that the HIP
library is checked against.  It is written in numpy (fp32 where the method
fixes fp32, fp64 for every dot product) from the pages' statement of the
method, and it shares no code with the GPU path: no kernels, headers,
helpers, tables or constant generators.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (``int4_weight_only_amd``) never does.

Sources, cited by title and section throughout:

* "Quantization basics: from FP32 to INT4" (量化基础：从 FP32 到 INT4 的压缩艺术,
  wsisp.com tutorial) -- §1.3 format table (INT4 grid [-8, 7]), §2.1 affine
  map, §2.2 symmetric quantization, §2.4 error bound |x_hat - x| <= s/2,
  §3 granularity (per-group), §5 error sources (rounding mode), §6.1 the
  worked numpy INT8 example and its printed output, §6.2 (torch.round is
  half-to-even), FAQ Q2/Q5.
* "INT4 QAT end-to-end for RL" (SGLang RL / slime / Miles write-up, Chinese
  copy on miaoxiaomiao.cn) -- §2.1 fake quantization and STE, §3.2
  quantization at weight update and the 8 x INT4 -> INT32 packing (Fig. 4),
  §4 inference (W4A16, moe_align_block_size, fused MoE / gating).
* "Quantization-aware training" tag summary (量化感知训练, reportify.cn) --
  bullets [8]-[11] (training/inference scheme, 1x32 scale granularity),
  [32] (compact INT4 storage), [35] (dynamic moe_align_block_size, fused
  gating).

Modules:

* ``bf16``  -- bfloat16 round-to-nearest-even and widening.
* ``quant`` -- symmetric group quantization, pack/unpack, dequant, fake quant.
* ``gemm``  -- fp64-accumulated W4A16 reference product.
* ``moe``   -- routing, block-size rule, moe_align_block_size, grouped
  expert GEMM, SwiGLU activation, top-k combine, the whole MoE layer.

Every function is pinned by ``tests/test_oracle_*.py`` against something
other than itself (the tutorial's printed numbers, exact rational
arithmetic, closed forms, brute force).  Functions without such a pin say
"parity unpinned" in their docstring.
"""

from . import bf16, quant, gemm, moe  # noqa: F401
