"""CPU oracle for the DeepSeekMoE FP8 block-scaled layer forward.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plainly written reference
that the HIP library is checked against.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import it; the library and its Python
binding never do, and nothing here imports them.  It shares no code, tables or
constants with the HIP kernels.

Everything is NumPy, evaluated in float64 unless a step is defined in float32
(quantisation scales, affinities, keys), and each function cites the passage
of the source pages it follows.  Citation shorthand used in this package:

* "V3 notes" -- the xutianle.me blog post "DeepSeek-V3 技术报告：从 671B MoE 到
  低成本训练系统" (a walk-through of the DeepSeek-V3 technical report); sections
  are that post's own numbering (§2 DeepSeekMoE, §4 auxiliary-loss-free load
  balancing, §4.2 node-limited routing, §6 FP8 mixed precision, §6.1
  fine-grained quantisation, §6.2 higher-precision accumulation).
* "infra answer" -- the second answer ("from the infra point of view") on the
  51itzy.com DeepSeek-V3 Q&A page, paragraphs on FP8 and on group routing.
* "evolution post" -- the "deepseek-evolution" blog post, V3 sections
  "FP8 mixed-precision training" and "auxiliary-loss-free load balancing".

Where those pages are silent or their formulas were lost, the reading taken
is stated at the function that implements it.

Modules
-------
e4m3   -- the OCP E4M3FN codec (encode with round-to-nearest-even, decode)
quant  -- 1x128 activation and 128x128 weight quantisation
gemm   -- block-scaled FP8 GEMM with per-128-K promotion (float64)
route  -- sigmoid affinity, bias-adjusted group-limited top-K, gates, permute
layer  -- expert SwiGLU FFN and the whole MoE layer forward
bias   -- auxiliary-loss-free bias update
"""

from . import e4m3, quant, gemm, route, layer, bias  # noqa: F401
