"""CPU oracle for the blockwise-FP8 linear layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
restatement of what the FP8 linear path computes.  It exists to check the HIP
kernels; it is never part of the product path.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code, tables or helpers with the HIP library and
imports nothing from ``blockwise_fp8_linear_quant_amd``.

Sources (the Puro-2B report as summarised on the web):

* arxiv-wiki summary "Puro-2B: Poor Lab's Qwen2-1.5B Trained on RTX 5090
  within $5090", section "접근 방법" (approach), item (4): the main linear
  operations run in blockwise E4M3 FP8; activations carry one scale per 1-D
  group of 128, weights one scale per 128x128 block; master weights and
  optimizer state stay BF16/FP32.  Same page, section "개발자 관점"
  (developer view): the main GEMMs use this grouping, which follows the
  DeepSeek-V3 scheme.
* paperlayer.ai summary of arXiv 2608.27370v1, appendix C "生産学習の詳細"
  (production training details), item "FP8実装pipeline": blockwise E4M3 is
  applied to the linear-layer GEMMs -- forward, data-gradient and
  weight-gradient -- while hidden/residual flow stays BF16 and gradients stay
  FP32.

What the pages leave open (scale formula, rounding, saturation, layouts) is
fixed by the readings listed in the design notes; each function states the
reading it implements.

Modules:
    e4m3     -- OCP E4M3 decode/encode (round-to-nearest-even, saturating).
    quant    -- 1x128 group quantisers (both orientations), 128x128 blocks.
    gemm     -- the block-scaled GEMM as dequantise-then-matmul in float64,
                plus the per-element error budget sum |a*b|.
    compare  -- the acceptance tests applied to GPU results.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
closed forms, brute force and invariants that do not reuse its code.
"""

from . import e4m3, quant, gemm, compare  # noqa: F401
