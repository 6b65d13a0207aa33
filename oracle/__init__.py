"""CPU oracle for the 8-bit quantized, optionally block-sparse attention forward.

TEST INFRASTRUCTURE ONLY. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package; the product path never
calls it and shares no code with it (the HIP kernels, the C ABI and the Python
binding are written separately and import nothing from here).

Everything here is plain numpy (fp64 unless a step fixes another precision),
written for reading, not for speed:

* ``exact_attention``     -- the result the method approximates: softmax
  attention in fp64, optionally restricted to a block mask.
* ``smooth_quant``        -- the K smoothing and per-block INT8 quantization of
  Q and K, with optional mean-pooled block vectors.
* ``block_mask``          -- the mean-pooled block score and the per-query-block
  keep list.
* ``emulate_attention``   -- the quantized path step by step: INT8 scores,
  online base-2 softmax, rounded probabilities, fp64 accumulation.
* ``emulate_promoted_attention`` / ``promote_plan`` -- promote instead of
  skip: the kept blocks at 16-bit Q K^T, every other visible block through
  the INT8 path, merged by the same online softmax.
* ``emulate_promoted_fp4_attention`` (module ``promote_fp4``) -- promote
  instead of skip with an MX FP4 low path: the kept blocks at 16-bit Q K^T,
  every other visible block at 4-bit Q K^T, the same online softmax.
* ``lowbit_block_mask`` (module ``lowbit``) -- the element-level 4-bit
  block estimator: MX FP4 Q and smoothed K, the block score as the largest
  estimated product over the block's visible pairs, the same selection rule.
* ``predict_patterns`` (module ``patterns``) -- vertical and slash lines
  predicted from the votes of the per-query-block selections, added to every
  query block's plan.
* ``stripe_select`` / ``emulate_stripe_attention`` (module ``stripes``) --
  anchor-based stripe selection (keys within a threshold of the anchor taken
  over the initial tokens and the local window) and the quantized path over
  the gathered keys.
* ``head_error`` / ``adaptive_lists`` -- adaptive per-head precision: a
  sampled RMS logit error of the INT8 path per head, and the kept lists that
  run the heads above a threshold entirely at 16-bit Q K^T.

Sources (the explainer pages these follow):

* SageAttention explainer, aibr.jp/archives/102657, sections 2-3: smooth K,
  quantize the attention inputs to 8 bits, INT8 matrix products for Q K^T and
  16-bit products for P V, FlashAttention-style tiling (section 4).
* ThriftAttention summary, gist.science/ja/paper/2605.23081, technical summary,
  method: block importance from the dot product of the block mean vectors,
  top-k block pairs, online softmax merge as in FlashAttention-2.
* AnchorAttention explainer, aibr.jp/archives/118418, section 3: an anchor
  from the initial tokens and a local window, keys selected by their
  difference to it without a sort, discrete key gathers.
* SALE explainer, aibr.jp/archives/118208, sections 1-3: a cheap low-bit
  estimate turned into a block-sparse plan that skips the rest, with the sink
  (first) and local (diagonal) stripes kept; element-level 4-bit estimates of
  the query-key products; vertical and slash lines predicted from the
  attention map's tendencies.

Parity pins: every function here is pinned by CPU tests against closed forms,
invariants, a library routine that computes the same definition, brute force
or hand-worked cases (tests/test_oracle_*.py, tests/golden/). The pages print
no worked example, so no pin is a printed value; the exponentials are numpy's
fp64 exp2 rounded once to fp32, checked by the closed forms up to that
rounding.
"""

from .rounding import bf16_rne, f16_rne, round_to_dtype  # noqa: F401
from .quant import (k_channel_mean, quantize_block, smooth_quant,  # noqa: F401
                    pool_vector_quant)
from .mask import block_mask, max_keep, select_blocks  # noqa: F401
from .attention import (exact_attention, emulate_attention, emulate_promoted_attention,  # noqa: F401
                        promote_plan, softmax_scale_log2, head_error, head_error_sample,
                        adaptive_lists)
from .lowbit import lowbit_block_mask, lowbit_scores, mxfp4_quantize  # noqa: F401,E402
from .stripes import stripe_select, emulate_stripe_attention  # noqa: F401,E402
from .promote_fp4 import emulate_promoted_fp4_attention  # noqa: F401,E402
from .patterns import predict_patterns, pattern_votes  # noqa: F401,E402
