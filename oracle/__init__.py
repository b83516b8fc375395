"""Reference oracle for cluster-smoothed progressive residual KV-cache quantization.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It is a plain, slow, CPU
implementation (numpy; fp64 for reductions, IEEE fp32 for the codec) written
from the method's description, and it shares no code, table or constant
generator with the HIP library.

Sources, cited by page title and section throughout:

* "Quant VideoGen: Auto-Regressive Long Video Generation via 2-Bit KV-Cache
  Quantization" (Italian explainer, gist.science/it/paper/2602.02958), below
  "QVG explainer".  Its "Sommario tecnico" section 2.A describes
  Semantic-Aware Smoothing (k-means over the sequence axis, centroid
  subtraction), section 2.B Progressive Residual Quantization (repeat the
  quantization on what remains, coarse to fine; decode dequantizes and adds
  centroids back), section 3 the centroid caching and fused dequantization
  kernels.
* "Coral-KV ..." news article (news.hamidun.com/ru/news/13833 and its
  Portuguese copy /pt/news/13833), section on cross-layer prediction: predict
  the next layer's K/V from one layer's cache with a block-diagonal plus
  low-rank ("block-DPLR") matrix and quantize only the prediction residual.
* "Q-ARVD: Quantizing Autoregressive Video Diffusion Models" (explainer,
  gist.science), section on outlier-aware adaptive dual-scale quantization:
  channels whose L2 norm a MAD-based modified z-score flags get a quantizer
  of their own (stated for weights; carried over to the KV residual).
* "KV Cache Quantization for Self-Forcing Video Generation: A 33-Method
  Empirical Study" (abstract, fugumt.com/fugumt/paper_check/2603.27469v1):
  reconstructing BF16 buffers during attention defeats the compression.

The pages give no formulas.  Every numerical choice the pages leave open
(quantizer form, rounding, metadata precision, group axis, k-means
initialisation and tie-breaking, summation order) is a stated reading; the
module docstrings list each one where it is used.

Modules:
  numerics  -- IEEE rounding helpers (bf16/fp16 round-to-nearest-even, fmaf)
  sas       -- k-means assignment, update, loop; centroid subtraction
  prq       -- progressive residual stages, bit packing, reconstruction
  attend    -- attention over the reconstructed cache (fp64)
  xlayer    -- cross-layer block-diagonal + low-rank prediction
  outlier   -- outlier-channel flags and the dual-scale stages
  stream    -- one (layer, K|V) stream encoded chunk by chunk
  bits      -- closed-form storage cost per element

Parity unpinned: nothing here.  Every function is pinned by a CPU test
(brute force, closed forms, invariants or textbook reductions).
"""
