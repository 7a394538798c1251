"""fp64 CPU oracle for BLASST block-sparse attention (TEST INFRASTRUCTURE ONLY).

This package is the independent checker of the HIP library.  Only the test suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.
The product path (``long_context_online_amd``) never imports, links or runs anything here,
and nothing here imports the product path: the two share no code.  The only shared module is
the seeded input generator ``synth``, which holds none of the method's arithmetic.

Pages cited (all are web pages about the paper "BLASST: Dynamic BLocked Attention Sparsity via
Softmax Thresholding", arXiv 2512.12087):
  [xllm]  xllm-io.github.io paper review (Chinese), sections 解决方案概述, 整体框架图, 核心公式,
          模型组件, 预填充内核优化, 解码内核优化.
  [gist-de] gist.science German summary, sections "2. Methodik" (Kernidee, Kalibrierung) and
          "3. Kernel-Design".
  [nerve] nervesearch.ai commentary (Russian), the paragraph on online softmax and the figure
          with six blocks where the first is always processed.
  [fugu]  fugumt.com page with the English v1 abstract.
  [gist-ja] gist.science Japanese summary, sections 2.1 (skip condition) and 2.2 (calibration).

``oracle.backward`` (torch fp64 autograd on the CPU) gives the gradients of the sparse prefill with
the forward's decisions held fixed ([xllm] 训练流程: skipped blocks receive no gradient).

Parity pins: every public function is pinned by a ``-m "not gpu"`` test against something other
than itself (textbook dense softmax, hand-derived closed forms, invariants, reductions).  No
function here is "parity unpinned".
"""

from .blasst_oracle import (  # noqa: F401
    NOT_LIVE,
    KEPT,
    SKIPPED,
    ln_threshold,
    softmax_attention,
    tile_sequential,
    keep_mask_closed_form,
    prefill,
    prefill_tile,
    decode,
    decode_tile,
    gather_pages,
    combine_splits,
    sparsity,
)
from .calibration import (  # noqa: F401
    quantile_ln_lambda,
    fit_alpha_beta,
    lambda_for,
    achieved_sparsity,
)
from . import backward  # noqa: F401,E402
