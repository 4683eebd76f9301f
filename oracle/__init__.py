"""CPU oracle for decode-step attention over dense, int8 and Quest block-sparse
KV caches.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
statement of what the GPU path computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP library and imports nothing from it.

Conventions
-----------
* Attention arithmetic is float64.  Quantities the method defines in float32
  (int8 scales and codes, query quantization) are emulated exactly in float32
  with NumPy, whose float32 division and ``rint`` are IEEE correctly rounded
  and round-half-to-even.
* Where the method reaches a plain definition exactly (flash-decode and split-K
  are an exact reorganisation of softmax(q K^T * scale) V; Quest attention is
  that softmax restricted to the selected blocks), the oracle computes the
  definition directly: no online softmax, no split-K.
* Layouts mirror the library's: per sequence, K and V are ``[Hkv][L][D]`` and q
  is ``[H][D]``; query head h reads KV head ``h // (H // Hkv)``.

Modules
-------
``quant``      absmax int8 quantization (per row, and per 32-channel group for
               the q8_0 / q4_0 / q5_0 caches), directed float32 -> float16 rounding
``attention``  dense f16 / int8 (method-exact and dequantized-reference) attention,
               exact int32 logit dots, split-K combine
``quest``      per-block kmin/kmax side cache, channel-wise upper bound,
               fixed top-K + sink + recent selection
``sparse_v``   skipping the value rows of negligible softmax weight (static tau
               or the adaptive eps rule)
``scan4``      the 4-bit key index, its deterministic score bounds and the
               candidate tokens they give
``multi_token`` a chunk of T query tokens per sequence, each attending
               causally (dense, or through its own Quest block set)

Parity pins: every function is checked by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` against brute force, closed forms, invariants or
page-printed numbers.  Two choices have no such pin and are marked "parity
unpinned" where they are made: the near-tie report width (1e-5 relative) and
the reading that forced blocks are excluded from the top-K candidates.
"""
from . import quant, attention, quest, sparse_v, scan4, multi_token  # noqa: F401
from .quant import (quantize_rows, f16_round_down, f16_round_up,  # noqa: F401
                    quantize_groups, dequantize_groups, QMAX_Q8, QMAX_Q4, QMAX_Q5)
from .attention import (attend_f16, attend_i8, attend_i8_dequant, attend_grouped,  # noqa: F401
                        int8_logit_dots, combine_partials, softmax_partials)
from .quest import (block_bounds, upper_bounds, group_scores, select_blocks,  # noqa: F401
                    selected_tokens)
from .sparse_v import attend_f16_sparse_v, attend_grouped_sparse_v, attend_i8_sparse_v  # noqa: F401
