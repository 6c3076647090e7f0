"""Plain CPU oracle for the predictor-gated sparse FFN decode step.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test suite, the smoke
check in ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The HIP library and
its Python binding never import it, and it never imports them: the two share
no code, headers, tables or helpers.

Everything here is numpy float64 on the CPU.  Stored inputs (fp32, fp16, Q4_0
blocks) are converted exactly to float64 before any arithmetic, and the steps
follow the definitions in the order the pages describe the method.

Sources (three web pages about PowerInfer, from SJTU-IPADS):

  [GN] GeekNews, vi.news.hada.io topic 12458, "Phục vụ mô hình ngôn ngữ lớn
       tốc độ cao trên PC trang bị GPU tiêu dùng" (a summary of the project
       README followed by a Hacker News thread).
  [QB] QbitAI article on r-manual.ru, "2080 Ti может запускать большие модели
       70B, а новая платформа может увеличить скорость вывода LLM в 11 раз".
  [AB] aibars.net library profile "SJTU-IPADS/PowerInfer" (Portuguese).

Every function is pinned by a CPU test against something other than itself
(pure-Python brute force, hand-worked fixtures under tests/golden/, closed
forms and invariants).  No function here is "parity unpinned".
"""

from .reference import (  # noqa: F401
    ACTIVATIONS,
    to_f64,
    logit_threshold,
    sigmoid,
    dense_ffn,
    predict,
    compact,
    sparse_ffn,
    q4_0_dequant,
    Q4_0Matrix,
    layer,
)
