"""Float64 CPU oracle for hybrid compressed attention (CSA / HCA).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it. It shares no code, header, table or helper with the HIP
library; the two meet only at the seeded inputs from ``workloads``.

Every function follows a definition stated on the source pages and cites the
page and section it comes from. Page short names used in citations:

* [PACMAN]  "DeepSeek-V4 technical report share" (THU PACMAN group, 10100.com)
* [Qiaomu]  "DeepSeek-V4论文解析：百万上下文、水平接近闭源模型是如何做到的？" (乔木博客)
* [cdjax]   "未来科技" DeepSeek-V4 architecture / post-training essay (cdjax.com)
* [fwf]     "DeepSeek-V4: Towards Highly Efficient Million-Token Context
            Intelligence" (fengweifeng.com; low reliability, used only where
            it agrees with the others)
* [kwkr]    kwkr.cn DeepSeek-V4 report walk-through (news 508982)

Parity status of each function is stated in its docstring ("pinned by ..." or
"parity unpinned").
"""

from .lca_oracle import *  # noqa: F401,F403
from .lca_oracle import __all__  # noqa: F401
