"""fp64 CPU oracle of one MoE layer's forward pass (route, dispatch, expert FFN, combine).

TEST INFRASTRUCTURE ONLY. This package is the slow, plainly written definition that the
HIP path is checked against. Only the tests, the smoke check and the bench's CPU-baseline
leg may import it; the product library never does, and the two share no code. The one
module both sides use is `synth` (seeded inputs), which holds none of the arithmetic here.

Pages cited (titles as they appear on each page):
  [EP-concept]  "專家並行（Expert Parallelism, EP）" (compassingai.com concept page)
  [EP-notes]    "专家并行与 MoE" (note.yj-dis.top notes)
  [EP-serving]  "MoE 服務的專家並行性" (aiunderstanding.org)
  [EP-wiki]     "Expert-Parallelism" (Awesome System Papers Wiki)
  [EP-overview] "总览" (t6page.pages.dev, expert-parallelism chapter overview)

Pinned: every function here is pinned by CPU tests against brute force, closed forms,
the pages' printed values or library routines; see the test modules named in each
function's docstring. Parity unpinned: none.
"""
from .route import router_logits, route, RouteResult  # noqa: F401
from .dispatch import capacity, max_rows, dispatch, DispatchResult  # noqa: F401
from .ffn import swiglu_ffn, expert_ffn, shared_ffn  # noqa: F401
from .combine import combine  # noqa: F401
from .forward import forward  # noqa: F401
from . import volumes  # noqa: F401
from . import layout  # noqa: F401
from . import replicas  # noqa: F401
from . import fp8  # noqa: F401
