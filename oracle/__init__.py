"""CPU float64 oracle for the Wan-style video DiT denoise step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP library and
its Python binding) never calls it and must fail loudly when its native library
is missing; nothing here is a fallback.

Every function is the plain definition of one step, written in NumPy float64
from the pages' description (each docstring names the page and section it
follows).  It shares no code, table or constant generator with the HIP path.

Pages cited (titles as they appear on the pages):
  * "图解 Wan2.1 I2V：从一张图到一段视频，模型到底发生了什么" (liyongzhi.xyz),
    cited as [I2V-illustrated §n];
  * "Wan（通义万相）：大规模视频生成基础模型 — 技术深度解析 & Wan2.1 vs Wan2.2对比"
    (devpress.csdn.net), cited as [Wan-deep-dive §n];
  * "Wan2.2 TI2V-5B" (lnwmold.com), cited as [TI2V-5B §n].

Parity status per function is listed in ``PARITY``: "pinned" functions are
checked by the CPU tests against closed forms, invariants, brute force or
hand-worked fixtures; "parity unpinned" ones only against shape and the
special cases named there.  Parity unpinned: ``time_embed``, ``context_embed``
and ``head_fwd`` (the pages name these MLPs and the head's adaLN but not their
layers; the readings taken are implemented as stated and checked against
PyTorch modules of the same composition).
"""
from .wan_oracle import *  # noqa: F401,F403
from .wan_oracle import PARITY, __all__  # noqa: F401
