"""Plain CPU oracle for the joint audio-video DiT denoising step.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package. The
product path (the HIP library and its Python binding) never imports, calls or
links it, and this package imports nothing from the product.

Everything here is float64 NumPy, written as the plain definition of each step
so that it can be checked against the pages by eye. Per-function headers cite
the page and section each step follows; readings of passages the pages leave
open are listed in the repository's design notes.
"""

from .avdit_oracle import *  # noqa: F401,F403
