"""Plain fp64 CPU oracle for VideoMLA's latent KV cache and attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this package.  The product path
(the HIP library and its Python binding) never imports, calls or links it, and
this package imports nothing from the product path.

Sources (the pages this follows):
  * "VideoMLA: Low-Rank Latent KV Cache for Minute-Scale Autoregressive Video
    Diffusion", abstract (chatpaper.ai page).
  * The same paper's technical summary on gist.science (Japanese page),
    sections 問題定義 (problem definition) and 手法 (method), items 1-4.
  * The same summary on gist.science (Hindi page), methodology section.

Parity status: every function in ``oracle.mla`` is pinned by a CPU test
against something other than itself (closed forms printed on the pages, a
library routine it reduces to, invariants of rotations and of softmax, or a
brute-force scalar loop).  Constants the pages leave open (score scale, the
RoPE axis split and frequency ladder, the position origin) are pinned only to
the reading documented beside each function; against the paper itself they are
"parity unpinned".
"""

from . import mla  # noqa: F401
