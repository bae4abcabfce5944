"""CPU oracle for the HSMLA attention forward pass (test infrastructure only).

This package is a plain, slow, float64 NumPy statement of what the HSMLA
forward pass computes. It exists to check the HIP library and nothing else:
only the test suite, the smoke check of the build entry point and the CPU
baseline leg of the benchmark may import it. The product path never calls it
and shares no code with it.

Sources cited in this package (the same paper seen through two web pages):

* FT -- "HSMLA: Hierarchical Softmax Multi-scale Linear Attention for
  Efficient Vision Transformers", full text as rendered by paperpeel.com.
  Primary source. Sections, equations and tables are named as they appear
  there (equation numbers were lost in that rendering, so equations are named
  by their subsection and role, e.g. "FT 3.1, Z/D sums").
* EX -- the gist.science explainer of the same paper (Dutch), section
  "Technische Samenvatting". Used only where FT is silent.

Parity status of every function is stated in its docstring ("pinned by ..."
or "parity unpinned").
"""

from .hsmla_ref import *  # noqa: F401,F403
