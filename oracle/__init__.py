"""CPU oracle for paged decode attention -- test infrastructure, not product.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package. The HIP library and its Python binding never
import it; a product path that routed through it would void every parity
claim.

Every function is a plain float64 NumPy restatement of what the pages define
(see the module docstring of :mod:`oracle.paged_attention`). Pins that tie it
to facts outside itself live in ``tests/test_oracle.py``. No function here is
"parity unpinned".
"""
from .paged_attention import *  # noqa: F401,F403
from .paged_attention import __all__ as _pa_all
from .fp8 import *  # noqa: F401,F403
from .fp8 import __all__ as _fp8_all

__all__ = list(_pa_all) + list(_fp8_all)
