"""CPU oracle for the LLM.int8() decomposed int8 matmul (test infrastructure).

Only tests, the package smoke check and the benchmark's CPU-baseline leg may
import this package; the product path never does.
"""

from .llm_int8 import *  # noqa: F401,F403
from .llm_int8 import __all__ as _main_all
from .variants import *  # noqa: F401,F403
from .variants import __all__ as _variant_all

__all__ = list(_main_all) + list(_variant_all)
