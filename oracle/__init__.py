"""CPU oracle of the sparse-KV decode step -- test infrastructure only.

Only tests/, the entry point's smoke() check and bench.py's cpu_baseline leg
may import this package.  The GPU library neither imports it nor shares any
code with it.
"""

from .step import *  # noqa: F401,F403
from .step import PINS  # noqa: F401
from . import append  # noqa: F401
from . import multiquery  # noqa: F401
from . import prefill  # noqa: F401
from . import residency  # noqa: F401
