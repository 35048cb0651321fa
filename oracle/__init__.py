"""fp64 CPU oracle of the retention operator and its gated layer -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may
import this package.  It shares no code with the HIP library and imports nothing from
it.  Pins: every public function is checked in ``tests/test_oracle.py`` against exact
rational arithmetic, closed forms, textbook special cases and hand-worked fixtures
(``tests/golden/``); no function here is "parity unpinned".
"""
from .retention_oracle import *  # noqa: F401,F403
from .retention_oracle import __all__ as _ops_all
from .msr_oracle import *  # noqa: F401,F403
from .msr_oracle import __all__ as _msr_all

__all__ = list(_ops_all) + list(_msr_all)
