"""CPU oracle (test infrastructure only): see ``oracle/rq_oracle.py``.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does.
"""
from .rq_oracle import *  # noqa: F401,F403
from .rq_oracle import __all__  # noqa: F401
