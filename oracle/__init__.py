"""CPU oracle for MoE token dispatch and combine (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path.
"""

from .epdc_oracle import *  # noqa: F401,F403
from .epdc_oracle import __all__  # noqa: F401
