"""fp64 CPU oracle for the multi-LoRA SGMV delta. Test infrastructure only: imported by
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``;
never by the library."""
from .sgmv_oracle import *  # noqa: F401,F403
from .sgmv_oracle import __all__  # noqa: F401
