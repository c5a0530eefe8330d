"""fp64 CPU oracle for the Muon step.  Test infrastructure only: the test
suite, the smoke check and the benchmark's CPU-baseline leg may use it; the
library never imports it.  See ``oracle/muon_oracle.py`` for the sources it
follows and the readings it takes."""
from .muon_oracle import *  # noqa: F401,F403
from .muon_oracle import __all__  # noqa: F401
