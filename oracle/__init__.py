"""CPU oracle for AdaS-Attn -- test infrastructure only.

Only tests, the package smoke check and the benchmark's CPU-baseline leg may
import this package.  See ``oracle.adas_oracle`` for the definitions.
"""
from .adas_oracle import *  # noqa: F401,F403
from .adas_oracle import __all__  # noqa: F401
