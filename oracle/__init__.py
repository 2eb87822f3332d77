"""fp64 CPU oracle of the K-FAC step. TEST INFRASTRUCTURE ONLY: imported by the test
suite, the smoke check and bench.py's CPU baseline, never by the product path."""
from .kfac_oracle import *  # noqa: F401,F403
from .kfac_oracle import __all__  # noqa: F401
