"""fp64 CPU oracle of the ZGCM-1 hybrid attention path (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package; the product path never does.
"""
from .zg_oracle import *  # noqa: F401,F403
