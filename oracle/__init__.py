"""CPU oracle for the MiKV mixed-precision KV-cache path (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package. The product path never imports it.
"""
from .mikv_oracle import *  # noqa: F401,F403
from .mikv_oracle import __all__  # noqa: F401
