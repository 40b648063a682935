"""fp64 CPU oracle for the HSTU attention layer (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package. The library and its Python binding never do.
"""
from .hstu import *  # noqa: F401,F403
