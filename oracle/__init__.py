"""fp64 CPU oracle of the selective scan (S6). TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark
import this package. It shares no code with the GPU library.
"""
from .ref import (Oracle, bwd, build, conv1d, conv1d_bwd, conv1d_step, default, default_threads, fwd,  # noqa: F401
                  scaled_error, ssd, ssd_step, step)
