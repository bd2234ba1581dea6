"""fp64 CPU oracle of the selective scan (S6). TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark
import this package. It shares no code with the GPU library.
"""
from .ref import Oracle, build, default, default_threads, fwd, scaled_error, step  # noqa: F401
