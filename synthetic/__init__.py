"""Seeded synthetic inputs shared by the oracle tests, the HIP parity tests and
the benchmark.

This package holds only random draws and their cast to the input dtype; none of
the attention method's arithmetic lives here, so both sides can import it
without sharing any computation.
"""

from .gen import CONFIGS, Problem, make_config, make_case, config_problem  # noqa: F401
