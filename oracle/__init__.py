"""Plain CPU oracle for the verify step of speculative sampling.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library (``rejection_sampling_verification_spec_amd``) never imports it and
shares no code with it.

The arithmetic lives in ``spec_verify_oracle.c`` (single-threaded fp64 C, built
by ``oracle.build.build()``); this package only marshals numpy arrays to it.
"""
from .oracle import (OracleResult, TreeResult, build, load, run_workload, sample, spec_verify,  # noqa: F401
                     spec_verify_tree)
