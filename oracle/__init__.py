"""CPU oracle for the GDN large-beam decode path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  The HIP library and its Python binding never do.
"""

from .gdn_oracle import *  # noqa: F401,F403
