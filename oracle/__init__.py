"""CPU float64 oracle for FAVOR+ attention.

TEST INFRASTRUCTURE ONLY: imported by the test-suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py``; never by the library.  It shares no code with the HIP
path.  Every function is pinned by ``tests/test_oracle.py`` or ``tests/test_feature_draw.py``
(closed forms, identities, brute force, known-answer vectors), the parity metric
``rowwise_rel_err`` included (hand-computed rows); none is "parity unpinned".
"""
from .favor_oracle import *  # noqa: F401,F403
