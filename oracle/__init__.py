"""fp64 CPU oracle for trie_tree label scoring.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this package:
only the tests, the smoke check and the bench's CPU-baseline leg call it.  It
shares no code with the HIP library.
"""
from .tcs_oracle import *  # noqa: F401,F403
from .tcs_oracle import __all__  # noqa: F401
