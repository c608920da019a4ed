"""CPU oracle for Dynamic Bifocal RoPE attention -- test infrastructure only.

Imported by the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU
baseline leg; never by the product path.  See ``bifocal_ref`` for what each
function follows on the pages, and ``brute`` for the loop-only twin used to
pin it on tiny inputs.
"""
from .bifocal_ref import *  # noqa: F401,F403
from .bifocal_ref import __all__  # noqa: F401
