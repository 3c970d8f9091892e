"""CPU oracle for the Ozaki Scheme II FP64 GEMM emulation.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
routes through it and shares no code, tables or constants with it.

Every function is a plain, slow, exact restatement of one step of the method;
see ``oracle.method`` for the steps and the passages they follow.
"""
from .method import *  # noqa: F401,F403
from .method import __all__  # noqa: F401
