"""fp64 CPU oracle for the lightning indexer path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import or call anything in this
package.  The product (the HIP library and its Python binding) never routes
through it, and it shares no code with the product: it reads the storage
formats with its own decoders and computes everything in float64 with plain
numpy.  See ``oracle.indexer`` for what each function follows.
"""
from .indexer import *  # noqa: F401,F403
