"""CPU oracle for condensate-set (Topological) attention.

TEST INFRASTRUCTURE ONLY. Only tests/, the smoke check of __graft_entry__ and the CPU-baseline leg of
bench.py may import it. The product path (the HIP library and its Python binding) never imports,
calls or links anything here, and shares no code with it.
"""
from .topo_oracle import *  # noqa: F401,F403
from .topo_oracle import __all__  # noqa: F401
