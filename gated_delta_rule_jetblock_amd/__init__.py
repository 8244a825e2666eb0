"""libjetblock: the JetBlock token mixer on one AMD MI355X (gfx950).

The compute lives in a C-ABI shared library built from hand-written HIP
(``csrc/``); ``jetblock`` is its thin ctypes binding (argument marshalling
only) and ``inputs`` draws the seeded synthetic workloads.  The binding is
imported lazily so that the input generator works on machines without the
library.
"""

__all__ = ["inputs", "jetblock"]
