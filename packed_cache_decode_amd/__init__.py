"""MI355X (gfx950) TurboQuant packed KV-cache store and paged decode.

The work happens in hand-written HIP kernels behind the C ABI of
``include/tq.h`` (library ``libtq_mi355x.so`` in this directory).  Python
only marshals arguments (``_lib``) and keeps a small convenience wrapper
(``runtime``) that holds a context and a decode workspace in torch memory.

``synth`` draws the seeded synthetic inputs; it holds none of the method's
arithmetic.  Nothing in this package imports the CPU oracle.
"""

__all__ = ["_lib", "synth"]
