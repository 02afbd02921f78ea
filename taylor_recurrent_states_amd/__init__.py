"""MI355X (gfx950) truncated-Taylor recurrent-state attention.

The compute lives in ``libtaylor_states.so`` (hand-written HIP kernels behind
a C ABI, declared in ``include/taylor_states.h``).  ``taylor_recurrent_states_amd.ops``
is a thin ctypes binding with the same call names; importing this package
does not load the library.
"""

__all__ = ["ops", "workloads"]
