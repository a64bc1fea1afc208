"""Dynamic any-precision MoE expert FFN for MI355X (gfx950).

The compute path lives in the HIP library libmoe_anyprec.so (csrc/), reached
through the thin ctypes binding in `binding`.  `workloads` holds the seeded
synthetic inputs and the offline bitplane encoder."""

__all__ = ["binding", "workloads"]


def __getattr__(name):
    if name == "binding":
        from . import binding
        return binding
    if name == "workloads":
        from . import workloads
        return workloads
    raise AttributeError(name)
