"""Dynamic any-precision MoE expert FFN for MI355X (gfx950).

The compute path lives in the HIP library libmoe_anyprec.so (csrc/), reached
through the thin ctypes binding in `binding`.  `workloads` holds the seeded
synthetic inputs and the offline bitplane encoder.  Submodules are imported
on demand: `from dynamic_any_precision_amd import binding`."""
