"""collective_communication_amd -- one-GPU collectives over R virtual ranks on
MI355X (gfx950): AllReduce, ReduceScatter, AllGather, Gather, Broadcast,
All-to-All-v and the MoE dispatch/combine helpers.

The compute lives in ``libcoll.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/coll.h``); ``collective_communication_amd.coll`` is the
thin ctypes binding.  Importing the package does not load the library; the
first call does, and fails loudly when it has not been built.
"""
