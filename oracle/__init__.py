"""Reference oracle for draft/verify attention and the greedy accept step — TEST INFRASTRUCTURE.

Plain, slow, fp64 CPU code (numpy) written from the VeriCache pages, used only to check the GPU
path.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import or run anything in this package; the product library never does.

It shares no code with the HIP path.  The only thing both sides use is the seeded input
generator package ``vcsynth`` (draws of random numbers and workload shapes, no method
arithmetic).

Modules
-------
numerics   fp64 -> fp16 round-to-nearest-even, bf16 bit decoding
compress   token-drop kept sets and KIVI-style asymmetric quantisation
attention  verify (causal multi-query, full KV) and draft (single query, compressed KV)
accept     argmax with top-2 gap, greedy longest-prefix accept, near-tie flags
workload   one (request, layer) instance of a workload end to end, from vcsynth inputs
costs      byte accounting (KV size formula, per-iteration HBM bytes of the throughput model)

Parity pins: every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
invariants, library routines, brute force on tiny inputs and the pages' worked numbers.
"""
