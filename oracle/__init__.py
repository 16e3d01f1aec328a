"""CPU oracle for the dense matrix product C = A·B.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import, call, link or execute anything in
this package.  It shares no code with the GPU path (``dense_gemm_run_amd``) and
imports nothing from it; the GPU path imports nothing from here.

Modules
-------
``gemm64``     ctypes binding of ``oracle_gemm.c``: the fp64 three-loop product,
               sampled dot products and fp64 -> fp16/bf16/fp32 round-to-nearest-even.
``exact``      pure-Python exact arithmetic (``fractions.Fraction``) for tiny
               shapes, round-to-nearest-even from a rational, the half-open
               ``tile_ranges`` partition, the tiled K-walk with its load count,
               the grouped program ordering, and the traffic / intensity models.
``tolerance``  the per-element acceptance rule for comparing a GPU result with
               the rounded oracle.
``build``      compiles ``oracle_gemm.c`` with gcc (no HIP, no GPU code).

Every function cites the passage of the pages it follows.  Parity status of
each function is listed in its module docstring; nothing here is "parity
unpinned": every function has at least one CPU test against values the pages
print, closed forms, a library routine or brute force.
"""
