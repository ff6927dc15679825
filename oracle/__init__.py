"""CPU oracle for the pipelined tile stream -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. It shares no code with the HIP path
(``async_stage_tile_amd``) and never imports it; both sides receive the same
input bits from ``synth``.

Contents
  results   -- what the path computes: tile copy, per-tile checksums, exact
               row sums rounded once to fp32, fp64 GEMM, tolerance checks.
  protocol  -- the pipeline cursor (index, phase, count), the mbarrier model
               (pending arrivals, phase, transaction bytes) and an
               explicit-state checker of the full/empty producer/consumer
               protocol over all interleavings.
  swizzle   -- the XOR swizzle on 16-byte chunks, the page's CuTe swizzle
               functor, and a parametric LDS bank model.

Pinning: every function here is checked by ``tests/test_oracle_*.py``
against values the pages print, closed forms, or brute force. The LDS bank
model (``swizzle.bank_conflicts``) is parity unpinned against hardware: the
real gfx950 bank geometry is taken from a counter measurement, not from the
model.
"""
from . import protocol, results, swizzle  # noqa: F401
