"""CPU oracle of the link step of position-independent KV reuse.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  This package is a plain, slow,
float64 numpy statement of what the method computes, written from the pages
(CacheSlide, FAST'26 notes: Weighted Correction Attention, Algorithm 2 and the
SLIDE page manager; EPIC, ICML'25 notes: the compile/link framing and
LegoLink, section 4).  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it.  It shares no code with the HIP path and
imports nothing from it; the only module both sides use is `workloads`, which
draws the seeded synthetic inputs and holds none of the method's arithmetic.

Modules:
  model   - decoder-layer arithmetic and storage rounding
  select  - deviation, alpha, top-k ranking, fusion, CKSim, refresh
  pages   - deterministic page allocator and slot maps
  link    - compile step, CacheSlide link, LegoLink / full / naive static links

Every function is pinned by tests under tests/ (closed forms, special cases
that reduce to library routines, brute force on tiny inputs, worked examples
under tests/golden/).  Parts with no such pin are the readings marked there as
"parity unpinned": the alpha lag order and the refresh direction (the hidden
state of refilled tokens is pinned by the hand-worked refresh schedule, the
absence of key re-rotation by the layer-1 closed form).
"""
from . import model, pages, select, link  # noqa: F401
