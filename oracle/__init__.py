"""CPU oracle for the parallel-Newton forward of diagonal GRU/LSTM cells.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package; only the tests, the smoke check and the bench's CPU
baseline leg use it.  It shares no code with the HIP library.

Plain NumPy in float64, written to be checked by eye:

  cells    the two cells and their closed-form per-channel Jacobians
  proj     the input projection  x @ W^T + bias
  newton   the sequential unroll (the truth) and the K-iteration Newton
           method with an explicit serial affine recurrence, plus the
           residual max|F(H)|
  backward gradients through the recurrence: the reverse-time adjoint
           recurrence at a given trajectory
  headmix  the head-mix GRU (dense d_head x d_head recurrent blocks): cell,
           Jacobian blocks, unroll and Newton
  scan     exact (rational) affine-map composition, every bracketing, and
           the chunked three-phase scan
  rounding storage-dtype rounding (fp32, bf16 round-to-nearest-even)

Each function says which passage of the pararnn-torch pages (the FAQs page,
the "Numerics contract" page, and the shapes/layout page on contiguity and
ragged packs) it follows, or which definition it writes out where the pages
leave the step open.
"""
from . import backward, cells, headmix, newton, proj, rounding, scan  # noqa: F401
