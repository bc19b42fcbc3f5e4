"""CPU oracle for the AWQ int4 MoE expert stage (test infrastructure).

This package is a plain, slow, float64 NumPy statement of what the stage
computes. It exists to check the HIP path and is not part of it: only the
tests, the package smoke check and the benchmark's CPU-baseline leg may
import it. It shares no code, tables or constants with the HIP library; the
two meet only at the seeded input generators and at the documented bank
byte layout, which each side implements on its own.

Modules:
  layout  -- packer / decoder of the prepared weight bank (byte layout spec)
  ref     -- float64 reference of dequantisation, routing compaction,
             W13 + SwiGLU, W2 + router-weighted reduction, router top-k
  loops   -- scalar pure-Python loop versions used to pin ``ref`` on tiny shapes
"""
