"""fp64 CPU oracle for the Kimi Delta Attention (KDA) recurrence.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import, call, link or execute anything in this package.
It shares no code with the HIP library and imports nothing from it.

Contents:
  kda_oracle.c  plain per-token recurrence in C, double precision, threaded over
                independent (batch, head) units; also a value-column-subset form
                for sampled checks of very long sequences.
  c_oracle.py   ctypes wrapper for kda_oracle.c (builds it on demand with gcc).
  ref.py        NumPy fp64 forms: the sequential definition and the naive
                chunked form written out matrix by matrix.
  exact.py      exact rational (fractions) and high-precision (mpmath) forms of
                the sequential definition, for pinning the fp64 forms.
"""
