"""CPU oracle for the SpMM path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  It shares no code with ``window_spmm_amd`` (the GPU
library) and never imports it.

Contents, each written from the AsyncSparse paper (Liu, Pu, Zhang,
"AsyncSparse: Accelerating Sparse Matrix-Matrix Multiplication on
Asynchronous GPU Architectures"):

* ``spmm`` -- the plain fp64 definition of C = A * B from COO triplets
  (Section II-C, problem statement), with the acceptance scale
  Bound = |A| * |B|; implemented in plain C (``spmm_oracle.c``).
* ``decode16`` -- exact value of binary16 / bfloat16 codes (same C file).
* ``encode_bcsr`` / ``encode_wcsr`` -- the two sparse formats written from
  their definitions (Section II-C, "Block Compressed Sparse Row" and "Window
  Compressed Sparse Row", Fig. 2), plus the matching decoders.
* ``wcsr_tasks`` -- the window-splitting rule (Section III-C: long windows are
  cut into fixed-size sub-tasks, and one task descriptor per thread block).
* ``within_tolerance`` -- the acceptance test |C_gpu - C| <= tol * Bound.
* ``dense_bruteforce`` -- a dense triple loop for tiny inputs.
* ``rcm_order`` / ``permute_symmetric`` / ``bandwidth`` -- reverse
  Cuthill-McKee reordering, the preprocessing of Section IV-A (``reorder.py``).
"""

from .reference import (  # noqa: F401
    ORACLE_LIB,
    decode16,
    decode_bcsr,
    decode_wcsr,
    dense_bruteforce,
    encode_bcsr,
    encode_wcsr,
    fill_ratio,
    padded_width,
    spmm,
    wcsr_tasks,
    within_tolerance,
)
from .reorder import bandwidth, permute_symmetric, rcm_order  # noqa: F401,E402
