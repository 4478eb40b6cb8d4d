"""CPU oracle for the NVFP4 block-scaled MoE grouped GEMM and its quantiser.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import, call, link or run anything in this
package.  The HIP library never does, and this package imports nothing from it.

  fp4_oracle.c   plain C99 + OpenMP: E2M1 / E4M3 codecs, the quantiser, the
                 grouped GEMM as an exact int64 sum and as an FP64 sum.
  oracle.py      ctypes wrapper over the C oracle (numpy in, numpy out), and in
                 plain numpy FP64 the steps around the GEMM: the token-order
                 combine (finalize) and the SwiGLU activation of the gate+up
                 projection.
  bruteforce.py  exact rational (Fractions) brute force for tiny shapes.

Parity status: every function is pinned by the tests in ``tests/test_oracle_*``
(golden format tables from the OCP specifications, torch's float8_e4m3fn
conversion, numpy matmul on dequantised matrices, the brute force, closed forms
and invariants).  The scale recipe itself (tensor scale amax/2688, RNE block
scale, IEEE division) is a reading of what the pages leave open; it is pinned by
self-consistency and invariants only, not by any value the pages print.
"""
