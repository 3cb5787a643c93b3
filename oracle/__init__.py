"""CPU oracle for the bit-reproducible block-scaled int8 GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing under ``oracle/`` is part of the product
path: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import it.  It shares no code with the HIP library in
``int8_gemm_amd/`` and never imports it.

Modules
-------
``ieee32``       exact-rational IEEE-754 binary32 rounding (the referee).
``ref``          the method in plain numpy, one IEEE binary32 operation per step.
``brute``        the method in pure Python on tiny shapes, every rounding done
                 by ``ieee32``.
``hashref``      the output-hash definition (numpy uint64 and pure Python).
``adversarial``  searches that build tie and near-tie inputs (uses ``ref``).
``formats``      power-of-two scales and int4 values (two per byte), numpy
                 and exact-rational versions.
``probe``        the seeded inputs and hash of the kernel probe.
``requant``      the requantizing epilogue (int8 codes and row scales of the output).

The method is the block-scaled int8 GEMM of the DaisyChain-Train page
"Verification — why you can trust the numbers", section "The verified INT8
units" (steps 1-3): per-row / per-column absmax scales floored at 1e-8,
int8 values, exact int32 accumulation and the epilogue
f32(f32(f32(acc)*s_row)*s_col).
"""
