"""CPU oracle for one rank's shard of a tensor-parallel transformer layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call or link anything in this package; only
the test-suite, the smoke check and the CPU-baseline leg of the benchmark do.

Independent implementations live here:

* ``oracle.layer``  -- NumPy float64, whole-tensor operations (matmul as the
  only library primitive), with optional bf16 storage-point mirroring.
* ``oracle.brute``  -- pure-Python scalar loops for tiny shapes, written
  separately, used only to pin ``oracle.layer``.
* ``oracle.fp8``    -- E4M3 encoding from the format definition and the
  per-row weight quantisation of the fp8 decode shard.
* ``oracle.sp``     -- the sequence-parallel variant: reduce-scatter over
  token rows, per-rank norms, all-gather of the normalised rows.

None of them shares any code with the GPU path.
"""

from . import layer, brute, fp8, sp  # noqa: F401
