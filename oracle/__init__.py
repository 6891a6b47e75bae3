"""CPU fp64 oracle for the fused NF4-LoRA linear — TEST INFRASTRUCTURE ONLY.

Only the tests under tests/, the smoke check in __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import, call or execute anything in this
package. The product path (the HIP library and its Python binding) never does,
and this package imports nothing from the product path.

It is a plain, slow, obviously-correct restatement of what the method computes:

* ``oracle.nf4``  — the 4-bit NormalFloat codebook, blockwise absmax
  quantization, packing and dequantization.
* ``oracle.lora`` — the LoRA linear over the dequantized frozen base, forward
  and backward, in float64.
* ``oracle.optim`` — the AdamW step of the LoRA factors and the rank-stabilized
  scale.
* ``oracle.dq``   — double quantization of the NF4 block scales (8-bit E4M3
  codes in blocks of 256).

Pinned by the ``-m "not gpu"`` tests (tests/test_oracle_*.py) against closed
forms, independent library routines, exact rational brute force and finite
differences. Parity unpinned: equality with any third-party NF4 table or file
format (the pages give no worked example of one).
"""
from . import dq, lora, nf4, optim  # noqa: F401
