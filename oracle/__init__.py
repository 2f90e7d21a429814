"""CPU oracle for the quantized-expert MoE step (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this package. The product library never does, and this
package imports nothing from the product.

* ``oracle.ref``   -- ctypes wrapper over ``qmoe_oracle.c`` (fp64, index-order
  accumulation) plus the layer / stack / prefill orchestration.
* ``oracle.brute`` -- an independent pure-Python (lists and loops) version of
  the decode layer for tiny shapes, used as a pin.

Parity status of each function is listed in ``oracle/ref.py``'s header.
"""
