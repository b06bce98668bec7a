"""CPU oracle for the routed MoE FFN layer -- TEST INFRASTRUCTURE ONLY.

Imported by ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py``, and by nothing else.  It shares no code with the HIP
library (``sparse_moe_router_amd``) and never imports it.

* ``oracle.moe_oracle`` -- the layer's definition in float64 NumPy.
* ``oracle.bruteforce`` -- the same definition in scalar pure Python, for tiny
  inputs, used to pin the NumPy oracle.
"""
