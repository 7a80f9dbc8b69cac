"""CPU oracle for ordered block-sparse prefill attention -- TEST INFRASTRUCTURE.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
anything under oracle/.  The product path (the package block_sparse_long_osk_amd
and its HIP library) never imports, calls or links it, and the oracle imports
nothing from the product.

Parity status of each function (what pins it to something other than itself is
listed in tests/test_oracle_pins.py and tests/test_maskref.py):
  osk.support_set            pinned (worked example of the PageWeaver notes)
  osk.brute_force_attention  pinned (torch SDPA in fp64, closed forms)
  osk.osk_reference          pinned (brute force, dense equivalence, order
                             invariance, closed-form skip constructions)
  osk.ReplayDecisions        pinned (self-replay identity, brute force over the
                             replayed kept set)
  maskref.build_order_mask   pinned to brute-force loops and exact counts; the
                             builder's definition itself is a reading (the pages
                             print no numeric example of the proxy)
"""
