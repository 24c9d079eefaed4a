"""CPU oracle of the QSA indexer hot path — TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  It shares no code with the GPU library and the product path never calls it.
"""
