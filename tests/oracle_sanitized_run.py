"""Child process of test_oracle_sanitized.py: runs every oracle pin, and the tiny-prefill and
decode workloads, on an oracle build instrumented with AddressSanitizer and
UndefinedBehaviorSanitizer (the sanitizer runtime is preloaded by the parent).  Any invalid
access or undefined operation inside the oracle aborts this process.

usage: python -m tests.oracle_sanitized_run <instrumented libqsa_ref.so> [pins|workloads|oob]
"""
import sys

import numpy as np


def _workloads(O):
    from sparse_attention_indexer_qsa_amd import workloads as W
    from oracle.ref import Pool
    for wl in (W.config1(), W.config4()):
        pool = Pool(np.full(wl.pool.shape, W.SENTINEL_U16, np.uint16), wl.pool.pageTable,
                    wl.pool.numPages, wl.pool.headSize)
        if wl.run_q_prep:
            O.q_prep(wl.indexQk, wl.cosSin, wl.ctx, wl.wQ, wl.eps, wl.dt, debug=True)
        kb, _ = O.k_compress(wl.indexQk, wl.cosSin, wl.ctx, wl.wK, wl.eps, wl.numBlocks,
                             wl.blockBegin, wl.blockEnd, wl.pastLen, wl.dt, ranges=wl.ranges,
                             pool=pool, debug=True)
        O.persist(pool, wl.indexQk, kb, wl.ctx, wl.numBlocks, wl.blockBegin, wl.blockEnd,
                  wl.pastLen, ranges=wl.ranges)
        print(f"workload {wl.name}: clean", flush=True)


def main():
    from oracle.ref import Oracle
    lib, what = sys.argv[1], sys.argv[2]
    O = Oracle(lib)
    if what == "pins":
        from tests import oracle_pins
        for check in oracle_pins.ALL_CHECKS:
            check(O)
            print(f"{check.__name__}: clean", flush=True)
    elif what == "workloads":
        _workloads(O)
    elif what == "oob":
        # a build with a planted one-past-the-end write must be stopped by the sanitizer
        O.ids_fill(3, 5)
    print("done", flush=True)


if __name__ == "__main__":
    main()
