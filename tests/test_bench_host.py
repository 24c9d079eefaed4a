"""Host-side logic of bench.py, on the CPU: the algorithmic byte counts its roofline figures
use (against closed forms for the long prefill, whose lengths and page table are full), the
one-GPU guard, and the source hash that keys the committed traffic counters."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_attention_indexer_qsa_amd import workloads as W  # noqa: E402


@pytest.fixture(scope="module")
def long_prefill():
    return W.config3()


def test_long_prefill_byte_counts(long_prefill):
    """B = 1, S = 131072, every row live, 32768 complete blocks, every V-tail page mapped:
      q-prep    1024 (q read) + 256 (cosSin row) + 1024 (qNormed written) per token;
      compress  1024 (4 raw keys) + 256 (cosSin row 4g) + 256 (kbar written) per block;
      persist   256 per V-tail + 4 per page-table entry (1024 pages of 128 tokens), no tails;
      gammas 512, the length 4.
    The fused launch reads each block's cosSin row once (with q-prep), not twice."""
    wl = long_prefill
    S, nb = wl.S, wl.numBlocks
    assert (wl.B, S, nb) == (1, 131072, 32768) and int(wl.ctx[0]) == S
    pages = S // 128
    path = 2304 * S + 1536 * nb + 256 * nb + 4 * pages + 512 + 4
    fused = path - 256 * nb
    assert bench.path_bytes(wl) == path == 360_714_756
    assert bench.algorithmic_bytes(wl) == fused == 352_326_148


def test_next_row_byte_counts(long_prefill):
    """Scores over rows [65536, 73728) x 32768 blocks: 4 B per logit written, 1 KB of q per
    row, 256 B per kbar row any row sees; selection: 4 B per complete-block logit read plus the
    2051 int32 token slots of each row."""
    wl = long_prefill
    r0, n = bench.SCORE_ROWS
    t = r0 + np.arange(n, dtype=np.int64)
    vis = np.minimum((t + 1) // 4, wl.numBlocks)
    alg, visible, _ = bench.scores_alg(wl.S, wl.numBlocks, r0, n)
    assert visible == int(vis.sum())
    assert alg == 4 * n * wl.numBlocks + 1024 * n + 256 * int(vis.max())
    assert bench.select_alg(wl.S, wl.numBlocks, r0, n) == 4 * int(vis.sum()) + 4 * 2051 * n


def test_more_than_one_gpu_is_refused():
    """The benchmark measures one GPU: --gpus 2 exits with a message, before touching a GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_kernel_source_hash_is_stable():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert h == bench.kernel_source_hash()
