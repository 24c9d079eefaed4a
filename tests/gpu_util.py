"""Helpers of the GPU parity tests: device buffers with red zones, T comparisons, and the
oracle run of a workload.  Used only by tests marked ``gpu``."""
import numpy as np
import torch

from oracle.ref import Pool
from sparse_attention_indexer_qsa_amd.workloads import SENTINEL_U16

RED = 0x5A5A           # red-zone fill (int16 bit pattern)
MARGIN = 128           # elements of red zone on each side (256 B keeps 16-byte alignment)


class Guarded:
    """A contiguous device tensor with poisoned margins on both sides."""

    def __init__(self, shape, dtype, fill=0):
        n = int(np.prod(shape))
        self.n = n
        self.flat = torch.empty(n + 2 * MARGIN, dtype=dtype, device="cuda")
        self.flat[:MARGIN].fill_(RED if dtype == torch.int16 else 12345)
        self.flat[MARGIN + n:].fill_(RED if dtype == torch.int16 else 12345)
        self.t = self.flat[MARGIN:MARGIN + n].view(shape)
        self.t.fill_(fill)

    def check(self):
        pad = RED if self.flat.dtype == torch.int16 else 12345
        assert bool((self.flat[:MARGIN] == pad).all()), "front red zone overwritten"
        assert bool((self.flat[MARGIN + self.n:] == pad).all()), "back red zone overwritten"


def dev_bits(a):
    """uint16 numpy -> int16 cuda tensor (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bits(t):
    return t.cpu().numpy().view(np.uint16)


def ordered(bits):
    """T bit patterns -> integers whose difference counts ulps (+0 and -0 both map to 0)."""
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def is_nan(bits, dt):
    e, m = (0x7F80, 0x007F) if dt == "bf16" else (0x7C00, 0x03FF)
    return ((bits & e) == e) & ((bits & m) != 0)


def ulp_value(bits, dt):
    """Value of one unit in the last place of each T value (subnormal ulp at the bottom)."""
    mant = 7 if dt == "bf16" else 10
    bias, emin = (127, -126) if dt == "bf16" else (15, -14)
    e = ((bits.astype(np.int32) & 0x7FFF) >> mant) - bias
    e = np.maximum(e, emin)
    return np.ldexp(1.0, e - mant)


def widen(bits, dt):
    if dt == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


def rope_terms(pre, cs):
    """|y_a c| + |y_b s| for every element of roped vectors, the magnitude of the two products
    whose difference (or sum) is the element: o_a = y_a c - y_b s and o_b = y_b c + y_a s for
    the pair (a, b) = (i, i+32), i < 32.  The pre-rope pair (y_a, y_b) is recovered in float64
    from the oracle's pre-cast pair by the inverse rotation (y_a = o_a c + o_b s,
    y_b = o_b c - o_a s; the cosSin rows satisfy c^2 + s^2 = 1 to binary32 rounding).  Dims
    [64, 128) are not roped: their term is |o| itself.  `pre` [N, 128], `cs` [N, 64]."""
    pre = np.asarray(pre, np.float64).reshape(-1, 128)
    cs = np.asarray(cs, np.float64).reshape(-1, 64)
    c, s = cs[:, :32], cs[:, 32:]
    oa, ob = pre[:, :32], pre[:, 32:64]
    ya, yb = oa * c + ob * s, ob * c - oa * s
    M = np.abs(pre).copy()
    M[:, :32] = np.abs(ya * c) + np.abs(yb * s)
    M[:, 32:64] = np.abs(yb * c) + np.abs(ya * s)
    return M


def compare_T(got, ref, dt, pre=None, cs=None, what="", stats=None):
    """Normed/roped outputs: at most 1 ulp of T apart.  On rope dims where the two products
    cancel, |o| < 2^-6 (|y_a c| + |y_b s|), the allowance is 1 ulp(o) + 2^-22 (|y_a c| + |y_b s|)
    (rope_terms).  `pre` [..., 128] FP32 (the oracle's pre-cast values) and `cs` [..., 64] (the
    cosSin row of each vector) enable that clause.  Returns the number of elements that differ
    in any bit; with `stats` (a dict) also records how many elements are within 1 ulp only
    ("ulp1") and how many pass only by the cancellation clause ("cancel")."""
    got, ref = np.asarray(got).reshape(-1, 128), np.asarray(ref).reshape(-1, 128)
    both_nan = is_nan(got, dt) & is_nan(ref, dt)
    d = np.abs(ordered(got) - ordered(ref))
    bad = (d > 1) & ~both_nan
    n_cancel = 0
    if bad.any() and pre is not None:
        o = np.asarray(pre, np.float64).reshape(-1, 128)
        M = rope_terms(o, cs)
        M[:, 64:] = 0.0                      # the clause covers roped dims only
        cancel = np.abs(o) < 2.0 ** -6 * M
        allow = ulp_value(ref, dt) + 2.0 ** -22 * M
        ok = bad & cancel & (np.abs(widen(got, dt) - o) <= allow)
        n_cancel = int(ok.sum())
        bad &= ~ok
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond tolerance, e.g. at " \
        f"{np.argwhere(bad)[:5].tolist()} got {got[bad][:5]} ref {ref[bad][:5]}"
    if stats is not None:
        stats["ulp1"] = int(((d == 1) & ~both_nan).sum())
        stats["cancel"] = n_cancel
    return int((got != ref).sum())


def oracle_pool(spec):
    data = np.full(spec.shape, SENTINEL_U16, np.uint16)
    return Pool(data, spec.pageTable, spec.numPages, spec.headSize)


def device_pool(spec):
    import sparse_attention_indexer_qsa_amd.qsa as qsa
    pool = torch.full(spec.shape, SENTINEL_U16 - 65536, dtype=torch.int16, device="cuda")
    pt = dev(spec.pageTable.astype(np.int32))
    return qsa.PoolState(pool, pt, spec.numPages, spec.numKVHeads, spec.poolHeadDim,
                         spec.headSize)
