"""Pins of the oracle's own IEEE conversions against library routines.

The method widens T to FP32 exactly and narrows FP32 to T once per output (the "single cast to
T at the very end" of launchQsaIndexQPrep, and the bit-critical cast of the block mean in
launchQsaIndexKCompress, "Qsa Indexer Kernels").  The oracle implements both directions itself;
here they are checked against torch's bfloat16 cast and numpy's float16 cast, which round to
nearest even: exhaustively for widening, and for narrowing on every exact midpoint, its two
neighbours, the special values and a large random sample of all binary32 patterns.
"""
import numpy as np
import pytest
import torch


def _torch_bf16_bits(f32):
    return torch.from_numpy(np.ascontiguousarray(f32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def _np_f16_bits(f32):
    with np.errstate(over="ignore"):
        return np.ascontiguousarray(f32).astype(np.float16).view(np.uint16)


def _same_or_both_nan(a_bits_f32, b_bits_f32):
    a, b = a_bits_f32.view(np.float32), b_bits_f32.view(np.float32)
    nan = np.isnan(a)
    assert np.array_equal(nan, np.isnan(b))
    assert np.array_equal(a_bits_f32[~nan], b_bits_f32[~nan])


def test_widen_bf16_exhaustive(oracle):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.widen(bits, "bf16").view(np.uint32)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy().view(np.uint32)
    _same_or_both_nan(got, ref)


def test_widen_f16_exhaustive(oracle):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.widen(bits, "f16").view(np.uint32)
    ref = bits.view(np.float16).astype(np.float32).view(np.uint32)
    _same_or_both_nan(got, ref)


def _narrow_cases(dt, rng):
    """All exact midpoints between adjacent finite T values, +-1 binary32 ulp around them, the
    T values themselves, special values, and 4M random binary32 patterns."""
    t_bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if dt == "bf16":
        vals = (t_bits.astype(np.uint32) << 16)
        finite = (vals & 0x7F800000) != 0x7F800000
        mids = (vals[finite] + 0x8000).astype(np.uint32)       # halfway to the next pattern
    else:
        f = t_bits.view(np.float16).astype(np.float64)
        finite = np.isfinite(f)
        fin = np.sort(np.unique(f[finite]))
        mids64 = (fin[:-1] + fin[1:]) / 2.0                    # exact in binary32
        mids = mids64.astype(np.float32).view(np.uint32)
        assert np.array_equal(mids.view(np.float32).astype(np.float64), mids64)
        vals = t_bits.view(np.float16).astype(np.float32).view(np.uint32)
    around = np.concatenate([mids, mids + 1, mids - 1, vals])
    special = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001,
                        0x00000001, 0x807FFFFF, 0x7F7FFFFF, 0x477FF000, 0x477FEFFF, 0x477FF001,
                        0x33000000, 0x33000001, 0x32FFFFFF, 0x387FC000], dtype=np.uint32)
    rand = rng.integers(0, 2**32, 1 << 22, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([around, special, rand]).view(np.float32)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_narrow_matches_library_rne(oracle, dt):
    rng = np.random.default_rng(123)
    x = _narrow_cases(dt, rng)
    got = oracle.narrow(x, dt)
    ref = _torch_bf16_bits(x) if dt == "bf16" else _np_f16_bits(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    # NaN stays NaN (quiet): exponent all ones, non-zero fraction, quiet bit set
    e_mask, q_bit = (0x7F80, 0x0040) if dt == "bf16" else (0x7C00, 0x0200)
    g = got[nan]
    assert np.all((g & e_mask) == e_mask) and np.all(g & q_bit)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_narrow_widen_roundtrip_is_identity(oracle, dt):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    w = oracle.widen(bits, dt)
    back = oracle.narrow(w, dt)
    ok = ~np.isnan(w)
    assert np.array_equal(back[ok], bits[ok])
