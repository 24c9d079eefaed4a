"""The C ABI library on the host: it loads, exports every function include/qsa.h declares,
reports its version, and rejects every invalid argument with the documented code before any
launch.  The invalid-argument calls hand the library host addresses that are never
dereferenced; on a machine with a GPU they are skipped (the GPU suite covers the same checks
with device tensors)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = open(os.path.join(ROOT, "include", "qsa.h")).read()


def _declared_functions():
    body = re.sub(r"/\*.*?\*/", "", HEADER, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(qsa_\w+)\s*\(", body, re.M)))


def _header_int(name):
    m = re.search(rf"\b{name}\s*=\s*(-?\d+)", HEADER) or \
        re.search(rf"#define\s+{name}\s+\(?(-?\d+)\)?", HEADER)
    return int(m.group(1))


@pytest.fixture(scope="module")
def qsa():
    from sparse_attention_indexer_qsa_amd import qsa
    return qsa


def test_every_declared_symbol_is_exported(qsa):
    names = _declared_functions()
    assert set(names) >= {"qsa_index_q_prep", "qsa_index_k_compress", "qsa_index_persist",
                          "qsa_index_prefill", "qsa_last_error", "qsa_abi_version"}
    lib = ctypes.CDLL(qsa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_codes(qsa):
    assert qsa.qsa_abi_version() == _header_int("QSA_ABI_VERSION")
    for n in ("QSA_OK", "QSA_E_INVALID", "QSA_E_ALIGN", "QSA_E_DTYPE", "QSA_E_LAUNCH",
              "QSA_E_NO_DEVICE", "QSA_F16", "QSA_BF16"):
        assert getattr(qsa, n) == _header_int(n), n


def _gpu_visible():
    import torch
    return torch.cuda.is_available()


class _Host:
    """Aligned host buffers whose addresses stand in for device pointers (never used)."""

    def __init__(self):
        self.buf = np.zeros(1 << 16, np.uint8)
        base = self.buf.ctypes.data
        self.a = base + (-base) % 256          # 256-byte aligned

    def p(self, k=0, mis=0):
        return self.a + 1024 * k + mis


@pytest.fixture
def host(qsa):
    if _gpu_visible():
        pytest.skip("host stand-in pointers are only used where no GPU is visible")
    return _Host()


def _qprep(qsa, h, **kw):
    a = dict(q=h.p(0), x=h.p(1), cs=h.p(2), P=64, ctx=h.p(3), w=h.p(4), eps=1e-6, B=2, S=64,
             dt=qsa.QSA_BF16)
    a.update(kw)
    return qsa.lib.qsa_index_q_prep(a["q"], a["x"], a["cs"], a["P"], a["ctx"], a["w"], a["eps"],
                                    a["B"], a["S"], a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), "QSA_E_DTYPE"), (dict(B=-1), "QSA_E_INVALID"), (dict(S=-4), "QSA_E_INVALID"),
    (dict(q=None), "QSA_E_INVALID"), (dict(x=None), "QSA_E_INVALID"),
    (dict(cs=None), "QSA_E_INVALID"), (dict(ctx=None), "QSA_E_INVALID"),
    (dict(w=None), "QSA_E_INVALID"), (dict(mis_q=2), "QSA_E_ALIGN"),
    (dict(mis_x=8), "QSA_E_ALIGN"), (dict(mis_cs=4), "QSA_E_ALIGN"),
    (dict(mis_ctx=2), "QSA_E_ALIGN"), (dict(mis_w=2), "QSA_E_ALIGN"),
    (dict(P=63), "QSA_E_INVALID"), (dict(eps=float("nan")), "QSA_E_INVALID"),
    (dict(eps=-1e-6), "QSA_E_INVALID"), (dict(eps=math.inf), "QSA_E_INVALID"),
    (dict(B=0, q=None, x=None), "QSA_OK"), (dict(S=0, cs=None), "QSA_OK"),
])
def test_q_prep_validation(qsa, host, kw, code):
    for k in list(kw):
        if k.startswith("mis_"):
            name = k[4:]
            kw[name] = host.p(["q", "x", "cs", "ctx", "w"].index(name), kw.pop(k))
    assert _qprep(qsa, host, **kw) == getattr(qsa, code)
    if code != "QSA_OK":
        assert qsa.qsa_last_error()


def _pool(qsa, h, **kw):
    a = dict(poolPtr=h.p(5), pageTable=h.p(6), maxPagesPerSeq=4, numPages=16, numKVHeads=2,
             poolHeadDim=384, headSize=256)
    a.update(kw)
    return qsa.qsa_pool_state_t(a["poolPtr"], a["pageTable"], a["maxPagesPerSeq"],
                                a["numPages"], a["numKVHeads"], a["poolHeadDim"], a["headSize"])


def _kcomp(qsa, h, pool=None, ranges=None, **kw):
    a = dict(kb=h.p(0), x=h.p(1), cs=h.p(2), P=64, ctx=h.p(3), w=h.p(4), eps=1e-6, B=2, S=64,
             nb=16, bB=0, bE=16, p=0, dt=qsa.QSA_BF16)
    a.update(kw)
    return qsa.lib.qsa_index_k_compress(
        a["kb"], a["x"], a["cs"], a["P"], a["ctx"], a["w"], a["eps"], a["B"], a["S"], a["nb"],
        a["bB"], a["bE"], a["p"], None if ranges is None else ctypes.byref(ranges),
        None if pool is None else ctypes.byref(pool), a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=-1), "QSA_E_DTYPE"), (dict(bB=5, bE=4), "QSA_E_INVALID"),
    (dict(bE=17), "QSA_E_INVALID"), (dict(bB=-1), "QSA_E_INVALID"),
    (dict(p=-1), "QSA_E_INVALID"), (dict(nb=-1, bE=0), "QSA_E_INVALID"),
    (dict(P=60), "QSA_E_INVALID"), (dict(P=61), "QSA_OK_IF_NO_GPU"),
    (dict(kb=None), "QSA_E_INVALID"), (dict(kb=1024 + 8), "QSA_E_ALIGN"),
    (dict(eps=float("nan")), "QSA_E_INVALID"),
    (dict(bB=3, bE=3, kb=None, x=None), "QSA_OK"), (dict(B=0, kb=None), "QSA_OK"),
])
def test_k_compress_validation(qsa, host, kw, code):
    rc = _kcomp(qsa, host, **kw)
    if code == "QSA_OK_IF_NO_GPU":
        # maxPositions = 4*blockEnd - 3 passes validation; with no GPU nothing is launched
        assert rc == qsa.QSA_E_NO_DEVICE
    else:
        assert rc == getattr(qsa, code)


@pytest.mark.parametrize("kw,code", [
    (dict(numPages=0), "QSA_E_INVALID"), (dict(maxPagesPerSeq=0), "QSA_E_INVALID"),
    (dict(numKVHeads=0), "QSA_E_INVALID"), (dict(headSize=257), "QSA_E_INVALID"),
    (dict(headSize=-8), "QSA_E_INVALID"), (dict(headSize=252), "QSA_E_ALIGN"),
    (dict(poolHeadDim=387, headSize=256), "QSA_E_ALIGN"),
    (dict(numKVHeads=1, poolHeadDim=390), "QSA_E_ALIGN"),
    (dict(poolPtr=None), "QSA_E_INVALID"), (dict(pageTable=None), "QSA_E_INVALID"),
    (dict(poolPtr=8), "QSA_E_ALIGN"), (dict(numPages=2**30), "QSA_E_INVALID"),
])
def test_pool_validation(qsa, host, kw, code):
    for k in ("poolPtr", "pageTable"):
        if k in kw and kw[k] is not None:
            kw[k] = host.p(5) + kw[k]
    rc = _kcomp(qsa, host, pool=_pool(qsa, host, **kw))
    assert rc == getattr(qsa, code)
    rc = qsa.lib.qsa_index_persist(ctypes.byref(_pool(qsa, host, **kw)), host.p(1), None,
                                   host.p(3), 2, 64, 16, 0, 16, 0, None, qsa.QSA_BF16, None)
    assert rc == getattr(qsa, code)


def test_ranges_validation(qsa, host):
    r = qsa.qsa_seq_ranges_t(host.p(7), host.p(8), None, 1)
    assert _kcomp(qsa, host, ranges=r) == qsa.QSA_E_INVALID
    r = qsa.qsa_seq_ranges_t(host.p(7), host.p(8), host.p(9), -1)
    assert _kcomp(qsa, host, ranges=r) == qsa.QSA_E_INVALID
    r = qsa.qsa_seq_ranges_t(host.p(7), host.p(8), host.p(9, 2), 1)
    assert _kcomp(qsa, host, ranges=r) == qsa.QSA_E_ALIGN
    r = qsa.qsa_seq_ranges_t(host.p(7), host.p(8), host.p(9), 0)
    # scalars are ignored in ranges mode, so a bad scalar triplet does not matter
    assert _kcomp(qsa, host, ranges=r, bB=9, bE=2, kb=None) == qsa.QSA_OK


def test_persist_and_prefill_validation(qsa, host):
    L = qsa.lib
    assert L.qsa_index_persist(None, host.p(1), None, host.p(3), 2, 64, 16, 0, 16, 0, None,
                               qsa.QSA_BF16, None) == qsa.QSA_E_INVALID
    assert L.qsa_index_persist(ctypes.byref(_pool(qsa, host)), host.p(1), None, host.p(3), 2, 0,
                               16, 0, 16, 0, None, qsa.QSA_BF16, None) == qsa.QSA_OK
    assert L.qsa_index_persist(ctypes.byref(_pool(qsa, host)), host.p(1), host.p(2, 4),
                               host.p(3), 2, 64, 16, 0, 16, 0, None, qsa.QSA_BF16,
                               None) == qsa.QSA_E_ALIGN

    def pre(**kw):
        a = dict(q=host.p(0), kb=host.p(1), x=host.p(2), cs=host.p(3), P=64, ctx=host.p(4),
                 wq=host.p(5), wk=host.p(6), eps=1e-6, pool=None, B=2, S=64, nb=16,
                 dt=qsa.QSA_F16)
        a.update(kw)
        return L.qsa_index_prefill(a["q"], a["kb"], a["x"], a["cs"], a["P"], a["ctx"], a["wq"],
                                   a["wk"], a["eps"], a["pool"], a["B"], a["S"], a["nb"],
                                   a["dt"], None)
    assert pre(nb=15) == qsa.QSA_E_INVALID
    assert pre(S=61, nb=15) == qsa.QSA_E_INVALID         # ceilDiv(61, 4) = 16 > 15
    assert pre(S=60, nb=15) == qsa.QSA_E_NO_DEVICE       # valid; no GPU here: no launch
    assert pre(P=63) == qsa.QSA_E_INVALID
    assert pre(wk=None) == qsa.QSA_E_INVALID
    assert pre(dt=2) == qsa.QSA_E_DTYPE
    assert pre(B=0, q=None) == qsa.QSA_OK
    assert "maxPositions" in (pre(P=10) and qsa.qsa_last_error())


def test_next_rows_validation(qsa, host):
    """Decode pre-pass, scores, ids fill, expand and the selections: every invalid argument is
    rejected with its code before any launch, empty calls return QSA_OK."""
    L, h, BF = qsa.lib, host, qsa.QSA_BF16
    pool = ctypes.byref(_pool(qsa, h))
    E, A, D, OK = qsa.QSA_E_INVALID, qsa.QSA_E_ALIGN, qsa.QSA_E_DTYPE, qsa.QSA_OK

    def pre(**kw):
        a = dict(q=h.p(0), x=h.p(1), cs=h.p(2), P=64, ctx=h.p(3), nl=None, wq=h.p(4), wk=h.p(8),
                 eps=1e-6, pool=pool, B=2, S=4, dt=BF)
        a.update(kw)
        return L.qsa_index_pre_decode(a["q"], a["x"], a["cs"], a["P"], a["ctx"], a["nl"],
                                      a["wq"], a["wk"], a["eps"], a["pool"], a["B"], a["S"],
                                      a["dt"], None)
    assert pre(dt=3) == D and pre(S=0) == E and pre(P=-1) == E and pre(B=-1) == E
    assert pre(q=None) == E and pre(x=h.p(1, 2)) == A and pre(nl=h.p(9, 2)) == A
    assert pre(eps=-1.0) == E and pre(pool=None) == E and pre(B=0, q=None, pool=None) == OK
    assert pre(B=2**24) == E                                  # more workgroups than a launch

    def sc(**kw):
        a = dict(lg=h.p(0), q=h.p(1), kb=h.p(2), ctx=h.p(3), B=2, S=64, nb=16, r0=0, n=128, dt=BF)
        a.update(kw)
        return L.qsa_index_scores(a["lg"], a["q"], a["kb"], a["ctx"], a["B"], a["S"], a["nb"],
                                  a["r0"], a["n"], a["dt"], None)
    assert sc(dt=-2) == D and sc(B=-1) == E and sc(r0=-1) == E and sc(n=-1) == E
    assert sc(r0=1) == E and sc(n=129) == E                   # chunk past B*S rows
    assert sc(nb=2**26 + 1) == E and sc(lg=None) == E and sc(q=h.p(1, 8)) == A
    assert sc(kb=h.p(2, 4)) == A and sc(ctx=h.p(3, 2)) == A and sc(lg=h.p(0, 2)) == A
    assert sc(n=0, lg=None, q=None) == OK and sc(nb=0, lg=None) == OK

    def scd(**kw):
        a = dict(lg=h.p(0), q=h.p(1), ctx=h.p(3), pool=pool, B=2, mb=16, dt=BF)
        a.update(kw)
        return L.qsa_index_scores_decode(a["lg"], a["q"], a["ctx"], a["pool"], a["B"], a["mb"],
                                         a["dt"], None)
    assert scd(dt=9) == D and scd(B=-1) == E and scd(mb=-1) == E
    # B * ceil(maxBlocks / 128) workgroups of 64 threads, at most 2^26 - 1
    assert scd(B=2**19, mb=2**14 + 1) == E and scd(B=2**19 - 1, mb=2**14) != E
    assert scd(lg=None) == E and scd(q=h.p(1, 2)) == A and scd(pool=None) == E
    assert scd(B=2**26) == E and scd(B=0, pool=None) == OK and scd(mb=0, lg=None) == OK

    assert L.qsa_index_ids_fill(None, 4, 16, None) == E
    assert L.qsa_index_ids_fill(h.p(0, 2), 4, 16, None) == A
    assert L.qsa_index_ids_fill(h.p(0), -1, 16, None) == E
    assert L.qsa_index_ids_fill(None, 0, 16, None) == OK and L.qsa_index_ids_fill(None, 4, 0, None) == OK

    def ex(**kw):
        a = dict(out=h.p(0), ids=h.p(1), ctx=h.p(3), B=2, S=64, nb=16, r0=0, n=128)
        a.update(kw)
        return L.qsa_index_expand(a["out"], a["ids"], a["ctx"], a["B"], a["S"], a["nb"],
                                  a["r0"], a["n"], None)
    assert ex(nb=15) == E                                     # fewer sorted ids than S/4
    assert ex(S=4096, nb=511, n=64) == E and ex(S=4096, nb=512, n=64, out=None) == E
    assert ex(r0=100, n=29) == E and ex(out=h.p(0, 2)) == A and ex(ids=None) == E
    assert ex(S=3, nb=0, n=6, ids=None, r0=0) != E            # no id is read when S/4 = 0
    assert ex(n=0, out=None) == OK

    def tk(**kw):
        a = dict(out=h.p(0), lg=h.p(1), ctx=h.p(3), B=2, S=64, nb=16, r0=0, n=128)
        a.update(kw)
        return L.qsa_index_topk_expand(a["out"], a["lg"], a["ctx"], a["B"], a["S"], a["nb"],
                                       a["r0"], a["n"], None)
    assert tk(B=-1) == E and tk(r0=120, n=9) == E and tk(out=None) == E
    assert tk(lg=h.p(1, 2)) == A and tk(ctx=None) == E and tk(n=0, out=None) == OK

    def tkd(**kw):
        a = dict(out=h.p(0), lg=h.p(1), ctx=h.p(3), sc=None, H=0, B=2, mb=1000)
        a.update(kw)
        return L.qsa_index_topk_expand_decode(a["out"], a["lg"], a["ctx"], a["sc"], a["H"],
                                              a["B"], a["mb"], None)
    assert tkd(B=-1) == E and tkd(mb=-1) == E and tkd(sc=h.p(4), H=-1) == E
    assert tkd(sc=h.p(4, 2), H=2) == A and tkd(out=None) == E and tkd(lg=None) == E
    assert tkd(B=2**23) == E                                  # 512-thread workgroups
    # rows of more than 32768 blocks take one workgroup per chunk of up to 8 (8192 to 32768
    # keys each): the grid is batchSize * chunks (valid calls: no device here, no launch)
    ND = qsa.QSA_E_NO_DEVICE
    far = h.p(0) + (2**20) * 65536 * 4 + 4096                 # outIdx past the largest logits
    assert tkd(B=2**20 - 1, mb=65536, out=far) == ND          # 8 chunks: 2^23 - 8 workgroups
    assert tkd(B=2**20, mb=65536, out=far) == E
    assert tkd(B=2**21, mb=32772, out=far) == E               # 5 chunks of 8192
    assert tkd(B=2**21 - 1, mb=262145) == ND                  # longer rows: one per sequence
    # split rows stage candidates in outIdx: it may not overlap logits
    assert tkd(out=h.p(1), lg=h.p(1), mb=65536) == E
    assert tkd(out=h.p(1), lg=h.p(1), mb=32768) == ND          # one workgroup per row: allowed
    assert tkd(mb=512, lg=None) != E                          # nVis <= 512 reads no logits
    assert tkd(B=0, out=None) == OK


def test_stream_copy_validation(qsa, host):
    L, h = qsa.lib, host
    assert L.qsa_stream_copy(h.p(0), h.p(1), 24, None) == qsa.QSA_E_INVALID
    assert L.qsa_stream_copy(h.p(0), h.p(1), -16, None) == qsa.QSA_E_INVALID
    assert L.qsa_stream_copy(None, h.p(1), 32, None) == qsa.QSA_E_INVALID
    assert L.qsa_stream_copy(h.p(0, 8), h.p(1), 32, None) == qsa.QSA_E_ALIGN
    assert L.qsa_stream_copy(h.p(0), h.p(1, 4), 32, None) == qsa.QSA_E_ALIGN
    assert L.qsa_stream_copy(None, None, 0, None) == qsa.QSA_OK


def test_valid_calls_report_no_device(qsa, host):
    """Every entry point, given valid arguments and work to do on a machine with no GPU,
    returns QSA_E_NO_DEVICE (nothing launched) with a message naming the cause."""
    L, h, BF = qsa.lib, host, qsa.QSA_BF16
    pool = ctypes.byref(_pool(qsa, h))
    ND = qsa.QSA_E_NO_DEVICE
    calls = {
        "q_prep": lambda: _qprep(qsa, h),
        "k_compress": lambda: _kcomp(qsa, h),
        "k_compress_paged": lambda: _kcomp(qsa, h, pool=_pool(qsa, h)),
        "persist": lambda: L.qsa_index_persist(pool, h.p(1), None, h.p(3), 2, 64, 16, 0, 16, 0,
                                               None, BF, None),
        "prefill": lambda: L.qsa_index_prefill(h.p(0), h.p(1), h.p(2), h.p(3), 64, h.p(4),
                                               h.p(5), h.p(6), 1e-6, None, 2, 64, 16, BF, None),
        "pre_decode": lambda: L.qsa_index_pre_decode(h.p(0), h.p(1), h.p(2), 64, h.p(3), None,
                                                     h.p(4), h.p(8), 1e-6, pool, 2, 4, BF,
                                                     None),
        "scores": lambda: L.qsa_index_scores(h.p(0), h.p(1), h.p(2), h.p(3), 2, 64, 16, 0, 128,
                                             BF, None),
        "scores_decode": lambda: L.qsa_index_scores_decode(h.p(0), h.p(1), h.p(3), pool, 2, 16,
                                                           BF, None),
        "ids_fill": lambda: L.qsa_index_ids_fill(h.p(0), 4, 16, None),
        "expand": lambda: L.qsa_index_expand(h.p(0), h.p(1), h.p(3), 2, 64, 16, 0, 128, None),
        "topk_expand": lambda: L.qsa_index_topk_expand(h.p(0), h.p(1), h.p(3), 2, 64, 16, 0,
                                                       128, None),
        "topk_expand_decode": lambda: L.qsa_index_topk_expand_decode(h.p(0), h.p(1), h.p(3),
                                                                     None, 0, 2, 1000, None),
        "stream_copy": lambda: L.qsa_stream_copy(h.p(0), h.p(1), 64, None),
    }
    for name, call in calls.items():
        assert call() == ND, name
        assert "no usable HIP device" in qsa.qsa_last_error(), name
