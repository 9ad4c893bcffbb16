"""CPU tests of the C ABI: the library loads, exports what include/kda.h
declares, and rejects bad arguments on the host without launching anything."""

import ctypes
import os
import re

import pytest

from gated_delta_rule_fwd_amd import kda as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*|size_t)\s+(kda_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(K.LIB_PATH):
        pytest.skip("libkda.so not built")
    return K.lib()


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for fn in ("kda_fwd_chunked", "kda_fwd_recurrent", "kda_decode_step", "kda_status_string"):
        assert fn in names


def test_library_exports_every_declared_symbol(L):
    for fn in declared_functions():
        assert hasattr(L, fn), fn


def test_status_strings_and_version(L):
    assert L.kda_abi_version() == 202
    assert L.kda_status_string(0) == b"ok"
    for code in (1, 2, 3, 4, 5, 6):
        assert len(L.kda_status_string(code)) > 3
    assert L.kda_status_string(99) == b"unknown status"


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
BIG = 1 << 40                    # a workspace size no validation rejects


def chunked(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, decay=None, kind=0, init=None, o=FAKE, fs=FAKE,
             B=1, T=8, H=1, HV=None, DK=64, DV=64, dtype=1, scale=0.0, l2=1, vf=0, chunk=64,
             A=None, dt=None, lb=0.0, tf=0, ws=FAKE, wsb=BIG)
    a.update(kw)
    hv = a["H"] if a["HV"] is None else a["HV"]
    return L.kda_fwd_chunked(a["q"], a["k"], a["v"], a["beta"], a["decay"], a["kind"], a["init"],
                             a["o"], a["fs"], a["B"], a["T"], a["H"], hv, a["DK"], a["DV"],
                             a["dtype"], a["scale"], a["l2"], a["vf"], a["chunk"], a["A"], a["dt"],
                             a["lb"], a["tf"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(fs=None), 1), (dict(beta=None), 1),
    (dict(kind=1, decay=None), 1), (dict(kind=2, decay=None), 1),
    (dict(B=0), 2), (dict(H=0), 2), (dict(T=-1), 2), (dict(B=1 << 20, T=1 << 12, H=8), 2),
    (dict(DK=48), 3), (dict(DV=256), 3), (dict(dtype=7), 3), (dict(kind=5), 3),
    (dict(chunk=128), 3), (dict(chunk=8), 3),
    # input transforms: KDA_TF_GATE 1, LOWER_BOUND 2, BETA_SIGMOID 4, NEG_EIGVAL 8
    (dict(tf=16), 4),                                            # unknown bit
    (dict(tf=1, A=FAKE), 4),                                     # raw gate, no decay tensor
    (dict(tf=2, kind=1, decay=FAKE), 4),                         # floor without the raw gate
    (dict(tf=3, kind=1, decay=FAKE, A=FAKE, lb=0.5), 4),         # floor above zero
    (dict(tf=3, kind=2, decay=FAKE, A=FAKE, lb=float("nan")), 4),
    (dict(tf=8), 4),                                             # 2 sigmoid without sigmoid
    (dict(tf=1, kind=1, decay=FAKE), 1),                         # raw gate without A_log
    # value heads: a multiple of the q/k heads; state layout flag 0 or 1
    (dict(H=2, HV=3), 2), (dict(H=2, HV=0), 2), (dict(H=4, HV=2), 2), (dict(HV=65536), 2),
    (dict(vf=2), 4), (dict(vf=-1), 4),
    # caller-owned workspace: present, 16-byte aligned, at least one chunk of every head
    (dict(ws=None), 6), (dict(ws=ctypes.c_void_p(0x1008)), 6), (dict(wsb=0), 6),
    (dict(B=2, H=3, wsb=6 * 9000), 6),
])
def test_chunked_rejects_bad_arguments(L, kw, code):
    assert chunked(L, **kw) == code


def test_recurrent_and_decode_reject_bad_arguments(L):
    assert L.kda_fwd_recurrent(None, FAKE, FAKE, FAKE, None, 0, None, FAKE, FAKE,
                               1, 4, 1, 1, 64, 64, 1, 0.0, 1, 0, None, None, 0.0, 0, None) == 1
    assert L.kda_fwd_recurrent(FAKE, FAKE, FAKE, FAKE, None, 0, None, FAKE, FAKE,
                               1, 4, 1, 1, 96, 64, 1, 0.0, 1, 0, None, None, 0.0, 0, None) == 3
    assert L.kda_fwd_recurrent(FAKE, FAKE, FAKE, FAKE, None, 0, None, FAKE, FAKE,
                               1, 4, 1, 1, 64, 64, 1, 0.0, 1, 0, None, None, 0.0, 8, None) == 4
    assert L.kda_fwd_recurrent(FAKE, FAKE, FAKE, FAKE, None, 0, None, FAKE, FAKE,
                               1, 4, 2, 3, 64, 64, 1, 0.0, 1, 0, None, None, 0.0, 0, None) == 2
    assert L.kda_decode_step(FAKE, FAKE, FAKE, FAKE, None, 0, None, FAKE,
                             1, 1, 1, 64, 64, 1, 0.0, 1, 0, None, None, 0.0, 0, None) == 1
    assert L.kda_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, 2, FAKE, FAKE,
                             0, 1, 1, 64, 64, 1, 0.0, 1, 0, None, None, 0.0, 0, None) == 2
    assert L.kda_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, 2, FAKE, FAKE,
                             1, 1, 1, 64, 64, 1, 0.0, 1, 0, None, None, 0.0, 1, None) == 1
    assert L.kda_decode_step(FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, FAKE,
                             1, 1, 1, 64, 64, 1, 0.0, 1, 3, None, None, 0.0, 0, None) == 4


def varlen(L, cu, N, T=8, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, decay=None, kind=0, init=None, o=FAKE, fs=FAKE,
             cud=FAKE, H=1, HV=1, DK=64, DV=64, dtype=1, scale=0.0, l2=1, vf=0, chunk=64,
             A=None, dt=None, lb=0.0, tf=0, ws=FAKE, wsb=BIG)
    a.update(kw)
    cuh = None if cu is None else (ctypes.c_int * len(cu))(*cu)
    return L.kda_fwd_chunked_varlen(a["q"], a["k"], a["v"], a["beta"], a["decay"], a["kind"],
                                    a["init"], a["o"], a["fs"], a["cud"], cuh, N, T, a["H"],
                                    a["HV"], a["DK"], a["DV"], a["dtype"], a["scale"], a["l2"],
                                    a["vf"], a["chunk"], a["A"], a["dt"], a["lb"], a["tf"],
                                    a["ws"], a["wsb"], None)


@pytest.mark.parametrize("cu,N,T,kw,code", [
    (None, 2, 8, {}, 1),                       # no host offsets
    ([0, 4, 8], 2, 8, dict(cud=None), 1),      # no device offsets
    ([0, 4, 8], 2, 8, dict(fs=None), 1),
    ([0, 8], 0, 8, {}, 2),                     # N < 1
    ([1, 4, 8], 2, 8, {}, 2),                  # does not start at 0
    ([0, 4, 7], 2, 8, {}, 2),                  # does not end at T
    ([0, 6, 4, 8], 3, 8, {}, 2),               # decreasing
    ([0, 4, 8], 2, 8, dict(chunk=128), 3),
    ([0, 4, 8], 2, 8, dict(DK=48), 3),
    ([0, 4, 8], 2, 8, dict(tf=12 | 16), 4),
    ([0, 4, 8], 2, 8, dict(ws=None), 6),
    ([0, 4, 8], 2, 8, dict(wsb=100), 6),
])
def test_varlen_rejects_bad_arguments(L, cu, N, T, kw, code):
    assert varlen(L, cu, N, T, **kw) == code


def _rec(L, DK, C, dtype, kind, heads=1):
    """record bytes of one chunk (T = chunk_size) for `heads` value heads"""
    return L.kda_fwd_chunked_workspace_bytes(1, C, heads, heads, DK, DK, dtype, kind, C)


def test_workspace_size_query(L):
    q = L.kda_fwd_chunked_workspace_bytes
    for dtype in (0, 1):
        for kind in (0, 1, 2):
            for C in (16, 32, 64):
                one = _rec(L, 128, C, dtype, kind)
                assert one > 0 and one % 256 == 0
                # one record per (batch, value head, chunk); a ragged tail is a whole chunk
                assert q(3, 5 * C + 1, 2, 4, 128, 128, dtype, kind, C) == one * 3 * 4 * 6
                assert q(3, C, 2, 4, 128, 128, dtype, kind, C) == one * 3 * 4
    # what the request does not support, and no tokens, give 0
    assert q(1, 0, 1, 1, 128, 128, 1, 1, 64) == 0
    assert q(1, 64, 1, 1, 96, 128, 1, 1, 64) == 0
    assert q(1, 64, 1, 1, 128, 128, 1, 1, 128) == 0
    assert q(1, 64, 2, 3, 128, 128, 1, 1, 64) == 0
    assert q(1, 64, 1, 1, 128, 128, 5, 1, 64) == 0


def test_varlen_workspace_size_query(L):
    q = L.kda_fwd_chunked_varlen_workspace_bytes
    one = _rec(L, 64, 32, 1, 2, heads=2)
    cu = (ctypes.c_int * 5)(0, 0, 33, 97, 100)     # 0, 2, 2 and 1 chunks of 32
    need = q(cu, 4, 1, 2, 64, 64, 1, 2, 32)
    assert need >= one * 5 and need - one * 5 >= 5 * 4 and need - one * 5 < 5 * 4 + 16
    assert q(cu, 4, 1, 2, 64, 64, 1, 2, 128) == 0
    assert q((ctypes.c_int * 2)(0, 0), 1, 1, 1, 64, 64, 1, 2, 32) == 0
    assert q((ctypes.c_int * 3)(0, 9, 4), 2, 1, 1, 64, 64, 1, 2, 32) == 0


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 1, 32)
    with pytest.raises(ValueError):
        K.fwd_chunked(x, x, x, torch.zeros(1, 4, 1))


def test_noalloc_constant_and_size_limit(L):
    text = open(HEADER).read()
    import re as _re
    m = _re.search(r"#define\s+KDA_NOALLOC_WORKSPACE_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == K.NOALLOC_WORKSPACE_BYTES
    # one chunk of 2048 per-channel D128 heads needs more than the scratch: refused on the
    # host before any HIP call
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 2, None, FAKE, FAKE,
            1, 64, 2048, 2048, 128, 128, 1, 0.0, 1, 0, 64, None, None, 0.0, 0, None]
    assert L.kda_fwd_chunked_workspace_bytes(1, 64, 2048, 2048, 128, 128, 1, 2, 64) > \
        K.NOALLOC_WORKSPACE_BYTES
    assert L.kda_fwd_chunked_noalloc(*args) == 6
    args[2] = None
    assert L.kda_fwd_chunked_noalloc(*args) == 1


def test_backward_rejects_bad_arguments(L):
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, decay=None, kind=0, init=None, do=FAKE,
                 dfin=None, dq=FAKE, dk=FAKE, dv=FAKE, db=FAKE, dg=None, dinit=None, B=1, T=8,
                 H=1, HV=1, DK=64, DV=64, dtype=1, vfirst=0, A_log=None, bias=None, tf=0,
                 dA=None, dbias=None, ws=FAKE, wsb=BIG)
        a.update(kw)
        return L.kda_bwd(a["q"], a["k"], a["v"], a["beta"], a["decay"], a["kind"], a["init"],
                         a["do"], a["dfin"], a["dq"], a["dk"], a["dv"], a["db"], a["dg"],
                         a["dinit"], a["B"], a["T"], a["H"], a["HV"], a["DK"], a["DV"],
                         a["dtype"], 0.0, 1, a["vfirst"], a["A_log"], a["bias"], 0.0, a["tf"],
                         a["dA"], a["dbias"], a["ws"], a["wsb"], None)
    assert call(do=None) == 1
    assert call(dq=None) == 1
    assert call(kind=1, decay=FAKE) == 1          # a decay needs its gradient
    assert call(DK=48) == 3
    assert call(H=2, HV=3) == 2
    assert call(ws=None) == 6
    assert call(wsb=L.kda_bwd_workspace_bytes(1, 8, 1, 64, 64) - 1) == 6
    # the raw gate: A_log and its gradient are required, and a dt_bias needs its gradient
    gate = dict(kind=1, decay=FAKE, dg=FAKE, tf=1)
    assert call(**gate) == 1                      # no A_log
    assert call(**gate, A_log=FAKE) == 1          # no dA_log
    assert call(**gate, A_log=FAKE, dA=FAKE, bias=FAKE) == 1
    assert call(tf=1, A_log=FAKE, dA=FAKE) == 4   # a raw gate needs a decay
    assert call(tf=64) == 4                       # an unknown flag
    # the chunked form's records (chunks of 32): five per-token factors, T
    # and P per chunk, each in whole 64-float blocks, the state and its
    # gradient at every chunk start, and a cumulative decay per token and
    # key channel
    def chunked(B, T, HV, DK, DV):
        blk = lambda n: -(-n // 64) * 64
        ch = B * HV * -(-T // 32)
        return 4 * (5 * blk(B * T * HV) + 2 * blk(ch * 32 * 32) + 2 * ch * DK * DV + B * T * HV * DK)
    for args in ((2, 33, 3, 64, 32), (1, 100, 2, 128, 128), (3, 7, 1, 32, 64)):
        assert L.kda_bwd_workspace_bytes(*args) == chunked(*args), args
    assert L.kda_bwd_workspace_bytes(1, 0, 1, 64, 64) == 0
