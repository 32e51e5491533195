"""The C ABI: the library loads, exports every declared symbol, and rejects bad
arguments on the host before enqueueing anything.  No GPU is touched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wf_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wf_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def wf():
    import video_diffusion_dit_amd as wf
    return wf


def test_every_declared_symbol_is_exported(wf):
    names = declared_functions()
    assert "wf_attn_dense" in names and "wf_vsa_coarse_topk" in names and "wf_vsa_fine" in names
    assert len(names) == 20
    for n in names:
        assert hasattr(wf.lib, n), f"{n} declared in wf_attn.h but not exported"


def test_status_strings(wf):
    assert wf.lib.wf_status_string(0) == b"WF_OK"
    assert wf.lib.wf_status_string(4) == b"WF_ERR_BAD_INDEX"
    assert wf.lib.wf_status_string(99) == b"WF_UNKNOWN_STATUS"
    assert wf.lib.wf_abi_version() == 4


def test_geometry_queries(wf):
    assert wf.num_cubes(21, 30, 52) == 624
    assert wf.num_cubes(21, 45, 80) == 1440
    assert wf.num_cubes(1, 1, 1) == 1
    assert wf.num_cubes(0, 4, 4) == 0
    assert wf.dense_workspace_bytes(2, 40, 32760, 128) == 2 * 40 * 128 * 32768 * 2
    assert wf.dense_workspace_bytes(1, 1, 0, 128) == 0
    ws = wf.vsa_workspace_bytes(1, 40, 21, 30, 52, 128)
    assert ws >= 3 * 40 * 624 * 64 * 128 * 2 + 2 * 40 * 624 * 128 * 4 + 40 * 624 * 624 * 4
    assert wf.vsa_workspace_bytes(1, 40, 21, 30, 52, 64) == 0


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def dense(wf, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, Hh=1, N=64, D=128, scale=0.1,
             ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return wf.lib.wf_attn_dense(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hh"], a["N"],
                                a["D"], a["scale"], a["ws"], a["wsb"], a["stream"])


def test_dense_argument_errors(wf):
    assert dense(wf, q=None) == 1
    assert b"q is NULL" in wf.lib.wf_last_error_detail()
    assert dense(wf, o=FAKE + 4) == 1
    assert b"aligned" in wf.lib.wf_last_error_detail()
    assert dense(wf, lse=FAKE + 8) == 1
    assert dense(wf, N=0) == 1
    assert dense(wf, B=-1) == 1
    assert dense(wf, N=1 << 24) == 1          # N*D does not fit in int32
    assert dense(wf, N=1 << 23) == 2          # one head's K reaches 2 GiB (32-bit descriptors)
    assert dense(wf, N=(1 << 23) - 64) == 3   # just below: accepted, but the workspace is short
    assert dense(wf, N=1 << 24, D=64) == 2    # the same bound at D = 64
    assert dense(wf, D=96) == 2
    assert dense(wf, scale=float("nan")) == 1
    assert dense(wf, scale=0.0) == 1
    assert dense(wf, ws=None) == 3
    assert dense(wf, wsb=16) == 3
    assert b"need" in wf.lib.wf_last_error_detail()


def coarse(wf, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, B=1, Hh=2, T=5, H=6, W=7, D=128, scale=0.1, topk=3,
             idx=FAKE, scores=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return wf.lib.wf_vsa_coarse_topk(a["q"], a["k"], a["v"], a["B"], a["Hh"], a["T"], a["H"], a["W"],
                                     a["D"], a["scale"], a["topk"], a["idx"], a["scores"], a["ws"],
                                     a["wsb"], None)


def test_launch_grid_limits(wf):
    """Shapes whose launch grids would not fit in 31 bits are refused up front, whatever workspace
    size the caller declares."""
    big = (1 << 62)
    # dense: B * Hh * ceil(N / 64) workgroups for the V^T transpose
    assert wf.lib.wf_attn_dense(FAKE, FAKE, FAKE, FAKE, None, 1, 1 << 23, 1 << 20, 128, 0.1, FAKE, big, None) == 2
    assert b"too many workgroups" in wf.lib.wf_last_error_detail()
    # VSA: B * Hh * C workgroups (C = 4096 here)
    assert coarse(wf, B=1, Hh=1 << 20, T=61, H=62, W=63, wsb=big) == 2
    assert b"too many workgroups" in wf.lib.wf_last_error_detail()


def test_vsa_argument_errors(wf):
    assert coarse(wf, idx=None) == 1
    assert coarse(wf, topk=0) == 1
    assert coarse(wf, topk=9) == 1            # 5x6x7 pads to 8x8x8: 8 cubes
    assert b"topk 9" in wf.lib.wf_last_error_detail()
    assert coarse(wf, D=64) == 2
    assert coarse(wf, T=0) == 1
    assert coarse(wf, T=80, H=80, W=48) == 2      # 4800 cubes: more than 4096
    assert coarse(wf, T=400, H=400, W=400) == 1   # padded tokens x D overflow int32
    assert coarse(wf, wsb=100) == 3
    assert coarse(wf, scores=FAKE + 2) == 1
    fine = wf.lib.wf_vsa_fine
    assert fine(FAKE, 1 << 30, None, 1, 2, 5, 6, 7, 128, 0.1, 3, FAKE, None, None) == 1
    assert fine(FAKE, 1 << 30, FAKE, 1, 2, 5, 6, 7, 128, 0.1, 0, FAKE, None, None) == 1
    assert fine(FAKE, 10, FAKE, 1, 2, 5, 6, 7, 128, 0.1, 3, FAKE, None, None) == 3
    assert fine(FAKE, 1 << 30, FAKE, 1, 2, 5, 6, 7, 128, float("inf"), 3, FAKE, None, None) == 1
    one = wf.lib.wf_vsa  # the one-call path: the coarse stage's checks, plus o, gate and o_coarse
    assert one(FAKE, FAKE, FAKE, 1, 2, 5, 6, 7, 128, 0.1, 3, FAKE, None, None, None, None, FAKE, 1 << 30, None) == 1
    assert one(FAKE, FAKE, FAKE, 1, 2, 5, 6, 7, 128, 0.1, 9, FAKE, None, FAKE, None, None, FAKE, 1 << 30, None) == 1
    assert one(FAKE, FAKE, FAKE, 1, 2, 5, 6, 7, 64, 0.1, 3, FAKE, None, FAKE, None, None, FAKE, 1 << 30, None) == 2
    assert one(FAKE, FAKE, FAKE, 1, 2, 5, 6, 7, 128, 0.1, 3, FAKE, None, FAKE, None, None, FAKE, 100, None) == 3
    assert one(FAKE, FAKE, FAKE, 1, 2, 5, 6, 7, 128, 0.1, 3, FAKE, None, FAKE, FAKE + 2, None, FAKE, 1 << 30,
               None) == 1
    assert one(FAKE, FAKE, FAKE, 1, 2, 5, 6, 7, 128, 0.1, 3, FAKE, None, FAKE, None, FAKE, FAKE, 1 << 30, None) == 1
    assert b"o_coarse given without a gate" in wf.lib.wf_last_error_detail()
    assert one(FAKE, FAKE, FAKE, 1, 2, 5, 6, 7, 128, 0.1, 3, FAKE, FAKE + 2, FAKE, None, None, FAKE, 1 << 30,
               None) == 1
    rope = wf.lib.wf_rope_qk
    assert rope(FAKE, FAKE, FAKE, FAKE, 1, 2, 5, 6, 7, 128, 0.0, 32, None) == 1
    assert rope(FAKE, FAKE, FAKE, FAKE, 1, 2, 5, 6, 7, 96, 1e4, 32, None) == 2
    assert rope(None, FAKE, FAKE, FAKE, 1, 2, 5, 6, 7, 128, 1e4, 32, None) == 1
    assert rope(FAKE, FAKE, FAKE + 2, FAKE, 1, 2, 5, 6, 7, 128, 1e4, 32, None) == 1
    assert rope(FAKE, FAKE, FAKE, FAKE, 1, 2, 0, 6, 7, 128, 1e4, 32, None) == 1
    assert rope(FAKE, FAKE, FAKE, FAKE, 1, 2, 5, 6, 7, 128, 1e4, 16, None) == 1
    cr = wf.lib.wf_vsa_coarse_topk_rope
    assert cr(FAKE, FAKE, FAKE, 1, 2, 5, 6, 7, 128, 0.1, 3, float("inf"), 32, FAKE, None, FAKE, 1 << 30, None) == 1
    assert cr(FAKE, FAKE, FAKE, 1, 2, 5, 6, 7, 128, 0.1, 3, -1.0, 32, FAKE, None, FAKE, 1 << 30, None) == 1
    assert cr(FAKE, FAKE, FAKE, 1, 2, 5, 6, 7, 128, 0.1, 9, 1e4, 32, FAKE, None, FAKE, 1 << 30, None) == 1
    assert cr(FAKE, FAKE, FAKE, 1, 2, 5, 6, 7, 128, 0.1, 3, 1e4, 48, FAKE, None, FAKE, 1 << 30, None) == 1
    dex = wf.lib.wf_attn_dense_ex
    assert dex(FAKE, FAKE, FAKE, FAKE, None, 1, 1, 64, 128, 0.1, 3, FAKE, 1 << 30, None) == 1
    assert dex(FAKE, FAKE, FAKE, FAKE, None, 1, 1, 64, 128, 0.1, -1, FAKE, 1 << 30, None) == 1
    assert dex(FAKE, FAKE, FAKE, FAKE, None, 1, 1, 64, 96, 0.1, 1, FAKE, 1 << 30, None) == 2
    fex = wf.lib.wf_vsa_fine_ex
    assert fex(FAKE, 1 << 30, FAKE, 1, 2, 5, 6, 7, 128, 0.1, 3, 7, FAKE, None, None) == 1
    assert fex(FAKE, 10, FAKE, 1, 2, 5, 6, 7, 128, 0.1, 3, 2, FAKE, None, None) == 3
    sta = wf.lib.wf_sta
    G = (18, 48, 80)                                       # a tuned grid: 3 x 6 x 10 tiles of 6x8x8
    assert sta(FAKE, FAKE, FAKE, 1, 2, *G, 128, 0.1, 4, 1, 1, FAKE, None, None, FAKE, 1 << 30, None) == 1
    assert sta(FAKE, FAKE, FAKE, 1, 2, *G, 128, 0.1, 1, 7, 1, FAKE, None, None, FAKE, 1 << 30, None) == 1
    assert sta(FAKE, FAKE, FAKE, 1, 2, *G, 128, 0.1, 0, 1, 1, FAKE, None, None, FAKE, 1 << 30, None) == 1
    assert sta(FAKE, FAKE, FAKE, 1, 2, *G, 64, 0.1, 1, 1, 1, FAKE, None, None, FAKE, 1 << 30, None) == 2
    assert sta(FAKE, FAKE, FAKE, 1, 2, *G, 128, 0.1, 2, 2, 2, FAKE, None, None, FAKE, 10, None) == 3
    assert sta(FAKE, FAKE, FAKE, 1, 2, *G, 128, 0.1, 2, 2, 2, FAKE, None, FAKE + 2, FAKE, 1 << 30, None) == 1
    for grid in ((5, 6, 7), (31, 22, 40), (36, 48, 40), (24, 48, 48)):   # not tuned: refused, no GPU work
        assert sta(FAKE, FAKE, FAKE, 1, 2, *grid, 128, 0.1, 1, 1, 1, FAKE, None, None, FAKE, 1 << 30, None) == 2
        assert b"tuned grids" in wf.lib.wf_last_error_detail()
        assert wf.lib.wf_sta_workspace_bytes(1, 2, *grid, 128, 1, 1, 1) == 0
    assert wf.lib.wf_sta_workspace_bytes(1, 40, 36, 48, 48, 128, 3, 3, 3) > 0
    assert wf.lib.wf_sta_workspace_bytes(1, 40, 36, 48, 48, 128, 7, 1, 1) == 0
    gated = wf.lib.wf_vsa_fine_gated
    assert gated(FAKE, 1 << 30, FAKE, None, 1, 2, 5, 6, 7, 128, 0.1, 3, FAKE, None, None, None) == 1
    assert gated(FAKE, 1 << 30, FAKE, FAKE + 4, 1, 2, 5, 6, 7, 128, 0.1, 3, FAKE, None, None, None) == 1
    assert gated(FAKE, 1 << 30, FAKE, FAKE, 1, 2, 5, 6, 7, 128, 0.1, 3, FAKE, None, FAKE + 8, None) == 1
    assert gated(FAKE, 1 << 30, None, FAKE, 1, 2, 5, 6, 7, 128, 0.1, 3, FAKE, None, None, None) == 1
    assert gated(FAKE, 1 << 30, FAKE, FAKE, 1, 2, 5, 6, 7, 128, 0.1, 9, FAKE, None, None, None) == 1
    assert gated(FAKE, 1 << 30, FAKE, FAKE, 1, 2, 5, 6, 7, 64, 0.1, 3, FAKE, None, None, None) == 2
    assert gated(FAKE, 10, FAKE, FAKE, 1, 2, 5, 6, 7, 128, 0.1, 3, FAKE, None, None, None) == 3


def test_profile_query_without_records(wf):
    assert wf.lib.wf_profile_enable(1) == 0
    n, ms = ctypes.c_int64(), ctypes.c_double()
    assert wf.lib.wf_profile_query(b"wf_dense_fwd", ctypes.byref(n), ctypes.byref(ms)) == 1
    assert wf.lib.wf_profile_enable(0) == 0


def test_error_detail_is_per_thread(wf):
    """wf_last_error_detail is thread-local: concurrent failures each read back their own message."""
    import threading
    results = {}
    barrier = threading.Barrier(8)

    def worker(i):
        barrier.wait()
        for _ in range(200):
            topk = 9 + i                       # 5x6x7 has 8 cubes: every topk here is rejected
            st = wf.lib.wf_vsa_coarse_topk(FAKE, FAKE, FAKE, 1, 1, 5, 6, 7, 128, 0.1, topk, FAKE, None, FAKE,
                                           1 << 30, None)
            msg = wf.lib.wf_last_error_detail()
            if st != 1 or f"topk {topk} ".encode() not in msg:
                results[i] = msg
                return
        results[i] = b"ok"

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert all(v == b"ok" for v in results.values()) and len(results) == 8, results
