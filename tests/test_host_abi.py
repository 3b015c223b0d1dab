"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, sizes its buffers by the documented formulas, and rejects
invalid calls with the documented codes before any launch.  No call here
reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import align_moe_route_amd as amr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]

# aligned fake device addresses: never dereferenced, validation fails first
P = 0x10000
Q = 0x20000


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(moe_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    L = amr.lib()
    names = declared_functions()
    assert set(names) == set(amr.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_strerror_names_every_code():
    for c in range(-7, 1):
        s = amr.strerror(c)
        assert s and "unknown" not in s
    assert "unknown" in amr.strerror(-99)


def test_capacity_formulas():
    for M, E, k, block in [(1, 896, 16, 32), (8192, 896, 16, 128), (16384, 4096, 16, 128),
                           (4, 64, 4, 16), (0, 8, 2, 4), (3, 2, 2, 1), (512, 896, 16, 64)]:
        routes = M * k
        rows = routes + min(E, routes) * (block - 1)
        assert amr.max_rows(M, E, k, block) == rows
        assert amr.max_blocks(M, E, k, block) == rows // block
    assert amr.max_rows(1, 896, 16, 32) == 512                      # decode: exactly 512 rows
    assert amr.max_rows(2 ** 26, 4096, 64, 1) == -1                 # M*k overflows int32
    assert amr.max_rows(1 << 20, 4096, 16, 1 << 20) == -1           # padding overflows
    assert amr.max_rows(1, 0, 1, 1) == -1 and amr.max_rows(1, 8, 1, 0) == -1


def test_workspace_sizes():
    assert amr.workspace_bytes(0, 896, 16, 128) == 0
    a = amr.workspace_bytes(8192, 896, 16, 128)
    b = amr.workspace_bytes(16384, 4096, 16, 128)
    assert a > 0 and b > a
    # linear in the number of workgroup histogram rows: bounded by a few MB
    assert b < 16 << 20
    with pytest.raises(ValueError):
        amr.workspace_bytes(1, 5000, 1, 1)


def call(M=4, E=64, k=4, n_group=8, topk_group=4, block=16, logits=P, bias=P, ids=P, w=P,
         rows=P, eob=P, npp=P, dtype=0, ws=Q, ws_bytes=1 << 30, flags=0, stats=None):
    return amr.raw_call(logits, bias, M, E, k, n_group, topk_group, block, ids, w, rows, eob,
                        npp, dtype, ws, ws_bytes, None, flags, stats)


@pytest.mark.parametrize("kw", [
    dict(M=-1), dict(E=0), dict(E=4097, n_group=1, topk_group=1), dict(n_group=7),
    dict(n_group=0), dict(topk_group=0), dict(topk_group=9), dict(k=0), dict(k=65, E=128),
    dict(k=33, n_group=8, topk_group=4),     # only 4 groups x 8 experts = 32 candidates
    dict(block=0), dict(dtype=2), dict(dtype=-1), dict(flags=8), dict(flags=3),
    dict(M=100, flags=1),                     # single workgroup cannot take 100 tokens
])
def test_invalid_arguments(kw):
    assert call(**kw) == amr.MRS_ERR_INVALID_ARG


def test_overflow():
    assert call(M=2 ** 26, E=4096, k=64, n_group=1, topk_group=1, block=1) == amr.MRS_ERR_OVERFLOW
    assert call(M=1 << 20, E=4096, k=16, n_group=1, topk_group=1, block=1 << 20) == amr.MRS_ERR_OVERFLOW


@pytest.mark.parametrize("name", ["logits", "bias", "ids", "w", "rows", "eob", "npp"])
def test_null_pointers(name):
    assert call(**{name: None}) == amr.MRS_ERR_NULL_POINTER


def test_zero_tokens_needs_only_num_post_pad():
    assert call(M=0, npp=None) == amr.MRS_ERR_NULL_POINTER


@pytest.mark.parametrize("name,off", [("logits", 8), ("logits", 4), ("bias", 2), ("ids", 2),
                                      ("w", 1), ("rows", 2), ("eob", 3), ("npp", 2)])
def test_misaligned(name, off):
    assert call(**{name: P + off}) == amr.MRS_ERR_MISALIGNED


def test_workspace_checks():
    big = dict(M=8192, E=896, k=16, n_group=8, topk_group=4, block=128)
    need = amr.workspace_bytes(8192, 896, 16, 128)
    assert call(**big, ws=None) == amr.MRS_ERR_WORKSPACE
    assert call(**big, ws_bytes=need - 4) == amr.MRS_ERR_WORKSPACE
    assert call(**big, ws=Q + 4) == amr.MRS_ERR_MISALIGNED
    # a small call forced onto the multi-workgroup path needs the workspace too
    assert call(M=4, flags=amr.FLAG_FORCE_MULTI_WG, ws=None) == amr.MRS_ERR_WORKSPACE


def test_sigmoid_probe_validation():
    L = amr.lib()
    assert L.moe_route_sort_sigmoid_probe(P, -1, P, P, None) == amr.MRS_ERR_INVALID_ARG
    assert L.moe_route_sort_sigmoid_probe(P, 0, P, P, None) == amr.MRS_OK
    assert L.moe_route_sort_sigmoid_probe(None, 5, P, P, None) == amr.MRS_ERR_NULL_POINTER
    assert L.moe_route_sort_sigmoid_probe(P + 2, 5, P, P, None) == amr.MRS_ERR_MISALIGNED


def test_profiled_entry_validation():
    """The profiled entry point checks its event array before anything else and
    passes every other check through unchanged (no event is touched on error)."""
    L = amr.lib()
    ev = (ctypes.c_void_p * 6)(P, P, P, P, P, P)
    n = ctypes.c_int(-1)
    args = [P, P, 4, 64, 4, 8, 4, 16, P, P, P, P, P, amr.MRS_DTYPE_F32, None, 0, None, 0, None]
    assert L.moe_route_sort_profiled(*args, None, ctypes.byref(n)) == amr.MRS_ERR_NULL_POINTER
    assert L.moe_route_sort_profiled(*args, ev, None) == amr.MRS_ERR_NULL_POINTER
    holes = (ctypes.c_void_p * 6)(P, P, P, None, P, P)
    assert L.moe_route_sort_profiled(*args, holes, ctypes.byref(n)) == amr.MRS_ERR_NULL_POINTER
    bad = list(args)
    bad[3] = 0  # E = 0
    assert L.moe_route_sort_profiled(*bad, ev, ctypes.byref(n)) == amr.MRS_ERR_INVALID_ARG
    assert n.value == 0


def test_sigmoid_table_probe_validation():
    L = amr.lib()
    assert L.moe_route_sort_sigmoid_table_probe(P, -1, P, P, None) == amr.MRS_ERR_INVALID_ARG
    assert L.moe_route_sort_sigmoid_table_probe(P, 0, P, P, None) == amr.MRS_OK
    assert L.moe_route_sort_sigmoid_table_probe(None, 5, P, P, None) == amr.MRS_ERR_NULL_POINTER
    assert L.moe_route_sort_sigmoid_table_probe(P + 1, 5, P, P, None) == amr.MRS_ERR_MISALIGNED


def ids_call(**kw):
    """moe_sort_from_ids with fake aligned pointers (validation only)."""
    L = amr.lib()
    d = dict(ids=P, M=4, E=64, k=4, block=16, rows=P, eob=P, npp=P, ws=None, ws_bytes=0)
    d.update(kw)
    return L.moe_sort_from_ids(d["ids"], d["M"], d["E"], d["k"], d["block"], d["rows"], d["eob"], d["npp"],
                               d["ws"], d["ws_bytes"], None)


@pytest.mark.parametrize("kw", [dict(M=-1), dict(E=0), dict(E=4097), dict(k=0), dict(k=65), dict(block=0)])
def test_sort_from_ids_invalid_arguments(kw):
    assert ids_call(**kw) == amr.MRS_ERR_INVALID_ARG


def test_sort_from_ids_checks():
    assert ids_call(M=1 << 26, k=64, E=64) == amr.MRS_ERR_OVERFLOW
    for name in ("ids", "rows", "eob", "npp"):
        assert ids_call(**{name: None}) == amr.MRS_ERR_NULL_POINTER
    for name in ("ids", "rows", "eob", "npp"):
        assert ids_call(**{name: P + 2}) == amr.MRS_ERR_MISALIGNED
    need = amr.workspace_bytes(8192, 896, 16, 128)
    assert ids_call(M=8192, E=896, k=16, block=128) == amr.MRS_ERR_WORKSPACE
    assert ids_call(M=8192, E=896, k=16, block=128, ws=Q, ws_bytes=need - 4) == amr.MRS_ERR_WORKSPACE
    assert ids_call(M=8192, E=896, k=16, block=128, ws=Q + 4, ws_bytes=need + 64) == amr.MRS_ERR_MISALIGNED
    assert ids_call(M=0, npp=None) == amr.MRS_ERR_NULL_POINTER


def static_call(M=4, E=64, k=4, n_group=8, topk_group=4, block=16, logits=P, bias=P, ids=P, w=P, rows=P,
                eob=P, npp=P, dtype=0):
    return amr.lib().moe_route_sort_static(logits, bias, M, E, k, n_group, topk_group, block, ids, w, rows, eob,
                                           npp, dtype, None)


def test_static_entry_checks():
    """moe_route_sort_static validates like moe_route_sort and rejects shapes
    whose scratch would exceed its 8 MiB before any launch."""
    assert static_call(M=-1) == amr.MRS_ERR_INVALID_ARG
    assert static_call(n_group=7) == amr.MRS_ERR_INVALID_ARG
    assert static_call(dtype=3) == amr.MRS_ERR_INVALID_ARG
    for name in ("logits", "bias", "ids", "w", "rows", "eob", "npp"):
        assert static_call(**{name: None}) == amr.MRS_ERR_NULL_POINTER
    assert static_call(logits=P + 4) == amr.MRS_ERR_MISALIGNED
    big = dict(M=1 << 18, E=4096, k=16, n_group=16, topk_group=8, block=128)
    assert amr.workspace_bytes(1 << 18, 4096, 16, 128) > 8 << 20
    assert static_call(**big) == amr.MRS_ERR_SCRATCH
    assert "8 MiB" in amr.strerror(amr.MRS_ERR_SCRATCH)
    for M, E, k, blk in [(16384, 4096, 16, 128), (65536, 896, 16, 128), (8192, 896, 16, 128)]:
        assert amr.workspace_bytes(M, E, k, blk) <= 8 << 20


def counters_call(**kw):
    """moe_sort_from_ids_counters with fake aligned pointers (validation only)."""
    L = amr.lib()
    d = dict(ids=P, M=4, E=64, k=4, block=16, cnt=Q, cap=4096, rows=P, eob=P, npp=P, ws=None, ws_bytes=0)
    d.update(kw)
    return L.moe_sort_from_ids_counters(d["ids"], d["M"], d["E"], d["k"], d["block"], d["cnt"], d["cap"],
                                        d["rows"], d["eob"], d["npp"], d["ws"], d["ws_bytes"], None)


@pytest.mark.parametrize("kw", [dict(M=-1), dict(E=0), dict(E=4097), dict(k=0), dict(k=65), dict(block=0),
                                dict(cap=-1), dict(cap=2 ** 31 - 1, block=16), dict(cap=2 ** 40)])
def test_counters_invalid_arguments(kw):
    assert counters_call(**kw) == amr.MRS_ERR_INVALID_ARG


def test_counters_checks():
    assert counters_call(cnt=None) == amr.MRS_ERR_NULL_POINTER
    for name in ("ids", "rows", "eob", "npp"):
        assert counters_call(**{name: None}) == amr.MRS_ERR_NULL_POINTER
    for name in ("ids", "rows", "eob", "npp", "cnt"):
        assert counters_call(**{name: P + 2}) == amr.MRS_ERR_MISALIGNED
    assert counters_call(M=1 << 26, k=64) == amr.MRS_ERR_OVERFLOW
    need = amr.workspace_bytes(8192, 896, 16, 128)
    assert counters_call(M=8192, E=896, k=16, block=128) == amr.MRS_ERR_WORKSPACE
    assert counters_call(M=8192, E=896, k=16, block=128, ws=Q, ws_bytes=need - 4) == amr.MRS_ERR_WORKSPACE
    # the largest legal capacity is accepted by the argument checks (the call
    # then fails on the missing workspace, before any launch)
    assert counters_call(M=8192, E=896, k=16, block=128, cap=2 ** 31 - 128) == amr.MRS_ERR_WORKSPACE


def gemm_call(**kw):
    L = amr.lib()
    d = dict(x=P, w=P, sid=Q, eob=Q, npp=Q, M=64, k=8, E=64, K=256, N=256, block=64, y=P)
    d.update(kw)
    return L.moe_grouped_gemm1(d["x"], d["w"], d["sid"], d["eob"], d["npp"], d["M"], d["k"], d["E"], d["K"],
                               d["N"], d["block"], d["y"], None)


@pytest.mark.parametrize("kw", [dict(M=-1), dict(k=0), dict(k=65), dict(E=0), dict(E=4097), dict(K=0),
                                dict(K=96), dict(N=0), dict(N=192), dict(block=16), dict(block=48)])
def test_grouped_gemm1_invalid_arguments(kw):
    assert gemm_call(**kw) == amr.MRS_ERR_INVALID_ARG


def test_grouped_gemm1_checks():
    for name in ("x", "w", "sid", "eob", "npp", "y"):
        assert gemm_call(**{name: None}) == amr.MRS_ERR_NULL_POINTER
    for name in ("x", "w", "y"):
        assert gemm_call(**{name: P + 8}) == amr.MRS_ERR_MISALIGNED
    assert gemm_call(M=1 << 26, k=64) == amr.MRS_ERR_OVERFLOW
    assert gemm_call(M=0) == amr.MRS_OK  # no row can exist: returns before any launch
    L = amr.lib()
    assert L.moe_grouped_gemm1_profiled(P, P, Q, Q, Q, 64, 8, 64, 256, 256, 64, P, None, None, None) == \
        amr.MRS_ERR_NULL_POINTER


def local_call(**kw):
    L = amr.lib()
    d = dict(logits=P, bias=P, M=64, E=64, k=4, ng=8, tg=4, block=16, lb=0, lc=64, ids=Q, w=Q, rows=Q, eob=Q,
             npp=Q, dtype=amr.MRS_DTYPE_F32, ws=Q, ws_bytes=1 << 20)
    d.update(kw)
    return L.moe_route_sort_local(d["logits"], d["bias"], d["M"], d["E"], d["k"], d["ng"], d["tg"], d["block"],
                                  d["lb"], d["lc"], d["ids"], d["w"], d["rows"], d["eob"], d["npp"], d["dtype"],
                                  d["ws"], d["ws_bytes"], None)


@pytest.mark.parametrize("kw", [dict(lb=-1), dict(lc=0), dict(lb=60, lc=5), dict(lb=64, lc=1), dict(lc=65),
                                dict(E=0), dict(k=0)])
def test_local_invalid_ranges(kw):
    assert local_call(**kw) == amr.MRS_ERR_INVALID_ARG


def test_local_checks():
    assert local_call(npp=None) == amr.MRS_ERR_NULL_POINTER
    assert local_call(logits=None) == amr.MRS_ERR_NULL_POINTER
    assert local_call(logits=P + 4) == amr.MRS_ERR_MISALIGNED


def gate_call(**kw):
    L = amr.lib()
    d = dict(h=P, w=P, bias=Q, M=1, E=896, H=7168, k=16, ng=8, tg=4, block=32, logits=P, ids=Q, wt=Q, rows=Q,
             eob=Q, npp=Q)
    d.update(kw)
    return L.moe_gate_route_sort(d["h"], d["w"], d["bias"], d["M"], d["E"], d["H"], d["k"], d["ng"], d["tg"],
                                 d["block"], d["logits"], d["ids"], d["wt"], d["rows"], d["eob"], d["npp"], None)


@pytest.mark.parametrize("kw", [dict(M=-1), dict(M=65), dict(H=0), dict(H=12), dict(E=0), dict(E=900),
                                dict(k=0), dict(tg=9), dict(block=0)])
def test_gate_invalid_arguments(kw):
    assert gate_call(**kw) == amr.MRS_ERR_INVALID_ARG


def test_gate_checks():
    for name in ("h", "w", "bias", "logits", "ids", "wt", "rows", "eob", "npp"):
        assert gate_call(**{name: None}) == amr.MRS_ERR_NULL_POINTER, name
    for name in ("h", "w", "logits"):
        assert gate_call(**{name: P + 8}) == amr.MRS_ERR_MISALIGNED, name


def test_default_workspace_per_stream(monkeypatch):
    """The binding's default workspace: one per stream (calls on different
    streams may overlap), shared by the calls of a stream whatever their
    shape, grown in powers of two with outgrown buffers kept alive (a captured
    graph may still point at them)."""
    monkeypatch.setattr(amr, "_ws_cache", {})
    a = amr._workspace("cpu", 0, 1000)
    assert a.numel() == 1024 and int(a.sum()) == 0
    assert amr._workspace("cpu", 0, 700).data_ptr() == a.data_ptr()  # a smaller shape reuses it
    b = amr._workspace("cpu", 12345, 1000)  # another stream: a buffer of its own
    assert b.data_ptr() != a.data_ptr()
    c = amr._workspace("cpu", 0, 5000)  # outgrown: a larger buffer, the old one kept
    assert c.numel() == 8192 and c.data_ptr() != a.data_ptr()
    bufs = amr._ws_cache[("cpu", 0)]
    assert [t.data_ptr() for t in bufs] == [a.data_ptr(), c.data_ptr()]
    assert amr._workspace("cpu", 0, 1000).data_ptr() == c.data_ptr()
    for n in range(1, 40000, 997):
        amr._workspace("cpu", 7, n)
    sizes = [t.numel() for t in amr._ws_cache[("cpu", 7)]]
    assert sum(sizes) < 2 * sizes[-1] and all(s & (s - 1) == 0 for s in sizes)


def test_binding_rejects_buffers_before_any_call():
    """The binding's tensor checks (run before any library call): a buffer on
    another device, of another dtype, too small or not contiguous is refused,
    so no host address or short buffer reaches a kernel."""
    torch = pytest.importorskip("torch")
    dev = torch.device("cpu")
    M, k, rows, blocks = 3, 2, 40, 5
    good = amr.RouteSortOutput(torch.zeros((M, k), dtype=torch.int32), torch.zeros((M, k)),
                               torch.zeros(rows, dtype=torch.int32), torch.zeros(blocks, dtype=torch.int32),
                               torch.zeros(1, dtype=torch.int32))
    amr._check_route_output(good, M, k, rows, blocks, dev)
    bad = [
        good._replace(sorted_ids=torch.zeros(rows, dtype=torch.int32, device="meta")),  # another device
        good._replace(expert_of_block=torch.zeros(blocks - 1, dtype=torch.int32)),     # too small
        good._replace(num_post_pad=torch.zeros(1, dtype=torch.int64)),                 # wrong dtype
        good._replace(sorted_ids=torch.zeros(2 * rows, dtype=torch.int32)[::2]),       # strided view
        good._replace(ids=torch.zeros((k, M), dtype=torch.int32)),                     # wrong shape
        good._replace(weights=torch.zeros((M, k), dtype=torch.float64)),              # wrong dtype
        good._replace(ids=torch.zeros((M, k), dtype=torch.int32, device="meta")),      # another device
    ]
    for out in bad:
        with pytest.raises(ValueError):
            amr._check_route_output(out, M, k, rows, blocks, dev)
    with pytest.raises(ValueError):
        amr._check_tensor(torch.zeros(4, device="meta"), dev, None, 0, "workspace")
    with pytest.raises(ValueError):
        amr._check_tensor(torch.zeros(1, dtype=torch.int32), dev, torch.int32, 2, "stats")
    amr._check_tensor(torch.zeros(2, dtype=torch.int32), dev, torch.int32, 2, "stats")
