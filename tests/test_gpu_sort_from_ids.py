"""GPU parity of the sort-only entry point (moe_sort_from_ids) against the
oracle's sort metadata: exact counts, stable rows, padding, expert per block,
dropped routes (ids outside [0, E)), rows that repeat an expert, and agreement
with the full route-sort call on its own ids."""
import numpy as np
import pytest

import workloads
from oracle import route_sort as orc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
amr = pytest.importorskip("align_moe_route_amd")


def distinct_rows(rng, M, E, k, skew=0.0):
    """k distinct experts per row; with skew > 0 popular experts are likelier."""
    p = None
    if skew > 0:
        w = 1.0 / np.arange(1, E + 1) ** skew
        p = w[rng.permutation(E)] / w.sum()
    return np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(M)]).astype(np.int32)


def run_and_check(ids, E, block):
    M, k = ids.shape
    print(f"[gpu] sort_from_ids M={M} E={E} k={k} block={block} dropped={int(((ids < 0) | (ids >= E)).sum())}",
          flush=True)
    out = amr.sort_from_ids(torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda(), E, block)
    torch.cuda.synchronize()
    npp = int(out.num_post_pad.item())
    rows = out.sorted_ids[:npp].cpu().numpy()
    eob = out.expert_of_block[:npp // block].cpu().numpy()
    ref = orc.sort_metadata(ids, E, block)
    assert npp == ref.num_post_pad
    assert np.array_equal(rows, ref.sorted_ids)
    assert np.array_equal(eob, ref.expert_of_block)
    assert orc.check_sort_invariants(ids, rows, eob, npp, E, block) == []
    return out


@pytest.mark.parametrize("M,E,k,block,skew", [
    (1, 896, 16, 32, 0.0), (4, 64, 4, 16, 0.0), (64, 896, 16, 128, 1.1), (65, 128, 8, 7, 0.0),
    (300, 4096, 16, 128, 0.5), (1000, 129, 5, 1, 0.0), (2517, 896, 16, 128, 1.1),
    (8192, 896, 16, 128, 1.1), (5000, 1, 1, 3, 0.0)])
def test_distinct_ids(M, E, k, block, skew):
    rng = np.random.default_rng(M + E)
    run_and_check(distinct_rows(rng, M, E, k, skew), E, block)


@pytest.mark.parametrize("M,E,k,block", [(3, 64, 8, 16), (64, 896, 16, 32), (700, 896, 16, 64),
                                         (9000, 512, 8, 128)])
def test_dropped_ids(M, E, k, block):
    rng = np.random.default_rng(7 * M + E)
    ids = distinct_rows(rng, M, E, k)
    mask = rng.random(ids.shape) < 0.2
    ids[mask] = rng.choice(np.array([-1, -7, E, E + 100, 2 ** 31 - 1, -2 ** 31]), size=int(mask.sum()))
    run_and_check(ids, E, block)


@pytest.mark.parametrize("M", [5, 600])
def test_all_dropped(M):
    ids = np.full((M, 4), -1, dtype=np.int32)
    out = run_and_check(ids, 32, 8)
    assert int(out.num_post_pad.item()) == 0


@pytest.mark.parametrize("M,E,k,block", [(10, 16, 6, 4), (200, 24, 8, 16)])
def test_rows_repeating_an_expert(M, E, k, block):
    """Each slot takes its own row even when a row names an expert twice."""
    rng = np.random.default_rng(M * k)
    ids = rng.integers(0, E, size=(M, k)).astype(np.int32)
    ids[:, 1] = ids[:, 0]
    run_and_check(ids, E, block)


# Drawn once by a seeded generator and kept as a fixed list:
# M, E, k, block, share of dropped ids, rows may repeat an expert, Zipf skew.
RANDOM_IDS = [
    (11, 1, 1, 128, 0.5, False, 0.8),
    (2795, 4096, 21, 2, 0.0, False, 1.3),
    (396, 100, 47, 128, 0.5, False, 0.0),
    (16105, 1000, 24, 2, 0.05, False, 0.0),
    (28, 3, 1, 2, 0.0, False, 0.8),
    (6, 64, 25, 32, 0.5, True, 0.0),
    (1, 100, 5, 300, 0.0, False, 1.3),
    (7, 3, 45, 128, 0.0, True, 0.0),
    (79, 1000, 28, 128, 0.5, True, 0.0),
    (518, 896, 52, 2, 0.0, False, 0.0),
    (1980, 896, 30, 1, 0.0, True, 0.0),
    (107, 64, 29, 2, 0.5, True, 0.0),
    (9156, 4096, 50, 2, 0.0, False, 0.0),
    (4, 64, 33, 128, 0.5, True, 0.0),
    (1714, 512, 63, 5, 0.05, False, 0.0),
    (71, 896, 3, 300, 0.5, False, 0.8),
    (874, 4096, 53, 128, 0.0, False, 1.3),
    (2388, 1000, 20, 128, 0.5, False, 1.3),
    (6141, 1, 50, 5, 0.05, True, 0.0),
    (101, 257, 4, 32, 0.5, False, 0.8),
    (4178, 64, 35, 2, 0.5, False, 1.3),
    (19, 1000, 42, 5, 0.5, True, 0.0),
    (72, 3, 3, 128, 0.0, False, 0.0),
    (43, 1000, 25, 128, 0.0, True, 0.0),
    (1, 2048, 64, 5, 0.0, False, 0.8),
    (17752, 128, 2, 1, 0.05, True, 0.0),
    (221, 1, 1, 16, 0.5, False, 0.8),
    (2, 896, 12, 1, 0.05, True, 0.0),
    (41, 896, 50, 2, 0.0, True, 0.0),
    (1097, 1, 1, 5, 0.05, False, 0.8),
    (2730, 1000, 8, 2, 0.0, False, 1.3),
    (2434, 896, 34, 300, 0.0, True, 0.0),
]


@pytest.mark.parametrize("case", RANDOM_IDS, ids=lambda c: "M{}_E{}_k{}_b{}_drop{}_rep{}_skew{}".format(*c))
def test_random_ids(case):
    M, E, k, block, drop, repeat, skew = case
    rng = np.random.default_rng(M * 31 + E * 7 + k)
    ids = rng.integers(0, E, size=(M, k)).astype(np.int32) if repeat else distinct_rows(rng, M, E, k, skew)
    if drop > 0:
        mask = rng.random(ids.shape) < drop
        ids[mask] = rng.choice(np.array([-1, E, -2 ** 31, 2 ** 31 - 1]), size=int(mask.sum()))
    run_and_check(ids, E, block)

def test_matches_full_route_sort():
    cfg = workloads.custom(3000, 896, 16, 8, 4, 128, "bf16", "log_zipf", seed=12)
    inp = workloads.make_inputs(cfg)
    x = torch.from_numpy(inp.logits_storage.view(np.int16)).view(torch.bfloat16).cuda()
    b = torch.from_numpy(inp.bias).cuda()
    full = amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block)
    srt = amr.sort_from_ids(full.ids, cfg.E, cfg.block)
    torch.cuda.synchronize()
    npp = int(full.num_post_pad.item())
    assert int(srt.num_post_pad.item()) == npp
    assert torch.equal(srt.sorted_ids[:npp], full.sorted_ids[:npp])
    assert torch.equal(srt.expert_of_block[:npp // cfg.block], full.expert_of_block[:npp // cfg.block])


def test_poisoned_tails_untouched():
    rng = np.random.default_rng(5)
    M, E, k, block = 500, 896, 16, 64
    ids = distinct_rows(rng, M, E, k, 1.1)
    rows, blocks = amr.max_rows(M, E, k, block), amr.max_blocks(M, E, k, block)
    poison = -99
    out = amr.SortOutput(torch.full((rows + 32,), poison, dtype=torch.int32, device="cuda"),
                         torch.full((blocks + 32,), poison, dtype=torch.int32, device="cuda"),
                         torch.full((1,), poison, dtype=torch.int32, device="cuda"))
    g = torch.from_numpy(ids).cuda()
    g0 = g.clone()
    amr.sort_from_ids(g, E, block, out=out)
    torch.cuda.synchronize()
    npp = int(out.num_post_pad.item())
    ref = orc.sort_metadata(ids, E, block)
    assert npp == ref.num_post_pad
    assert np.array_equal(out.sorted_ids[:npp].cpu().numpy(), ref.sorted_ids)
    assert torch.all(out.sorted_ids[npp:] == poison)
    assert torch.all(out.expert_of_block[npp // block:] == poison)
    assert torch.equal(g, g0)


# ---------------------------------------------------------------------------
# Caller-provided initial counters (moe_sort_from_ids_counters).
# ---------------------------------------------------------------------------
POISON = -123456789


def _run_counters(ids, E, block, c0, cap=None, out=None):
    M, k = ids.shape
    need = int(((c0 + np.bincount(ids[(ids >= 0) & (ids < E)].reshape(-1), minlength=E) + block - 1)
                // block * block).sum())
    cap = need + 3 * block if cap is None else cap
    print(f"[gpu] sort_from_ids counters M={M} E={E} k={k} block={block} sum(c0)={int(c0.sum())} cap={cap}",
          flush=True)
    if out is None:
        out = amr.SortOutput(torch.full((max(cap, 1),), POISON, dtype=torch.int32, device="cuda"),
                             torch.full((max(cap // block, 1),), POISON, dtype=torch.int32, device="cuda"),
                             torch.full((1,), POISON, dtype=torch.int32, device="cuda"))
    cnt = torch.from_numpy(np.asarray(c0, dtype=np.int32)).cuda()
    ids_d = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    amr.sort_from_ids(ids_d, E, block, out=out, counters=cnt, rows_capacity=cap)
    torch.cuda.synchronize()
    return out, cnt, need, cap


def _check_counters(ids, E, block, c0, out, cnt, cap):
    ref = orc.sort_metadata_counters(ids, E, block, c0)
    npp = int(out.num_post_pad.item())
    rows = out.sorted_ids.cpu().numpy()
    eob = out.expert_of_block.cpu().numpy()
    assert npp == ref.meta.num_post_pad
    w = ref.written
    assert np.array_equal(rows[:npp][w], ref.meta.sorted_ids[w])
    assert np.all(rows[:npp][~w] == POISON)          # the caller's rows are untouched
    assert np.all(rows[npp:] == POISON)              # nothing past num_post_pad
    assert np.array_equal(eob[:npp // block], ref.meta.expert_of_block)
    assert np.all(eob[npp // block:] == POISON)
    assert np.array_equal(cnt.cpu().numpy(), ref.counters_out)


@pytest.mark.parametrize("M,E,k,block,maxc", [
    (1, 896, 16, 32, 40), (4, 64, 4, 16, 5), (64, 896, 16, 128, 300), (65, 128, 8, 7, 20),
    (150, 896, 16, 64, 200), (700, 896, 16, 64, 1), (5000, 896, 16, 128, 500), (9000, 512, 8, 128, 3),
    (3000, 4096, 16, 128, 50), (2000, 1, 1, 3, 10)])
def test_counters_nonzero_initial(M, E, k, block, maxc):
    rng = np.random.default_rng(M * 3 + E)
    ids = distinct_rows(rng, M, E, k, 0.8)
    ids[rng.random(ids.shape) < 0.1] = -1
    c0 = rng.integers(0, maxc + 1, E) * (rng.random(E) < 0.7)
    out, cnt, _, cap = _run_counters(ids, E, block, c0)
    _check_counters(ids, E, block, c0, out, cnt, cap)


@pytest.mark.parametrize("M,E,k,block", [(8, 64, 4, 16), (500, 896, 16, 128), (0, 896, 16, 32)])
def test_counters_all_dropped_and_empty(M, E, k, block):
    rng = np.random.default_rng(M + 5)
    ids = np.full((M, k), -1, np.int32)
    c0 = rng.integers(0, 50, E)
    out, cnt, _, cap = _run_counters(ids, E, block, c0)
    _check_counters(ids, E, block, c0, out, cnt, cap)


@pytest.mark.parametrize("M", [10, 100, 5000])
def test_counters_fail_closed(M):
    """A negative counter, or rows past the capacity: num_post_pad = -1 and
    nothing else written (counters included)."""
    E, k, block = 896, 16, 64
    rng = np.random.default_rng(M)
    ids = distinct_rows(rng, M, E, k)
    c0 = rng.integers(0, 30, E)
    for case in ("negative", "capacity"):
        c = c0.copy()
        if case == "negative":
            c[E // 2] = -1
            cap = None
        else:
            cap = int(((c + np.bincount(ids.reshape(-1), minlength=E) + block - 1) // block * block).sum()) - 1
        out, cnt, _, cap = _run_counters(ids, E, block, c, cap=cap)
        assert int(out.num_post_pad.item()) == -1, case
        assert np.all(out.sorted_ids.cpu().numpy() == POISON), case
        assert np.all(out.expert_of_block.cpu().numpy() == POISON), case
        assert np.array_equal(cnt.cpu().numpy(), c), case


@pytest.mark.parametrize("M", [40, 3000])
def test_counters_graph_replay_with_changed_inputs(M):
    """Eight replays of a captured call, each with new ids and new counters
    written into the captured buffers; every replay checked."""
    E, k, block = 896, 16, 64
    rng = np.random.default_rng(M + 11)
    cap = M * k + E * (block - 1) + E * 64 + block
    out = amr.SortOutput(torch.full((cap,), POISON, dtype=torch.int32, device="cuda"),
                         torch.full((cap // block,), POISON, dtype=torch.int32, device="cuda"),
                         torch.full((1,), POISON, dtype=torch.int32, device="cuda"))
    ids_d = torch.zeros((M, k), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((E,), dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):  # the stream's workspace, allocated outside the capture
        amr.sort_from_ids(ids_d, E, block, out=out, counters=cnt, rows_capacity=cap, stream=stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        amr.sort_from_ids(ids_d, E, block, out=out, counters=cnt, rows_capacity=cap, stream=stream)
    torch.cuda.synchronize()
    print(f"[gpu] graph replay M={M} E={E} x8", flush=True)
    for rep in range(8):
        ids = distinct_rows(rng, M, E, k, 0.5 * (rep % 3))
        ids[rng.random(ids.shape) < 0.05 * (rep % 2)] = -1
        c0 = rng.integers(0, 64, E)
        out.sorted_ids.fill_(POISON)
        out.expert_of_block.fill_(POISON)
        ids_d.copy_(torch.from_numpy(ids))
        cnt.copy_(torch.from_numpy(c0.astype(np.int32)))
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        _check_counters(ids, E, block, c0, out, cnt, cap)
