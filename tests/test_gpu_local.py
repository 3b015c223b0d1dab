"""GPU parity of the expert-parallel local entry (moe_route_sort_local): the
selection equals the full call's, and the metadata equals the oracle's local
metadata (oracle.route_sort.local_metadata) bit for bit, for every rank of an
even split and for ranges that are not aligned to anything."""
import numpy as np
import pytest

import workloads
from oracle import route_sort as orc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
amr = pytest.importorskip("align_moe_route_amd")


def to_gpu(inp):
    if inp.cfg.dtype == "bf16":
        x = torch.from_numpy(inp.logits_storage.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        x = torch.from_numpy(inp.logits_storage).cuda()
    return x, torch.from_numpy(inp.bias).cuda()


def check_rank(cfg, x, b, ref_ids, ids_full, w_full, lb, lc):
    print(f"[gpu] local {cfg.name} M={cfg.M} E={cfg.E} range=[{lb}, {lb + lc})", flush=True)
    out = amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block, local=(lb, lc))
    torch.cuda.synchronize()
    assert torch.equal(out.ids, ids_full) and torch.equal(out.weights, w_full)
    m = orc.local_metadata(ref_ids, lb, lc, cfg.block)
    npp = int(out.num_post_pad.item())
    assert npp == m.num_post_pad
    assert np.array_equal(out.sorted_ids[:npp].cpu().numpy(), m.sorted_ids)
    assert np.array_equal(out.expert_of_block[:npp // cfg.block].cpu().numpy(), m.expert_of_block)


CASES = [
    (workloads.CONFIGS["tiny"], 2),
    (workloads.CONFIGS["decode"], 8),
    (workloads.CONFIGS["threshold"], 4),
    (workloads.CONFIGS["prefill_skew"], 8),
    (workloads.custom(1000, 4096, 16, 16, 8, 128, "f32", "normal", 0.2, seed=4, name="wide_1000"), 16),
]


@pytest.mark.parametrize("cfg,ranks", CASES, ids=[c.name for c, _ in CASES])
def test_every_rank_of_an_even_split(cfg, ranks):
    inp = workloads.make_inputs(cfg)
    ref = orc.route_sort(inp.logits_storage, cfg.dtype, inp.bias, cfg.k, cfg.n_group, cfg.topk_group, cfg.block)
    x, b = to_gpu(inp)
    full = amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block)
    torch.cuda.synchronize()
    assert np.array_equal(full.ids.cpu().numpy(), ref.ids)
    EL = cfg.E // ranks
    for r in range(ranks):
        check_rank(cfg, x, b, ref.ids, full.ids, full.weights, r * EL, EL)


def test_unaligned_ranges_and_the_full_range():
    cfg = workloads.custom(700, 896, 16, 8, 4, 64, "bf16", "log_zipf", seed=2, name="skew_700")
    inp = workloads.make_inputs(cfg)
    ref = orc.route_sort(inp.logits_storage, cfg.dtype, inp.bias, cfg.k, cfg.n_group, cfg.topk_group, cfg.block)
    x, b = to_gpu(inp)
    full = amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block)
    torch.cuda.synchronize()
    for lb, lc in [(0, 896), (100, 37), (0, 1), (895, 1), (333, 500)]:
        check_rank(cfg, x, b, ref.ids, full.ids, full.weights, lb, lc)
    # the full range reproduces the global metadata
    whole = amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block, local=(0, cfg.E))
    torch.cuda.synchronize()
    npp = int(full.num_post_pad.item())
    assert int(whole.num_post_pad.item()) == npp
    assert torch.equal(whole.sorted_ids[:npp], full.sorted_ids[:npp])
    assert torch.equal(whole.expert_of_block[:npp // cfg.block], full.expert_of_block[:npp // cfg.block])


def test_rank_with_no_routes_and_untouched_tails():
    # a rank whose experts no token picks: num_post_pad = 0, nothing else written
    cfg = workloads.CONFIGS["decode"]
    inp = workloads.make_inputs(cfg)
    ref = orc.route_sort(inp.logits_storage, cfg.dtype, inp.bias, cfg.k, cfg.n_group, cfg.topk_group, cfg.block)
    x, b = to_gpu(inp)
    unused = np.setdiff1d(np.arange(cfg.E), ref.ids.reshape(-1))
    lb = int(unused[0])
    lc = 1
    rows = amr.max_rows(cfg.M, lc, cfg.k, cfg.block)
    blocks = amr.max_blocks(cfg.M, lc, cfg.k, cfg.block)
    out = amr.RouteSortOutput(torch.empty((cfg.M, cfg.k), dtype=torch.int32, device="cuda"),
                              torch.empty((cfg.M, cfg.k), dtype=torch.float32, device="cuda"),
                              torch.full((rows,), -77, dtype=torch.int32, device="cuda"),
                              torch.full((blocks,), -77, dtype=torch.int32, device="cuda"),
                              torch.full((1,), -77, dtype=torch.int32, device="cuda"))
    amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block, local=(lb, lc), out=out)
    torch.cuda.synchronize()
    assert int(out.num_post_pad.item()) == 0
    assert bool((out.sorted_ids == -77).all()) and bool((out.expert_of_block == -77).all())
