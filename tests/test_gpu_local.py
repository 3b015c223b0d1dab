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


# Drawn once by a seeded generator over the wave layouts and kept as a fixed
# list: M, E, k, n_group, topk_group, block, dtype, distribution, then two
# expert ranges (begin, count), the second one ending at E.
RANDOM_LOCAL = [
    (5, 896, 7, 32, 22, 4, "bf16", "shared", 19, 859, 217, 679),
    (10, 64, 20, 1, 1, 200, "bf16", "coarse", 4, 37, 31, 33),
    (298, 64, 31, 8, 5, 64, "bf16", "normal", 3, 61, 2, 62),
    (1252, 2240, 59, 64, 29, 128, "f32", "hot", 270, 1378, 967, 1273),
    (8, 1280, 23, 16, 6, 200, "bf16", "equal", 128, 832, 49, 1231),
    (872, 128, 62, 4, 3, 16, "f32", "dominant_group", 20, 71, 68, 60),
    (14527, 64, 19, 1, 1, 7, "bf16", "log_zipf", 35, 7, 42, 22),
    (1227, 512, 39, 16, 3, 7, "f32", "coarse", 10, 477, 386, 126),
    (142, 768, 12, 1, 1, 4, "bf16", "hot", 94, 463, 504, 264),
    (5700, 896, 37, 4, 4, 16, "bf16", "coarse", 375, 351, 653, 243),
    (1, 3072, 24, 2, 2, 1, "bf16", "normal", 100, 2787, 693, 2379),
    (3267, 896, 44, 16, 1, 1, "f32", "offset_normal", 40, 839, 557, 339),
    (1163, 64, 4, 8, 2, 7, "f32", "dominant_group", 17, 43, 15, 49),
    (244, 64, 28, 8, 4, 64, "bf16", "normal", 5, 3, 44, 20),
    (9, 4096, 42, 64, 20, 4, "bf16", "equal", 1856, 1455, 3724, 372),
    (122, 1792, 48, 8, 2, 7, "f32", "duplicated", 781, 811, 197, 1595),
]


@pytest.mark.parametrize("case", RANDOM_LOCAL, ids=lambda c: "M{}_E{}_k{}_g{}-{}_b{}_{}_{}_r{}+{}_r{}+{}".format(*c))
def test_random_shapes_and_ranges(case):
    M, E, k, ng, tg, block, dtype, dist, lb1, lc1, lb2, lc2 = case
    cfg = workloads.custom(M, E, k, ng, tg, block, dtype, dist, seed=M * 5 + E, name="random")
    inp = workloads.make_inputs(cfg)
    ref = orc.route_sort(inp.logits_storage, cfg.dtype, inp.bias, cfg.k, cfg.n_group, cfg.topk_group, cfg.block)
    x, b = to_gpu(inp)
    full = amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block)
    torch.cuda.synchronize()
    assert np.array_equal(full.ids.cpu().numpy(), ref.ids)
    for lb, lc in ((lb1, lc1), (lb2, lc2)):
        check_rank(cfg, x, b, ref.ids, full.ids, full.weights, lb, lc)
