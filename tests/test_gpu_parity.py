"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Expert ids and all sort metadata must be bit-exact;
weights within 1e-6 relative of the oracle's float64 weights.  Tokens whose
k-th/(k+1)-th (or group-boundary) gap is below 1e-6 are counted and printed
separately -- they are still required to match exactly."""
import numpy as np
import pytest

import workloads
from oracle import route_sort as orc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
amr = pytest.importorskip("align_moe_route_amd")

W_RTOL = 1e-6


def to_gpu(inp):
    if inp.cfg.dtype == "bf16":
        x = torch.from_numpy(inp.logits_storage.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        x = torch.from_numpy(inp.logits_storage).cuda()
    return x, torch.from_numpy(inp.bias).cuda()


def fetch(out, block):
    torch.cuda.synchronize()
    npp = int(out.num_post_pad.item())
    return dict(ids=out.ids.cpu().numpy(), w=out.weights.cpu().numpy(), npp=npp,
                rows=out.sorted_ids[:npp].cpu().numpy(),
                eob=out.expert_of_block[:npp // block].cpu().numpy())


def run(inp, flags=0, stats=None):
    cfg = inp.cfg
    x, b = to_gpu(inp)
    print(f"[gpu] {cfg.name} M={cfg.M} E={cfg.E} k={cfg.k} g={cfg.n_group}/{cfg.topk_group} "
          f"block={cfg.block} {cfg.dtype} {cfg.dist} flags={flags}", flush=True)
    out = amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block, flags=flags, stats=stats)
    return fetch(out, cfg.block)


def assert_metadata_matches_ids(g, cfg):
    """The oracle's sort stage run on the GPU's own ids equals the GPU metadata
    bit for bit, with no exemption."""
    meta = orc.sort_metadata(g["ids"], cfg.E, cfg.block)
    assert g["npp"] == meta.num_post_pad
    assert np.array_equal(g["rows"], meta.sorted_ids)
    assert np.array_equal(g["eob"], meta.expert_of_block)


def assert_parity(inp, g, tokens=None):
    cfg = inp.cfg
    ref = orc.route_sort(inp.logits_storage, cfg.dtype, inp.bias, cfg.k, cfg.n_group,
                         cfg.topk_group, cfg.block, tokens=tokens)
    gi = g["ids"] if tokens is None else g["ids"][tokens]
    gw = g["w"] if tokens is None else g["w"][tokens]
    near = (ref.gap_k < 1e-6) | (ref.gap_g < 1e-6)
    if near.any():
        print(f"  near-tie tokens (gap < 1e-6): {int(near.sum())} of {near.size}", flush=True)
    bad = np.flatnonzero(np.any(gi != ref.ids, axis=1))
    assert bad.size == 0, f"{bad.size} tokens differ, first {bad[:5]} near-tie={near[bad[:5]]}"
    err = np.abs(gw.astype(np.float64) - ref.weights) / np.abs(ref.weights)
    assert err.max() <= W_RTOL, err.max()
    if tokens is None:
        assert g["npp"] == ref.meta.num_post_pad
        assert np.array_equal(g["rows"], ref.meta.sorted_ids)
        assert np.array_equal(g["eob"], ref.meta.expert_of_block)
    assert_metadata_matches_ids(g, cfg)
    assert orc.check_sort_invariants(g["ids"], g["rows"], g["eob"], g["npp"], cfg.E, cfg.block) == []
    return ref


# ---------------------------------------------------------------------------
# The five workloads at full size.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_workload_parity(name):
    cfg = workloads.CONFIGS[name]
    inp = workloads.make_inputs(cfg)
    stats = torch.zeros(3, dtype=torch.int32, device="cuda")
    g = run(inp, stats=stats)
    st = stats.cpu().numpy()
    print(f"  exact-path tokens {st[0]}, fast-path tokens {st[1]}, exact group scores {st[2]}", flush=True)
    assert st[0] + st[1] == cfg.M
    assert_parity(inp, g)


@pytest.mark.parametrize("name", ["tiny", "decode", "threshold", "prefill_skew"])
def test_exact_path_parity(name):
    """Every token through the workgroup-wide exact selection."""
    cfg = workloads.CONFIGS[name]
    inp = workloads.make_inputs(cfg)
    g = run(inp, flags=amr.FLAG_FORCE_EXACT)
    assert_parity(inp, g)


@pytest.mark.parametrize("name,flags", [("tiny", 2), ("decode", 2), ("tiny", 1), ("decode", 1),
                                        ("decode", 6), ("tiny", 5)])
def test_forced_paths(name, flags):
    cfg = workloads.CONFIGS[name]
    inp = workloads.make_inputs(cfg)
    assert_parity(inp, run(inp, flags=flags))


# ---------------------------------------------------------------------------
# Sweeps over shapes, group layouts, block sizes and distributions.
# ---------------------------------------------------------------------------
SWEEP = [
    # M, E, k, n_group, topk_group, block, dtype, dist
    (1, 64, 4, 8, 4, 16, "f32", "normal"),
    (3, 64, 8, 64, 10, 1, "bf16", "normal"),         # group of one expert
    (65, 128, 8, 2, 1, 32, "f32", "hot"),             # just past the single-workgroup bound
    (63, 256, 16, 4, 2, 48, "bf16", "shared"),
    (130, 512, 16, 8, 3, 64, "bf16", "dominant_group"),
    (257, 896, 16, 8, 4, 128, "bf16", "log_zipf"),
    (300, 896, 16, 1, 1, 16, "f32", "coarse"),        # many exact ties
    (200, 896, 16, 8, 4, 32, "f32", "duplicated"),    # pairs of identical keys
    (64, 896, 16, 8, 4, 32, "f32", "equal"),          # all keys equal
    (100, 1024, 32, 16, 8, 64, "f32", "normal"),
    (50, 2048, 64, 32, 16, 16, "bf16", "normal"),
    (70, 4096, 16, 16, 8, 128, "f32", "normal"),
    (33, 4096, 8, 64, 2, 8, "bf16", "normal"),
    # shapes outside the wave layout: every token takes the exact selection
    (40, 100, 5, 5, 2, 7, "f32", "normal"),
    (20, 129, 5, 1, 1, 16, "bf16", "shared"),
    (17, 3000, 12, 12, 5, 20, "f32", "normal"),
    (9, 4095, 3, 3, 1, 3, "bf16", "hot"),
    (90, 768, 6, 96, 10, 24, "f32", "normal"),       # 96 groups of 8
    (12, 17, 1, 1, 1, 1, "f32", "normal"),
    (70, 4032, 8, 63, 30, 16, "f32", "normal"),        # staged rows too large for LDS
    (70, 2240, 16, 8, 4, 64, "bf16", "normal"),        # 35 experts per lane, staged
    # two tokens per wave (32-lane segments)
    (40, 896, 16, 8, 4, 32, "bf16", "normal"),         # one workgroup, staged rows, two buffers
    (4500, 128, 8, 4, 2, 8, "f32", "shared"),
    (5000, 896, 16, 8, 4, 128, "f32", "normal"),
    (6000, 512, 8, 16, 4, 32, "bf16", "hot"),
    (8300, 896, 16, 8, 4, 128, "bf16", "log_zipf"),   # staged rows, two buffers
    (9000, 1024, 8, 32, 8, 64, "bf16", "normal"),     # one lane per group
    (20000, 64, 4, 2, 1, 16, "f32", "normal"),        # three rounds per wave
    # FP32 vector loads, one token per wave: lanes interleave their 16-byte vectors
    (300, 1024, 16, 1, 1, 16, "f32", "normal"),       # the whole wave interleaved (no group stage)
    (500, 2048, 8, 4, 4, 32, "f32", "hot"),           # every group kept: the whole wave interleaved
    (150, 512, 8, 8, 3, 16, "f32", "shared"),         # the 8 lanes of each group interleaved
    (200, 1024, 16, 1, 1, 8, "f32", "coarse"),        # interleaved, many exact ties
    (16, 1024, 16, 1, 1, 32, "f32", "duplicated"),    # one workgroup, interleaved, pairs of equal keys
    (120, 1280, 16, 4, 2, 64, "f32", "normal"),       # 20 experts per lane (5 vectors), 16-lane blocks
    (90, 768, 8, 8, 3, 16, "f32", "hot"),             # 12 experts per lane (3 vectors), 8-lane blocks
    # 64 experts per lane: blocks of two groups (the two load batches)
    (85, 4096, 16, 4, 2, 64, "f32", "normal"),        # 16-lane groups, 32-lane blocks
    (90, 4096, 16, 8, 3, 64, "f32", "hot"),           # 8-lane groups, 16-lane blocks
    (75, 4096, 16, 16, 8, 128, "f32", "coarse"),      # 4-lane groups, 8-lane blocks, many exact ties
    (80, 4096, 8, 32, 10, 32, "f32", "shared"),       # 2-lane groups, 4-lane blocks
    # FP32 rows in the key registers with the next row requested early, the
    # tokens claimed by the waves: runs of 20 and 40 experts (run-time
    # length), and pairs of equal keys (group scores made exact in the wave)
    (5000, 1280, 16, 4, 2, 64, "f32", "normal"),
    (5000, 2560, 16, 8, 4, 64, "f32", "duplicated"),
    # 20 tokens per workgroup (four claimed after the first sixteen) and a
    # last workgroup of 4 tokens (twelve waves without a token)
    (4984, 4096, 16, 16, 8, 128, "f32", "normal"),
    # small batches with the keys computed by the whole workgroup up front
    (2, 896, 16, 8, 4, 32, "bf16", "shared"),         # 14 experts per lane, 8 lanes per group fixed
    (16, 128, 8, 4, 2, 16, "f32", "equal"),           # one token per wave, all keys equal
    (1, 2048, 16, 8, 4, 32, "f32", "normal"),         # 32 experts per lane (run-time length)
    # one workgroup, at most 64 experts: wave 0 writes the metadata up to 256
    # routes, the workgroup scan beyond
    (32, 64, 8, 8, 4, 16, "f32", "normal"),           # 256 routes
    (33, 64, 8, 8, 4, 16, "bf16", "hot"),             # 264 routes
    (56, 64, 4, 2, 1, 4, "f32", "duplicated"),        # 224 routes, four-row blocks
    # at the limits of the contract: k = 64 with E = 4096, thousands of groups,
    # groups of one expert, blocks larger than any expert's count
    (40, 4096, 64, 1, 1, 1024, "bf16", "normal"),      # one group, 1024-row blocks
    (3000, 4096, 64, 8, 8, 256, "f32", "hot"),         # every group kept, several workgroups
    (2, 4096, 64, 64, 64, 1, "f32", "equal"),          # all keys equal, every group kept
    (700, 896, 64, 8, 8, 4096, "bf16", "log_zipf"),    # block above M: one block per used expert
    (50, 4096, 64, 2048, 40, 32, "f32", "normal"),     # 2048 groups of two
    (1, 4096, 64, 4096, 64, 1, "bf16", "coarse"),      # 4096 groups of one
    (130, 4096, 64, 4096, 100, 16, "f32", "normal"),   # groups of one, several workgroups
]


@pytest.mark.parametrize("case", SWEEP, ids=lambda c: "M{}_E{}_k{}_g{}-{}_b{}_{}_{}".format(*c))
def test_sweep_parity(case):
    M, E, k, ng, tg, block, dtype, dist = case
    cfg = workloads.custom(M, E, k, ng, tg, block, dtype, dist, seed=M + E)
    inp = workloads.make_inputs(cfg)
    assert_parity(inp, run(inp))


# the single-workgroup path on every small sweep shape, whichever path the
# library would pick for it
@pytest.mark.parametrize("case", [c for c in SWEEP if c[0] <= 64],
                         ids=lambda c: "M{}_E{}_k{}_g{}-{}_b{}_{}_{}".format(*c))
def test_sweep_parity_single_workgroup(case):
    M, E, k, ng, tg, block, dtype, dist = case
    cfg = workloads.custom(M, E, k, ng, tg, block, dtype, dist, seed=M + E)
    inp = workloads.make_inputs(cfg)
    assert_parity(inp, run(inp, flags=amr.FLAG_FORCE_SINGLE_WG))


# Drawn once by seeded generators and kept as a fixed list.  The first 32 range
# over the whole contract (E from 64 to 4096 with odd sizes, n_group any
# divisor, topk_group and k anywhere in range, block 1 to 256, M log-uniform up
# to 6000); the other 64 over the wave layouts (E = 32 or 64 lanes times 1 to
# 64 experts per lane, n_group dividing the lanes, M up to 20000); both dtypes
# and every distribution.
RANDOM_SWEEP = [
    (14, 192, 4, 32, 3, 128, "bf16", "coarse"),
    (4, 4096, 56, 2, 1, 1, "bf16", "shared"),
    (213, 192, 38, 3, 2, 256, "f32", "dominant_group"),
    (4853, 640, 2, 80, 1, 24, "bf16", "duplicated"),
    (6, 512, 21, 32, 12, 100, "f32", "duplicated"),
    (10, 192, 54, 48, 42, 3, "bf16", "duplicated"),
    (1, 448, 18, 7, 1, 100, "f32", "coarse"),
    (838, 192, 40, 8, 8, 8, "f32", "dominant_group"),
    (2475, 512, 62, 16, 8, 3, "f32", "hot"),
    (123, 192, 9, 24, 5, 128, "bf16", "shared"),
    (376, 96, 4, 48, 5, 2, "f32", "normal"),
    (19, 64, 35, 2, 2, 8, "bf16", "hot"),
    (18, 999, 37, 9, 6, 2, "f32", "log_zipf"),
    (38, 160, 32, 160, 81, 32, "bf16", "shared"),
    (17, 4096, 4, 4096, 2239, 64, "bf16", "offset_normal"),
    (8, 768, 3, 1, 1, 256, "f32", "log_zipf"),
    (34, 64, 21, 1, 1, 1, "bf16", "dominant_group"),
    (53, 64, 46, 1, 1, 64, "bf16", "equal"),
    (35, 128, 36, 64, 52, 16, "bf16", "log_zipf"),
    (3, 128, 14, 4, 1, 64, "bf16", "shared"),
    (3, 100, 16, 5, 2, 3, "bf16", "dominant_group"),
    (11, 640, 49, 5, 4, 1, "bf16", "coarse"),
    (6, 640, 32, 640, 57, 32, "bf16", "shared"),
    (207, 512, 19, 4, 2, 24, "bf16", "hot"),
    (68, 64, 37, 16, 15, 3, "f32", "offset_normal"),
    (8, 2048, 51, 16, 1, 16, "bf16", "equal"),
    (84, 768, 57, 24, 16, 128, "f32", "offset_normal"),
    (1053, 257, 32, 257, 49, 8, "f32", "coarse"),
    (5, 160, 61, 20, 19, 32, "bf16", "shared"),
    (172, 256, 9, 8, 2, 8, "f32", "hot"),
    (134, 96, 29, 2, 1, 16, "bf16", "coarse"),
    (3, 2560, 10, 8, 7, 100, "f32", "dominant_group"),
    (3990, 1024, 62, 32, 13, 128, "bf16", "coarse"),
    (807, 64, 16, 4, 2, 200, "bf16", "hot"),
    (4, 256, 51, 4, 1, 4, "f32", "coarse"),
    (17, 768, 57, 2, 1, 16, "f32", "offset_normal"),
    (347, 128, 38, 1, 1, 32, "bf16", "dominant_group"),
    (122, 128, 19, 4, 2, 200, "bf16", "equal"),
    (15, 4096, 51, 32, 28, 200, "bf16", "offset_normal"),
    (4591, 64, 12, 32, 10, 200, "bf16", "dominant_group"),
    (3062, 256, 20, 4, 2, 7, "f32", "offset_normal"),
    (2929, 4096, 17, 8, 4, 4, "bf16", "dominant_group"),
    (24, 768, 58, 2, 1, 64, "f32", "normal"),
    (9375, 1280, 63, 32, 28, 128, "bf16", "shared"),
    (46, 4096, 9, 4, 4, 200, "f32", "log_zipf"),
    (116, 256, 8, 8, 5, 64, "bf16", "log_zipf"),
    (5, 192, 59, 1, 1, 1, "f32", "duplicated"),
    (11718, 1024, 27, 1, 1, 32, "bf16", "offset_normal"),
    (239, 128, 20, 16, 4, 200, "bf16", "normal"),
    (28, 1792, 61, 2, 2, 200, "bf16", "log_zipf"),
    (821, 128, 4, 2, 1, 16, "f32", "normal"),
    (3489, 256, 3, 32, 1, 32, "bf16", "dominant_group"),
    (10, 256, 7, 2, 1, 200, "bf16", "log_zipf"),
    (654, 896, 18, 16, 2, 7, "bf16", "duplicated"),
    (86, 1280, 15, 1, 1, 7, "bf16", "equal"),
    (95, 512, 41, 8, 3, 128, "bf16", "dominant_group"),
    (1, 896, 47, 2, 1, 32, "bf16", "hot"),
    (229, 1792, 36, 16, 16, 7, "bf16", "dominant_group"),
    (6, 512, 5, 64, 40, 32, "bf16", "normal"),
    (150, 512, 21, 1, 1, 128, "f32", "offset_normal"),
    (56, 512, 40, 4, 1, 16, "f32", "coarse"),
    (1, 192, 23, 4, 2, 64, "bf16", "normal"),
    (793, 64, 1, 64, 1, 4, "f32", "duplicated"),
    (20, 512, 44, 4, 3, 1, "bf16", "equal"),
    (22, 256, 61, 8, 6, 16, "f32", "log_zipf"),
    (14499, 128, 7, 4, 1, 7, "f32", "log_zipf"),
    (8, 3072, 19, 64, 18, 16, "bf16", "equal"),
    (44, 128, 24, 2, 1, 64, "bf16", "offset_normal"),
    (2491, 768, 41, 4, 2, 4, "f32", "log_zipf"),
    (3, 512, 30, 2, 2, 128, "f32", "equal"),
    (14, 1024, 47, 8, 5, 200, "f32", "offset_normal"),
    (13, 128, 26, 2, 2, 7, "f32", "duplicated"),
    (1, 64, 9, 1, 1, 200, "f32", "normal"),
    (3459, 1024, 3, 16, 12, 32, "bf16", "offset_normal"),
    (1, 4096, 58, 16, 5, 200, "bf16", "equal"),
    (31, 1792, 20, 1, 1, 128, "bf16", "offset_normal"),
    (1547, 64, 49, 32, 32, 128, "f32", "log_zipf"),
    (4, 128, 31, 1, 1, 128, "f32", "hot"),
    (6, 192, 23, 8, 1, 64, "bf16", "duplicated"),
    (2929, 4096, 27, 4, 3, 1, "f32", "duplicated"),
    (704, 896, 49, 8, 7, 200, "f32", "shared"),
    (13217, 896, 9, 1, 1, 1, "f32", "normal"),
    (18, 128, 24, 1, 1, 200, "f32", "shared"),
    (97, 896, 61, 8, 4, 128, "f32", "duplicated"),
    (72, 256, 24, 1, 1, 64, "f32", "offset_normal"),
    (7451, 512, 13, 8, 4, 7, "bf16", "log_zipf"),
    (1, 896, 4, 2, 2, 64, "bf16", "duplicated"),
    (228, 2048, 41, 1, 1, 1, "f32", "normal"),
    (307, 896, 20, 64, 12, 32, "f32", "log_zipf"),
    (7, 64, 19, 1, 1, 1, "f32", "dominant_group"),
    (1, 2240, 6, 1, 1, 32, "f32", "coarse"),
    (18502, 256, 52, 4, 3, 4, "bf16", "hot"),
    (12, 1280, 26, 2, 1, 16, "bf16", "log_zipf"),
    (6, 1024, 37, 1, 1, 32, "bf16", "equal"),
    (63, 256, 11, 32, 12, 16, "bf16", "shared"),
    (5, 896, 33, 4, 2, 64, "f32", "duplicated"),
]


@pytest.mark.parametrize("case", RANDOM_SWEEP, ids=lambda c: "M{}_E{}_k{}_g{}-{}_b{}_{}_{}".format(*c))
def test_random_sweep_parity(case):
    M, E, k, ng, tg, block, dtype, dist = case
    cfg = workloads.custom(M, E, k, ng, tg, block, dtype, dist, seed=M * 7 + E)
    inp = workloads.make_inputs(cfg)
    assert_parity(inp, run(inp))
    if M <= 64:
        assert_parity(inp, run(inp, flags=amr.FLAG_FORCE_SINGLE_WG))


@pytest.mark.parametrize("dist", ["normal", "hot", "shared", "dominant_group", "log_zipf", "equal",
                                  "duplicated", "coarse"])
def test_distributions_prefill_shape(dist):
    cfg = workloads.custom(1024, 896, 16, 8, 4, 128, "bf16", dist, seed=7)
    inp = workloads.make_inputs(cfg)
    assert_parity(inp, run(inp))


# ---------------------------------------------------------------------------
# Contract: untouched tails, zero tokens, immutability, reuse, determinism,
# graph replay with changed inputs.
# ---------------------------------------------------------------------------
def test_poisoned_outputs_tails_untouched():
    cfg = workloads.custom(300, 896, 16, 8, 4, 64, "bf16", "log_zipf", seed=3)
    inp = workloads.make_inputs(cfg)
    x, b = to_gpu(inp)
    rows, blocks = amr.max_rows(cfg.M, cfg.E, cfg.k, cfg.block), amr.max_blocks(cfg.M, cfg.E, cfg.k, cfg.block)
    poison = -123456
    out = amr.RouteSortOutput(
        torch.full((cfg.M, cfg.k), poison, dtype=torch.int32, device="cuda"),
        torch.full((cfg.M, cfg.k), float("nan"), dtype=torch.float32, device="cuda"),
        torch.full((rows + 64,), poison, dtype=torch.int32, device="cuda"),
        torch.full((blocks + 64,), poison, dtype=torch.int32, device="cuda"),
        torch.full((1,), poison, dtype=torch.int32, device="cuda"))
    x0, b0 = x.clone(), b.clone()
    amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block, out=out)
    g = fetch(out, cfg.block)
    assert_parity(inp, g)
    rows_all = out.sorted_ids.cpu().numpy()
    eob_all = out.expert_of_block.cpu().numpy()
    assert np.all(rows_all[g["npp"]:] == poison)
    assert np.all(eob_all[g["npp"] // cfg.block:] == poison)
    assert torch.equal(x, x0) and torch.equal(b, b0)   # inputs never written


def test_zero_tokens():
    x = torch.empty((0, 64), dtype=torch.float32, device="cuda")
    b = torch.zeros(64, dtype=torch.float32, device="cuda")
    out = amr.RouteSortOutput(torch.empty((0, 4), dtype=torch.int32, device="cuda"),
                              torch.empty((0, 4), dtype=torch.float32, device="cuda"),
                              torch.full((4,), 7, dtype=torch.int32, device="cuda"),
                              torch.full((4,), 7, dtype=torch.int32, device="cuda"),
                              torch.full((1,), 7, dtype=torch.int32, device="cuda"))
    amr.route_sort(x, b, 4, 8, 4, 16, out=out)
    torch.cuda.synchronize()
    assert int(out.num_post_pad.item()) == 0
    assert torch.all(out.sorted_ids == 7) and torch.all(out.expert_of_block == 7)


def test_binding_refuses_host_buffers():
    """Outputs, workspace or stats in host memory are refused before any
    launch, by route_sort and by sort_from_ids."""
    cfg = workloads.CONFIGS["tiny"]
    x, b = to_gpu(workloads.make_inputs(cfg))
    print(f"[gpu] host buffers refused, M={cfg.M} E={cfg.E}", flush=True)
    good = amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block)
    torch.cuda.synchronize()
    for field in good._fields:
        out = good._replace(**{field: getattr(good, field).cpu()})
        with pytest.raises(ValueError):
            amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block, out=out)
    with pytest.raises(ValueError):
        amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block,
                       workspace=torch.zeros(1 << 16, dtype=torch.uint8))
    with pytest.raises(ValueError):
        amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block,
                       stats=torch.zeros(3, dtype=torch.int32))
    srt = amr.sort_from_ids(good.ids, cfg.E, cfg.block)
    torch.cuda.synchronize()
    for field in srt._fields:
        with pytest.raises(ValueError):
            amr.sort_from_ids(good.ids, cfg.E, cfg.block, out=srt._replace(**{field: getattr(srt, field).cpu()}))


def test_determinism_across_runs_and_paths():
    cfg = workloads.custom(700, 896, 16, 8, 4, 128, "bf16", "log_zipf", seed=21)
    inp = workloads.make_inputs(cfg)
    base = run(inp)
    for flags in [0] * 10 + [amr.FLAG_FORCE_EXACT, amr.FLAG_FORCE_MULTI_WG]:
        g = run(inp, flags=flags)
        for key in ("ids", "rows", "eob"):
            assert np.array_equal(g[key], base[key])
        assert np.array_equal(g["w"].view(np.uint32), base["w"].view(np.uint32)) or flags


@pytest.mark.parametrize("shape", [
    (512, 896, 16, 8, 4, 64, "bf16"),    # three launches
    (1, 896, 16, 8, 4, 32, "bf16"),      # one token: keys precomputed, rows written by the idle waves
    (4, 64, 4, 8, 4, 16, "f32"),         # keys precomputed, FP32
    (5000, 2560, 16, 8, 4, 64, "f32"),   # FP32 rows in the key registers, next rows requested early
], ids=lambda c: "M{}_E{}_{}".format(c[0], c[1], c[6]))
def test_graph_replay_with_changed_inputs(shape):
    M, E, k, ng, tg, block, dtype = shape
    print(f"[gpu] graph replay M={M} E={E} {dtype}", flush=True)
    cfg = workloads.custom(M, E, k, ng, tg, block, dtype, "normal", seed=30)
    sets = [workloads.make_inputs(cfg, seed=s) for s in range(4)]
    x, b = to_gpu(sets[0])
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):  # warm up: outputs and the stream's workspace, outside the capture
        out = amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block, out=out)
    for rep in range(8):
        inp = sets[rep % 4]
        xs, bs = to_gpu(inp)
        x.copy_(xs)
        b.copy_(bs)
        torch.cuda.synchronize()
        graph.replay()
        g = fetch(out, cfg.block)
        assert_parity(inp, g)


def test_one_workspace_across_shapes():
    """One workspace serves calls of different shapes in turn (three launches,
    two launches with the folded scan, the sort-only entry, a smaller call after
    a larger one): no call reads workspace words that an earlier call left."""
    cfgs = [workloads.custom(6000, 896, 16, 8, 4, 128, "bf16", "log_zipf", seed=50),
            workloads.custom(100, 512, 8, 4, 2, 32, "f32", "hot", seed=51),
            workloads.custom(3000, 2048, 32, 16, 8, 64, "f32", "normal", seed=52),
            workloads.custom(180, 896, 16, 8, 4, 16, "bf16", "shared", seed=53)]
    need = max(amr.workspace_bytes(c.M, c.E, c.k, c.block) for c in cfgs)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for cfg in cfgs:
            inp = workloads.make_inputs(cfg)
            x, b = to_gpu(inp)
            print(f"[gpu] shared workspace, pass {rep}, M={cfg.M} E={cfg.E} k={cfg.k}", flush=True)
            out = amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block, workspace=ws)
            ref = assert_parity(inp, fetch(out, cfg.block))
            srt = amr.sort_from_ids(out.ids, cfg.E, cfg.block, workspace=ws)
            torch.cuda.synchronize()
            npp = int(srt.num_post_pad.item())
            assert npp == ref.meta.num_post_pad
            assert np.array_equal(srt.sorted_ids[:npp].cpu().numpy(), ref.meta.sorted_ids)


def test_concurrent_streams_default_workspace():
    """Calls queued on two streams, free to overlap in time, each with the
    binding's default workspace (one per stream): both match the oracle."""
    cfg = workloads.custom(4096, 896, 16, 8, 4, 64, "bf16", "log_zipf", seed=40)
    inps = [workloads.make_inputs(cfg, seed=s) for s in (40, 41)]
    dev = [to_gpu(i) for i in inps]
    outs = [amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block) for x, b in dev]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    print(f"[gpu] two streams, M={cfg.M} E={cfg.E} x10 calls each", flush=True)
    for _ in range(10):
        for (x, b), out, s in zip(dev, outs, streams):
            with torch.cuda.stream(s):
                amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block, out=out)
    torch.cuda.synchronize()
    ws = {amr._ws_cache[(str(x.device), s.cuda_stream)][-1].data_ptr() for (x, _), s in zip(dev, streams)}
    assert len(ws) == 2
    for inp, out in zip(inps, outs):
        assert_parity(inp, fetch(out, cfg.block))


def test_stats_count_every_token():
    cfg = workloads.CONFIGS["threshold"]
    inp = workloads.make_inputs(cfg)
    stats = torch.zeros(3, dtype=torch.int32, device="cuda")
    run(inp, stats=stats)
    run(inp, flags=amr.FLAG_FORCE_EXACT, stats=stats)
    st = stats.cpu().numpy()
    assert st[0] + st[1] == 2 * cfg.M and st[0] >= cfg.M and st[2] == 0  # BF16 keys are exact already


@pytest.mark.parametrize("case", [
    # FP32 rows in the key registers, tokens claimed one at a time by each wave
    (5000, 2560, 16, 8, 4, 64, "f32", "duplicated"),
    # 32-lane segments (two tokens per wave)
    (5000, 896, 16, 8, 4, 128, "f32", "equal"),
    # one token per wave, rows staged in LDS (14 experts per lane)
    (200, 896, 16, 8, 4, 32, "f32", "equal"),
], ids=lambda c: "M{}_E{}".format(c[0], c[1]))
def test_exact_group_scores_in_the_wave(case):
    """Equal group scores (pairs of identical keys; all keys equal) leave the
    group boundary of the fast keys uncertain, so the wave makes those
    tokens' group scores exact: the refinement is taken on every layout, and
    every token still matches the oracle (with all keys equal the candidates
    then outnumber the lanes and the token goes to the workgroup-wide
    selection)."""
    M, E, k, ng, tg, block, dtype, dist = case
    print(f"[gpu] exact group scores M={M} E={E} {dtype} {dist}", flush=True)
    inp = workloads.make_inputs(workloads.custom(M, E, k, ng, tg, block, dtype, dist, seed=3))
    stats = torch.zeros(3, dtype=torch.int32, device="cuda")
    g = run(inp, stats=stats)
    st = stats.cpu().numpy()
    print(f"  exact-path tokens {st[0]}, fast-path tokens {st[1]}, exact group scores {st[2]}", flush=True)
    assert st[0] + st[1] == M
    assert st[2] > 0
    assert_parity(inp, g)


# ---------------------------------------------------------------------------
# The two sigmoid forms of the kernels.
# ---------------------------------------------------------------------------
def test_exact_sigmoid_bit_exact_on_all_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = orc.bf16_bits_to_f32(bits)
    x = x[np.isfinite(x)]
    f, e = amr.sigmoid_probe(torch.from_numpy(x).cuda())
    ref = orc.sigmoid_f32(x)
    e = e.cpu().numpy()
    bad = np.flatnonzero(e.view(np.uint32) != ref.view(np.uint32))
    assert bad.size == 0, (x[bad[:8]], e[bad[:8]], ref[bad[:8]])
    err = np.abs(f.cpu().numpy().astype(np.float64) - ref.astype(np.float64))
    print(f"  fast sigmoid max |err| over BF16 inputs: {err.max():.3e}", flush=True)
    assert err.max() < 2.0 ** -22


def test_sigmoid_table_bit_exact_on_all_bf16():
    """The LDS table that BF16 logits are scored with, through both address
    forms, equals the oracle's correctly rounded sigmoid on every finite BF16
    value (including zeros, subnormals and both clamped ends)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = orc.bf16_bits_to_f32(bits)
    fin = np.isfinite(x)
    o1, o2 = amr.sigmoid_table_probe(torch.from_numpy(bits.view(np.int16)).cuda())
    ref = orc.sigmoid_f32(x[fin])
    for o in (o1, o2):
        got = o.cpu().numpy()[fin]
        bad = np.flatnonzero(got.view(np.uint32) != ref.view(np.uint32))
        assert bad.size == 0, (x[fin][bad[:8]], got[bad[:8]], ref[bad[:8]])


def test_sigmoid_forms_on_fp32_grid():
    rng = np.random.default_rng(4)
    x = np.concatenate([np.linspace(-110, 40, 400001), rng.standard_normal(200000) * 3,
                        rng.standard_normal(50000) * 1e-3, rng.standard_normal(50000) * 1e-6]
                       ).astype(np.float32)
    f, e = amr.sigmoid_probe(torch.from_numpy(x).cuda())
    ref = orc.sigmoid_f32(x)
    e = e.cpu().numpy()
    mism = np.flatnonzero(e.view(np.uint32) != ref.view(np.uint32))
    print(f"  exact-form mismatches on {x.size} FP32 inputs: {mism.size}", flush=True)
    assert mism.size == 0, (x[mism[:8]], e[mism[:8]], ref[mism[:8]])
    err = np.abs(f.cpu().numpy().astype(np.float64) - ref.astype(np.float64))
    print(f"  fast sigmoid max |err| over FP32 grid: {err.max():.3e}", flush=True)
    assert err.max() < 2.0 ** -22


def _near_midpoint_fp32(n_per_chunk=48):
    """FP32 inputs whose float64 sigmoid lies closest to the midpoint between
    two FP32 neighbours, found by scanning whole binades (every FP32 value in
    them): the inputs on which a float64 evaluation alone can round wrongly."""
    picks = []
    for lo, hi in [(0x3a800000, 0x3b000000), (0x3f000000, 0x3f800000), (0x40000000, 0x40800000),
                   (0x41000000, 0x41800000), (0xbf800000, 0xc0000000), (0xc0800000, 0xc1000000),
                   (0xc2800000, 0xc2d00000)]:
        for start in range(lo, hi, 1 << 22):
            u = np.arange(start, min(hi, start + (1 << 22)), dtype=np.uint32)
            x = u.view(np.float32)
            r = 1.0 / (1.0 + np.exp(-x.astype(np.float64)))
            s = r.astype(np.float32)
            up = np.nextafter(s, np.float32(np.inf)).astype(np.float64)
            dn = np.nextafter(s, np.float32(-np.inf)).astype(np.float64)
            d = np.minimum(np.abs(r - 0.5 * (s + up)), np.abs(r - 0.5 * (s + dn))) / r
            picks.append(x[np.argsort(d)[:n_per_chunk]])
    return np.concatenate(picks)


def test_exact_sigmoid_near_rounding_midpoints():
    """The kernels' correctly rounded sigmoid on the hardest FP32 inputs: each
    sits within a few units of 2^-53 (relative) of an FP32 rounding midpoint,
    where the value is settled in double-double arithmetic."""
    x = _near_midpoint_fp32()
    print(f"  {x.size} near-midpoint FP32 inputs", flush=True)
    _, e = amr.sigmoid_probe(torch.from_numpy(x).cuda())
    ref = orc.sigmoid_f32(x)
    e = e.cpu().numpy()
    bad = np.flatnonzero(e.view(np.uint32) != ref.view(np.uint32))
    assert bad.size == 0, (x[bad[:8]], e[bad[:8]], ref[bad[:8]])
