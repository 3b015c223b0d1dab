"""GPU parity on shapes drawn at test time by a seeded generator: every expert
count from 8 to 4096 the layouts distinguish, any n_group dividing E, k and
topk_group anywhere in range, blocks from 1 to 256, both dtypes, every input
distribution, and now and then a forced path (exact selection, or one
workgroup).  Ids and metadata bit-exact against the oracle, weights within
1e-6; every unforced case also checks one random expert range of the
expert-parallel entry against the oracle's local metadata."""
import numpy as np
import pytest

import workloads
from oracle import route_sort as orc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
amr = pytest.importorskip("align_moe_route_amd")

W_RTOL = 1e-6
CHUNKS, PER_CHUNK = 8, 50
ES = [8, 16, 32, 48, 64, 96, 100, 128, 160, 192, 224, 256, 257, 320, 384, 448, 512, 640, 768, 896, 999,
      1024, 1280, 1536, 1792, 2048, 2240, 2560, 3072, 3584, 4032, 4096]
BLOCKS = [1, 2, 3, 4, 7, 8, 16, 24, 32, 48, 64, 100, 128, 200, 256]
DISTS = ["normal", "offset_normal", "hot", "shared", "dominant_group", "log_zipf", "equal", "duplicated",
         "coarse"]


def draw_cases(seed, n):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        E = int(rng.choice(ES))
        divs = [d for d in range(1, E + 1) if E % d == 0]
        ng = int(rng.choice(divs))
        tg = int(rng.integers(1, ng + 1))
        k = int(rng.integers(1, min(64, tg * (E // ng)) + 1))
        M = int(np.exp(rng.uniform(0, np.log(9000))))
        M = max(1, min(M, 3_000_000 // E))
        block = int(rng.choice(BLOCKS))
        dtype = str(rng.choice(["f32", "bf16"]))
        dist = str(rng.choice(DISTS))
        r = float(rng.random())
        flags = amr.FLAG_FORCE_EXACT if r < 0.1 else (amr.FLAG_FORCE_SINGLE_WG if (r < 0.25 and M <= 64) else 0)
        lb = int(rng.integers(0, E))
        lc = int(rng.integers(1, E - lb + 1))
        cases.append((M, E, k, ng, tg, block, dtype, dist, flags, int(rng.integers(1 << 30)), lb, lc))
    return cases


CASES = draw_cases(20261203, CHUNKS * PER_CHUNK)


def to_gpu(inp):
    if inp.cfg.dtype == "bf16":
        x = torch.from_numpy(inp.logits_storage.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        x = torch.from_numpy(inp.logits_storage).cuda()
    return x, torch.from_numpy(inp.bias).cuda()


@pytest.mark.parametrize("chunk", range(CHUNKS))
def test_random_shapes(chunk):
    bad = []
    for M, E, k, ng, tg, block, dtype, dist, flags, seed, lb, lc in CASES[chunk * PER_CHUNK:(chunk + 1) * PER_CHUNK]:
        name = f"M={M} E={E} k={k} g={ng}/{tg} block={block} {dtype} {dist} flags={flags} seed={seed}"
        print(f"[gpu] random shape {name}", flush=True)
        cfg = workloads.custom(M, E, k, ng, tg, block, dtype, dist, seed=seed)
        inp = workloads.make_inputs(cfg)
        x, b = to_gpu(inp)
        out = amr.route_sort(x, b, k, ng, tg, block, flags=flags)
        torch.cuda.synchronize()
        ref = orc.route_sort(inp.logits_storage, cfg.dtype, inp.bias, k, ng, tg, block)
        npp = int(out.num_post_pad.item())
        w = out.weights.cpu().numpy().astype(np.float64)
        ok = (np.array_equal(out.ids.cpu().numpy(), ref.ids) and npp == ref.meta.num_post_pad
              and np.array_equal(out.sorted_ids[:npp].cpu().numpy(), ref.meta.sorted_ids)
              and np.array_equal(out.expert_of_block[:npp // block].cpu().numpy(), ref.meta.expert_of_block)
              and float((np.abs(w - ref.weights) / np.abs(ref.weights)).max()) <= W_RTOL)
        if not ok:
            bad.append(name)
        if flags == 0:
            lo = amr.route_sort(x, b, k, ng, tg, block, local=(lb, lc))
            torch.cuda.synchronize()
            m = orc.local_metadata(ref.ids, lb, lc, block)
            n2 = int(lo.num_post_pad.item())
            if not (n2 == m.num_post_pad and np.array_equal(lo.sorted_ids[:n2].cpu().numpy(), m.sorted_ids)
                    and np.array_equal(lo.expert_of_block[:n2 // block].cpu().numpy(), m.expert_of_block)):
                bad.append(f"{name} local=({lb},{lc})")
    assert not bad, bad
