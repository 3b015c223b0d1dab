"""GPU parity of the grouped GEMM that reads the route-sort metadata
(moe_grouped_gemm1) against the oracle (oracle/moe_gemm.py).

The metadata fed to the kernel is the oracle's own (sort_metadata of seeded
ids), so every expected value comes from the oracle.  Integer-valued inputs
must match bit for bit; random inputs must lie within the tolerance derived
from FP32 accumulation and BF16 rounding (oracle.moe_gemm.tolerance)."""
import numpy as np
import pytest

import workloads
from oracle import moe_gemm as og
from oracle import route_sort as orc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
amr = pytest.importorskip("align_moe_route_amd")

POISON = 0x7FBF  # a BF16 NaN pattern: any row the kernel writes replaces it


def distinct_rows(rng, M, E, k, skew=0.0):
    p = None
    if skew > 0:
        w = 1.0 / np.arange(1, E + 1) ** skew
        p = w[rng.permutation(E)] / w.sum()
    return np.stack([np.sort(rng.choice(E, k, replace=False, p=p)) for _ in range(M)]).astype(np.int32)


def bits_to_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def device_meta(ref, M, E, k, block):
    """The oracle's metadata in buffers of the library's capacity; the unused
    tails hold values that would be out of range if the kernel read them."""
    rows, blocks = amr.max_rows(M, E, k, block), amr.max_blocks(M, E, k, block)
    sid = np.full(max(rows, 1), -12345, dtype=np.int32)
    sid[:ref.num_post_pad] = ref.sorted_ids
    eob = np.full(max(blocks, 1), 1 << 30, dtype=np.int32)
    eob[:ref.num_post_pad // block] = ref.expert_of_block
    npp = np.array([ref.num_post_pad], dtype=np.int32)
    return [torch.from_numpy(a).cuda() for a in (sid, eob, npp)]


def run_gemm(xb, wb, ref, M, E, k, block):
    N = wb.shape[1]
    sid, eob, npp = device_meta(ref, M, E, k, block)
    y = torch.full((max(amr.max_rows(M, E, k, block), 1), N), POISON, dtype=torch.int16,
                   device="cuda").view(torch.bfloat16)
    amr.grouped_gemm1(bits_to_bf16(xb).cuda(), bits_to_bf16(wb).cuda(), sid, eob, npp, k, block, out=y)
    torch.cuda.synchronize()
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


SHAPES = [  # M, E, k, K, N, block
    (64, 16, 4, 128, 128, 32),
    (200, 24, 6, 256, 256, 64),
    (300, 8, 2, 192, 128, 128),
    (1, 32, 16, 3584, 768, 32),
    (513, 64, 8, 512, 384, 128),
    (97, 40, 5, 64, 128, 96),
    (150, 12, 4, 64, 512, 64),     # one K step; 64 x 256 tiles
    (90, 20, 3, 128, 256, 256),    # two 128-row tiles per padding block
    # drawn once by a seeded generator (K a multiple of 64 up to 1024, N a
    # multiple of 128 up to 768, block a multiple of 32 up to 256) and kept
    (675, 13, 11, 832, 256, 96),
    (493, 51, 4, 128, 128, 64),
    (308, 56, 11, 704, 128, 32),
    (162, 47, 10, 576, 768, 32),
    (375, 34, 2, 448, 384, 160),
    (610, 35, 9, 64, 512, 96),
    (462, 54, 15, 128, 768, 256),
    (544, 18, 2, 256, 384, 160),
    (601, 34, 16, 128, 384, 32),
    (13, 27, 7, 960, 384, 128),
    (3, 14, 10, 128, 768, 128),    # a few tokens: nearly every tile is padding
    (1, 29, 11, 768, 512, 64),
    (2, 36, 14, 64, 512, 96),
    (10, 61, 13, 704, 512, 256),
]


@pytest.mark.parametrize("M,E,k,K,N,block", SHAPES)
def test_integer_inputs_bit_exact(M, E, k, K, N, block):
    print(f"[gpu] gemm1 integer M={M} E={E} k={k} K={K} N={N} block={block}", flush=True)
    rng = np.random.default_rng(M * 7 + K)
    xb = workloads.f32_to_bf16_bits(rng.integers(-6, 7, size=(M, K)).astype(np.float32))
    wb = workloads.f32_to_bf16_bits(rng.integers(-6, 7, size=(E, N, K)).astype(np.float32))
    ref = orc.sort_metadata(distinct_rows(rng, M, E, k), E, block)
    y = run_gemm(xb, wb, ref, M, E, k, block)
    exact = og.gemm1_sorted(xb, wb, ref.sorted_ids, ref.expert_of_block, ref.num_post_pad, M, k, block)
    assert np.array_equal(y[:ref.num_post_pad], og.f64_to_bf16_bits(exact))
    assert np.all(y[ref.num_post_pad:] == POISON)


@pytest.mark.parametrize("M,E,k,K,N,block", SHAPES)
def test_random_inputs_within_tolerance(M, E, k, K, N, block):
    print(f"[gpu] gemm1 random M={M} E={E} k={k} K={K} N={N} block={block}", flush=True)
    rng = np.random.default_rng(M * 11 + E)
    xb = workloads.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    wb = workloads.f32_to_bf16_bits((rng.standard_normal((E, N, K)) * K ** -0.5).astype(np.float32))
    ref = orc.sort_metadata(distinct_rows(rng, M, E, k, skew=1.1), E, block)
    y = run_gemm(xb, wb, ref, M, E, k, block)
    npp = ref.num_post_pad
    rows = np.arange(npp)
    exact = og.gemm1_rows(xb, wb, ref.sorted_ids, ref.expert_of_block, M, k, block, rows)
    absp = og.abs_products(xb, wb, ref.sorted_ids, ref.expert_of_block, M, k, block, rows)
    got = og.bf16_to_f64(y[:npp])
    tol = og.tolerance(exact, absp, K)
    bad = np.abs(got - exact) > tol
    assert not bad.any(), f"{int(bad.sum())} elements outside tolerance, first at {np.argwhere(bad)[0]}"
    pad = ref.sorted_ids == M * k
    assert np.all(y[:npp][pad] == 0)
    assert np.all(y[npp:] == POISON)


def test_dropped_routes_and_empty_metadata():
    # metadata of ids with dropped routes (fewer rows), and of ids that are all
    # dropped (num_post_pad = 0: nothing is written)
    M, E, k, K, N, block = 150, 32, 4, 128, 128, 32
    rng = np.random.default_rng(3)
    xb = workloads.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    wb = workloads.f32_to_bf16_bits(rng.standard_normal((E, N, K)).astype(np.float32) * 0.1)
    ids = distinct_rows(rng, M, E, k)
    ids[rng.random(ids.shape) < 0.3] = -1
    ref = orc.sort_metadata(ids, E, block)
    y = run_gemm(xb, wb, ref, M, E, k, block)
    rows = np.arange(ref.num_post_pad)
    exact = og.gemm1_rows(xb, wb, ref.sorted_ids, ref.expert_of_block, M, k, block, rows)
    absp = og.abs_products(xb, wb, ref.sorted_ids, ref.expert_of_block, M, k, block, rows)
    assert np.all(np.abs(og.bf16_to_f64(y[:ref.num_post_pad]) - exact) <= og.tolerance(exact, absp, K))
    ref0 = orc.sort_metadata(np.full((M, k), -1, dtype=np.int32), E, block)
    assert ref0.num_post_pad == 0
    y0 = run_gemm(xb, wb, ref0, M, E, k, block)
    assert np.all(y0 == POISON)


def test_route_sort_then_gemm_matches_oracle_chain():
    # the product path end to end (route-sort kernels, then the GEMM on their
    # device metadata) against the oracle's route-sort followed by its GEMM
    M, E, k, ng, tg, block, K, N = 700, 896, 16, 8, 4, 128, 256, 256
    cfg = workloads.custom(M, E, k, ng, tg, block, "bf16", "log_zipf", seed=5)
    inp = workloads.make_inputs(cfg)
    ref = orc.route_sort(inp.logits_storage, cfg.dtype, inp.bias, k, ng, tg, block)
    rng = np.random.default_rng(9)
    xb = workloads.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    wb = workloads.f32_to_bf16_bits(rng.standard_normal((E, N, K)).astype(np.float32) * 0.06)
    logits = torch.from_numpy(inp.logits_storage.view(np.int16)).view(torch.bfloat16).cuda()
    out = amr.route_sort(logits, torch.from_numpy(inp.bias).cuda(), k, ng, tg, block)
    y = amr.grouped_gemm1(bits_to_bf16(xb).cuda(), bits_to_bf16(wb).cuda(), out.sorted_ids,
                          out.expert_of_block, out.num_post_pad, k, block)
    torch.cuda.synchronize()
    npp = ref.meta.num_post_pad
    assert int(out.num_post_pad.item()) == npp
    got = og.bf16_to_f64(y[:npp].view(torch.int16).cpu().numpy().view(np.uint16))
    rows = np.arange(npp)
    m = ref.meta
    exact = og.gemm1_rows(xb, wb, m.sorted_ids, m.expert_of_block, M, k, block, rows)
    absp = og.abs_products(xb, wb, m.sorted_ids, m.expert_of_block, M, k, block, rows)
    assert np.all(np.abs(got - exact) <= og.tolerance(exact, absp, K))


def test_full_size_prefill_sampled_rows():
    # Kimi-K3 TP8 shapes: 8192 tokens, 896 experts, top-16, K = 3584,
    # N = 2 * 384, block 128, metadata of the skewed prefill workload; the
    # oracle recomputes a sample of rows one by one
    cfg = workloads.CONFIGS["prefill_skew"]
    M, E, k, block, K, N = cfg.M, cfg.E, cfg.k, cfg.block, 3584, 768
    print(f"[gpu] gemm1 full size M={M} E={E} k={k} K={K} N={N}", flush=True)
    inp = workloads.make_inputs(cfg)
    ids = orc.route_sort(inp.logits_storage, cfg.dtype, inp.bias, k, cfg.n_group, cfg.topk_group, block).ids
    ref = orc.sort_metadata(ids, E, block)
    g = torch.Generator(device="cuda").manual_seed(0)
    x = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn((E, N, K), generator=g, device="cuda") * K ** -0.5).to(torch.bfloat16)
    sid, eob, npp = device_meta(ref, M, E, k, block)
    y = amr.grouped_gemm1(x, w, sid, eob, npp, k, block)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    nppv = ref.num_post_pad
    rows = np.unique(np.concatenate([rng.choice(nppv, 96, replace=False), [0, nppv - 1]]))
    experts = np.unique(ref.expert_of_block[rows // block])
    remap = np.full(E, -1, dtype=np.int32)
    remap[experts] = np.arange(experts.size)
    xb = x.view(torch.int16).cpu().numpy().view(np.uint16)
    wsub = w[torch.from_numpy(experts).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
    eobm = remap[ref.expert_of_block]
    exact = og.gemm1_rows(xb, wsub, ref.sorted_ids, eobm, M, k, block, rows)
    absp = og.abs_products(xb, wsub, ref.sorted_ids, eobm, M, k, block, rows)
    got = og.bf16_to_f64(y[torch.from_numpy(rows).cuda()].view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.all(np.abs(got - exact) <= og.tolerance(exact, absp, K))


def test_route_sort_and_gemm_in_one_graph_with_changed_inputs():
    # the handoff needs no host round trip: route-sort and the GEMM captured in
    # one HIP graph, replayed with new logits and hidden states each time
    M, E, k, ng, tg, block, K, N = 300, 896, 16, 8, 4, 64, 128, 256
    cfg = workloads.custom(M, E, k, ng, tg, block, "bf16", "log_zipf", seed=11)
    sets = [workloads.make_inputs(cfg, seed=s) for s in range(3)]
    rng = np.random.default_rng(12)
    xbs = [workloads.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)) for _ in range(3)]
    wb = workloads.f32_to_bf16_bits(rng.standard_normal((E, N, K)).astype(np.float32) * 0.08)
    logits = torch.from_numpy(sets[0].logits_storage.view(np.int16)).view(torch.bfloat16).cuda()
    bias = torch.from_numpy(sets[0].bias).cuda()
    xg = bits_to_bf16(xbs[0]).cuda()
    wg = bits_to_bf16(wb).cuda()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):  # the stream's workspace, allocated outside the capture
        out = amr.route_sort(logits, bias, k, ng, tg, block)
        y = amr.grouped_gemm1(xg, wg, out.sorted_ids, out.expert_of_block, out.num_post_pad, k, block)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        amr.route_sort(logits, bias, k, ng, tg, block, out=out)
        amr.grouped_gemm1(xg, wg, out.sorted_ids, out.expert_of_block, out.num_post_pad, k, block, out=y)
    for rep in range(6):
        inp, xb = sets[rep % 3], xbs[rep % 3]
        logits.copy_(torch.from_numpy(inp.logits_storage.view(np.int16)).view(torch.bfloat16).cuda())
        bias.copy_(torch.from_numpy(inp.bias).cuda())
        xg.copy_(bits_to_bf16(xb).cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = orc.route_sort(inp.logits_storage, cfg.dtype, inp.bias, k, ng, tg, block).meta
        npp = int(out.num_post_pad.item())
        assert npp == ref.num_post_pad
        rows = np.arange(npp)
        exact = og.gemm1_rows(xb, wb, ref.sorted_ids, ref.expert_of_block, M, k, block, rows)
        absp = og.abs_products(xb, wb, ref.sorted_ids, ref.expert_of_block, M, k, block, rows)
        got = og.bf16_to_f64(y[:npp].view(torch.int16).cpu().numpy().view(np.uint16))
        assert np.all(np.abs(got - exact) <= og.tolerance(exact, absp, K)), rep
