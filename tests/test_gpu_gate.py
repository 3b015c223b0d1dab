"""GPU parity of the gate projection + route-sort entry (moe_gate_route_sort)
against the oracle: the FP32 logits equal the exactly rounded dot products
(oracle.gate.gate_logits), and the routing on them equals the oracle's routing
of the same logits bit for bit."""
import numpy as np
import pytest

import workloads
from oracle import gate as ogate
from oracle import route_sort as orc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
amr = pytest.importorskip("align_moe_route_amd")


def bits_to_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


CASES = [  # M, E, H, k, n_group, topk_group, block
    (1, 896, 7168, 16, 8, 4, 32),   # Kimi-K3 batch-1 decode
    (4, 896, 7168, 16, 8, 4, 32),
    (7, 64, 512, 4, 8, 4, 16),
    (64, 64, 256, 8, 1, 1, 8),
    (3, 4096, 1024, 16, 16, 8, 128),
    (2, 160, 8, 6, 4, 2, 5),
    # drawn once by a seeded generator (M up to 64, H any multiple of 8,
    # groups, k and block anywhere in range) and kept
    (39, 896, 528, 55, 7, 1, 16),
    (33, 64, 7920, 17, 2, 1, 1),
    (25, 1024, 2328, 51, 16, 9, 32),
    (61, 4096, 16, 58, 32, 10, 64),
    (38, 128, 3616, 16, 32, 10, 64),
    (50, 1024, 240, 64, 16, 15, 64),
    (5, 128, 3400, 15, 8, 4, 128),
    (39, 64, 3336, 25, 8, 5, 128),
    (52, 96, 5768, 35, 48, 44, 16),
    (19, 384, 1816, 31, 1, 1, 16),
]


@pytest.mark.parametrize("M,E,H,k,ng,tg,block", CASES)
def test_gate_then_route_matches_oracle(M, E, H, k, ng, tg, block):
    print(f"[gpu] gate M={M} E={E} H={H} k={k}", flush=True)
    rng = np.random.default_rng(M * 1000 + E + H)
    hb = workloads.f32_to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    wb = workloads.f32_to_bf16_bits((rng.standard_normal((E, H)) * H ** -0.5).astype(np.float32))
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    logits, out = amr.gate_route_sort(bits_to_bf16(hb).cuda(), bits_to_bf16(wb).cuda(), torch.from_numpy(bias).cuda(),
                                      k, ng, tg, block)
    torch.cuda.synchronize()
    got = logits.cpu().numpy()
    ref = ogate.gate_logits(hb, wb)
    diff = got != ref
    if diff.any():
        # only where the exact value is within the float64 accumulation bound
        # of an FP32 rounding midpoint may the kernel round the other way
        margin = ogate.midpoint_margin(hb, wb, ref)
        assert np.all(margin[diff] < 8 * H * 2.0 ** -53), "logit differs away from a rounding midpoint"
        ulps = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
        assert np.all(ulps[diff] <= 1)
        print(f"[gpu]   {int(diff.sum())} logits one ulp apart at a rounding midpoint", flush=True)
    same = ~diff.any(axis=1)
    r = orc.route_sort(ref, "f32", bias, k, ng, tg, block)
    ids = out.ids.cpu().numpy()
    w = out.weights.cpu().numpy().astype(np.float64)
    assert np.array_equal(ids[same], r.ids[same])
    assert np.all(np.abs(w[same] - r.weights[same]) <= 1e-6 * np.abs(r.weights[same]))
    npp = int(out.num_post_pad.item())
    rows = out.sorted_ids[:npp].cpu().numpy()
    eob = out.expert_of_block[:npp // block].cpu().numpy()
    if same.all():
        assert npp == r.meta.num_post_pad
        assert np.array_equal(rows, r.meta.sorted_ids)
        assert np.array_equal(eob, r.meta.expert_of_block)
    else:
        # tokens with a logit at a rounding midpoint: reported, and their
        # metadata must still be consistent with the kernel's own picks
        print(f"[gpu]   {int((~same).sum())} tokens with a midpoint logit", flush=True)
        assert orc.check_sort_invariants(ids, rows, eob, npp, E, block) == []


def test_zero_tokens():
    E, H = 896, 7168
    h = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((E, H), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((E,), dtype=torch.float32, device="cuda")
    logits, out = amr.gate_route_sort(h, w, b, 16, 8, 4, 32)
    torch.cuda.synchronize()
    assert int(out.num_post_pad.item()) == 0
