"""The entry point that allocates nothing (moe_route_sort_static): its output
equals moe_route_sort's (caller workspace) bit for bit, on two calls in a row,
the second with a smaller input, and matches the oracle."""
import ctypes

import numpy as np
import pytest

import workloads
from oracle import route_sort as orc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
amr = pytest.importorskip("align_moe_route_amd")


def _to_gpu(inp):
    if inp.cfg.dtype == "bf16":
        x = torch.from_numpy(inp.logits_storage.view(np.int16)).view(torch.bfloat16).cuda()
        dt = amr.MRS_DTYPE_BF16
    else:
        x = torch.from_numpy(inp.logits_storage).cuda()
        dt = amr.MRS_DTYPE_F32
    return x, torch.from_numpy(inp.bias).cuda(), dt


def _fresh(M, E, k, block):
    rows, blocks = amr.max_rows(M, E, k, block), amr.max_blocks(M, E, k, block)
    return amr.RouteSortOutput(torch.full((M, k), -7, dtype=torch.int32, device="cuda"),
                               torch.full((M, k), -7.0, dtype=torch.float32, device="cuda"),
                               torch.full((rows,), -7, dtype=torch.int32, device="cuda"),
                               torch.full((blocks,), -7, dtype=torch.int32, device="cuda"),
                               torch.full((1,), -7, dtype=torch.int32, device="cuda"))


def _static_call(cfg, x, b, dt, out):
    """Straight through the C ABI (no binding logic in between)."""
    stream = torch.cuda.current_stream().cuda_stream
    return int(amr.lib().moe_route_sort_static(
        x.data_ptr(), b.data_ptr(), cfg.M, cfg.E, cfg.k, cfg.n_group, cfg.topk_group, cfg.block,
        out.ids.data_ptr(), out.weights.data_ptr(), out.sorted_ids.data_ptr(), out.expert_of_block.data_ptr(),
        out.num_post_pad.data_ptr(), dt, ctypes.c_void_p(stream)))


@pytest.mark.parametrize("names", [("wide", "prefill_skew"), ("prefill_skew", "threshold")])
def test_static_entry_matches_workspace_entry(names):
    for name in names:  # the second call takes a smaller input than the first
        cfg = workloads.CONFIGS[name]
        inp = workloads.make_inputs(cfg, seed=3)
        x, b, dt = _to_gpu(inp)
        print(f"[gpu] static entry {name} M={cfg.M} E={cfg.E}", flush=True)
        st = _fresh(cfg.M, cfg.E, cfg.k, cfg.block)
        assert _static_call(cfg, x, b, dt, st) == amr.MRS_OK
        ws = torch.zeros(amr.workspace_bytes(cfg.M, cfg.E, cfg.k, cfg.block), dtype=torch.uint8, device="cuda")
        ref = amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block, workspace=ws,
                             out=_fresh(cfg.M, cfg.E, cfg.k, cfg.block))
        torch.cuda.synchronize()
        npp = int(st.num_post_pad.item())
        assert npp == int(ref.num_post_pad.item())
        assert torch.equal(st.ids, ref.ids)
        assert torch.equal(st.weights.view(torch.int32), ref.weights.view(torch.int32))
        assert torch.equal(st.sorted_ids, ref.sorted_ids)            # tails untouched alike
        assert torch.equal(st.expert_of_block, ref.expert_of_block)
        # and the oracle: ids and metadata bit for bit, weights to 1e-6
        o = orc.route_sort(inp.logits_storage, cfg.dtype, inp.bias, cfg.k, cfg.n_group, cfg.topk_group,
                           cfg.block)
        assert np.array_equal(st.ids.cpu().numpy(), o.ids)
        w = st.weights.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(w - o.weights) / o.weights) <= 1e-6
        assert npp == o.meta.num_post_pad
        assert np.array_equal(st.sorted_ids[:npp].cpu().numpy(), o.meta.sorted_ids)
        assert np.array_equal(st.expert_of_block[:npp // cfg.block].cpu().numpy(), o.meta.expert_of_block)


def test_static_entry_small_and_zero_tokens():
    """One-workgroup shapes need no scratch; zero tokens write num_post_pad only."""
    cfg = workloads.CONFIGS["decode"]
    inp = workloads.make_inputs(cfg)
    x, b, dt = _to_gpu(inp)
    st = _fresh(cfg.M, cfg.E, cfg.k, cfg.block)
    assert _static_call(cfg, x, b, dt, st) == amr.MRS_OK
    ref = amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block)
    torch.cuda.synchronize()
    assert torch.equal(st.ids, ref.ids) and int(st.num_post_pad.item()) == int(ref.num_post_pad.item())
    empty = workloads.custom(0, 896, 16, 8, 4, 32, "bf16", "normal", seed=0, name="empty")
    x0 = torch.empty((0, 896), dtype=torch.bfloat16, device="cuda")
    out0 = amr.RouteSortOutput(*(torch.full((1,), -7, dtype=t, device="cuda")
                                 for t in (torch.int32, torch.float32, torch.int32, torch.int32, torch.int32)))
    assert _static_call(empty, x0, b, dt, out0) == amr.MRS_OK
    torch.cuda.synchronize()
    assert int(out0.num_post_pad.item()) == 0
