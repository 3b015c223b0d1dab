"""Hand-worked fixtures under tests/golden/ (each states its source and the
derivation of every expected value): the CPU oracle must reproduce them, and,
on a GPU, so must the HIP path through the C ABI."""
import glob
import json
import os

import numpy as np
import pytest

from oracle import route_sort as orc

GOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "*.json")))


def _load(path):
    fx = json.load(open(path))
    logits = np.asarray(fx["logits_f32"], dtype=np.float32)
    bias = np.asarray(fx["bias_f32"], dtype=np.float32)
    return fx, logits, bias


def _check(fx, ids, w, npp, sorted_ids, eob):
    ex = fx["expected"]
    assert np.array_equal(np.asarray(ids), np.asarray(ex["ids"]))
    assert np.allclose(np.asarray(w, dtype=np.float64), np.asarray(ex["weights"]), rtol=1e-6, atol=0)
    assert npp == ex["num_post_pad"]
    assert np.array_equal(np.asarray(sorted_ids)[:npp], np.asarray(ex["sorted_ids"]))
    assert np.array_equal(np.asarray(eob)[:npp // fx["block"]], np.asarray(ex["expert_of_block"]))


@pytest.mark.parametrize("path", GOLDEN, ids=os.path.basename)
def test_golden_oracle(path):
    fx, logits, bias = _load(path)
    r = orc.route_sort(logits, "f32", bias, fx["k"], fx["n_group"], fx["topk_group"], fx["block"])
    _check(fx, r.ids, r.weights, r.meta.num_post_pad, r.meta.sorted_ids, r.meta.expert_of_block)


@pytest.mark.gpu
@pytest.mark.parametrize("path", GOLDEN, ids=os.path.basename)
def test_golden_gpu(path):
    import torch
    import align_moe_route_amd as amr
    fx, logits, bias = _load(path)
    out = amr.route_sort(torch.from_numpy(logits).cuda(), torch.from_numpy(bias).cuda(), fx["k"],
                         fx["n_group"], fx["topk_group"], fx["block"])
    torch.cuda.synchronize()
    _check(fx, out.ids.cpu().numpy(), out.weights.cpu().numpy(), int(out.num_post_pad.item()),
           out.sorted_ids.cpu().numpy(), out.expert_of_block.cpu().numpy())
