"""entmaxkv_score_select_noalloc (the library's static scratch in place of a
workspace) against entmaxkv_score_select on the same inputs: selections and
reported bounds bit for bit equal, on two calls in a row, the second with a
smaller input (the scratch keeps the first call's bounds), for bf16 and
float32 boxes; sampled heads also against the oracle."""
import numpy as np
import pytest
import torch

from sparse_long_context_page_amd import synth
from parity_util import Dev, announce, check_selection, check_meta_sequence, meta_to_f64

pytestmark = pytest.mark.gpu


def _both(dev, budget):
    from sparse_long_context_page_amd import entmaxkv as E
    w = dev.w
    sel_ref, ub_ref = dev.select(budget)
    sel = torch.full((w.batch, w.num_q_heads, budget), -7, dtype=torch.int32, device="cuda")
    ub = torch.full((w.batch, w.num_q_heads, budget), float("nan"), device="cuda")
    E.entmaxkv_score_select_noalloc(dev.shape, dev.q, dev.meta, dev.bt, dev.lens, budget, sel, ub)
    torch.cuda.synchronize()
    assert torch.equal(sel.cpu(), sel_ref.cpu())
    assert torch.equal(ub.cpu().view(torch.int32), ub_ref.cpu().view(torch.int32))
    return sel.cpu().numpy(), ub.cpu().numpy()


@pytest.mark.parametrize("kv_dtype", ["bf16", "f32"])
def test_noalloc_select_matches_workspace_select(kv_dtype):
    first = synth.Workload("noalloc_a", 3, 32, 8, 128, 32, 40000, kv_dtype, (1.5,), (82,),
                           4.0 / np.sqrt(128), plant="group_mean", n_planted=16,
                           seq_lens=(40000, 23000, 1000))
    second = synth.Workload("noalloc_b", 1, 8, 2, 64, 16, 3000, kv_dtype, (1.5,), (20,),
                            4.0 / np.sqrt(64), plant="group_mean", n_planted=8)
    for w, budget in ((first, 82), (second, 20)):
        inp = synth.generate(w, 71)
        dev = Dev(inp)
        announce(f"noalloc select {kv_dtype} {w.name} budget {budget}")
        meta = dev.build_meta()
        sel, ub = _both(dev, budget)
        meta64 = meta_to_f64(meta, kv_dtype)
        G = w.num_q_heads // w.num_kv_heads
        for b, h in ((0, 0), (w.batch - 1, w.num_q_heads - 1)):
            seq_meta = check_meta_sequence(inp, meta64, b, h // G)
            check_selection(inp, b, h, budget, sel[b, h], ub[b, h], seq_meta)
