"""More than 256 (sequence, query head) pairs in one call: the threshold
kernel then holds at most 4096 window members per head in LDS (two
workgroups fit a compute unit), and longer lists take the global-memory
path. Selection of every head and sampled sparse and full decodes against
the oracle, at alpha = 1.5 and at alpha = 1.05 (window 20 in z: lists of
thousands of entries)."""
import numpy as np
import pytest
import torch

from oracle import entmax_oracle as O
from sparse_long_context_page_amd import synth
from parity_util import Dev, announce, check_decode, check_selection

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("alpha", [1.5, 1.05])
def test_more_than_256_heads(alpha):
    w = synth.shrink(synth.WORKLOADS["gqa_32k"], context=6000, batch=9, n_planted=8)
    assert w.batch * w.num_q_heads > 256
    inp = synth.generate(w, 12)
    dev = Dev(inp)
    budget = 64
    announce(f"many heads alpha {alpha}")
    sel, sel_ub = dev.select(budget)
    sp = dev.sparse(sel, budget, alpha)
    fu = dev.full(alpha)
    torch.cuda.synchronize()
    sel_np, ub_np = sel.cpu().numpy(), sel_ub.cpu().numpy()
    so, st, ss = (x.cpu().numpy() for x in sp)
    fo, ft, fs = (x.cpu().numpy() for x in fu)
    for b in range(w.batch):
        for h in range(w.num_q_heads):
            check_selection(inp, b, h, budget, sel_np[b, h], ub_np[b, h])
    rng = np.random.default_rng(3)
    heads = sorted({(int(rng.integers(0, w.batch)), int(rng.integers(0, w.num_q_heads)))
                    for _ in range(10)})
    for b, h in heads:
        announce(f"many heads alpha {alpha}: oracle b{b} h{h}")
        check_decode(O.decode_sparse(inp, b, h, alpha, sel_np[b, h]), so[b, h], st[b, h],
                     ss[b, h], w.kv_dtype, alpha, f"sparse b{b} h{h}")
        check_decode(O.decode_full(inp, b, h, alpha), fo[b, h], ft[b, h], fs[b, h], w.kv_dtype,
                     alpha, f"full b{b} h{h}")
