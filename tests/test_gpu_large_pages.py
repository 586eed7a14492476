"""Sequences with more pages than the kernels stage on chip: 20000 pages of
16 tokens (over the select kernel's 16384 keys in LDS, so its passes re-read
the bounds row; over the Gaussian solve's 4096 pages in LDS, so its steps
re-read the page statistics). Boxes, top-k selection, sparse and full
decode, and the Gaussian-aware selection against the oracle."""
import numpy as np
import pytest
import torch

from oracle import entmax_oracle as O
from oracle import gauss_oracle as GO
from sparse_long_context_page_amd import synth
from parity_util import Dev, announce, check_decode, check_meta_sequence, check_selection, \
    meta_to_f64

pytestmark = pytest.mark.gpu


def test_more_pages_than_staged_on_chip():
    from sparse_long_context_page_amd import entmaxkv as E
    ps, P = 16, 20000
    lens = (P * ps - 5,)
    w = synth.Workload("many_pages", 1, 2, 1, 128, ps, lens[0], "bf16", (1.5,), (40,),
                       4.0 / np.sqrt(128), plant="group_mean", n_planted=16, seq_lens=lens)
    announce("many pages: generate")
    inp = synth.generate(w, 77)
    dev = Dev(inp)
    budget, alpha = 40, 1.5
    announce("many pages: meta/select/sparse/full")
    meta = dev.build_meta()
    sel, sel_ub = dev.select(budget)
    sp = dev.sparse(sel, budget, alpha)
    fu = dev.full(alpha)
    mom = torch.full_like(meta, float("nan"))
    E.entmaxkv_build_page_moments(dev.shape, dev.k, dev.bt, dev.lens, mom)
    cap = 64
    gsel = torch.empty((1, 2, cap), dtype=torch.int32, device="cuda")
    gtau = torch.empty((1, 2), device="cuda")
    E.entmaxkv_gauss_select(dev.shape, dev.q, mom, dev.bt, dev.lens, alpha, 3.0, cap, gsel, gtau)
    torch.cuda.synchronize()

    seq_meta = check_meta_sequence(inp, meta_to_f64(meta, "bf16"), 0, 0)
    moments = GO.page_moments(inp["k_pool"], inp["block_table"], inp["seq_lens"], ps, "bf16")
    sel_np, ub_np = sel.cpu().numpy(), sel_ub.cpu().numpy()
    so, st, ss = (x.cpu().numpy() for x in sp)
    fo, ft, fs = (x.cpu().numpy() for x in fu)
    gsel_np, gtau_np = gsel.cpu().numpy(), gtau.cpu().numpy()
    for h in range(2):
        announce(f"many pages: oracle head {h}")
        check_selection(inp, 0, h, budget, sel_np[0, h], ub_np[0, h], seq_meta=seq_meta)
        check_decode(O.decode_sparse(inp, 0, h, alpha, sel_np[0, h]), so[0, h], st[0, h],
                     ss[0, h], "bf16", alpha, f"sparse h{h}")
        check_decode(O.decode_full(inp, 0, h, alpha), fo[0, h], ft[0, h], fs[0, h], "bf16",
                     alpha, f"full h{h}")
        tau_ref, est, ref = GO.gauss_select_for_head(inp, 0, h, alpha, 3.0, cap, moments=moments)
        assert abs(float(gtau_np[0, h]) - tau_ref) <= 1e-6 * max(1.0, abs(tau_ref))
        got = [int(j) for j in gsel_np[0, h]]
        n = sum(1 for j in got if j >= 0)
        assert got[n:] == [-1] * (cap - n) and got[:n] == sorted(got[:n])
        diff = set(got[:n]) ^ {j for j in ref if j >= 0}
        if diff:
            assert diff <= GO.gauss_near_threshold(est, tau_ref, 3.0, cap), sorted(diff)


def test_budget_beyond_the_sequence():
    """A budget of more pages than the sequence has (25000 for 20000): every
    page is kept (then -1), the selection no longer fits the score kernel's
    LDS copy, and the sparse decode equals the full-cache one."""
    ps, P = 16, 20000
    lens = (P * ps - 9,)
    w = synth.Workload("many_pages_all", 1, 2, 1, 128, ps, lens[0], "bf16", (1.5,), (25000,),
                       4.0 / np.sqrt(128), plant="group_mean", n_planted=16, seq_lens=lens)
    inp = synth.generate(w, 78)
    dev = Dev(inp)
    budget, alpha = 25000, 1.5
    announce("budget beyond the sequence: select/sparse/full")
    sel, _ = dev.select(budget)
    sp = dev.sparse(sel, budget, alpha)
    fu = dev.full(alpha)
    torch.cuda.synchronize()
    s = sel.cpu().numpy()
    assert (s[:, :, :P] == np.arange(P)).all() and (s[:, :, P:] == -1).all()
    so, st, ss = (x.cpu().numpy() for x in sp)
    fo, ft, fs = (x.cpu().numpy() for x in fu)
    for h in range(2):
        ref = O.decode_full(inp, 0, h, alpha)
        check_decode(ref, so[0, h], st[0, h], ss[0, h], "bf16", alpha, f"sparse (all pages) h{h}")
        check_decode(ref, fo[0, h], ft[0, h], fs[0, h], "bf16", alpha, f"full h{h}")
