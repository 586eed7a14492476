"""Sequences that share a prefix of physical pages (a paged cache's prefix
sharing: the block tables of three sequences list the same first four
physical pages): page boxes, page moments, top-k selection, sparse and full
decode and the Gaussian-aware selection of every head against the oracle,
which reads the same block tables."""
import numpy as np
import pytest
import torch

from oracle import entmax_oracle as O
from oracle import gauss_oracle as GO
from sparse_long_context_page_amd import synth
from parity_util import (Dev, announce, check_decode, check_meta_sequence, check_selection,
                         meta_to_f64)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv_dtype", ["bf16", "f32"])
def test_shared_prefix_pages(kv_dtype):
    from sparse_long_context_page_amd import entmaxkv as E
    ps, D, Hkv, G = 16, 128, 2, 2
    lens = (200, 170, 90)
    w = synth.Workload("shared", len(lens), G * Hkv, Hkv, D, ps, max(lens), kv_dtype, (1.5,),
                       (3,), 4.0 / np.sqrt(D), plant="group_mean", n_planted=3, seq_lens=lens)
    inp = dict(synth.generate(w, 61))
    bt = inp["block_table"].copy()
    shared = 4  # full pages: every sequence holds all ps rows of each
    bt[1, :shared] = bt[0, :shared]
    bt[2, :shared] = bt[0, :shared]
    inp["block_table"] = bt
    dev = Dev(inp)
    budget, alpha, delta = 3, 1.5, 2.0
    announce(f"shared prefix {kv_dtype}")
    meta = dev.build_meta()
    sel, sel_ub = dev.select(budget)
    sp = dev.sparse(sel, budget, alpha)
    fu = dev.full(alpha)
    mom = torch.full_like(meta, float("nan"))
    E.entmaxkv_build_page_moments(dev.shape, dev.k, dev.bt, dev.lens, mom)
    P0 = O.num_pages(lens[0], ps)
    gsel = torch.empty((w.batch, w.num_q_heads, P0), dtype=torch.int32, device="cuda")
    gtau = torch.empty((w.batch, w.num_q_heads), device="cuda")
    E.entmaxkv_gauss_select(dev.shape, dev.q, mom, dev.bt, dev.lens, alpha, delta, P0, gsel,
                            gtau)
    torch.cuda.synchronize()

    meta64 = meta_to_f64(meta, kv_dtype)
    moments = GO.page_moments(inp["k_pool"], bt, inp["seq_lens"], ps, kv_dtype)
    mom64 = meta_to_f64(mom, kv_dtype)
    # the Gaussian selection is compared with the oracle run on the GPU's
    # moments (themselves checked against the oracle's within one unit in
    # the last place below): a one-ulp moment difference would otherwise
    # move tau_hat by far more than the float64 summation-order band
    gpu_moments = (mom64[:, :, 0], mom64[:, :, 1])
    sel_np, ub_np = sel.cpu().numpy(), sel_ub.cpu().numpy()
    so, st, ss = (x.cpu().numpy() for x in sp)
    fo, ft, fs = (x.cpu().numpy() for x in fu)
    gsel_np, gtau_np = gsel.cpu().numpy(), gtau.cpu().numpy()
    for b in range(w.batch):
        phys = bt[b, :O.num_pages(lens[b], ps)]
        for side, ref in ((0, moments[0]), (1, moments[1])):
            got, want = mom64[phys, :, side], ref[phys]
            sp_ = np.spacing(np.maximum(np.abs(want), 1e-30).astype(np.float32)).astype(np.float64)
            sp_ *= 65536.0 if kv_dtype == "bf16" else 1.0
            assert (np.abs(got - want) <= sp_).all(), f"moments b{b} side {side}"
        for g in range(Hkv):
            seq_meta = check_meta_sequence(inp, meta64, b, g)
            for hh in range(G):
                h = g * G + hh
                what = f"{kv_dtype} b{b} h{h}"
                check_selection(inp, b, h, budget, sel_np[b, h], ub_np[b, h], seq_meta=seq_meta)
                check_decode(O.decode_sparse(inp, b, h, alpha, sel_np[b, h]), so[b, h], st[b, h],
                             ss[b, h], kv_dtype, alpha, "sparse " + what)
                check_decode(O.decode_full(inp, b, h, alpha), fo[b, h], ft[b, h], fs[b, h],
                             kv_dtype, alpha, "full " + what)
                tau_ref, est, ref = GO.gauss_select_for_head(inp, b, h, alpha, delta, P0,
                                                             moments=gpu_moments)
                assert abs(float(gtau_np[b, h]) - tau_ref) <= 1e-6 * max(1.0, abs(tau_ref))
                got_sel = {int(j) for j in gsel_np[b, h] if j >= 0}
                diff = got_sel ^ {j for j in ref if j >= 0}
                if diff:
                    near = GO.gauss_near_threshold(est, tau_ref, delta, P0)
                    assert diff <= near, f"gauss {what}: {sorted(diff)}"
