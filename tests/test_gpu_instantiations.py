"""Every kernel instantiation against the oracle: cache dtype (bf16, float32)
x head_dim (64, 128) x query heads per KV head (1, 2, 4, 8) x page size
(16, 32, 64), each on a small ragged batch (a partial last page, a
one-page sequence): page boxes value for value, the top-k selection, the
sparse and the full decode of every head, and the Gaussian-aware selection
with its page moments."""
import itertools

import numpy as np
import pytest
import torch

from oracle import entmax_oracle as O
from oracle import gauss_oracle as GO
from sparse_long_context_page_amd import synth
from parity_util import (Dev, announce, check_decode, check_meta_sequence, check_selection,
                         meta_to_f64)

pytestmark = pytest.mark.gpu

COMBOS = list(itertools.product(("bf16", "f32"), (64, 128), (1, 2, 4, 8), (16, 32, 64)))


@pytest.mark.parametrize("kv_dtype,D,G,ps", COMBOS)
def test_instantiation(kv_dtype, D, G, ps):
    from sparse_long_context_page_amd import entmaxkv as E
    Hkv = 2
    lens = (5 * ps + 3, ps - 1)
    w = synth.Workload("inst", len(lens), G * Hkv, Hkv, D, ps, max(lens), kv_dtype, (1.5,),
                       (3,), 4.0 / np.sqrt(D), plant="group_mean", n_planted=3, seq_lens=lens)
    inp = synth.generate(w, 100 + D + G + ps)
    dev = Dev(inp)
    budget, alpha = 3, 1.5
    announce(f"instantiation {kv_dtype} D{D} G{G} ps{ps}")
    meta = dev.build_meta()
    sel, sel_ub = dev.select(budget)
    sp = dev.sparse(sel, budget, alpha)
    fu = dev.full(alpha)
    mom = torch.full_like(meta, float("nan"))
    E.entmaxkv_build_page_moments(dev.shape, dev.k, dev.bt, dev.lens, mom)
    P0 = O.num_pages(lens[0], ps)
    gsel = torch.empty((w.batch, w.num_q_heads, P0), dtype=torch.int32, device="cuda")
    gtau = torch.empty((w.batch, w.num_q_heads), device="cuda")
    E.entmaxkv_gauss_select(dev.shape, dev.q, mom, dev.bt, dev.lens, alpha, 2.0, P0, gsel, gtau)
    torch.cuda.synchronize()

    meta64 = meta_to_f64(meta, kv_dtype)
    mom64 = meta_to_f64(mom, kv_dtype)
    # the Gaussian selection is compared with the oracle run on the GPU's
    # moments (themselves checked against the oracle's within one unit in
    # the last place below): a one-ulp moment difference would otherwise
    # move tau_hat by far more than the float64 summation-order band
    gpu_moments = (mom64[:, :, 0], mom64[:, :, 1])
    moments = GO.page_moments(inp["k_pool"], inp["block_table"], inp["seq_lens"], ps, kv_dtype)
    sel_np, ub_np = sel.cpu().numpy(), sel_ub.cpu().numpy()
    so, st, ss = (x.cpu().numpy() for x in sp)
    fo, ft, fs = (x.cpu().numpy() for x in fu)
    gsel_np, gtau_np = gsel.cpu().numpy(), gtau.cpu().numpy()
    for b in range(w.batch):
        P = O.num_pages(lens[b], ps)
        phys = inp["block_table"][b, :P]
        for g in range(Hkv):
            seq_meta = check_meta_sequence(inp, meta64, b, g)
            # moments of full pages of bf16 keys are exact; elsewhere within
            # one unit in the last place of the stored dtype
            for side, ref in ((0, moments[0]), (1, moments[1])):
                got, want = mom64[phys, g, side], ref[phys, g]
                spacing = np.spacing(np.maximum(np.abs(want), 1e-30).astype(np.float32))
                spacing = spacing.astype(np.float64) * (65536.0 if kv_dtype == "bf16" else 1.0)
                assert (np.abs(got - want) <= spacing).all(), f"moments side {side}"
            for hh in range(G):
                h = g * G + hh
                check_selection(inp, b, h, budget, sel_np[b, h], ub_np[b, h], seq_meta=seq_meta)
                what = f"{kv_dtype} D{D} G{G} ps{ps} b{b} h{h}"
                check_decode(O.decode_sparse(inp, b, h, alpha, sel_np[b, h]), so[b, h], st[b, h],
                             ss[b, h], kv_dtype, alpha, "sparse " + what)
                check_decode(O.decode_full(inp, b, h, alpha), fo[b, h], ft[b, h], fs[b, h],
                             kv_dtype, alpha, "full " + what)
                # Gaussian selection (no cap binding): against the oracle on
                # the oracle's own moments, near-threshold pages excused
                tau_ref, est, ref = GO.gauss_select_for_head(inp, b, h, alpha, 2.0, P0,
                                                             moments=gpu_moments)
                assert abs(float(gtau_np[b, h]) - tau_ref) <= 1e-6 * max(1.0, abs(tau_ref))
                got_sel = {int(j) for j in gsel_np[b, h] if j >= 0}
                diff = got_sel ^ {j for j in ref if j >= 0}
                if diff:
                    near = GO.gauss_near_threshold(est, tau_ref, 2.0, P0)
                    assert diff <= near, f"gauss {what}: {sorted(diff)}"
