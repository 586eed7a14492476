"""Parity at the workloads' full sizes (the configuration the benchmark
times: entmaxkv_decode_topk for the sparse path, entmaxkv_decode_full), on
sampled (sequence, head) outputs the oracle computes one by one, plus
properties that hold at any size for every head. The two-call sparse path
(entmaxkv_score_select, entmaxkv_decode_sparse) is checked beside it, and the
one-call path must select the same pages bit for bit."""
import numpy as np
import pytest
import torch

from oracle import entmax_oracle as O
from sparse_long_context_page_amd import synth
from parity_util import Dev, announce, check_decode, check_meta_sequence, check_selection, \
    meta_to_f64

pytestmark = pytest.mark.gpu

N_SAMPLES = 6


def sample_heads(w, n, seed):
    rng = np.random.default_rng(seed)
    return sorted({(int(rng.integers(0, w.batch)), int(rng.integers(0, w.num_q_heads)))
                   for _ in range(n)})


def whole_batch_properties(w, sel, sel_ub, out, tau, sup, budget, lens):
    """Checks that hold for every head at any size: kept pages strictly
    ascending and inside the sequence, -1 padding after them, a non-empty
    support, finite outputs and thresholds."""
    P = (lens + w.page_size - 1) // w.page_size
    s = sel.cpu().numpy()
    for b in range(w.batch):
        keep = min(budget, int(P[b]))
        rows = s[b]
        assert (rows[:, keep:] == -1).all()
        kept = rows[:, :keep]
        assert (np.diff(kept, axis=1) > 0).all() and (kept >= 0).all() and (kept < P[b]).all()
    o = out.cpu().numpy()
    assert np.isfinite(o).all()
    assert (sup.cpu().numpy() >= 1).all()
    assert np.isfinite(tau.cpu().numpy()).all()


@pytest.mark.parametrize("name", ["tiny_4k_f32", "gqa_32k", "long_128k", "extreme_512k", "extreme_1m"])
def test_full_size_workload(name):
    w = synth.WORKLOADS[name]
    announce(f"full size {name}: generate")
    inp = synth.generate(w, synth.WORKLOAD_SEEDS[name])
    dev = Dev(inp)
    alpha, budget = w.alphas[0], w.budgets[0]
    announce(f"full size {name}: meta/select/sparse/full/topk")
    meta = dev.build_meta()
    sel, sel_ub = dev.select(budget)
    sp = dev.sparse(sel, budget, alpha)
    fu = dev.full(alpha)
    tk_sel, tk_ub, *tk = dev.topk(budget, alpha)
    torch.cuda.synchronize()
    whole_batch_properties(w, sel, sel_ub, *sp, budget, inp["seq_lens"])
    whole_batch_properties(w, sel, sel_ub, *fu, budget, inp["seq_lens"])
    # the one-call sparse path selects the same pages bit for bit
    assert torch.equal(tk_sel, sel) and torch.equal(tk_ub, sel_ub)
    whole_batch_properties(w, sel, sel_ub, *tk, budget, inp["seq_lens"])
    to, tt, ts = (x.cpu().numpy() for x in tk)
    meta64 = meta_to_f64(meta, w.kv_dtype)
    sel_np, ub_np = sel.cpu().numpy(), sel_ub.cpu().numpy()
    so, st, ss = (x.cpu().numpy() for x in sp)
    fo, ft, fs = (x.cpu().numpy() for x in fu)
    G = w.num_q_heads // w.num_kv_heads
    near = differing = 0
    for b, h in sample_heads(w, N_SAMPLES, 7):
        seq_meta = check_meta_sequence(inp, meta64, b, h // G)
        n_near, n_diff = check_selection(inp, b, h, budget, sel_np[b, h], ub_np[b, h], seq_meta)
        near += n_near
        differing += n_diff
        ref = O.decode_sparse(inp, b, h, alpha, sel_np[b, h])
        check_decode(ref, so[b, h], st[b, h], ss[b, h], w.kv_dtype, alpha, f"{name} sparse b{b} h{h}")
        check_decode(ref, to[b, h], tt[b, h], ts[b, h], w.kv_dtype, alpha, f"{name} topk b{b} h{h}")
        check_decode(O.decode_full(inp, b, h, alpha), fo[b, h], ft[b, h], fs[b, h],
                     w.kv_dtype, alpha, f"{name} full b{b} h{h}")
    announce(f"full size {name}: near-tie pages {near}, pages where the selections "
             f"differ {differing}")


def test_full_size_alpha_sweep():
    """Every (alpha, budget) cell of the 64K sweep at full size; the oracle
    checks sampled heads of each cell."""
    name = "alpha_sweep_64k"
    w = synth.WORKLOADS[name]
    announce(f"full size {name}: generate")
    inp = synth.generate(w, synth.WORKLOAD_SEEDS[name])
    dev = Dev(inp)
    meta = dev.build_meta()
    meta64 = None
    G = w.num_q_heads // w.num_kv_heads
    heads = sample_heads(w, 4, 11)
    seq_meta = {}
    for budget in w.budgets:
        announce(f"full size {name}: select budget={budget}")
        sel, sel_ub = dev.select(budget)
        torch.cuda.synchronize()
        if meta64 is None:
            meta64 = meta_to_f64(meta, w.kv_dtype)
        sel_np, ub_np = sel.cpu().numpy(), sel_ub.cpu().numpy()
        for b, h in heads:
            if (b, h // G) not in seq_meta:
                seq_meta[(b, h // G)] = check_meta_sequence(inp, meta64, b, h // G)
            n_near, n_diff = check_selection(inp, b, h, budget, sel_np[b, h], ub_np[b, h],
                                             seq_meta[(b, h // G)])
            announce(f"full size {name}: budget {budget} b{b} h{h}: near-tie pages {n_near}, "
                     f"differing {n_diff}")
        for alpha in w.alphas:
            announce(f"full size {name}: decode budget={budget} alpha={alpha}")
            sp = dev.sparse(sel, budget, alpha)
            fu = dev.full(alpha) if budget == w.budgets[0] else None
            tk_sel, tk_ub, *tk = dev.topk(budget, alpha)
            torch.cuda.synchronize()
            whole_batch_properties(w, sel, sel_ub, *sp, budget, inp["seq_lens"])
            assert torch.equal(tk_sel, sel) and torch.equal(tk_ub, sel_ub)
            whole_batch_properties(w, sel, sel_ub, *tk, budget, inp["seq_lens"])
            so, st, ss = (x.cpu().numpy() for x in sp)
            to, tt, ts = (x.cpu().numpy() for x in tk)
            sparse_checked = list(heads)
            if alpha == min(w.alphas) and budget == max(w.budgets):
                # the sparse heads with the largest supports (the longest
                # window lists of the sparse threshold step)
                order = np.argsort(-ss.reshape(-1), kind="stable")[:8]
                sparse_checked += [(int(i) // w.num_q_heads, int(i) % w.num_q_heads)
                                   for i in order]
                announce(f"full size {name}: sparse decode alpha={alpha} budget={budget}, "
                         f"the 8 largest supports "
                         f"{sorted(int(x) for x in ss.reshape(-1)[order])} checked")
            for b, h in dict.fromkeys(sparse_checked):
                ref = O.decode_sparse(inp, b, h, alpha, sel_np[b, h])
                check_decode(ref, so[b, h], st[b, h], ss[b, h], w.kv_dtype, alpha,
                             f"sweep sparse a{alpha} B{budget} b{b} h{h}")
                check_decode(ref, to[b, h], tt[b, h], ts[b, h], w.kv_dtype, alpha,
                             f"sweep topk a{alpha} B{budget} b{b} h{h}")
            if fu is not None:
                fo, ft, fs = (x.cpu().numpy() for x in fu)
                checked = list(heads)
                if alpha == min(w.alphas):
                    # the heads with the largest supports are those with the
                    # longest window lists (over 1024 members, over 2048
                    # candidates at alpha 1.25): the threshold step's long-list
                    # solve and wide gathers
                    order = np.argsort(-fs.reshape(-1), kind="stable")[:16]
                    longest = [(int(i) // w.num_q_heads, int(i) % w.num_q_heads) for i in order]
                    assert fs.reshape(-1)[order[-1]] >= 250, fs.reshape(-1)[order[-1]]
                    checked += [bh for bh in longest if bh not in checked]
                    announce(f"full size {name}: full decode alpha={alpha}, the 16 largest "
                             f"supports {sorted(int(x) for x in fs.reshape(-1)[order])} checked")
                for b, h in checked:
                    check_decode(O.decode_full(inp, b, h, alpha), fo[b, h], ft[b, h], fs[b, h],
                                 w.kv_dtype, alpha, f"sweep full a{alpha} b{b} h{h}")


def test_containment_report_matches_oracle():
    """The GPU containment criterion used by the sweep report (equal support
    size and tau) against the oracle's definition (the support's pages are a
    subset of the selection) on every trial of a shrunk alpha sweep; they may
    differ only where the oracle's support has a marginal token."""
    import bench
    from parity_util import marginal_tokens
    w = synth.shrink(synth.WORKLOADS["alpha_sweep_64k"], context=4096, batch=2, name="sweep_small")
    inp = synth.generate(w, synth.WORKLOAD_SEEDS["alpha_sweep_64k"])
    dev = Dev(inp)
    dev.build_meta()
    B, H = w.batch, w.num_q_heads
    announce("containment criterion")
    for budget in (16, 64):
        sel, _ = dev.select(budget)
        torch.cuda.synchronize()
        sel_np = sel.cpu().numpy()
        for alpha in w.alphas:
            _, ts, ss = dev.sparse(sel, budget, alpha)
            _, tf, sf = dev.full(alpha)
            torch.cuda.synchronize()
            c = bench.contained(ss.cpu().numpy(), sf.cpu().numpy(), ts.cpu().numpy(),
                                tf.cpu().numpy())
            mismatches = 0
            for b in range(B):
                for h in range(H):
                    res = O.decode_full(inp, b, h, alpha)
                    ref = set(O.support_pages(res, w.page_size)) <= set(int(j) for j in sel_np[b, h])
                    if ref != bool(c[b, h]):
                        assert marginal_tokens(res, alpha, 1e-6) > 0, (alpha, budget, b, h)
                        mismatches += 1
            assert mismatches <= 2, (alpha, budget, mismatches)
