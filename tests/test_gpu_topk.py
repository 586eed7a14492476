"""GPU parity of entmaxkv_decode_topk (bounds, top-k and sparse decode in
one call) against the oracle and against the two-call path.

With bf16 caches and at least 128 query heads the call runs the per-head
select-and-decode kernel; with fewer heads its split form (several
workgroups per head, each selecting the head's pages and scoring a share,
then the threshold kernel); with float32 caches the four kernels of
entmaxkv_score_select and entmaxkv_decode_sparse. In both cases the selection must equal
entmaxkv_score_select's bit for bit (same bounds, same radix select), the
outputs must match the oracle run on that selection at the tolerances of the
other parity tests, and the two paths' outputs must agree. Shapes cover both
head sizes, every page size, GQA groups of 1, 4 and 8, ragged and empty
sequences, budgets below and above the page count, the chunked selection
(few long rows), alpha in {1.25, 1.5, 2, 3}, and all-equal scores (q = 0:
every token in the window, the per-wave spill areas and the global window
list)."""
import numpy as np
import pytest
import torch

from oracle import entmax_oracle as O
from sparse_long_context_page_amd import synth
from parity_util import Dev, announce, check_decode, check_meta_sequence, check_selection, \
    meta_to_f64

pytestmark = pytest.mark.gpu


def compare(inp, budget, alpha, heads=None, dev=None):
    """decode_topk vs the two calls (selection bit for bit, outputs close)
    and vs the oracle on the listed (or every) head."""
    w = inp["workload"]
    dev = dev or Dev(inp)
    if dev.meta is None:
        dev.build_meta()
    announce(f"{w.name}: decode_topk budget={budget} alpha={alpha}")
    sel, sel_ub, out, tau, sup = dev.topk(budget, alpha)
    sel2, ub2 = dev.select(budget)
    out2, tau2, sup2 = dev.sparse(sel2, budget, alpha)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel2), "selection differs from entmaxkv_score_select"
    assert torch.equal(sel_ub, ub2), "sel_ub differs from entmaxkv_score_select"
    o, t, s = out.cpu().numpy(), tau.cpu().numpy(), sup.cpu().numpy()
    o2, t2, s2 = out2.cpu().numpy(), tau2.cpu().numpy(), sup2.cpu().numpy()
    # the two paths: the same float32 scores, the same window; only the order
    # of the threshold's float64 sums and of the P.V float32 sums differ
    empty = s2 == 0
    assert (s[empty] == 0).all() and np.isnan(t[empty]).all() and (o[empty] == 0).all()
    live = ~empty
    assert np.abs(t[live] - t2[live]).max(initial=0.0) <= 1e-5 * max(1.0, np.abs(t2[live]).max(initial=1.0))
    norm = np.linalg.norm(o2, axis=-1, keepdims=True)
    assert (np.abs(o - o2) <= 1e-4 * np.maximum(norm, 1e-30) + 1e-7).all(), \
        f"paths differ by {np.abs(o - o2).max():.3e}"
    sel_np, ub_np = sel.cpu().numpy(), sel_ub.cpu().numpy()
    meta64 = meta_to_f64(dev.meta, w.kv_dtype)
    G = w.num_q_heads // w.num_kv_heads
    heads = heads or [(b, h) for b in range(w.batch) for h in range(w.num_q_heads)]
    seq_meta = {}
    near = differing = 0
    for b, h in heads:
        g = h // G
        if (b, g) not in seq_meta:
            seq_meta[(b, g)] = check_meta_sequence(inp, meta64, b, g)
        n_near, n_diff = check_selection(inp, b, h, budget, sel_np[b, h], ub_np[b, h],
                                         seq_meta[(b, g)])
        near += n_near
        differing += n_diff
        ref = O.decode_sparse(inp, b, h, alpha, sel_np[b, h])
        check_decode(ref, o[b, h], t[b, h], s[b, h], w.kv_dtype, alpha, f"topk b{b} h{h}")
    announce(f"{w.name}: {len(heads)} heads checked, near-tie pages {near}, differing {differing}")
    return dev


def sample(w, n, seed):
    rng = np.random.default_rng(seed)
    return sorted({(int(rng.integers(0, w.batch)), int(rng.integers(0, w.num_q_heads)))
                   for _ in range(n)})


@pytest.mark.parametrize("alpha", [1.5, 1.25, 2.0, 3.0])
def test_long_128k_shrunk(alpha):
    """128 heads (the per-head kernel), 32-token pages, several budgets."""
    w = synth.shrink(synth.WORKLOADS["long_128k"], context=6000, n_planted=32)
    inp = synth.generate(w, synth.WORKLOAD_SEEDS["long_128k"])
    dev = None
    P = (6000 + 31) // 32
    for budget in (1, 40, P, P + 9):
        dev = compare(inp, budget, alpha, sample(w, 24, budget), dev)


@pytest.mark.parametrize("D,ps,H,Hkv,lens", [
    (128, 16, 32, 8, (3000, 1, 16, 17, 0, 2500)),
    (64, 64, 64, 8, (4000, 64, 65, 1)),
    (64, 32, 128, 128, (900,)),
    (128, 64, 16, 4, (5000,) * 8),
])
def test_shapes_ragged(D, ps, H, Hkv, lens):
    w = synth.Workload("topk_ragged", len(lens), H, Hkv, D, ps, max(lens), "bf16", (1.5,), (9,),
                       4.0 / np.sqrt(D), plant="group_mean", n_planted=16, seq_lens=lens)
    inp = synth.generate(w, 31)
    dev = None
    for budget in (9, 33):
        dev = compare(inp, budget, 1.5, sample(w, 30, budget), dev)


def test_gqa_32k_shrunk():
    """256 heads with 16-token pages (four page buffers per wave)."""
    w = synth.shrink(synth.WORKLOADS["gqa_32k"], context=8000, n_planted=32)
    inp = synth.generate(w, synth.WORKLOAD_SEEDS["gqa_32k"])
    compare(inp, 256, 1.5, sample(w, 24, 5))


def test_chunked_selection_per_head():
    """128 rows of 8192+ pages: the bounds kernel keeps each chunk's top
    pages and the per-head kernel selects among them."""
    lens = (8192 * 16 + 77, 8192 * 16 - 300)
    w = synth.Workload("topk_chunked", 2, 64, 8, 64, 16, max(lens), "bf16", (1.5,), (64,),
                       4.0 / 8.0, plant="group_mean", n_planted=64, run_len=4, seq_lens=lens)
    inp = synth.generate(w, 37)
    dev = compare(inp, 64, 1.5, sample(w, 12, 1))
    compare(inp, 100, 2.0, sample(w, 12, 2), dev)


def test_all_equal_scores_spill_and_global_list():
    """q = 0: every bound and every score is 0, so each head keeps its first
    pages, every token is in the window and in the support (per-wave lists
    overflow to their spill areas; 1024 pages of 16 tokens exceed the LDS
    window list), and the output is the mean of the kept V rows."""
    lens = (1024 * 16 + 5, 700 * 16)
    w = synth.Workload("topk_flat", 2, 64, 8, 64, 16, max(lens), "bf16", (1.5,), (1024,),
                       0.5, plant="none", seq_lens=lens)
    inp = synth.generate(w, 41)
    inp["q"][:] = 0.0
    compare(inp, 1024, 1.5, sample(w, 6, 3))


def test_split_form_few_heads():
    """Fewer than 128 heads: the split form (bounds, several workgroups per
    head writing candidate regions, the threshold kernel)."""
    w = synth.shrink(synth.WORKLOADS["extreme_512k"], context=9000, n_planted=32)
    inp = synth.generate(w, synth.WORKLOAD_SEEDS["extreme_512k"])
    dev = None
    for budget, alpha in ((20, 1.5), (64, 1.25), (200, 2.0)):
        dev = compare(inp, budget, alpha, dev=dev)


@pytest.mark.parametrize("D,ps,H,Hkv,lens", [
    (128, 16, 8, 2, (3000, 1, 0, 2500)),
    (64, 32, 16, 16, (900, 4000)),
    (128, 64, 4, 1, (7000,)),
])
def test_split_form_shapes_ragged(D, ps, H, Hkv, lens):
    w = synth.Workload("topk_split", len(lens), H, Hkv, D, ps, max(lens), "bf16", (1.5,), (9,),
                       4.0 / np.sqrt(D), plant="group_mean", n_planted=16, seq_lens=lens)
    inp = synth.generate(w, 43)
    dev = None
    for budget in (3, 37):
        dev = compare(inp, budget, 1.5, dev=dev)


def test_split_form_chunked_selection():
    """32 rows of 8192+ pages: chunk candidates selected by every split."""
    lens = (8192 * 16 + 33,)
    w = synth.Workload("topk_split_chunked", 1, 32, 8, 64, 16, max(lens), "bf16", (1.5,), (64,),
                       4.0 / 8.0, plant="group_mean", n_planted=64, run_len=4, seq_lens=lens)
    inp = synth.generate(w, 47)
    compare(inp, 64, 1.5)


def test_fallback_path_matches():
    """float32 caches: the four-kernel path behind the same call."""
    w = synth.WORKLOADS["tiny_4k_f32"]
    inp = synth.generate(w, synth.WORKLOAD_SEEDS["tiny_4k_f32"])
    compare(inp, 32, 1.5)
