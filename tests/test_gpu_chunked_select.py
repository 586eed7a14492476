"""GPU parity of the chunked page selection against the oracle, every head.

When the per-row selection would scan many pages per compute unit (about
8192 or more: few, long rows) and the budget is at most half a bounds chunk,
the bounds kernel keeps each chunk's top pages itself and the select kernel
picks the budget largest of those candidates. These shapes are sized so that
path runs: bf16 boxes, at least 8192 pages per sequence and at most 256
(sequence, head) rows. They cover one, four and eight query heads per KV
head, both head sizes, ragged last chunks (fewer pages than the chunk, more
or fewer than the budget), a sequence shorter than one chunk, one whose last
chunk holds a single page, an empty one, and all-equal bounds (q = 0), where
ties must go to the lower pages."""
import numpy as np
import pytest
import torch

from sparse_long_context_page_amd import synth
from parity_util import Dev, announce, check_meta_sequence, check_selection, meta_to_f64

pytestmark = pytest.mark.gpu

PS = 16
LONG = 8192 * PS  # tokens of an 8192-page sequence

CASES = {
    # B=4, G=4, D=128: 256-page chunks; last chunks of 220 pages, of 1 page,
    # and a 7-page sequence
    "g4_d128": dict(H=8, Hkv=2, D=128,
                    lens=(LONG, LONG - 37 * PS + 5, 100, 2 * 128 * PS + 1), budgets=(16, 64)),
    # B=1, G=1, D=64: 320-page chunks, a 243-page last chunk
    "g1_d64": dict(H=8, Hkv=8, D=64, lens=(LONG + 50 * PS + 3,), budgets=(7, 100)),
    # B=2, G=8, D=128: 192-page chunks, a 110-page last chunk, an empty sequence
    "g8_d128": dict(H=16, Hkv=2, D=128, lens=(140000, 0), budgets=(40,)),
}


def make_inputs(name):
    c = CASES[name]
    lens = c["lens"]
    w = synth.Workload(f"chunked_{name}", len(lens), c["H"], c["Hkv"], c["D"], PS, max(lens),
                       "bf16", (1.5,), c["budgets"], 4.0 / np.sqrt(c["D"]), plant="group_mean",
                       n_planted=64, run_len=4, seq_lens=lens)
    return synth.generate(w, 23)


def check_all_heads(inp, budget, dev):
    w = inp["workload"]
    announce(f"{w.name}: select budget={budget}")
    sel, sel_ub = dev.select(budget)
    torch.cuda.synchronize()
    meta64 = meta_to_f64(dev.meta, w.kv_dtype)
    sel_np, ub_np = sel.cpu().numpy(), sel_ub.cpu().numpy()
    G = w.num_q_heads // w.num_kv_heads
    seq_meta = {}
    near = differing = 0
    for b in range(w.batch):
        for h in range(w.num_q_heads):
            g = h // G
            if (b, g) not in seq_meta:
                seq_meta[(b, g)] = check_meta_sequence(inp, meta64, b, g)
            n_near, n_diff = check_selection(inp, b, h, budget, sel_np[b, h], ub_np[b, h],
                                             seq_meta[(b, g)])
            near += n_near
            differing += n_diff
    announce(f"{w.name}: budget {budget}: near-tie pages {near}, differing {differing}")


@pytest.mark.parametrize("name", sorted(CASES))
def test_chunked_selection_every_head(name):
    inp = make_inputs(name)
    dev = Dev(inp)
    dev.build_meta()
    for budget in CASES[name]["budgets"]:
        check_all_heads(inp, budget, dev)


def test_chunked_selection_all_ties_take_lower_pages():
    """q = 0: every page's bound is exactly 0, so each head keeps its first
    min(budget, pages) pages."""
    inp = make_inputs("g4_d128")
    inp["q"][:] = 0.0
    dev = Dev(inp)
    dev.build_meta()
    budget = 64
    announce(f"{inp['workload'].name}: q = 0, select budget={budget}")
    sel, sel_ub = dev.select(budget)
    torch.cuda.synchronize()
    sel_np, ub_np = sel.cpu().numpy(), sel_ub.cpu().numpy()
    pages = (inp["seq_lens"] + PS - 1) // PS
    for b in range(inp["workload"].batch):
        keep = min(budget, int(pages[b]))
        want = list(range(keep)) + [-1] * (budget - keep)
        for h in range(inp["workload"].num_q_heads):
            assert sel_np[b, h].tolist() == want, f"b{b} h{h}"
            assert (ub_np[b, h, :keep] == 0.0).all(), f"b{b} h{h}"
