"""Seeded synthetic inputs for paged-KV decode (the only module both the HIP
path's tests and the CPU oracle consume).

It draws q, a paged K/V pool, a block table and sequence lengths, in the
stored dtypes the library takes. It holds none of the decode arithmetic: no
scores, bounds, thresholds or probabilities are computed here. The one use
of q is to aim the planted keys at a query direction, which is part of how
the workload is shaped, not part of the method.

Workload shapes follow the long-context decode settings of the EntmaxKV
summary page (gist.science/it/paper/2605.21649, section 4, efficiency
paragraph): long contexts, paged caches, grouped-query heads. The pages run
RULER / Passkey / PG19 with trained models; those are not available, and
these seeded Gaussian workloads stand in for them.

Layout of what `generate` returns (all numpy, C-contiguous):
  q           float32 [B, H, D]
  k_pool      uint16 (bf16 bit patterns) or float32 [P_phys, H_kv, ps, D]
  v_pool      same as k_pool
  block_table int32 [B, max_pages]   (-1 beyond a sequence's last page)
  seq_lens    int32 [B]
Rows of a sequence's last page beyond its length hold the value 30.0, so any
kernel that wrongly reads them produces visibly wrong results.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

TAIL_FILL = 30.0


@dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic decode batch."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    context: int  # tokens per sequence unless seq_lens overrides
    kv_dtype: str  # "bf16" or "f32"
    alphas: tuple
    budgets: tuple  # page budgets
    q_scale: float
    plant: str = "none"  # "none" | "query" (single head) | "group_mean"
    n_planted: int = 0  # planted keys per (sequence, KV head)
    run_len: int = 1  # planted keys come in contiguous runs of this length
    plant_magnitude: float = 3.0
    plant_noise: float = 0.1
    block_table: str = "permuted"  # or "contiguous"
    seq_lens: tuple | None = None  # ragged lengths, one per sequence

    def lengths(self) -> np.ndarray:
        if self.seq_lens is not None:
            assert len(self.seq_lens) == self.batch
            return np.asarray(self.seq_lens, dtype=np.int32)
        return np.full(self.batch, self.context, dtype=np.int32)

    def pages_per_seq(self) -> np.ndarray:
        return (self.lengths() + self.page_size - 1) // self.page_size

    def max_pages(self) -> int:
        return max(1, int(self.pages_per_seq().max()))

    def num_phys_pages(self) -> int:
        return max(1, int(self.pages_per_seq().sum()))


_S128 = 1.0 / math.sqrt(128.0)

# The decode workloads. Names say what they are.
WORKLOADS = {
    # Single head, fp32 cache, 4K tokens; small enough for a pure-CPU check.
    "tiny_4k_f32": Workload(
        "tiny_4k_f32", 1, 1, 1, 64, 16, 4096, "f32", (1.5,), (32,), 4.0 / 8.0,
        plant="query", n_planted=8, block_table="contiguous"),
    # Grouped-query decode at 32K.
    "gqa_32k": Workload(
        "gqa_32k", 8, 32, 8, 128, 16, 32768, "bf16", (1.5,), (256,), 4.0 * _S128,
        plant="group_mean", n_planted=64),
    # Long-context decode at 128K, 2% page budget (82 of 4096 pages).
    "long_128k": Workload(
        "long_128k", 4, 32, 8, 128, 32, 131072, "bf16", (1.5,), (82,), 4.0 * _S128,
        plant="group_mean", n_planted=128, run_len=8),
    # alpha / budget sweep at 64K without planted keys.
    "alpha_sweep_64k": Workload(
        "alpha_sweep_64k", 16, 32, 8, 128, 16, 65536, "bf16", (1.25, 1.5, 2.0),
        (64, 256, 1024), 2.0 * _S128),
    # One sequence of 512K tokens, 64-token pages.
    "extreme_512k": Workload(
        "extreme_512k", 1, 32, 8, 128, 64, 524288, "bf16", (1.5,), (64,), 4.0 * _S128,
        plant="group_mean", n_planted=256),
    # The same recipe at 1,048,576 tokens (16384 pages of 64 tokens), the
    # longest context the EntmaxKV page measures.
    "extreme_1m": Workload(
        "extreme_1m", 1, 32, 8, 128, 64, 1048576, "bf16", (1.5,), (64,), 4.0 * _S128,
        plant="group_mean", n_planted=256),
    # Extra, not one of the sizing workloads above: long_128k with planted runs
    # of magnitude 32 instead of 3, so a planted key's coordinates (about 2.8
    # each) leave the random keys' per-page range and its score (about 64)
    # tops the random maximum (about 17): the peaked attention regime of a
    # trained model, where the entmax support sits in a few pages the box
    # bound can find. Used by the discarded-mass report.
    "long_128k_peaked": Workload(
        "long_128k_peaked", 4, 32, 8, 128, 32, 131072, "bf16", (1.5,), (82,), 4.0 * _S128,
        plant="group_mean", n_planted=128, run_len=8, plant_magnitude=32.0),
}

# Seeds: each workload has a fixed seed so every run sees the same data.
WORKLOAD_SEEDS = {"tiny_4k_f32": 1, "gqa_32k": 2, "long_128k": 3,
                  "alpha_sweep_64k": 4, "extreme_512k": 5, "extreme_1m": 6,
                  "long_128k_peaked": 7}


def shrink(w: Workload, context: int | None = None, batch: int | None = None,
           seq_lens: tuple | None = None, n_planted: int | None = None,
           name: str | None = None) -> Workload:
    """Same recipe at a smaller size (for parity runs the oracle finishes quickly)."""
    kw = {}
    if context is not None:
        kw["context"] = context
    if batch is not None:
        kw["batch"] = batch
    if seq_lens is not None:
        kw["seq_lens"] = tuple(int(x) for x in seq_lens)
        kw["batch"] = len(seq_lens)
    if n_planted is not None:
        kw["n_planted"] = n_planted
    kw["name"] = name or (w.name + "_small")
    return replace(w, **kw)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16, returned as uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x32: np.ndarray, kv_dtype: str) -> np.ndarray:
    if kv_dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if kv_dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    raise ValueError(kv_dtype)


def _planted_positions(rng: np.random.Generator, length: int, n: int, run_len: int) -> np.ndarray:
    """Token positions of the planted keys: n/run_len non-overlapping runs."""
    if n <= 0 or length <= 0:
        return np.zeros(0, dtype=np.int64)
    if run_len <= 1:
        return np.sort(rng.choice(length, size=min(n, length), replace=False))
    n_runs = n // run_len
    starts: list[int] = []
    taken = np.zeros(length, dtype=bool)
    tries = 0
    while len(starts) < n_runs:
        tries += 1
        if tries > 100000:
            raise RuntimeError("could not place planted runs")
        s = int(rng.integers(0, length - run_len + 1))
        if taken[s:s + run_len].any():
            continue
        taken[s:s + run_len] = True
        starts.append(s)
    pos = np.concatenate([np.arange(s, s + run_len) for s in sorted(starts)])
    return pos.astype(np.int64)


def generate(w: Workload, seed: int, threads: int | None = None) -> dict:
    """Draw one batch of the workload `w` from `seed` (deterministic)."""
    B, H, Hkv, D, ps = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size
    assert H % Hkv == 0
    G = H // Hkv
    lens = w.lengths()
    pages = w.pages_per_seq()
    max_pages = w.max_pages()
    n_phys = w.num_phys_pages()

    root = np.random.SeedSequence(seed)
    q_ss, perm_ss, k_ss, v_ss, pl_ss = root.spawn(5)
    k_kids = k_ss.spawn(B * Hkv)
    v_kids = v_ss.spawn(B * Hkv)
    pl_kids = pl_ss.spawn(B * Hkv)

    q = (np.random.Generator(np.random.PCG64(q_ss)).standard_normal((B, H, D))
         * w.q_scale).astype(np.float32)

    if w.block_table == "contiguous":
        phys = np.arange(n_phys, dtype=np.int64)
    else:
        phys = np.random.Generator(np.random.PCG64(perm_ss)).permutation(n_phys)
    block_table = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        block_table[b, :pages[b]] = phys[off:off + pages[b]]
        off += int(pages[b])

    store_dt = np.uint16 if w.kv_dtype == "bf16" else np.float32
    fill = _store(np.full(1, TAIL_FILL, np.float32), w.kv_dtype)[0]
    k_pool = np.full((n_phys, Hkv, ps, D), fill, dtype=store_dt)
    v_pool = np.full((n_phys, Hkv, ps, D), fill, dtype=store_dt)
    planted = {}

    def one_block(idx: int):
        b, g = divmod(idx, Hkv)
        L = int(lens[b])
        if L == 0:
            return idx, None
        kb = np.random.Generator(np.random.PCG64(k_kids[idx])).standard_normal(
            (L, D), dtype=np.float32)
        vb = np.random.Generator(np.random.PCG64(v_kids[idx])).standard_normal(
            (L, D), dtype=np.float32)
        pos = np.zeros(0, dtype=np.int64)
        if w.plant != "none" and w.n_planted > 0:
            prng = np.random.Generator(np.random.PCG64(pl_kids[idx]))
            pos = _planted_positions(prng, L, w.n_planted, w.run_len)
            if w.plant == "query":
                u = q[b, g * G].astype(np.float64)
            elif w.plant == "group_mean":
                u = q[b, g * G:(g + 1) * G].astype(np.float64).mean(axis=0)
            else:
                raise ValueError(w.plant)
            u = u / np.linalg.norm(u)
            noise = prng.standard_normal((len(pos), D))
            kb[pos] = (w.plant_magnitude * u[None, :] + w.plant_noise * noise).astype(np.float32)
        P = int(pages[b])
        pad = P * ps - L
        ks = _store(kb, w.kv_dtype)
        vs = _store(vb, w.kv_dtype)
        if pad:
            ks = np.concatenate([ks, np.full((pad, D), fill, dtype=store_dt)])
            vs = np.concatenate([vs, np.full((pad, D), fill, dtype=store_dt)])
        rows = block_table[b, :P]
        k_pool[rows, g] = ks.reshape(P, ps, D)
        v_pool[rows, g] = vs.reshape(P, ps, D)
        return idx, pos

    n_threads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=n_threads) as ex:
        for idx, pos in ex.map(one_block, range(B * Hkv)):
            if pos is not None and len(pos):
                planted[divmod(idx, Hkv)] = pos

    return {
        "workload": w,
        "seed": seed,
        "q": q,
        "k_pool": k_pool,
        "v_pool": v_pool,
        "block_table": block_table,
        "seq_lens": lens.copy(),
        "planted": planted,
        "num_phys_pages": n_phys,
        "max_pages": max_pages,
    }


def constructed_selection(pages_needed, n_pages: int, budget: int, seed: int) -> list:
    """A page selection that contains `pages_needed`, filled up to `budget` with
    other random pages, ascending, padded with -1 (used to exercise the
    support-recovery case with a selection known to hold the support)."""
    need = sorted(set(int(j) for j in pages_needed))
    if len(need) > budget:
        raise ValueError("budget smaller than required page set")
    rng = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(n_pages), np.asarray(need, dtype=np.int64))
    extra = rng.choice(rest, size=min(len(rest), budget - len(need)), replace=False) if len(rest) else []
    sel = sorted(need + [int(x) for x in extra])
    return sel + [-1] * (budget - len(sel))
