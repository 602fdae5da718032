"""Oracle: the host-side dispatch contract of the routed fused-MoE kernel.

TEST INFRASTRUCTURE ONLY -- imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

Source: tutorial page "moe_dispatch_contract.py" (chapter 18, MoE inference
dispatch/combine contract), function ``build_contract`` steps 1-4 and the
three self-checks ``check_coverage``, ``check_padded_covers_compact`` and
``check_kernel_addressing``; the kernel side of the contract is the kernel
signature and the Step-1/Step-2 row predicate in "Fused MoE GEMM 提交说明",
section 完整算子代码, plus the section 实现要点 (padded vs compact indexing).

Plain Python lists, loops and standard-library primitives (a bucket sort,
prefix sums, a bisection) on purpose: this is the definition, not a fast
implementation.

Readings of points the pages leave open:
  * group_offsets / group_padded_offsets carry E+1 entries, the last being the
    total (the kernel signature declares num_experts+1 entries; the tutorial
    script builds only E).  The kernel reads entries [0, E) only.
  * Ties inside an expert group keep ascending pair index p = t*k + j (the
    tutorial sorts with Python's stable ``sorted``), which makes every table
    unique.
  * The padding block size is 128 and equals the kernel's block_token.
"""
from __future__ import annotations

import bisect
import collections
import itertools

BLOCK = 128  # block_token == padding_M in both pages


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def build_contract(topk_ids, n_experts: int, block: int = BLOCK) -> dict:
    """Group tables for a routing ``topk_ids`` (T rows of k expert ids).

    What the tutorial's ``build_contract`` defines, step by step:
      1. the routed pairs are the (token, slot) entries in token-major then
         slot order, pair p = t*k + j;
      2. the pairs sorted by expert, ties in ascending p -> ``order``; the
         expert group sizes; their exclusive prefix sums -> ``group_offsets``
         (where each expert's rows start in compact order);
      3. each expert occupies ceil((count + 1) / block) * block padded rows
         (the "+1" leaves one slack row), their prefix sums ->
         ``group_padded_offsets``;
      4. ``m_blocks = ceil(pairs / block) + E`` blocks, block bx belonging to
         the last expert whose padded start is <= bx * block.
    Packing (where each pair lands) follows section 实现要点 of the
    submission notes: tokens use padded row indices, routed weights use
    compact indices ``group_offsets[e] + token_offset``.
    """
    E = int(n_experts)
    if E < 1:
        raise ValueError("need at least one expert")
    # 1) the routed pairs, p = t*k + j
    pair_list = [(t, int(e)) for t, row in enumerate(topk_ids) for e in row]
    for _, e in pair_list:
        if not 0 <= e < E:
            raise ValueError(f"expert id {e} out of range [0, {E})")
    flat_token = [t for t, _ in pair_list]
    flat_expert = [e for _, e in pair_list]
    pairs = len(pair_list)

    # 2) counting sort: one bucket per expert, filled in ascending p (stable)
    buckets: list[list[int]] = [[] for _ in range(E)]
    for p, e in enumerate(flat_expert):
        buckets[e].append(p)
    order = [p for bucket in buckets for p in bucket]
    counts = [len(bucket) for bucket in buckets]
    group_offsets = list(itertools.accumulate(counts, initial=0))        # E+1 entries

    # 3) padded spans and their prefix sums (E+1 entries)
    spans = [ceil_div(c + 1, block) * block for c in counts]
    group_padded_offsets = list(itertools.accumulate(spans, initial=0))

    # 4) blocks: the padded starts are strictly increasing, so "the last
    #    expert whose start is <= bx*block" is a right bisection
    m_blocks = ceil_div(pairs, block) + E
    starts = group_padded_offsets[:E]
    group_idx_for_bx = [bisect.bisect_right(starts, bx * block) - 1 for bx in range(m_blocks)]

    # packing maps: the r-th pair of expert e (in sorted order)
    padded_row_of_pair = [0] * pairs
    compact_pos_of_pair = [0] * pairs
    for e, bucket in enumerate(buckets):
        for r, p in enumerate(bucket):
            padded_row_of_pair[p] = group_padded_offsets[e] + r
            compact_pos_of_pair[p] = group_offsets[e] + r

    return {
        "n_experts": E,
        "block": block,
        "pairs": pairs,
        "flat_expert": flat_expert,
        "flat_token": flat_token,
        "order": order,
        "group_sizes": counts,
        "group_offsets": group_offsets,
        "group_padded_offsets": group_padded_offsets,
        "num_blocks_m": m_blocks,
        "group_idx_for_bx": group_idx_for_bx,
        "padded_row_of_pair": padded_row_of_pair,
        "compact_pos_of_pair": compact_pos_of_pair,
        "total_padded_tokens": m_blocks * block,
    }


def block_rows(c: dict, bx: int) -> tuple[int, int, int]:
    """(expert, token_offset, actual_rows) of block bx -- the kernel's row
    predicate from both Step-1 and Step-2 grids (section 完整算子代码):
    actual_rows = max(0, min(block, group_size - (bx*block - padded_start)))."""
    e = c["group_idx_for_bx"][bx]
    token_offset = bx * c["block"] - c["group_padded_offsets"][e]
    rows = max(0, min(c["block"], c["group_sizes"][e] - token_offset))
    return e, token_offset, rows


def valid_rows(c: dict):
    """Yield (padded_row, expert, compact_index) for every row the kernel
    computes, block by block, using only the kernel-side addressing."""
    for bx in range(c["num_blocks_m"]):
        e, off, rows = block_rows(c, bx)
        for i in range(rows):
            yield bx * c["block"] + i, e, c["group_offsets"][e] + off + i


# ---------------------------------------------------------------- invariants
def check_coverage(c: dict) -> None:
    """Every (token, expert) pair appears exactly once (tutorial check 1),
    and ``order`` is a permutation of the pairs."""
    tally = collections.Counter((c["flat_token"][p], c["flat_expert"][p]) for p in c["order"])
    assert all(n == 1 for n in tally.values()), "a (token, expert) pair appears twice"
    assert sum(tally.values()) == sum(c["group_sizes"]) == c["pairs"]
    assert collections.Counter(c["order"]) == collections.Counter(range(c["pairs"])), \
        "order is not a permutation"


def check_padded_covers_compact(c: dict) -> None:
    """Each expert's padded interval holds its whole compact interval plus at
    least one slack row, intervals are block-aligned, disjoint and in order,
    and all of them fit inside num_blocks_m blocks (tutorial check 2, in the
    strict form: the page's literal inequality is implied by these)."""
    B, E = c["block"], c["n_experts"]
    go, gpo, gs = c["group_offsets"], c["group_padded_offsets"], c["group_sizes"]
    assert go[0] == 0 and gpo[0] == 0
    for e in range(E):
        assert go[e + 1] - go[e] == gs[e]
        assert gpo[e] % B == 0
        assert gpo[e + 1] - gpo[e] >= gs[e] + 1
        assert gpo[e + 1] - gpo[e] == (gs[e] // B + 1) * B
    assert go[E] == c["pairs"]
    assert gpo[E] <= c["num_blocks_m"] * B <= c["total_padded_tokens"]


def check_kernel_addressing(c: dict) -> None:
    """Kernel addressing stays inside each group (tutorial check 3): the
    compact row ``padded - group_padded_offsets[g] + group_offsets[g]`` of
    every computed row lies in expert g's compact interval, and the map from
    computed padded rows to compact rows is a bijection onto [0, pairs)."""
    go, gs = c["group_offsets"], c["group_sizes"]
    hit = [0] * c["pairs"]
    for r, e, ci in valid_rows(c):
        assert go[e] <= ci < go[e] + gs[e]
        assert ci == r - c["group_padded_offsets"][e] + go[e]
        hit[ci] += 1
    assert all(h == 1 for h in hit), "compact rows not covered exactly once"
    # packing maps agree with the kernel addressing
    for p in range(c["pairs"]):
        e = c["flat_expert"][p]
        r = c["padded_row_of_pair"][p]
        assert c["group_idx_for_bx"][r // c["block"]] == e
        assert c["compact_pos_of_pair"][p] == r - c["group_padded_offsets"][e] + go[e]


def check_all(c: dict) -> None:
    check_coverage(c)
    check_padded_covers_compact(c)
    check_kernel_addressing(c)


# ------------------------------------------------------------------ packing
def pack_rows(c: dict, x_rows, topk_w_flat, pad_row):
    """Expert-sorted padded token matrix and compact routed weights.

    ``x_rows`` is a list-like of T token rows, ``topk_w_flat`` the routed
    weight of each pair p = t*k + j.  Returns (stacked, w_compact) where
    stacked[padded_row_of_pair[p]] = x_rows[flat_token[p]] and every other
    row is ``pad_row``; w_compact[compact_pos_of_pair[p]] = topk_w_flat[p].
    """
    stacked = [pad_row] * c["total_padded_tokens"]
    w_compact = [0.0] * c["pairs"]
    for p in range(c["pairs"]):
        stacked[c["padded_row_of_pair"][p]] = x_rows[c["flat_token"][p]]
        w_compact[c["compact_pos_of_pair"][p]] = topk_w_flat[p]
    return stacked, w_compact
