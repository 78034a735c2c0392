"""Page tables of the oracle: deterministic allocator and slot maps.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The KV cache is paged with 16 tokens per page (the vLLM default quoted in the
CS349D lecture notes, section 4 "Strata").  CacheSlide's SLIDE manager
(CacheSlide page, "Method details", SLIDE implementation paragraph) preallocates
extra pages for layers 2..n sized by the number of tokens selected at layer 1,
registers them in the request's block table and slot mapping, and writes the
selected tokens' K/V there instead of into the reused pages.

Readings taken where the pages are silent:
  * one layer-agnostic pool; a page holds 16 tokens of one layer;
  * allocation is deterministic, lowest free page id first, in call order;
  * compile allocates chunk instance by chunk instance, layer 1..L within each;
  * link allocates request by request, layer 1..L within each, with
      CacheSlide: N_r pages' worth at layer 1 (full recompute), and
                  floor(ratio * N_r) tokens' worth at every later layer
                  (the selection capacity, known before any kernel runs);
                  the CacheBlend-style selection the same with its ratio;
      LegoLink:   |S_r| tokens' worth at every layer;
  * the j-th selected token (ascending token index) of a layer goes to slot
    page[j // 16] * 16 + j % 16 of that layer's new pages.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np


class CapacityError(RuntimeError):
    pass


class PageAllocator:
    """Lowest-free-id-first page allocator over pages 0..n_pages-1."""

    def __init__(self, n_pages: int):
        self.used = np.zeros(int(n_pages), dtype=bool)

    def alloc(self, n: int) -> List[int]:
        free = np.flatnonzero(~self.used)
        if free.shape[0] < n:
            raise CapacityError(f"need {n} pages, {free.shape[0]} free")
        ids = free[:n]
        self.used[ids] = True
        return [int(i) for i in ids]

    def release(self, ids) -> None:
        ids = np.asarray(list(ids), dtype=np.int64)
        if ids.size and not self.used[ids].all():
            raise ValueError("releasing a page that is not allocated")
        self.used[ids] = False


def n_pages_for(n_tokens: int, page_size: int = 16) -> int:
    return (int(n_tokens) + page_size - 1) // page_size


def slot_of(pages: List[int], j, page_size: int = 16):
    """Slot of the j-th token placed into the page list `pages`."""
    j = np.asarray(j, dtype=np.int64)
    return np.asarray(pages, dtype=np.int64)[j // page_size] * page_size + j % page_size


def capacity(workload_mode: str, n_tok: int, ratio: float, lego_rows: int, layer: int) -> int:
    """Tokens' worth of new pages a request gets at 1-based `layer` of the link step."""
    if workload_mode in ("cacheslide", "cacheblend"):
        return n_tok if layer == 1 else int(np.floor(ratio * n_tok))
    if workload_mode == "legolink":
        return lego_rows
    raise ValueError(workload_mode)


def compile_plan(chunks, n_layers: int, alloc: PageAllocator, page_size: int = 16) -> Dict[int, List[List[int]]]:
    """pages[uid][layer-1] for every compiled chunk instance, in compile order."""
    plan = {}
    for c in chunks:
        if c.cached:
            plan[c.uid] = [alloc.alloc(n_pages_for(len(c), page_size)) for _ in range(n_layers)]
    return plan


def reuse_slots(request, plan, layer: int, page_size: int = 16) -> np.ndarray:
    """Slot of each spliced token's compile-step KV at 1-based `layer`: int64 [N];
    -1 for the tokens of an uncached query chunk."""
    out = []
    for c in request.chunks:
        if c.cached:
            out.append(slot_of(plan[c.uid][layer - 1], np.arange(len(c)), page_size))
        else:
            out.append(np.full(len(c), -1, dtype=np.int64))
    return np.concatenate(out)


def slot_map(reuse_slot_l: np.ndarray, selected: np.ndarray, new_pages_l: List[int],
             page_size: int = 16) -> np.ndarray:
    """Layer slot map: new slot for the j-th selected token (ascending), reuse slot otherwise."""
    m = np.array(reuse_slot_l, dtype=np.int64, copy=True)
    sel = np.asarray(selected, dtype=np.int64)
    if sel.size:
        m[sel] = slot_of(new_pages_l, np.arange(sel.size), page_size)
    return m


# ---------------------------------------------------------------- dirty pages (SLIDE)

def dirty_counts(n_pages: int, layer_routes, decode_slots=(), page_size: int = 16) -> np.ndarray:
    """SLIDE's per-page dirty counters after a link step and its decode tokens.

    CacheSlide page, SLIDE paragraphs: from layer 2 on, a page that holds
    selected tokens is dirty, and its counter goes up each time the slot
    mapping routes a selected token to it; decode follows the same policy.
    layer_routes[l-1] = (slot_map of layer l, tokens selected at layer l) for
    l = 1..L; layer 1 is not counted.  decode_slots: every slot a decode
    token's K/V was written to (all layers).  Returns int64 [n_pages].
    """
    counts = np.zeros(int(n_pages), dtype=np.int64)
    for layer, (smap, S) in enumerate(layer_routes, start=1):
        if layer < 2:
            continue
        for i in S:
            counts[int(smap[int(i)]) // page_size] += 1
    for slot in decode_slots:
        counts[int(slot) // page_size] += 1
    return counts


def spill_order(counts, pages) -> List[int]:
    """The order SLIDE evicts `pages` in: clean pages (counter 0) first, then
    dirty pages by counter, largest first.  Ties: lower page id first."""
    pages = sorted(int(p) for p in pages)
    clean = [p for p in pages if counts[p] == 0]
    dirty = [p for p in pages if counts[p] != 0]
    dirty.sort(key=lambda p: (-int(counts[p]), p))
    return clean + dirty
