"""Reused KV in a host tier (pinned memory), loaded layer by layer during the link step.

The link step with the compile pages in host memory (their device copies
zeroed, so the step can only see what it loads) must give bitwise the same
result as the step with the pages resident in HBM: hidden state, deviation,
alpha, selected rows and every new page.  Overlapped loads (copy stream ahead
of the recompute) and serial loads (copy, then layer) both; CacheSlide and
LegoLink; two steps in a row.
"""
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402
from selective_kv_cache_amd.link import LinkConfig, LinkEngine, Model  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def engine(w, mode, tier, overlap=True):
    s = w.shape
    E = wl.embedding_table(w, DEV)
    layers = [wl.layer_weights(w, l, DEV) for l in range(1, s.n_layers + 1)]
    cfg = LinkConfig(mode=mode, ratio=w.ratio, tau=w.tau, period=w.period, lego_k=w.lego_k, reuse_tier=tier,
                     tier_overlap=overlap)
    return LinkEngine(Model(s, E, layers), w.requests, cfg, device=DEV)


def outputs(eng):
    torch.cuda.synchronize()
    n = eng.n_compile_pages
    out = dict(hidden=eng.hidden.clone(), d=eng.d.clone(), alpha=eng.alpha.clone(),
               k_new=eng.k_pool[n:].clone(), v_new=eng.v_pool[n:].clone())
    if eng.cfg.mode == "cacheslide":
        out["sel"] = [x.copy() for x in eng.selected()]
    return out


@pytest.mark.parametrize("mode", ["cacheslide", "legolink"])
@pytest.mark.parametrize("overlap", [True, False])
def test_host_tier_matches_resident(mode, overlap):
    w = wl.small_bf16(n_layers=8, mode=mode)
    ref_eng = engine(w, mode, "hbm")
    ref_eng.run_compile()
    ref_eng.run_link()
    ref = outputs(ref_eng)
    ref_eng.close()

    eng = engine(w, mode, "host", overlap)
    eng.run_compile()
    eng.stage_reuse_to_host(evict=True)
    assert int(torch.count_nonzero(eng.k_pool[: eng.n_compile_pages])) == 0
    for step in range(2):
        eng.run_link()
        got = outputs(eng)
        for key in ("hidden", "d", "alpha", "k_new", "v_new"):
            assert torch.equal(got[key], ref[key]), (step, key)
        if mode == "cacheslide":
            assert all(np.array_equal(a, b) for a, b in zip(got["sel"], ref["sel"]))
    eng.close()


def test_host_tier_needs_staging():
    w = wl.small_bf16(n_layers=2)
    eng = engine(w, "cacheslide", "host")
    eng.run_compile()
    with pytest.raises(RuntimeError):
        eng.run_link()
    eng.close()
