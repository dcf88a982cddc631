"""Host-side capacity planning: vt_plan_patches (the analogue of the pages'
derive_max_patches, "init.rs (VisionEncoder::new)") and vt_pack_items.
No GPU: both are host functions of the library; their answers are checked
against the workspace sizes the library asks for, by invariants."""
import numpy as np
import pytest

import synth
import vision_transformer_encoder_tiled_amd as vt

TB = 1 << 40


def test_area_bound_gives_area_over_patch_squared():
    cfg = vt.config()
    # "patches = area / patch^2": 448^2 -> 32 x 32, 2016^2 -> 144 x 144 (ample budget: no clamp)
    assert vt.vt_plan_patches(cfg, TB, 1, 448 * 448) == (1024, 0)
    assert vt.vt_plan_patches(cfg, TB, 1, 2016 * 2016) == (20736, 0)
    assert vt.vt_plan_patches(cfg, TB, 1, 1) == (1, 0)  # at least one patch
    p, w = vt.vt_plan_patches(cfg, TB, 1, 0)          # no area bound: the budget decides
    assert w == 0 and p % 4 == 0 and p > 10 ** 6


def test_budget_clamps_and_reports_the_request():
    cfg = vt.config()
    budget = vt.vt_tower_workspace_size(cfg, [(1, 144, 144)])  # what 2016^2 needs
    p, w = vt.vt_plan_patches(cfg, budget, 1, 4096 * 4096)
    assert w == 4096 * 4096 // 196 and 0.8 * 20736 < p <= 20736 and p % 4 == 0
    # the granted count fits for the least favourable grid shape of that many tokens
    for grid in ([(1, 2, p // 2)], [(1, 2 * int(np.sqrt(p / 4)), 2 * int(np.sqrt(p / 4)))], [(p // 4, 2, 2)]):
        assert vt.vt_tower_workspace_size(cfg, grid) <= budget
    # more budget never grants fewer patches
    p2, _ = vt.vt_plan_patches(cfg, 2 * budget, 1, 0)
    p1, _ = vt.vt_plan_patches(cfg, budget, 1, 0)
    assert p1 <= p2
    # the planner's bound is conservative, but by at most the split-K bound (64 MiB) of the
    # block and of the projector buffers plus a RoPE table for every position
    assert vt.vt_tower_workspace_size(cfg, [(1, 2, (p1 + 4) // 2)]) > budget - 2 * (64 << 20) - 40 * 8 * (p1 + 4)


def test_budget_too_small_is_an_error():
    cfg = vt.config()
    with pytest.raises(vt.VtError) as e:
        vt.vt_plan_patches(cfg, 1 << 20, 1, 448 * 448)
    assert e.value.status == vt.VT_ERR_WORKSPACE


def test_pack_items_in_order_and_maximal():
    cfg = vt.config()
    grids = list(synth.WORKLOADS["tower_mixed8"].grids) + [(1, 32, 32)] * 5 + [(3, 16, 16)]
    budget = vt.vt_tower_workspace_size(cfg, grids[:3])
    batch, nb = vt.vt_pack_items(cfg, grids, budget)
    assert batch[0] == 0 and batch[-1] == nb - 1
    assert all(b1 - b0 in (0, 1) for b0, b1 in zip(batch, batch[1:]))
    for b in range(nb):
        items = [g for g, k in zip(grids, batch) if k == b]
        assert vt.vt_tower_workspace_size(cfg, items) <= budget
        last = max(i for i, k in enumerate(batch) if k == b)
        if last + 1 < len(grids):  # maximal: the next item would not fit
            assert vt.vt_tower_workspace_size(cfg, items + [grids[last + 1]]) > budget
    # one call for everything when the budget allows it
    assert vt.vt_pack_items(cfg, grids, vt.vt_tower_workspace_size(cfg, grids)) == ([0] * len(grids), 1)


def test_pack_items_refuses_an_item_that_cannot_fit():
    cfg = vt.config()
    grids = [(1, 16, 16), (1, 144, 144)]
    budget = vt.vt_tower_workspace_size(cfg, grids[:1])
    with pytest.raises(vt.VtError) as e:
        vt.vt_pack_items(cfg, grids, budget)
    assert e.value.status == vt.VT_ERR_WORKSPACE and "item 1" in str(e.value)
