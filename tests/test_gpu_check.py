"""std_check_idx counts exactly the index-list entries that break the draft
call's preconditions (outside the visual span, or not above the previous
entry of the same head), against a count written from that definition."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_draft_speculative_amd as sd
    sd.load()
    return sd


def count_bad(idx, vis_start, vis_len):
    bad = 0
    for row in idx:
        for j, x in enumerate(row):
            if not (vis_start <= x < vis_start + vis_len) or (j > 0 and x <= row[j - 1]):
                bad += 1
    return bad


def valid_list(rng, hkv, topk, vis_start, vis_len):
    return np.stack([np.sort(rng.choice(vis_len, topk, replace=False)) + vis_start
                     for _ in range(hkv)]).astype(np.int32)


@pytest.mark.parametrize("hkv,topk,vis_start,vis_len", [(4, 4096, 0, 140000), (1, 1, 5, 1),
                                                        (7, 300, 37, 1000), (2, 0, 0, 10)])
def test_check_idx_counts(lib, hkv, topk, vis_start, vis_len):
    rng = np.random.default_rng(hkv * 1000 + topk)
    idx = valid_list(rng, hkv, topk, vis_start, vis_len)
    print(f"check_idx {hkv}x{topk} span [{vis_start}, +{vis_len})", flush=True)
    got = lib.std_check_idx(torch.from_numpy(idx).cuda(), vis_start, vis_len)
    assert int(got.item()) == 0
    if topk == 0:
        return
    bad = idx.copy()
    h = hkv - 1
    bad[h, 0] = vis_start - 1                               # below the span
    bad[h, -1] = vis_start + vis_len                        # past the span
    if topk >= 4:
        bad[0, 2] = bad[0, 1]                               # a repeat
        bad[0, 3] = 2 ** 31 - 1                              # out of span, then a descent
    ref = count_bad(bad.tolist(), vis_start, vis_len)
    assert ref > 0
    got = lib.std_check_idx(torch.from_numpy(bad).cuda(), vis_start, vis_len)
    assert int(got.item()) == ref
