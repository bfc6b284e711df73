"""The allocation-free importance mask (gs_active_mask_static) against the
workspace entry point (gs_active_mask), through the C ABI: bit-identical
masks on consecutive calls that share the library's fixed scratch array, the
second call smaller than the first (so nothing left in the array from the
first call may leak into the second), plus the oracle's full sort as a
third opinion."""

import numpy as np
import pytest
import torch

import oracle
from gaussian_splatting_tile_amd import binding as B
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _both(scores: np.ndarray, keep: int):
    n = scores.shape[0]
    s = torch.from_numpy(scores).cuda()
    pad = 64
    m_ws = torch.full((n + pad,), 7, dtype=torch.uint8, device="cuda")
    m_st = torch.full((n + pad,), 9, dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(B.active_mask_workspace_bytes(n), 1), dtype=torch.uint8, device="cuda")
    B.active_mask(s, n, keep, m_ws[:n], ws)
    B.active_mask_static(s, n, keep, m_st[:n])
    torch.cuda.synchronize()
    a, b = m_ws.cpu().numpy(), m_st.cpu().numpy()
    assert np.all(a[n:] == 7) and np.all(b[n:] == 9), "write past the mask"
    return a[:n], b[:n]


@pytest.mark.parametrize("first,second", [(3_000_017, 70_001), (1_048_576, 4_097)])
def test_static_mask_equals_workspace_mask_on_consecutive_calls(first, second):
    rng = np.random.default_rng(first)
    for n, kind in ((first, "exp"), (second, "ties")):
        if kind == "exp":
            s = rng.exponential(1.0, n).astype(np.float32)
        else:
            s = rng.integers(0, 7, n).astype(np.float32)       # heavy ties: the tie ranks use the scratch
        keep = (3 * n) // 10
        say(f"[gpu] static mask n={n} keep={keep} ({kind})")
        ref = oracle.topk_mask(s, keep)
        a, b = _both(s, keep)
        assert np.array_equal(a, ref)
        assert np.array_equal(b, a), f"static mask differs at {np.nonzero(b != a)[0][:5]}"
        assert int(b.sum()) == keep


def test_static_mask_degenerate_sizes():
    rng = np.random.default_rng(3)
    for n in (1, 5, 4096, 4097):
        s = rng.exponential(1.0, n).astype(np.float32)
        for keep in (0, 1, n // 2, n):
            a, b = _both(s, keep)
            assert np.array_equal(a, b) and int(b.sum()) == keep
    B.active_mask_static(None, 0, 0, None)             # n = 0: nothing to do
    torch.cuda.synchronize()
