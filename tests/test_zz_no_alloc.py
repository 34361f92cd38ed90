"""The allocation-free permute (scratch in the library's fixed device array) against
moe_permute with a caller workspace: bit-exact counts, offsets, restoration map and
packed rows, on two calls in a row, the second with a smaller input, so the second call
runs on scratch the first one left behind."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _routes(rng, T, N, K):
    """K distinct experts per token, skewed toward low indices (so capacity drops)."""
    w = 1.0 / np.arange(1, N + 1) ** 1.1
    keys = np.log(w)[None, :] - np.log(-np.log(rng.random((T, N))))   # Gumbel top-K
    return np.argsort(-keys, axis=1, kind="stable")[:, :K].astype(np.int32)


CASES = [  # T, d_model, N, K, capacity, capacity_group, dtype
    (4096, 2048, 64, 4, 256, 0, torch.bfloat16),
    (700, 256, 16, 3, -1, 0, torch.float32),
]


def test_noalloc_permute_matches_workspace_permute_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_gemm_amd import moe
    rng = np.random.default_rng(11)
    for (T, d, N, K, cap, grp, dt) in CASES:
        print(f"noalloc permute T={T} d={d} N={N} K={K} capacity={cap}", flush=True)
        x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(dt).cuda()
        idx = torch.from_numpy(_routes(rng, T, N, K)).cuda()
        ref = moe.moe_permute(x, idx, N, cap, copy_rows=True, capacity_group=grp)
        got = moe.moe_permute_noalloc(x, idx, N, cap, copy_rows=True, capacity_group=grp)
        torch.cuda.synchronize()
        for k in ("C_req", "C_keep", "offsets", "dest_row"):
            assert torch.equal(got[k], ref[k]), k
        R = int(ref["offsets"][-1].item())
        assert R > 0
        assert torch.equal(got["row_token"][:R], ref["row_token"][:R])
        iv = torch.int16 if dt == torch.bfloat16 else torch.int32
        assert torch.equal(got["x_perm"][:R].view(iv), ref["x_perm"][:R].view(iv))
        if cap >= 0:
            assert int(ref["C_keep"].max().item()) == cap   # the skew forces drops
