"""moe_permute_noalloc (static scratch, no allocation in the call) against
moe_permute (caller workspace), through the C ABI: two calls in a row, the
second smaller, each bit for bit equal to the workspace path and to the
oracle; sizes past the static scratch are rejected without enqueuing."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synthetic import bf16_bits, generate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_grouped_router_amd as mod
    mod.load_library()
    return mod


def _outputs(T, H, E, k, precision, with_w):
    rows = T * k
    dev = "cuda"
    out = {
        "row_map": torch.empty(rows, dtype=torch.int32, device=dev),
        "src_row": torch.empty(rows, dtype=torch.int32, device=dev),
        "split_sizes": torch.empty(E, dtype=torch.int32, device=dev),
        "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
    }
    if precision == 0:
        out["x_perm"] = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    else:
        out["x_perm"] = torch.empty((rows, H), dtype=torch.uint8, device=dev)
        out["x_perm_scale"] = torch.empty((rows, H // 32), dtype=torch.uint8,
                                          device=dev)
    if with_w:
        out["w_perm"] = torch.empty(rows, dtype=torch.float32, device=dev)
    return out


def _check_equal(a, b, keys):
    for key in keys:
        x, y = a[key], b[key]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), key


@pytest.mark.parametrize("precision", [0, 1])
def test_permute_noalloc_equals_workspace_path(m, precision):
    # the first call larger than the second: the second must not see the
    # first call's histograms (the array keeps the last call's contents)
    for (T, H, E, k, zipf, seed) in [(20000, 256, 128, 8, 1.2, 1),
                                     (3000, 128, 64, 4, 0.0, 2)]:
        d = generate(T, H, 64, E, k, zipf=zipf, seed=seed,
                     want=("x", "logits"))
        x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).cuda()
        idx, w = m.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), k)
        ref = m.moe_permute(x, idx, E, topk_w=w, precision=precision)
        out = _outputs(T, H, E, k, precision, True)
        got = m.moe_permute_noalloc(x, idx, w, out, precision=precision)
        torch.cuda.synchronize()
        keys = ["x_perm", "row_map", "src_row", "split_sizes", "offsets",
                "w_perm"] + (["x_perm_scale"] if precision else [])
        _check_equal(got, ref, keys)
        want = O.permute_index(idx.cpu().numpy(), E)
        for key in ("split_sizes", "offsets", "row_map", "src_row"):
            np.testing.assert_array_equal(got[key].cpu().numpy(), want[key])


def test_permute_noalloc_rejects_sizes_past_scratch(m):
    # ceil(T*k / 1024) * E * 4 bytes > 4 MiB: E = 1024, T*k = 1025 * 1024
    E, k = 1024, 8
    T = 1025 * 1024 // k
    x = torch.zeros((T, 8), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    out = _outputs(T, 8, E, k, 0, False)
    out["offsets"].fill_(-7)
    torch.cuda.synchronize()
    with pytest.raises(m.MoEError) as ei:
        m.moe_permute_noalloc(x, idx, None, out)
    assert ei.value.status == 2 and "static array" in str(ei.value)
    torch.cuda.synchronize()
    assert int(out["offsets"][0].item()) == -7    # nothing was enqueued
