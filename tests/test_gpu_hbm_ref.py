"""The HBM reference streams (measurement aids the bench compares the
permute's gather and the combine with): their outputs are what the header
states, for every traffic mix, with a length that leaves a partial trip."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_grouped_router_amd as mod
    mod.load_library()   # raises if the HIP library is missing
    return mod


NBYTES = 16 * 5003   # not a whole number of 16 KiB block trips


def _src(seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, size=2 * NBYTES, dtype=np.uint8)


@pytest.mark.parametrize("r,w", [(1, 0), (0, 1), (1, 1), (1, 2), (2, 1),
                                 (2, 2), (0, 2)])
def test_hbm_stream_mix_outputs(m, r, w):
    src = _src(11 + 3 * r + w)
    d_src = torch.from_numpy(src).cuda()
    d_dst = torch.zeros(2 * NBYTES, dtype=torch.uint8, device="cuda")
    ctx = m._context(torch.device("cuda"))
    st = torch.cuda.current_stream().cuda_stream
    m._check(m.load_library().moe_hbm_stream_mix(
        ctx, d_src.data_ptr(), NBYTES, r, w, d_dst.data_ptr(), st))
    torch.cuda.synchronize()
    got = d_dst.cpu().numpy()
    if r == 0:
        want = np.frombuffer(np.full(NBYTES // 4, 1.0, np.float32).tobytes(),
                             np.uint8)
    else:
        want = src[:NBYTES].copy()
        if r == 2:
            want ^= src[NBYTES:]
    for j in range(2):
        part = got[j * NBYTES:(j + 1) * NBYTES]
        if j < w:
            np.testing.assert_array_equal(part, want)
        else:
            assert not part.any(), f"copy {j} written"


def test_hbm_stream_reference_copies(m):
    src = _src(5)[:NBYTES]
    d_src = torch.from_numpy(src).cuda()
    d_dst = torch.zeros(3 * NBYTES, dtype=torch.uint8, device="cuda")
    ctx = m._context(torch.device("cuda"))
    st = torch.cuda.current_stream().cuda_stream
    m._check(m.load_library().moe_hbm_stream_reference(
        ctx, d_src.data_ptr(), NBYTES, 3, d_dst.data_ptr(), st))
    torch.cuda.synchronize()
    got = d_dst.cpu().numpy().reshape(3, NBYTES)
    for j in range(3):
        np.testing.assert_array_equal(got[j], src)
