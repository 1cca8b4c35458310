"""The allocation-free forward (mra_attention_fwd_noalloc, through the C
ABI) against mra_attention_fwd with a caller workspace: the same kernels on
the library's fixed scratch, so the outputs must be bit-identical.  Two
calls in a row on one GPU, the second with smaller inputs (the scratch then
still holds the first call's contents), in both modes."""
import ctypes

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mra():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_approximate_amd as m
    m.lib()
    return m


def dev(w, name):
    return torch.from_numpy(w.raw(name).view(np.int16)).view(torch.bfloat16).cuda()


def case(mra, w):
    q, k, v = dev(w, "q"), dev(w, "k"), dev(w, "v")
    mask = None if w.mask is None else torch.from_numpy(w.mask).cuda()
    kw = dict(block_per_row=w.block_per_row, approx_mode=w.approx_mode,
              initial_prior_first_n_blocks=w.prior_first, initial_prior_diagonal_n_blocks=w.prior_diag)
    ref = mra.attention(q, k, v, mask, **kw)
    got = mra.attention_noalloc(q, k, v, mask, **kw)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), w.name
    return got


@pytest.mark.parametrize("mode", ["full", "sparse"])
def test_noalloc_matches_workspace_forward_twice(mra, mode):
    big = workloads.get("C4") if mode == "full" else workloads.get("C3")
    print("case", big.name, flush=True)
    case(mra, big)
    mask = np.zeros((2, 1024), np.uint8)
    mask[0, :700] = 1
    mask[1, :1024] = 1
    small = workloads.iid("noalloc-small-" + mode, 2, 3, 1024, dtype="bf16", seed=5, scale=0.7, mask=mask,
                          block_per_row=3, approx_mode=mode, prior_first=1, prior_diag=2)
    print("case", small.name, flush=True)
    case(mra, small)


def test_noalloc_rejects_sizes_beyond_its_scratch(mra):
    # N = 16384 with 16 heads needs 183 MiB of workspace: refused on the host
    d = mra._Dims(1, 16, 16384, 64, 1)
    x = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    st = mra.lib().mra_attention_fwd_noalloc(ctypes.byref(d), x.data_ptr(), x.data_ptr(), x.data_ptr(), None, 8,
                                             0, 0, 1, x.data_ptr(), None)
    assert st == 14
