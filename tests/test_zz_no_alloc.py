"""GPU check of df11_gpu_encode_noalloc, the encoder entry point that
allocates nothing (its workspace is the library's own device array): through
the C-ABI, its sections equal those of df11_gpu_encode with a caller
workspace, byte for byte, on two calls in a row (the second on a smaller
block, so the array still holds the first call's contents), with and without
window counts; they decode back to the input; and a plan that needs more
workspace than the array holds is refused before anything runs."""
import numpy as np
import pytest

import df11_inputs as di
import huffman_decode_block_amd as hdb

pytestmark = pytest.mark.gpu

SECTIONS = ("stream", "sign_mant", "gaps", "unit_pos", "counts")


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "the GPU tests need a GPU"
    return t


def encode_both(torch, x, window_counts):
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    ref = hdb.gpu_encode(xd, window_counts=window_counts)  # df11_gpu_encode, caller workspace
    t = ref.tensors
    # fresh outputs, poisoned, for the no-allocation call on the same plan
    out = {k: (torch.full_like(t[k], 0x5A) if t[k] is not None else None) for k in SECTIONS}
    hdb.df11_gpu_encode_noalloc(ref.plan, xd, t["chunk_hist"], out["stream"], out["sign_mant"], out["gaps"],
                                out["unit_pos"], out["counts"])
    torch.cuda.synchronize()
    return xd, ref, out


@pytest.mark.parametrize("window_counts", [False, True])
def test_noalloc_encoder_equals_workspace_encoder(torch, window_counts):
    for n, seed in ((6_000_007, 11), (1_000_003, 12)):  # the second call smaller
        x = di.random_normal(n, 0.02, seed)
        say(f"no-alloc encode n={n} counts={window_counts}")
        xd, ref, out = encode_both(torch, x, window_counts)
        for k in SECTIONS:
            if ref.tensors[k] is None:
                continue
            assert torch.equal(out[k], ref.tensors[k]), f"section {k} differs (n={n})"
        # and the sections decode back to the input
        blk = ref.block
        dec = torch.empty(n, dtype=torch.int16, device="cuda")
        hdb.df11_decode_block(blk, out=dec)
        torch.cuda.synchronize()
        assert torch.equal(dec, xd)


def test_noalloc_encoder_refuses_plans_beyond_its_workspace(torch):
    # a histogram of 2^31 weights spread over 30 exponents needs far more than
    # the array (about 0.04 byte per weight): refused on the host
    hist = np.zeros(256, dtype=np.uint64)
    hist[100:130] = (1 << 31) // 30
    plan = hdb.df11_gpu_plan_build(hist)
    assert plan.workspace_bytes > hdb.DF11_NOALLOC_WORKSPACE_BYTES
    small = torch.zeros(64, dtype=torch.uint8, device="cuda")
    x = torch.zeros(64, dtype=torch.int16, device="cuda")
    st = hdb.lib().df11_gpu_encode_noalloc(
        __import__("ctypes").byref(plan), x.data_ptr(), small.data_ptr(), small.data_ptr(), small.data_ptr(),
        small.data_ptr(), small.data_ptr(), None, None)
    assert st == hdb.DF11_E_BUFFER_TOO_SMALL
