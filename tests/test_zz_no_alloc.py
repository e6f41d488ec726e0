"""GPU: the allocation-free sampler (qw3_sample_noalloc, scratch in a device array inside the library)
against qw3_sample with a caller workspace, through the C ABI: two calls in a row, the second on a smaller
input (fewer rows, a smaller vocabulary), must give identical tokens, flags, statuses and generator states.
Collected last on purpose (test_zz_*): the array keeps the previous call's contents."""
import ctypes

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _call(lib, fn, logits, prm, hist, rng, ws=None):
    import torch
    import transformer_qwen3_block_amd as q
    rows, vocab = logits.shape
    tok = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    done = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    st = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    stop = (ctypes.c_int32 * 2)(5, 11)
    args = [ctypes.c_void_p(logits.data_ptr()), rows, vocab, logits.stride(0), ctypes.byref(prm),
            ctypes.c_void_p(hist.data_ptr()), hist.shape[1], None, 0, stop, 2, ctypes.c_void_p(rng.data_ptr()),
            ctypes.c_void_p(tok.data_ptr()), ctypes.c_void_p(done.data_ptr()), ctypes.c_void_p(st.data_ptr())]
    if ws is not None:
        args += [ctypes.c_void_p(ws[0]), ws[1]]
    args.append(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert getattr(lib, fn)(*args) == 0
    torch.cuda.synchronize()
    return tok.cpu().numpy(), done.cpu().numpy(), st.cpu().numpy()


@pytest.mark.parametrize("temperature", [0.9, 0.0])
def test_noalloc_sampler_matches_workspace_sampler(temperature):
    import torch
    import transformer_qwen3_block_amd as q
    lib = q.lib()
    nb = ctypes.c_uint64(0)
    assert lib.qw3_sample_workspace_bytes(16, ctypes.byref(nb)) == 0
    buf = torch.empty(int(nb.value) + 256, dtype=torch.uint8, device="cuda")
    ws = ((buf.data_ptr() + 255) & ~255, int(nb.value))
    prm = q.SampleParams(temperature, 0.9, 1.2, 64)
    for call, (rows, vocab) in enumerate([(16, 151936), (3, 5000)]):   # second call: smaller input
        lg = torch.from_numpy(synth.logits_rows(70 + call, 0, rows, vocab, 3.0)).cuda()
        lg[:, 5] = 50.0                                                  # a stop token is likely drawn
        hist = torch.from_numpy(synth.tokens(70 + call, 1, rows * 20, vocab).reshape(rows, 20)).cuda()
        seeds = np.array([q.pcg32_seed(900 + r, r) for r in range(rows)], np.uint64).view(np.int64)
        rng_a = torch.from_numpy(seeds.copy()).cuda()
        rng_b = torch.from_numpy(seeds.copy()).cuda()
        a = _call(lib, "qw3_sample", lg, prm, hist, rng_a, ws)
        b = _call(lib, "qw3_sample_noalloc", lg, prm, hist, rng_b)
        for x, y in zip(a, b):
            assert np.array_equal(x, y), (call, x, y)
        assert np.array_equal(rng_a.cpu().numpy(), rng_b.cpu().numpy())
        assert np.all(a[2] == 0) and np.all(a[0] >= 0)


def test_noalloc_sampler_rejects_requests_beyond_its_array():
    import torch
    import transformer_qwen3_block_amd as q
    lib = q.lib()
    prm = q.SampleParams(1.0, 1.0, 1.0, 8)
    lg = torch.zeros((17, 100), dtype=torch.float32, device="cuda")
    rng = torch.zeros((17, 2), dtype=torch.int64, device="cuda")
    tok = torch.zeros(17, dtype=torch.int32, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    assert lib.qw3_sample_noalloc(p(lg), 17, 100, 100, ctypes.byref(prm), None, 0, None, 0, None, 0, p(rng),
                                  p(tok), None, None, s) == 1            # rows beyond the array's 16
    big = torch.zeros((1, 262145), dtype=torch.float32, device="cuda")
    assert lib.qw3_sample_noalloc(p(big), 1, 262145, 262145, ctypes.byref(prm), None, 0, None, 0, None, 0,
                                  p(rng), p(tok), None, None, s) == 1    # vocabulary beyond 262,144
