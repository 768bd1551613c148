"""The entry point that allocates nothing (lla_forward_noalloc, scratch in the library's
static device buffer) against lla_forward_ws with a caller workspace: bit-identical outputs
on two calls in a row, the second smaller than the first (the buffer keeps the first call's
contents), and a problem beyond the buffer refused before any launch."""
import ctypes

import numpy as np
import pytest

from parity_util import require_gpu, to_device, workload_arrays

pytestmark = pytest.mark.gpu


def _call_noalloc(lib, tq, tk, tv, out, w, stream):
    return lib.lla_forward_noalloc(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(),
                                   w.B, w.H, w.n, w.d, float(w.h), float(w.lam), 1,
                                   ctypes.c_void_p(stream.cuda_stream), 0)


def test_noalloc_matches_workspace_entry_point_twice():
    torch = require_gpu()
    from local_linear_attention_amd import lla_forward_ws, lla_workspace_size, load_library
    lib = load_library()
    stream = torch.cuda.current_stream()
    for shape in ({"B": 2, "H": 4, "n": 1100}, {"B": 1, "H": 2, "n": 333}):
        w, q, k, v = workload_arrays("d24", **shape)
        print(f"[noalloc] d24 {shape}", flush=True)
        tq, tk, tv = (to_device(x, "bf16") for x in (q, k, v))
        nbytes = lla_workspace_size(w.B, w.H, w.n, w.d, "bf16", "auto")
        assert 0 < nbytes <= lib_limit()
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        ref = lla_forward_ws(tq, tk, tv, w.h, w.lam, ws, path="auto")
        out = torch.full(tq.shape, float("nan"), dtype=torch.float32, device="cuda")
        assert _call_noalloc(lib, tq, tk, tv, out, w, stream) == 0
        torch.cuda.synchronize()
        assert torch.isfinite(out).all().item()
        assert torch.equal(out, ref), float((out - ref).abs().max())


def test_noalloc_refuses_problems_beyond_its_buffer():
    torch = require_gpu()
    from local_linear_attention_amd import lla_workspace_size, load_library
    lib = load_library()
    w, _, _, _ = workload_arrays("d24", B=1, H=1, n=64)
    big = dict(B=4, H=16, n=8192)
    assert lla_workspace_size(big["B"], big["H"], big["n"], 64, "bf16", "auto") > lib_limit()
    t = torch.empty(1, dtype=torch.bfloat16, device="cuda")
    o = torch.empty(1, dtype=torch.float32, device="cuda")
    # pointers are never dereferenced: the size check comes before any launch
    st = lib.lla_forward_noalloc(t.data_ptr(), t.data_ptr() + 2 ** 30, t.data_ptr() + 2 ** 31, o.data_ptr() + 2 ** 32,
                                 big["B"], big["H"], big["n"], 64, 8.0, 0.01, 1, None, 0)
    assert st == 8


def lib_limit():
    return 256 << 20
