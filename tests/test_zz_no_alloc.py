"""flash_decode_full_noalloc, the entry point for callers that cannot
allocate, against flash_decode_full through the C ABI: two calls in a row,
the second with a smaller input, each bit for bit equal to the workspace
entry point (same kernels, same split counts; the static scratch keeps the
first call's records, which the second must not read), and the size limit
rejected on the host."""
import ctypes as C

import pytest
import torch

import int4_q4_gemv_amd as q4
from int4_q4_gemv_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ptr(t):
    return C.c_void_p(t.data_ptr())


def _both(q, k, v, pos0):
    L = q4.lib()
    n_rows, Hq, D = q.shape
    cap = k.shape[0]
    q, k, v = q.to(DEV).contiguous(), k.to(DEV).contiguous(), v.to(DEV).contiguous()
    pos = (C.c_int32 * 1)(pos0)
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    nb = int(L.flash_decode_workspace_size(1, n_rows, Hq, D))
    assert 0 < nb <= int(L.flash_decode_noalloc_max_bytes())
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    ref = torch.full((1, n_rows, Hq, D), float("nan"), device=DEV)
    got = torch.full((1, n_rows, Hq, D), float("nan"), device=DEV)
    rc = L.flash_decode_full(_ptr(q), _ptr(k), _ptr(v), 0, cap, Hq, D, pos, 1, n_rows, 1.0, _ptr(ref),
                             _ptr(ws), nb, st)
    assert rc == q4.Q4_OK
    rc = L.flash_decode_full_noalloc(_ptr(q), _ptr(k), _ptr(v), 0, cap, Hq, D, pos, 1, n_rows, 1.0,
                                     _ptr(got), st)
    assert rc == q4.Q4_OK
    torch.cuda.synchronize()
    return got, ref


def test_noalloc_matches_the_workspace_entry_point():
    print("noalloc full attention: 32768 x 4 rows, D 512, then 3000 x 1 row, D 256", flush=True)
    # the largest call the scratch holds (4 rows x 16 heads x 64 splits at D = 512) ...
    q, k, v = synth.full_attn_inputs(32768, 32768 + 8, 4, Hq=16, D=512, seed=21)
    got, ref = _both(q, k, v, 32768 - 4)
    assert torch.isfinite(got).all() and torch.equal(got, ref)
    # ... then a smaller one on the scratch the first call left behind
    q, k, v = synth.full_attn_inputs(3000, 3100, 1, Hq=16, D=256, seed=22)
    got, ref = _both(q, k, v, 2999)
    assert torch.isfinite(got).all() and torch.equal(got, ref)


def test_noalloc_rejects_calls_beyond_the_scratch():
    L = q4.lib()
    # 16 sequences x 4 rows need 16.9 MB of records: refused before any launch
    assert int(L.flash_decode_workspace_size(16, 4, 16, 512)) > int(L.flash_decode_noalloc_max_bytes())
    f = C.c_void_p(0x10000)
    pos = (C.c_int32 * 16)(*([100] * 16))
    rc = L.flash_decode_full_noalloc(f, f, f, 200 * 512, 200, 16, 512, pos, 16, 4, 1.0, f, None)
    assert rc == q4.Q4_ENOSPACE
