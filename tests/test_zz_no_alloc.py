"""The allocation-free decode attention (aatc_decode_attn_noalloc): the same kernels as
aatc_decode_attn, with partial records in the library's static per-GPU array instead of a
caller workspace.  Its results must equal aatc_decode_attn's bit for bit, on consecutive calls
whose second one is smaller (the array keeps the first call's records), and a step too large
for the array is refused before anything runs."""
import ctypes

import numpy as np
import pytest

import synth
from compressed_decode_attention_head_amd import _native as N
from gpu_helpers import Case

ATOL_ATTN = 2e-3


def test_noalloc_refuses_oversized_steps():
    """Host-side check, no device work: 256 sequences x 8 KV heads x 128K tokens need far more
    than the static array holds."""
    L = N.lib()
    c = N.Cache(batch=256, n_kv_heads=8, d=128, k_bits=170, v_bits=170, v_tiles=12, capacity_tokens=131072,
                k_calib=256, v_calib=512, k_codes=1024, v_codes=2048)
    need = L.aatc_decode_attn_workspace_bytes(ctypes.byref(c), 32, 131072)
    assert need > (8 << 20)
    st = L.aatc_decode_attn_noalloc(ctypes.byref(c), 4096, 0, 32, None, 131072, 0.0, 8192, None, None)
    assert N.STATUS[st] == "AATC_ERR_BUFFER_TOO_SMALL"
    assert b"static workspace" in L.aatc_last_error()


@pytest.mark.gpu
def test_noalloc_equals_decode_attn_on_consecutive_calls():
    import torch
    # first call: the 1.33-bit Walsh-Hadamard GQA-7 shape; second: a smaller 2.76-bit KLT layer
    cases = [Case(cfg=4, n_kv=2, group=7, n_tokens=2000, rotation="wht", bpe_k=1.33, marginal="t3"),
             Case(cfg=2, n_kv=2, group=4, n_tokens=333, rotation="klt", bpe_k=2.76)]
    for i, case in enumerate(cases):
        cache = case.make_cache()
        for t in (synth.K, synth.V):
            cache.encode(t, case.torch_x(t))
        q = torch.from_numpy(case.q.astype(np.float32)).cuda()
        ref, lref = cache.decode_attn(q, case.n)
        out = torch.full_like(ref, float("nan"))
        lse = torch.full_like(lref, float("nan"))
        cache.decode_attn_noalloc(q, case.n, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(lse, lref), i
        want, _ = case.oracle_attention()
        err = float(np.abs(out.cpu().numpy() - want).max())
        print("no-alloc call %d: %d tokens, equal to aatc_decode_attn, max abs err vs oracle %.2e" % (i, case.n, err),
              flush=True)
        assert err <= ATOL_ATTN
