"""pkv_paged_attn_decode_noalloc against pkv_paged_attn_decode.

The allocation-free decode runs the same kernels with its partials in the
library's fixed per-GPU array, so its outputs must equal the workspace
call's bit for bit.  Two calls in a row (the second smaller, over the array
the first left behind), three kernel paths (vector bf16, matrix-core bf16,
matrix-core fp8), the oracle's bar on the first, and the size limit.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_277_amd import binding as B
from paged_kv_cache_277_amd import device as dev
from paged_kv_cache_277_amd import workloads as wk
from tests import _support as sup
from tests.test_gpu_parity import check_close, check_lse

pytestmark = pytest.mark.gpu

CASES = [
    # (lens of the first call, lens of the second, Hq, Hkv, D, page, kv, split)
    ((3000, 17, 2048, 0, 1, 900, 2500, 64), (700, 5, 1200), 16, 16, 128, 64, "bf16", 256),
    ((4000, 33, 3100, 1, 2047, 256), (800, 300), 32, 8, 128, 32, "bf16", 128),
    ((5000, 4096, 100, 2900), (1500, 64, 3), 64, 8, 128, 64, "fp8", 512),
]


def _decode_inputs(lens, Hq, Hkv, D, P, kv, seed):
    spec = wk.custom_spec(lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P,
                          q_dtype="bf16", kv_dtype=kv, out_dtype="bf16")
    wl = wk.make_workload(spec, seed=seed)
    dw = dev.upload(wl)
    dw.setup()
    dw.append_step()
    return wl, dw


def _run_both(dw, split):
    max_len = int(dw.lens.max().item())
    ws = B.decode_workspace(dw.cache, dw.q.shape[0], dw.q.shape[1], max_len, split)
    assert ws is not None, "the case must need partials"
    assert ws.numel() <= B.NOALLOC_SCRATCH_BYTES
    want, want_lse = torch.empty_like(dw.out), torch.empty_like(dw.lse)
    B.pkv_paged_attn_decode(dw.cache, dw.q, want, dw.bt, dw.lens, max_len,
                            float(dw.wl.sm_scale), lse=want_lse, split_tokens=split, workspace=ws)
    got = torch.full_like(dw.out, float("nan"))
    got_lse = torch.full_like(dw.lse, float("nan"))
    B.pkv_paged_attn_decode_noalloc(dw.cache, dw.q, got, dw.bt, dw.lens, max_len,
                                    float(dw.wl.sm_scale), lse=got_lse, split_tokens=split)
    torch.cuda.synchronize()
    return got, got_lse, want, want_lse


@pytest.mark.parametrize("case", CASES)
def test_noalloc_decode_equals_workspace_decode(case):
    lens1, lens2, Hq, Hkv, D, P, kv, split = case
    print(f"[no-alloc] case {case}", flush=True)
    wl, dw = _decode_inputs(lens1, Hq, Hkv, D, P, kv, seed=61)
    got, got_lse, want, want_lse = _run_both(dw, split)
    assert torch.equal(got, want) and torch.equal(got_lse, want_lse)
    kp, vp = sup.oracle_pools(wl)
    ref, ref_lse = sup.oracle_decode(wl, kp, vp)
    check_close(got, ref, wl.spec)
    check_lse(got_lse, ref_lse, wl.spec)
    # a second, smaller call over the array the first one left behind
    wl2, dw2 = _decode_inputs(lens2, Hq, Hkv, D, P, kv, seed=62)
    got, got_lse, want, want_lse = _run_both(dw2, split)
    assert torch.equal(got, want) and torch.equal(got_lse, want_lse)


def test_noalloc_decode_rejects_calls_beyond_the_array():
    # 64 sequences x 64 query heads x 64 ranges of 16 tokens: 64 MiB of partials
    lens = (1024,) * 64
    spec = wk.custom_spec(lens, num_q_heads=64, num_kv_heads=64, head_dim=128, page_size=16,
                          q_dtype="bf16", kv_dtype="bf16", out_dtype="bf16", num_pages=4096)
    wl = wk.make_workload(spec, seed=63)
    dw = dev.upload(wl)
    need = B.pkv_decode_workspace_bytes(dw.cache, 64, 64, 1024, 16)
    assert need > B.NOALLOC_SCRATCH_BYTES
    dw.out.fill_(7.0)
    with pytest.raises(B.PkvError, match="scratch"):
        B.pkv_paged_attn_decode_noalloc(dw.cache, dw.q, dw.out, dw.bt, dw.lens, 1024,
                                        float(wl.sm_scale), split_tokens=16)
    torch.cuda.synchronize()
    assert bool((dw.out == 7.0).all()), "a refused call launched work"
    # the same call with 256-token ranges (8.5 MB of partials) fits and
    # matches the workspace call
    dw.setup()
    dw.append_step()
    got, got_lse, want, want_lse = _run_both(dw, 256)
    assert torch.equal(got, want) and torch.equal(got_lse, want_lse)
