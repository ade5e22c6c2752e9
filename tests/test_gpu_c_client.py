"""The C ABI on its own: a plain C program (tests/abi_c/decode_client.c,
built here with gcc against include/pagedkv.h and libpagedkv.so) appends one
decode step and decodes, runs the same step as one pkv_decode_step call, or
runs one pkv_mixed_step with chunked prefill on a second stream, in a
process with no Python and no PyTorch.  Its
pools must equal the oracle's byte for byte and its outputs must match the
oracle within the decode tolerances ("TensorRT-LLM框架解析与高性能推理优化实践"
§4.2 and §6.2: the block-table write and walk; §6.1: the one-pass softmax)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from paged_kv_cache_277_amd import binding as B
from paged_kv_cache_277_amd import workloads as wk

from tests import _support as sup

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "paged_kv_cache_277_amd")
SRC = os.path.join(ROOT, "tests", "abi_c", "decode_client.c")

# max |err|, mean |err| bars of the decode output (as in the parity tests)
TOL = {"bf16": (2e-2, 2e-3), "fp8": (6e-2, None), "int8": (2e-2, 2e-3)}
LSE_TOL = 2e-3

CASES = [
    # lens, Hq, Hkv, D, P, kv, and None, prefill (ctx_before per request,
    # chunk) or "fused"
    ((1, 33, 200, 700, 2100), 16, 4, 128, 32, "bf16", None),   # matrix-core decode, ranges
    ((5, 64, 65, 900), 8, 8, 128, 64, "bf16", None),           # vector decode (MHA)
    ((1, 129, 1500), 64, 8, 128, 64, "fp8", None),             # fp8 codes from f32 input
    # one pkv_mixed_step call: decode beside chunked prefill on a second stream
    ((5, 300, 1000), 32, 8, 128, 32, "bf16", ((0, 100, 1800), 200)),
    # one pkv_decode_step call (the append inside the attention launch)
    ((1, 33, 200, 700, 2100), 16, 4, 128, 32, "bf16", "fused"),
    ((1, 129, 1500), 64, 8, 128, 64, "fp8", "fused"),
    ((5, 64, 65, 900), 8, 8, 128, 64, "bf16", "fused"),
]


def _build(tmp_path) -> str:
    if not os.path.exists(os.path.join(PKG, "libpagedkv.so")):
        pytest.fail("libpagedkv.so is not built (python -m paged_kv_cache_277_amd.build)")
    exe = str(tmp_path / "decode_client")
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", "-I/opt/rocm/include", SRC, f"-L{PKG}",
           "-lpagedkv", "-L/opt/rocm/lib", "-lamdhip64", f"-Wl,-rpath,{PKG}",
           "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"gcc failed:\n{r.stdout}\n{r.stderr}"
    return exe


def _write_inputs(d, wl, kp0, vp0, fused=False):
    s = wl.spec
    st = wl.step
    kv = B.DTYPE_CODES[s.kv_dtype]
    meta = [wl.num_pages, s.num_kv_heads, s.page_size, s.head_dim, kv,
            wl.num_seqs, s.num_q_heads, wl.block_tables.shape[1], int(wl.context_lens.max()),
            repr(float(wl.sm_scale)), st.num_rows, st.num_tokens, st.block_tables.shape[1],
            B.DTYPE_CODES[s.kv_in_dtype]]
    (d / "meta.txt").write_text(" ".join(str(x) for x in meta) + "\n")
    k_step, v_step = st.k, st.v
    if fused:
        (d / "fused.txt").write_text("1\n")
        k_step, v_step = wk.decode_step_tokens(wl)
    files = {"kpool.bin": kp0, "vpool.bin": vp0, "knew.bin": k_step, "vnew.bin": v_step,
             "cu.bin": st.cu.astype(np.int32), "start.bin": st.start_pos.astype(np.int32),
             "stepbt.bin": st.block_tables.astype(np.int32), "q.bin": wl.q,
             "bt.bin": wl.block_tables.astype(np.int32),
             "lens.bin": wl.context_lens.astype(np.int32)}
    if s.kv_dtype in ("fp8", "int8"):
        files["kscale.bin"] = wl.k_scale.astype(np.float32)
        files["vscale.bin"] = wl.v_scale.astype(np.float32)
    if wl.num_prefill:
        tot = wl.pf_ctx_before + np.diff(wl.pf_cu)
        (d / "pfmeta.txt").write_text(" ".join(str(x) for x in (
            wl.num_prefill, int(wl.pf_cu[-1]), int(np.diff(wl.pf_cu).max()), int(tot.max()),
            wl.pf_block_tables.shape[1])) + "\n")
        files.update({"pfq.bin": wl.pf_q, "pfcu.bin": wl.pf_cu.astype(np.int32),
                      "pfctx.bin": wl.pf_ctx_before.astype(np.int32),
                      "pfbt.bin": wl.pf_block_tables.astype(np.int32)})
    for name, arr in files.items():
        (d / name).write_bytes(np.ascontiguousarray(arr).tobytes())


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES)
def test_c_client_append_and_decode_match_oracle(case, tmp_path):
    if shutil.which("gcc") is None:
        pytest.fail("gcc is needed to build the C client")
    lens, hq, hkv, hd, page, kv, mode = case
    fused = mode == "fused"
    pf = None if fused else mode
    extra = dict(prefill_ctx=pf[0], prefill_chunk=pf[1]) if pf else {}
    spec = wk.custom_spec(lens, num_q_heads=hq, num_kv_heads=hkv, head_dim=hd, page_size=page,
                          q_dtype="bf16", kv_dtype=kv, out_dtype="bf16", **extra)
    wl = wk.make_workload(spec, seed=77)
    kp0, vp0 = sup.oracle_pools(wl, with_step=False)
    kp1, vp1 = sup.oracle_pools(wl, with_step=True)
    ref, ref_lse = sup.oracle_decode(wl, kp1, vp1)

    exe = _build(tmp_path)
    d = tmp_path / "io"
    d.mkdir()
    _write_inputs(d, wl, kp0, vp0, fused)
    print(f"[c-client] case {case}", flush=True)
    r = subprocess.run([exe, str(d)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"decode_client failed:\n{r.stdout}\n{r.stderr}"

    # pools: the library's append equals the oracle's, byte for byte
    assert (d / "kpool_out.bin").read_bytes() == kp1.tobytes()
    assert (d / "vpool_out.bin").read_bytes() == vp1.tobytes()
    # outputs
    out = np.frombuffer((d / "out.bin").read_bytes(), dtype=np.uint16).reshape(ref.shape)
    g = sup.to_f64(out, "bf16")
    assert np.isfinite(g).all()
    err = np.abs(g - ref)
    mx, mean_bar = TOL[kv]
    assert err.max() <= mx, f"max |err| {err.max():.3g}"
    if mean_bar is not None:
        assert err.mean() <= mean_bar, f"mean |err| {err.mean():.3g}"
    lse = np.frombuffer((d / "lse.bin").read_bytes(), dtype=np.float32).reshape(ref_lse.shape)
    assert np.abs(lse.astype(np.float64) - ref_lse).max() <= LSE_TOL
    print(f"[c-client] max |err| {err.max():.3g}, mean {err.mean():.3g}", flush=True)
    if pf:
        pref, plse = sup.oracle_prefill(wl, kp1, vp1)
        pout = np.frombuffer((d / "pfout.bin").read_bytes(), dtype=np.uint16).reshape(pref.shape)
        pg = sup.to_f64(pout, "bf16")
        perr = np.abs(pg - pref)
        assert np.isfinite(pg).all()
        assert perr.max() <= mx and perr.mean() <= mean_bar, (perr.max(), perr.mean())
        pl = np.frombuffer((d / "pflse.bin").read_bytes(), dtype=np.float32).reshape(plse.shape)
        assert np.abs(pl.astype(np.float64) - plse).max() <= LSE_TOL
        print(f"[c-client] prefill max |err| {perr.max():.3g}, mean {perr.mean():.3g}", flush=True)
