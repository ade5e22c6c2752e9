"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Bars (from the workload statement): fp32 max |err| <= 1e-4; bf16 max |err| <=
2e-2 and mean |err| <= 2e-3; fp8 KV max |err| <= 6e-2 against the oracle on
the dequantised cache; append bit-exact over the whole pool (poison included).
The log-sum-exp output is held to 1e-4 (fp32) / 2e-3 (bf16, fp8): it is a
float32 reduction of exactly-represented products, far tighter than the
output bar.  Small cases compare every element; the five workloads at full
size compare sampled sequences / prefill rows in the launch configuration the
benchmark times.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_277_amd import binding as B
from paged_kv_cache_277_amd import device as dev
from paged_kv_cache_277_amd import workloads as wk
from oracle import attention as oa
from oracle import formats as of
from tests import _support as sup

pytestmark = pytest.mark.gpu

# int8: the codes widen exactly to bf16 and the arithmetic after that is the
# bf16 path's (scales applied in fp32), so the bf16 bar applies.
TOL = {"f32": (1e-4, None), "bf16": (2e-2, 2e-3), "fp8": (6e-2, None), "int8": (2e-2, 2e-3)}
LSE_TOL = {"f32": 1e-4, "bf16": 2e-3, "fp8": 2e-3, "int8": 2e-3}


def _kind(spec):
    return "fp8" if spec.kv_dtype == "fp8" else spec.kv_dtype


def check_close(gpu: torch.Tensor, ref: np.ndarray, spec, what="out"):
    g = sup.to_f64(dev.storage_to_numpy(gpu), spec.out_dtype)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite GPU values"
    err = np.abs(g - ref)
    mx, mean_bar = TOL[_kind(spec)]
    assert err.max() <= mx, f"{what}: max |err| {err.max():.3g} > {mx}"
    if mean_bar is not None:
        assert err.mean() <= mean_bar, f"{what}: mean |err| {err.mean():.3g} > {mean_bar}"
    return float(err.max())


def check_lse(gpu: torch.Tensor, ref: np.ndarray, spec):
    g = gpu.detach().cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(g), fin)
    assert np.array_equal(g[~fin], ref[~fin])
    if fin.any():
        assert np.abs(g[fin] - ref[fin]).max() <= LSE_TOL[_kind(spec)]


def spec_of(lens, Hq, Hkv, D, P, kv, **kw):
    qd = "f32" if kv == "f32" else "bf16"
    return wk.custom_spec(lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P,
                          q_dtype=qd, kv_dtype=kv, out_dtype=qd, **kw)


def gpu_cache_from(wl, kp, vp):
    s = wl.spec
    ks = vs = None
    if s.kv_dtype in ("fp8", "int8"):
        ks = torch.from_numpy(wl.k_scale).cuda()
        vs = torch.from_numpy(wl.v_scale).cuda()
    return B.PagedCache(dev._dev(kp, s.kv_dtype, "cuda"), dev._dev(vp, s.kv_dtype, "cuda"), ks, vs)


def gpu_decode(wl, cache, split=0, bt=None):
    s = wl.spec
    q = dev._dev(wl.q, s.q_dtype, "cuda")
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    bt = dev._dev(wl.block_tables if bt is None else bt, "i32", "cuda")
    lens = dev._dev(wl.context_lens, "i32", "cuda")
    max_len = int(wl.context_lens.max())
    ws = B.decode_workspace(cache, wl.num_seqs, s.num_q_heads, max_len, split)
    B.pkv_paged_attn_decode(cache, q, out, bt, lens, max_len, float(wl.sm_scale), lse=lse,
                            split_tokens=split, workspace=ws)
    torch.cuda.synchronize()
    return out, lse


# ------------------------------------------------------------- fp8 codec ----
def test_fp8_device_decode_matches_format_definition():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).cuda()
    out = torch.empty(256, dtype=torch.float32, device="cuda")
    B.pkv_fp8_e4m3fn_to_f32(codes, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = of.E4M3FN_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ---------------------------------------------------------------- append ----
APPEND_CASES = [
    ((7, 33, 64, 100), 4, 4, 64, 16, "f32"),
    ((1, 15, 16, 17, 63, 64, 65), 8, 2, 128, 64, "bf16"),
    ((5, 31, 32, 33, 200), 8, 1, 128, 32, "fp8"),
    ((3, 70, 129), 16, 4, 64, 16, "fp8"),
    ((5, 31, 32, 33, 200), 8, 1, 128, 32, "int8"),
    ((3, 70, 129), 16, 4, 64, 16, "int8"),
    ((5, 127, 128, 129, 300), 8, 2, 128, 128, "bf16"),   # 128-token pages
    ((3, 255, 256, 257), 8, 8, 64, 256, "fp8"),          # 256-token pages
]


@pytest.mark.parametrize("case", APPEND_CASES)
def test_append_bit_exact(case):
    spec = spec_of(*case)
    wl = wk.make_workload(spec, seed=31)
    dw = dev.upload(wl)
    dw.setup()
    dw.append_step()
    torch.cuda.synchronize()
    kp, vp = sup.oracle_pools(wl)
    assert dev.storage_to_numpy(dw.cache.k_pool).tobytes() == kp.tobytes()
    assert dev.storage_to_numpy(dw.cache.v_pool).tobytes() == vp.tobytes()


def test_append_fp8_rounding_edges():
    """Values at e4m3 rounding midpoints, saturation and tiny magnitudes."""
    spec = spec_of((40,), 2, 2, 64, 16, "fp8")
    wl = wk.make_workload(spec, seed=3)
    vals = np.unique(of.E4M3FN_TABLE[:0x7F])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    probe = np.concatenate([mids, np.nextafter(mids, np.float32(1e9)), np.nextafter(mids, np.float32(0)),
                            np.array([448, 449, 463.9, 464, 500, 1e30, 2.0 ** -10, 3 * 2.0 ** -10,
                                      1e-30, 0.0, -0.0], np.float32)])
    probe = np.concatenate([probe, -probe]).astype(np.float32)
    flat = wl.setup.k.reshape(-1)
    flat[:] = np.resize(probe, flat.shape)          # the scale is 1/448 of the original amax
    wl.setup.v.reshape(-1)[:] = np.resize(probe[::-1], flat.shape)
    wl.k_scale[:] = 1.0
    wl.v_scale[:] = 1.0
    dw = dev.upload(wl)
    dw.setup()
    torch.cuda.synchronize()
    kp, vp = sup.oracle_pools(wl, with_step=False)
    assert dev.storage_to_numpy(dw.cache.k_pool).tobytes() == kp.tobytes()
    assert dev.storage_to_numpy(dw.cache.v_pool).tobytes() == vp.tobytes()


def test_append_int8_rounding_edges():
    """Quotients at and around every half-integer tie, saturation, infinities
    and NaN (which encodes as 0); scale 1 so the quotient is the value."""
    spec = spec_of((40,), 2, 2, 64, 16, "int8")
    wl = wk.make_workload(spec, seed=4)
    ties = (np.arange(-130, 131) + 0.5).astype(np.float32)
    probe = np.concatenate([ties, np.nextafter(ties, np.float32(1e9)),
                            np.nextafter(ties, np.float32(-1e9)),
                            np.array([127.0, 127.49, 127.5, 128.0, 1e30, np.inf, np.nan, 0.0, -0.0,
                                      1e-30], np.float32)])
    probe = np.concatenate([probe, -probe]).astype(np.float32)
    flat = wl.setup.k.reshape(-1)
    flat[:] = np.resize(probe, flat.shape)
    wl.setup.v.reshape(-1)[:] = np.resize(probe[::-1], flat.shape)
    wl.k_scale[:] = 1.0
    wl.v_scale[:] = 1.0
    dw = dev.upload(wl)
    dw.setup()
    torch.cuda.synchronize()
    kp, vp = sup.oracle_pools(wl, with_step=False)
    assert dev.storage_to_numpy(dw.cache.k_pool).tobytes() == kp.tobytes()
    assert dev.storage_to_numpy(dw.cache.v_pool).tobytes() == vp.tobytes()


# ---------------------------------------------------------------- decode ----
DECODE_CASES = [
    # lens, Hq, Hkv, D, P, kv
    ((7, 33, 64, 100), 4, 4, 64, 16, "f32"),            # the tiny fp32 workload's shape
    ((1, 63, 64, 65, 129, 700), 8, 8, 128, 64, "bf16"),   # MHA, 13B-like head_dim / page
    ((16, 31, 32, 33, 1000), 32, 8, 128, 32, "bf16"),     # GQA 4
    ((1, 64, 65, 1500), 64, 8, 128, 64, "fp8"),           # GQA 8, fp8 KV
    ((15, 16, 17, 300), 4, 2, 64, 16, "bf16"),            # G 2, D 64
    ((5, 100), 16, 1, 64, 32, "bf16"),                    # G 16
    ((5, 100, 333), 8, 1, 64, 16, "fp8"),
    ((2, 3, 40), 4, 1, 128, 16, "f32"),
    ((1, 31, 200), 4, 2, 128, 32, "fp8"),                 # G 2: fp8 on the vector path
    ((1, 31, 200), 12, 4, 128, 32, "fp8"),                # G 3: smallest matrix-core group
    ((17, 250), 48, 4, 64, 64, "bf16"),                   # G 12, D 64
    ((1, 64, 65, 1500), 64, 8, 128, 64, "int8"),          # GQA 8, int8 KV (matrix cores)
    ((5, 100, 333), 8, 1, 64, 16, "int8"),                # G 8, D 64, page 16
    ((1, 31, 200), 4, 2, 128, 32, "int8"),                # G 2: int8 on the vector path
    ((7, 33, 64), 4, 4, 64, 16, "int8"),                  # G 1, D 64
    ((1, 127, 128, 129, 700), 8, 8, 128, 128, "bf16"),    # 128-token pages, MHA (vector path)
    ((16, 255, 256, 257, 1000), 32, 8, 128, 256, "bf16"), # 256-token pages, G 4 (matrix cores)
    ((1, 129, 1500), 64, 8, 128, 128, "fp8"),             # 128-token pages, G 8, fp8
    ((5, 300, 513), 4, 2, 64, 256, "int8"),               # 256-token pages, G 2, int8 (vector)
    ((3, 200), 4, 4, 64, 128, "f32"),                     # 128-token pages, fp32
    # with split 64: rows of 3, 4, 5, 5 and 1 ranges, across the merge's
    # one-round limit of four ranges (vector path, then matrix cores)
    ((192, 256, 257, 320, 1), 8, 2, 128, 64, "bf16"),
    ((192, 256, 257, 320, 1), 16, 4, 128, 32, "bf16"),
]


@pytest.mark.parametrize("case", DECODE_CASES)
@pytest.mark.parametrize("split", [0, 64])
def test_decode_parity_small(case, split):
    """split 64 cuts contexts into many ranges (one page each for pages of
    more than 64 tokens: ranges are page multiples)."""
    spec = spec_of(*case)
    split = max(split, spec.page_size) if split else 0
    wl = wk.make_workload(spec, seed=101)
    kp, vp = sup.oracle_pools(wl)
    ref, ref_lse = sup.oracle_decode(wl, kp, vp)
    out, lse = gpu_decode(wl, gpu_cache_from(wl, kp, vp), split=split)
    check_close(out, ref, spec)
    check_lse(lse, ref_lse, spec)


def test_decode_tiny_workload_exact_config():
    wl = wk.make_workload(wk.C1)
    kp, vp = sup.oracle_pools(wl)
    ref, ref_lse = sup.oracle_decode(wl, kp, vp)
    dw = dev.upload(wl)
    dw.setup()
    dw.step()
    torch.cuda.synchronize()
    check_close(dw.out, ref, wl.spec)
    check_lse(dw.lse, ref_lse, wl.spec)


def test_decode_empty_context():
    spec = spec_of((0, 5, 0, 17), 4, 2, 64, 16, "bf16")
    wl = wk.make_workload(spec, seed=4)
    kp, vp = sup.oracle_pools(wl)
    ref, ref_lse = sup.oracle_decode(wl, kp, vp)
    out, lse = gpu_decode(wl, gpu_cache_from(wl, kp, vp))
    check_close(out, ref, spec)
    check_lse(lse, ref_lse, spec)
    assert (out[0] == 0).all() and torch.isneginf(lse[0]).all()


def test_decode_page_permutation_bit_identical():
    spec = spec_of((17, 200, 333, 64), 16, 4, 128, 32, "bf16")
    wl = wk.make_workload(spec, seed=9)
    kp, vp = sup.oracle_pools(wl)
    out1, lse1 = gpu_decode(wl, gpu_cache_from(wl, kp, vp))
    pi = np.random.default_rng(5).permutation(wl.num_pages)
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[pi], vp2[pi] = kp, vp
    bt2 = np.where(wl.block_tables >= 0, pi[np.maximum(wl.block_tables, 0)], -1).astype(np.int32)
    out2, lse2 = gpu_decode(wl, gpu_cache_from(wl, kp2, vp2), bt=bt2)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_decode_split_invariance_and_determinism():
    spec = spec_of((40, 900, 2000), 8, 2, 128, 32, "bf16")
    wl = wk.make_workload(spec, seed=19)
    kp, vp = sup.oracle_pools(wl)
    cache = gpu_cache_from(wl, kp, vp)
    outs = [gpu_decode(wl, cache, split=s)[0].float() for s in (32, 64, 256, 2048)]
    for o in outs[1:]:
        assert (o - outs[0]).abs().max().item() <= 2 * 2 ** -8   # bf16 output rounding only
    a, la = gpu_decode(wl, cache, split=64)
    b, lb = gpu_decode(wl, cache, split=64)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_shared_prefix_equal_queries_equal_outputs():
    spec = spec_of((40, 100, 128, 128, 300), 8, 2, 128, 32, "bf16", shared_prefix_pages=4)
    wl = wk.make_workload(spec, seed=23)
    wl.q[2] = wl.q[3]               # two sequences of length 128 = the shared prefix only
    kp, vp = sup.oracle_pools(wl)
    ref, _ = sup.oracle_decode(wl, kp, vp)
    out, _ = gpu_decode(wl, gpu_cache_from(wl, kp, vp))
    check_close(out, ref, spec)
    assert torch.equal(out[2], out[3])


# --------------------------------------------------------------- prefill ----
PREFILL_CASES = [
    # lens(decode), Hq, Hkv, D, P, kv, prefill_ctx, chunk
    ((9,), 8, 2, 128, 32, "bf16", (0, 16, 33), 24),
    ((9,), 32, 8, 128, 32, "bf16", (0, 512), 130),
    ((9,), 4, 4, 64, 16, "f32", (0, 5), 17),
    ((9,), 16, 2, 128, 64, "fp8", (64, 1), 70),
    ((9,), 8, 8, 64, 16, "bf16", (7,), 1),                    # single-token chunk
    ((9,), 12, 4, 64, 16, "bf16", (3, 40), 33),               # G 3, page 16, ragged tiles
    ((9,), 16, 16, 128, 64, "bf16", (100,), 77),              # G 1 on the matrix cores
    ((9,), 8, 1, 64, 32, "fp8", (31,), 45),                   # G 8, fp8, head_dim 64
    ((9,), 16, 2, 128, 64, "int8", (64, 1), 70),              # int8 KV
    ((9,), 8, 1, 64, 32, "int8", (31, 100), 45),              # int8, head_dim 64
    ((9,), 16, 4, 64, 32, "bf16", (0, 37, 250), 90),          # bf16 head_dim 64, ragged ranges
    ((9,), 8, 2, 128, 16, "bf16", (5, 70), 40),               # bf16 head_dim 128, page 16
    ((9,), 8, 2, 64, 16, "bf16", (14000,), 20),               # long context, page 16: ranges capped at 511 pages
    ((9,), 16, 4, 128, 128, "bf16", (0, 200), 150),           # 128-token pages, ranges start mid-page
    ((9,), 8, 2, 64, 256, "fp8", (300,), 70),                 # 256-token pages, fp8
    ((9,), 8, 8, 128, 256, "bf16", (0, 600), 65),             # 256-token pages, G 1
]


@pytest.mark.parametrize("psplit", [0, 64])
@pytest.mark.parametrize("case", PREFILL_CASES)
def test_prefill_parity_small(case, psplit):
    """psplit 64 cuts every context longer than 64 keys into ranges (partials
    + merge); 0 takes the library's default (one range at these sizes)."""
    lens, Hq, Hkv, D, P, kv, ctx, chunk = case
    spec = spec_of(lens, Hq, Hkv, D, P, kv, prefill_ctx=ctx, prefill_chunk=chunk)
    wl = wk.make_workload(spec, seed=41)
    if kv == "f32":
        psplit = 0                                  # the generic path takes one range
    dw = dev.upload(wl, prefill_split=psplit)
    dw.setup()
    dw.step()
    torch.cuda.synchronize()
    kp, vp = sup.oracle_pools(wl)
    ref, ref_lse = sup.oracle_prefill(wl, kp, vp)
    check_close(dw.pf["out"], ref, spec, "prefill")
    check_lse(dw.pf["lse"], ref_lse, spec)
    dref, dlse = sup.oracle_decode(wl, kp, vp)
    check_close(dw.out, dref, spec, "decode")


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("psplit", [0, 128])
def test_prefill_schedules_agree(D, psplit):
    """The bf16 prefill kernel reads a tile's LDS operands in one of two
    orders, chosen by the launch's workgroup count.  The same requests with
    128 empty ones added (their workgroups exit at once) cross the threshold;
    the real rows must come out bit for bit the same, and match the oracle."""
    spec = spec_of((9,), 16, 4, D, 32, "bf16", prefill_ctx=(0, 70, 300), prefill_chunk=96)
    wl = wk.make_workload(spec, seed=47)
    dw = dev.upload(wl, prefill_split=psplit)
    dw.setup()
    dw.append_step()
    p = dw.pf
    kp, vp = sup.oracle_pools(wl)
    ref, ref_lse = sup.oracle_prefill(wl, kp, vp)
    outs = []
    for extra in (0, 128):
        R = wl.num_prefill + extra
        cu = torch.cat([p["cu"], p["cu"][-1:].repeat(extra)])
        ctx = torch.cat([p["ctx"], torch.zeros(extra, dtype=torch.int32, device="cuda")])
        bt = torch.cat([p["bt"], torch.full((extra, p["bt"].shape[1]), -1, dtype=torch.int32,
                                            device="cuda")])
        ws = B.prefill_workspace(dw.cache, R, p["q"].shape[0], spec.num_q_heads, p["max_chunk"],
                                 p["max_total"], psplit)
        out = torch.full_like(p["out"], float("nan"))
        lse = torch.full_like(p["lse"], float("nan"))
        B.pkv_paged_attn_chunked_prefill(dw.cache, p["q"], out, cu, ctx, bt, p["max_chunk"],
                                         p["max_total"], float(wl.sm_scale), lse=lse,
                                         split_tokens=psplit, workspace=ws)
        torch.cuda.synchronize()
        check_close(out, ref, spec, f"prefill with {extra} empty requests")
        check_lse(lse, ref_lse, spec)
        outs.append((out, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_prefill_ranges_loose_bound_and_invariance():
    """A loose max_total_len bound (more ranges than any row needs) gives the
    same rows as the exact one; range sizes change only rounding."""
    spec = spec_of((9,), 16, 4, 128, 32, "bf16", prefill_ctx=(0, 300, 700), prefill_chunk=150)
    wl = wk.make_workload(spec, seed=43)
    dw = dev.upload(wl)
    dw.setup()
    dw.append_step()
    p = dw.pf
    kp, vp = sup.oracle_pools(wl)
    ref, ref_lse = sup.oracle_prefill(wl, kp, vp)
    outs = []
    for split, total in ((64, p["max_total"]), (64, p["max_total"] + 400), (256, p["max_total"]),
                         (1024, p["max_total"])):
        total = min(total, wl.pf_block_tables.shape[1] * spec.page_size)
        ws = B.prefill_workspace(dw.cache, wl.num_prefill, p["q"].shape[0], spec.num_q_heads,
                                 p["max_chunk"], total, split)
        out = torch.full_like(p["out"], float("nan"))
        lse = torch.full_like(p["lse"], float("nan"))
        B.pkv_paged_attn_chunked_prefill(dw.cache, p["q"], out, p["cu"], p["ctx"], p["bt"],
                                         p["max_chunk"], total, float(wl.sm_scale), lse=lse,
                                         split_tokens=split, workspace=ws)
        torch.cuda.synchronize()
        check_close(out, ref, spec, f"prefill split {split} bound {total}")
        check_lse(lse, ref_lse, spec)
        outs.append(out)
    assert torch.equal(outs[0], outs[1]), "a looser bound changed the result"


# ---------------------------------------------- the workloads at full size --
# Every sequence and every prefill row of the five workloads (and the int8
# variant of the 70B-shaped one), in the launch configuration the benchmark
# times, against the oracle; the bars apply to the whole output.  The whole K
# and V pools after the step's append are compared byte for byte.  The oracle
# runs on a thread pool (tests/_support.py); the 70B-shaped fp8 workload,
# whose 2.3 GB of codes the oracle encodes by table search, is the slowest
# (about a minute on 16 cores).
def _sample(n, k, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(n, size=min(n, k), replace=False))


def _pools_equal(dw, kp, vp, what):
    for name, gpu, ref in (("K", dw.cache.k_pool, kp), ("V", dw.cache.v_pool, vp)):
        got = dev.storage_to_numpy(gpu)
        assert got.shape == ref.shape
        same = got.view(np.uint8) == ref.view(np.uint8)
        if not same.all():
            bad = np.argwhere(~same.reshape(ref.shape[0], -1).all(axis=1)).ravel()
            raise AssertionError(f"{what}: {name} pool differs in {bad.size} pages, first {bad[:5]}")


def _report(what, gpu, ref, spec):
    g = sup.to_f64(dev.storage_to_numpy(gpu), spec.out_dtype)
    err = np.abs(g - ref)
    print(f"[full-size] {what}: {ref.shape[0]} rows, max |err| {err.max():.3e}, "
          f"mean |err| {err.mean():.3e}", flush=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [2, 3, 4, "4-int8"])
def test_decode_full_size_every_sequence(cfg):
    spec = wk.CONFIGS[cfg] if cfg in wk.CONFIGS else wk.variant(cfg)
    wl = wk.make_workload(spec)
    print(f"[full-size decode] workload {cfg} B={wl.num_seqs} pages={wl.num_pages}", flush=True)
    dw = dev.upload(wl)
    dw.setup()
    dw.mixed_step(side_stream=torch.cuda.Stream())     # the benchmark's launch
    torch.cuda.synchronize()
    kp, vp = sup.oracle_pools(wl)
    _pools_equal(dw, kp, vp, f"workload {cfg}")
    ref, ref_lse = sup.oracle_decode(wl, kp, vp)
    _report(f"workload {cfg} decode", dw.out, ref, spec)
    check_close(dw.out, ref, spec)
    check_lse(dw.lse, ref_lse, spec)


@pytest.mark.timeout(900)
def test_mixed_step_full_size_every_row():
    spec = wk.C5
    wl = wk.make_workload(spec)
    dw = dev.upload(wl)
    dw.setup()
    dw.mixed_step(side_stream=torch.cuda.Stream())     # the benchmark's launch
    torch.cuda.synchronize()
    kp, vp = sup.oracle_pools(wl)
    _pools_equal(dw, kp, vp, "mixed step")
    ref, ref_lse = sup.oracle_decode(wl, kp, vp)
    _report("mixed step decode", dw.out, ref, spec)
    check_close(dw.out, ref, spec, "decode")
    check_lse(dw.lse, ref_lse, spec)
    pref, plse = sup.oracle_prefill(wl, kp, vp)
    _report("mixed step prefill", dw.pf["out"], pref, spec)
    check_close(dw.pf["out"], pref, spec, "prefill")
    check_lse(dw.pf["lse"], plse, spec)


# Mixed steps with an append part whose decode has at least 1024 (sequence,
# range, KV head) workgroups run the decode from a work list (longest ranges
# first) built by one extra workgroup of the append launch.  40 rows of edge
# lengths (empty, one token, page and range boundaries) in 64-token ranges,
# on both decode kernels.
WORKLIST_LENS = (0, 1, 63, 64, 65, 128, 129, 500, 1000, 2047) * 4
WORKLIST_CASES = [
    (WORKLIST_LENS, 32, 8, 128, 32, "bf16"),    # matrix cores, G 4
    (WORKLIST_LENS, 8, 8, 128, 64, "bf16"),     # vector path, MHA
    (WORKLIST_LENS, 64, 8, 128, 64, "fp8"),     # matrix cores, 8-bit codes
    (WORKLIST_LENS, 4, 4, 64, 16, "f32"),       # vector path, fp32
    (WORKLIST_LENS, 4, 2, 128, 32, "int8"),     # vector path, G 2
    (WORKLIST_LENS, 32, 8, 128, 128, "bf16"),   # matrix cores, 128-token pages
    (WORKLIST_LENS, 8, 8, 128, 256, "bf16"),    # vector path, 256-token pages
]


@pytest.mark.parametrize("case", WORKLIST_CASES)
def test_mixed_step_work_list_parity_bits_and_graph(case):
    """The decode of a mixed step run from its work list matches the oracle,
    equals bit for bit the same step as separate calls (whose decode grid
    walks (row, range) itself), and so do replays of the step captured as a
    graph."""
    spec = spec_of(*case)
    wl = wk.make_workload(spec, seed=31)
    kp, vp = sup.oracle_pools(wl)
    ref, ref_lse = sup.oracle_decode(wl, kp, vp)
    dw = dev.upload(wl, split_tokens=max(64, spec.page_size))   # ranges are whole pages
    dw.setup()
    dw.step()
    torch.cuda.synchronize()
    check_close(dw.out, ref, spec)
    check_lse(dw.lse, ref_lse, spec)
    out0, lse0 = dw.out.clone(), dw.lse.clone()
    side = torch.cuda.Stream()

    def clear():
        dw.out.fill_(float("nan"))
        dw.lse.fill_(float("nan"))
        torch.cuda.synchronize()

    clear()
    dw.mixed_step(side_stream=side)
    torch.cuda.synchronize()
    assert torch.equal(dw.out, out0) and torch.equal(dw.lse, lse0)
    # separate calls: the list built on its own, the listed partial pass, the merge
    clear()
    dw.build_work_list()
    dw.decode_partial(listed=True)
    dw.merge()
    torch.cuda.synchronize()
    assert torch.equal(dw.out, out0) and torch.equal(dw.lse, lse0)
    g = dw.capture_step(side_stream=side)
    for rep in range(3):
        clear()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dw.out, out0) and torch.equal(dw.lse, lse0), f"graph replay {rep}"
        dw.step()                                   # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("shared", [True, False])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_sequential_mixed_step_shared_workspace(shared, kv):
    """The mixed step with no side stream runs append, decode (from its work
    list: 40 rows x 32 ranges x 8 KV heads) and a multi-range prefill one
    after another on one stream.  With one workspace buffer shared by the
    decode and the prefill, and with separate ones, it matches the oracle
    and equals the separate calls bit for bit."""
    spec = spec_of(WORKLIST_LENS, 32, 8, 128, 32, kv, prefill_ctx=(0, 40, 200), prefill_chunk=96)
    wl = wk.make_workload(spec, seed=43)
    kp, vp = sup.oracle_pools(wl)
    ref, ref_lse = sup.oracle_decode(wl, kp, vp)
    pref, plse = sup.oracle_prefill(wl, kp, vp)
    dw = dev.upload(wl, split_tokens=64, prefill_split=64)
    p = dw.pf
    assert dw.workspace is not None and p["ws"] is not None
    dw.setup()
    dw.step()                                       # separate calls
    torch.cuda.synchronize()
    want = [t.clone() for t in (dw.out, dw.lse, p["out"], p["lse"])]
    if shared:
        n = max(dw.workspace.numel(), p["ws"].numel())
        ws_d = ws_p = torch.empty(n, dtype=torch.uint8, device="cuda")
    else:
        ws_d, ws_p = dw.workspace, p["ws"]
    a = dw.step_batch
    batches = (B.append_batch(a.k, a.v, a.cu, a.start, a.bt),
               B.decode_batch(dw.q, dw.out, dw.bt, dw.lens, dw.max_len, lse=dw.lse,
                              split_tokens=dw.split_tokens, workspace=ws_d),
               B.prefill_batch(p["q"], p["out"], p["cu"], p["ctx"], p["bt"], p["max_chunk"],
                               p["max_total"], lse=p["lse"], split_tokens=p["split"],
                               workspace=ws_p))
    for t in (dw.out, dw.lse, p["out"], p["lse"]):
        t.fill_(float("nan"))
    B.pkv_mixed_step(dw.cache, *batches, float(wl.sm_scale), side_stream=None)
    torch.cuda.synchronize()
    check_close(dw.out, ref, spec, "decode")
    check_lse(dw.lse, ref_lse, spec)
    check_close(p["out"], pref, spec, "prefill")
    check_lse(p["lse"], plse, spec)
    for got, w in zip((dw.out, dw.lse, p["out"], p["lse"]), want):
        assert torch.equal(got, w)
    # concurrent parts must not share a workspace
    if shared:
        with pytest.raises(B.PkvError):
            B.pkv_mixed_step(dw.cache, *batches, float(wl.sm_scale),
                             side_stream=torch.cuda.Stream())


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_mixed_step_work_list_full_size_bits(cfg):
    """At full size, the mixed step (decode from its work list, beside the
    prefill for the mixed workload) reproduces the separate calls' bits."""
    wl = wk.make_workload(wk.CONFIGS[cfg])
    dw = dev.upload(wl)
    dw.setup()
    dw.step()
    torch.cuda.synchronize()
    ref = [dw.out.clone(), dw.lse.clone()] + ([dw.pf["out"].clone(), dw.pf["lse"].clone()]
                                              if dw.pf else [])
    outs = [dw.out, dw.lse] + ([dw.pf["out"], dw.pf["lse"]] if dw.pf else [])
    for t in outs:
        t.fill_(float("nan"))
    dw.mixed_step(side_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    for a, b in zip(outs, ref):
        assert torch.equal(a, b)


# ---------------------------------------------------------- graph replay ----
@pytest.mark.parametrize("cfg", [1, 5])
def test_step_graph_replays_match_eager(cfg):
    """The captured step, replayed several times with eager work in between,
    reproduces the eager step bit for bit (outputs cleared before each replay)."""
    wl = wk.make_workload(wk.CONFIGS[cfg]) if cfg == 1 else wk.make_workload(
        spec_of((40, 300, 1000), 32, 8, 128, 32, "bf16", prefill_ctx=(0, 100), prefill_chunk=70),
        seed=5)
    dw = dev.upload(wl)
    dw.setup()
    dw.step()
    torch.cuda.synchronize()
    ref_out, ref_lse = dw.out.clone(), dw.lse.clone()
    ref_pf = dw.pf["out"].clone() if dw.pf else None
    g = dw.capture_step()
    for rep in range(3):
        dw.out.zero_()
        dw.lse.zero_()
        if dw.pf:
            dw.pf["out"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dw.out, ref_out), f"replay {rep}: decode output differs"
        assert torch.equal(dw.lse, ref_lse)
        if dw.pf:
            assert torch.equal(dw.pf["out"], ref_pf), f"replay {rep}: prefill output differs"
        dw.step()                                   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(dw.out, ref_out)
    kp, vp = sup.oracle_pools(wl)
    ref, _ = sup.oracle_decode(wl, kp, vp)
    check_close(dw.out, ref, wl.spec)


@pytest.mark.parametrize("cfg", [1, 5])
def test_mixed_step_call_and_overlapped_graph_match_eager(cfg):
    """pkv_mixed_step with the prefill forked onto a second stream, called
    directly and replayed from a captured graph, gives the eager step's bits."""
    wl = wk.make_workload(wk.CONFIGS[cfg]) if cfg == 1 else wk.make_workload(
        spec_of((40, 300, 1000), 32, 8, 128, 32, "bf16", prefill_ctx=(0, 100, 700),
                prefill_chunk=70), seed=6)
    dw = dev.upload(wl, prefill_split=64)
    dw.setup()
    dw.step()
    torch.cuda.synchronize()
    ref = [dw.out.clone(), dw.lse.clone()] + ([dw.pf["out"].clone(), dw.pf["lse"].clone()]
                                              if dw.pf else [])

    def outs():
        return [dw.out, dw.lse] + ([dw.pf["out"], dw.pf["lse"]] if dw.pf else [])

    def clear():
        for t in outs():
            t.fill_(float("nan"))
        torch.cuda.synchronize()

    side = torch.cuda.Stream()
    for rep in range(2):
        clear()
        dw.mixed_step(side_stream=side)
        torch.cuda.synchronize()
        for a, b in zip(outs(), ref):
            assert torch.equal(a, b), f"mixed_step call {rep} differs from the eager step"
    g = dw.capture_step(side_stream=side)
    for rep in range(3):
        clear()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs(), ref):
            assert torch.equal(a, b), f"graph replay {rep} differs from the eager step"
        dw.step()                                   # eager work between replays
        torch.cuda.synchronize()


# ---------------------------------------------- context attention (FMHA) --
CONTEXT_CASES = [
    # lens, Hq, Hkv, D, split
    ((1, 31, 200, 700), 32, 8, 128, 0),
    ((1, 31, 200, 700), 32, 8, 128, 64),                   # many key ranges + merge
    ((5, 100, 129), 8, 8, 64, 0),                          # G 1, head_dim 64
    ((257,), 16, 1, 128, 128),                             # G 16
    ((64, 3), 12, 4, 64, 64),                              # G 3
    ((300, 45), 16, 4, 64, 0),                             # head_dim 64: 1..10 tiles per block, ragged
    ((300, 45), 16, 4, 64, 128),                           # ranges of 1..4 tiles around the pipeline depth
]


def _ctx_inputs(lens, Hq, Hkv, D, seed):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    bits = [wk.bf16_bits_rne(rng.standard_normal(sh, dtype=np.float32))
            for sh in ((T, Hq, D), (T, Hkv, D), (T, Hkv, D))]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return bits, cu


@pytest.mark.parametrize("case", CONTEXT_CASES)
def test_context_fmha_parity(case):
    lens, Hq, Hkv, D, split = case
    (q, k, v), cu = _ctx_inputs(lens, Hq, Hkv, D, 71)
    scale = 1.0 / np.sqrt(D)
    qd, kd, vd = (dev._dev(x, "bf16", "cuda") for x in (q, k, v))
    out = torch.full_like(qd, float("nan"))
    lse = torch.full(qd.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    cud = dev._dev(cu, "i32", "cuda")
    ws = B.context_workspace(len(lens), q.shape[0], Hq, Hkv, D, max(lens), split)
    B.pkv_context_fmha(qd, kd, vd, out, cud, max(lens), scale, lse=lse, split_tokens=split,
                       workspace=ws)
    torch.cuda.synchronize()
    ref, ref_lse = oa.context_attention(q, k, v, "bf16", cu, scale)
    spec = spec_of((1,), Hq, Hkv, D, 16, "bf16")
    check_close(out, ref, spec, "context")
    check_lse(lse, ref_lse, spec)


@pytest.mark.parametrize("split", [0, 4096])
def test_context_fmha_full_size_sampled(split):
    """Whole-prompt attention at the long-prompt benchmark shape (4 prompts of
    8192 tokens, 32/8 heads, head_dim 128): the default (one key range per
    row) and 4096-key ranges (rows past the first range combine two
    partials), checked on sampled rows: tile, range and prompt boundaries
    plus random rows."""
    lens, Hq, Hkv, D = (8192, 8192, 8192, 8192), 32, 8, 128
    (q, k, v), cu = _ctx_inputs(lens, Hq, Hkv, D, 73)
    print(f"[full-size context] {len(lens)} x {lens[0]} tokens, split {split}", flush=True)
    scale = 1.0 / np.sqrt(D)
    qd, kd, vd = (dev._dev(x, "bf16", "cuda") for x in (q, k, v))
    out = torch.full_like(qd, float("nan"))
    lse = torch.full(qd.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    cud = dev._dev(cu, "i32", "cuda")
    ws = B.context_workspace(len(lens), q.shape[0], Hq, Hkv, D, max(lens), split)
    B.pkv_context_fmha(qd, kd, vd, out, cud, max(lens), scale, lse=lse, split_tokens=split,
                       workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    local = [0, 1, 31, 32, 1023, 4095, 4096, 4097, 4927, 4928, 8190, 8191]
    rows = np.unique(np.concatenate([[int(cu[s]) + i for s in (0, 3) for i in local],
                                     _sample(int(cu[-1]), 8, 74)]))
    ref, ref_lse = oa.context_attention(q, k, v, "bf16", cu, scale, rows=rows)
    spec = spec_of((1,), Hq, Hkv, D, 16, "bf16")
    sel = torch.from_numpy(rows).cuda()
    check_close(out[sel], ref, spec, "context (full size)")
    check_lse(lse[sel], ref_lse, spec)


def test_context_fmha_bit_identical_to_prefill_with_nothing_cached():
    """The same kernel over contiguous K/V and over pages (whole prompts as
    one chunk, ctx_before = 0, same key ranges) gives the same bits."""
    lens, Hq, Hkv, D, P, split = (3, 150, 400), 32, 8, 128, 32, 128
    (q, k, v), cu = _ctx_inputs(lens, Hq, Hkv, D, 72)
    scale = 1.0 / np.sqrt(D)
    qd, kd, vd = (dev._dev(x, "bf16", "cuda") for x in (q, k, v))
    cud = dev._dev(cu, "i32", "cuda")
    T, R = q.shape[0], len(lens)
    out_c = torch.empty_like(qd)
    lse_c = torch.empty(qd.shape[:2], dtype=torch.float32, device="cuda")
    ws = B.context_workspace(R, T, Hq, Hkv, D, max(lens), split)
    B.pkv_context_fmha(qd, kd, vd, out_c, cud, max(lens), scale, lse=lse_c, split_tokens=split,
                       workspace=ws)
    # the same K/V in pages (reversed page order per request), appended by the library
    pages = [-(-n // P) for n in lens]
    stride = max(pages)
    bt = np.full((R, stride), -1, np.int32)
    nxt = 0
    for r, n in enumerate(pages):
        bt[r, :n] = np.arange(nxt, nxt + n)[::-1]
        nxt += n
    kp = dev.poisoned_pool(nxt, Hkv, P, D, "bf16", "cuda")
    vp = dev.poisoned_pool(nxt, Hkv, P, D, "bf16", "cuda")
    cache = B.PagedCache(kp, vp)
    btd = dev._dev(bt, "i32", "cuda")
    ctx = torch.zeros(R, dtype=torch.int32, device="cuda")
    B.pkv_kv_cache_append(cache, kd, vd, cud, ctx, btd)
    out_p = torch.empty_like(qd)
    lse_p = torch.empty_like(lse_c)
    wsp = B.prefill_workspace(cache, R, T, Hq, max(lens), max(lens), split)
    B.pkv_paged_attn_chunked_prefill(cache, qd, out_p, cud, ctx, btd, max(lens), max(lens),
                                     scale, lse=lse_p, split_tokens=split, workspace=wsp)
    torch.cuda.synchronize()
    assert torch.equal(out_c, out_p) and torch.equal(lse_c, lse_p)
