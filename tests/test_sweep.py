"""GPU parity over seeded random batches (bat_attn_prefill through the C ABI
against the CPU oracle, every output compared).

The targeted cases in test_parity name one axis at a time.  Each case here
draws all of them together from its own seed: dtype and head dim, batch
size and heads, every request's suffix and prefix length (zero included),
its prefix mode (user history or gathered items, Bat page, "This paper's
idea"), the user pool's page size, and the launch choices a caller can
force through the environment: workgroup shape (BAT_WAVES), gather form
(BAT_GATHER) and a prefix split with its log-sum-exp merge (BAT_SPLIT_CHUNK).
Bars as in test_parity: max-abs 1e-5 (fp32) / 2e-2 with relative RMS 1e-2
(bf16) on out, 1e-5 / 1e-3 on lse.
"""
import numpy as np
import pytest

from helpers import as_f64, check_close, oracle_full
from prefix_reuse_attention_amd import workloads as W

N_CASES = 24


def draw_case(case):
    """The workload and the environment of sweep case `case` (host only)."""
    rng = np.random.default_rng(9000 + case)
    dtype = str(rng.choice(["bf16", "bf16", "f32"]))
    D = int(rng.choice([64, 128] if dtype == "bf16" else [32, 64, 128]))
    B = int(rng.integers(1, 6))
    H = int(rng.choice([1, 2, 3]))
    n_s = np.where(rng.random(B) < 0.2, 0, rng.integers(1, 520, size=B))
    n_s[rng.integers(B)] = rng.integers(1, 520)  # at least one row to write
    mode = rng.integers(0, 2, size=B).astype(np.uint8)
    n_p = np.where(rng.random(B) < 0.15, 0, rng.integers(1, 2400, size=B))
    n_p = np.where(mode == W.ITEM, (n_p // W.ITEM_TOKENS) * W.ITEM_TOKENS, n_p)
    bs = int(rng.choice([1, 2, 4, 16, 64, 128]))
    env = {
        "BAT_WAVES": str(rng.choice(["", "4", "8"])),
        "BAT_GATHER": str(rng.choice(["", "flat"])),
        "BAT_SPLIT_CHUNK": str(rng.choice(["", "", "256", "704"])),
    }
    q_scale = float(rng.choice([1.0, 1.0, 4.0]))
    wl = W.make_custom(dtype=dtype, H=H, D=D, n_s=n_s, n_p=n_p, mode=mode, seed=9100 + case,
                       user_block_size=bs, num_items=700, q_scale=q_scale,
                       name=f"sweep{case}")
    return wl, {k: v for k, v in env.items() if v}


def test_sweep_draws_cover_the_axes():
    """Host only: the drawn cases reach both dtypes and head dims, both
    prefix modes, per-key and whole-page pools, each forced launch choice,
    and empty suffixes and prefixes."""
    seen = set()
    for c in range(N_CASES):
        wl, env = draw_case(c)
        seen.add(("dtype", wl.dtype))
        seen.add(("D", wl.D))
        seen.update(("mode", int(m)) for m in wl.mode)
        seen.add(("bs<64", int(wl.user_block_size) < 64))
        seen.update(("env", k) for k in env)
        if (wl.n_s == 0).any():
            seen.add("empty suffix")
        if (wl.n_p == 0).any():
            seen.add("empty prefix")
    for want in [("dtype", "bf16"), ("dtype", "f32"), ("D", 64), ("D", 128), ("mode", 0),
                 ("mode", 1), ("bs<64", True), ("bs<64", False), ("env", "BAT_WAVES"),
                 ("env", "BAT_GATHER"), ("env", "BAT_SPLIT_CHUNK"), "empty suffix",
                 "empty prefix"]:
        assert want in seen, want


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(N_CASES))
def test_random_batch(gpu_ready, monkeypatch, case):
    from prefix_reuse_attention_amd.device import DeviceWorkload, to_host
    import torch
    wl, env = draw_case(case)
    for k in ("BAT_WAVES", "BAT_GATHER", "BAT_SPLIT_CHUNK"):
        monkeypatch.delenv(k, raising=False)
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    print(f"[sweep] case {case}: dtype={wl.dtype} B={wl.B} H={wl.H} D={wl.D} "
          f"bs={wl.user_block_size} n_s={wl.n_s.tolist()} n_p={wl.n_p.tolist()} "
          f"mode={wl.mode.tolist()} env={env}", flush=True)
    dw = DeviceWorkload(wl)
    out, lse = dw.run()
    torch.cuda.synchronize()
    got = as_f64(to_host(out, wl.dtype), wl.dtype)
    lse = lse.cpu().numpy().astype(np.float64)
    ref_o, ref_l = oracle_full(wl)
    check_close(got, ref_o, wl.dtype)
    tol = 1e-5 if wl.dtype == "f32" else 1e-3
    assert np.abs(lse - ref_l).max() <= tol, f"lse max-abs {np.abs(lse - ref_l).max():.3e}"


# ---- the other entry points, drawn the same way ---------------------------

N_GQA, N_ISO, N_ROWS, N_FP8 = 8, 8, 6, 6


def _lengths(rng, B, max_s, max_p, mode, T=1):
    n_s = np.where(rng.random(B) < 0.2, 0, rng.integers(1, max_s, size=B)) * T
    n_s[rng.integers(B)] = rng.integers(1, max_s) * T
    n_p = np.where(rng.random(B) < 0.15, 0, rng.integers(1, max_p, size=B))
    n_p = np.where(mode == W.ITEM, (n_p // W.ITEM_TOKENS) * W.ITEM_TOKENS, n_p)
    return n_s, n_p


def draw_gqa(case):
    """Grouped heads: H_kv key/value heads, hg query heads each."""
    rng = np.random.default_rng(9300 + case)
    dtype = str(rng.choice(["bf16", "bf16", "f32"]))
    D = int(rng.choice([64, 128] if dtype == "bf16" else [32, 64, 128]))
    H_kv, hg = int(rng.choice([1, 2, 4])), int(rng.choice([2, 4, 8]))
    B = int(rng.integers(1, 5))
    mode = rng.integers(0, 2, size=B).astype(np.uint8)
    n_s, n_p = _lengths(rng, B, 520, 2000, mode)
    env = {"BAT_WAVES": str(rng.choice(["", "4", "8"])),
           "BAT_SPLIT_CHUNK": str(rng.choice(["", "", "512"]))}
    wl = W.make_custom(dtype=dtype, H=H_kv, D=D, n_s=n_s, n_p=n_p, mode=mode, seed=9400 + case,
                       user_block_size=int(rng.choice([4, 16, 64, 128])), num_items=600,
                       name=f"sweep_gqa{case}")
    return wl, H_kv * hg, {k: v for k, v in env.items() if v}


def draw_isolated(case):
    """Candidate-isolated rows: every request's suffix is whole candidates of T tokens."""
    rng = np.random.default_rng(9500 + case)
    dtype = str(rng.choice(["bf16", "bf16", "f32"]))
    D = int(rng.choice([64, 128] if dtype == "bf16" else [32, 64, 128]))
    T = (1, 2, 4, 8)[case % 4]
    B = int(rng.integers(1, 5))
    mode = rng.integers(0, 2, size=B).astype(np.uint8)
    n_s, n_p = _lengths(rng, B, 400 // T + 2, 2000, mode, T)
    env = {"BAT_WAVES": str(rng.choice(["", "4", "8"]))}
    wl = W.make_custom(dtype=dtype, H=int(rng.choice([1, 2])), D=D, n_s=n_s, n_p=n_p, mode=mode,
                       seed=9600 + case, user_block_size=int(rng.choice([2, 16, 64])),
                       num_items=600, q_scale=float(rng.choice([1.0, 4.0])),
                       name=f"sweep_iso{case}")
    return wl, T, {k: v for k, v in env.items() if v}


def draw_prefix_rows(case):
    """Prefix rows: each request's prefix group attends within itself."""
    rng = np.random.default_rng(9700 + case)
    dtype = str(rng.choice(["bf16", "f32"]))
    D = int(rng.choice([64, 128] if dtype == "bf16" else [32, 64, 128]))
    B = int(rng.integers(1, 6))
    lens = np.where(rng.random(B) < 0.2, 0, rng.integers(1, 1500, size=B))
    lens[rng.integers(B)] = rng.integers(1, 1500)
    return dtype, D, int(rng.choice([1, 2, 3])), lens, float(rng.choice([1.0, 4.0]))


def draw_fp8(case):
    """E4M3 pools read back into bf16 tiles."""
    rng = np.random.default_rng(9800 + case)
    D = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 5))
    mode = rng.integers(0, 2, size=B).astype(np.uint8)
    n_s, n_p = _lengths(rng, B, 520, 2000, mode)
    env = {"BAT_WAVES": str(rng.choice(["", "4", "8"])),
           "BAT_SPLIT_CHUNK": str(rng.choice(["", "", "512"]))}
    wl = W.make_custom(dtype="bf16", H=int(rng.choice([1, 2])), D=D, n_s=n_s, n_p=n_p, mode=mode,
                       seed=9900 + case, user_block_size=int(rng.choice([16, 64, 128])),
                       num_items=600, name=f"sweep_fp8_{case}")
    return wl, {k: v for k, v in env.items() if v}


def _set_env(monkeypatch, env):
    for k in ("BAT_WAVES", "BAT_GATHER", "BAT_SPLIT_CHUNK"):
        monkeypatch.delenv(k, raising=False)
    for k, v in env.items():
        monkeypatch.setenv(k, v)


def test_other_draws_are_valid():
    """Host only: every drawn case is a valid call (whole candidates per
    request, item prefixes of whole items, at least one row), and the draws
    reach both dtypes, every T and both workgroup shapes."""
    seen = set()
    for c in range(N_GQA):
        wl, H, env = draw_gqa(c)
        assert H % wl.H == 0 and wl.n_s.sum() > 0
        seen.update({("gqa", wl.dtype), ("gqa_hg", H // wl.H)})
    for c in range(N_ISO):
        wl, T, env = draw_isolated(c)
        assert (wl.n_s % T == 0).all() and wl.n_s.sum() > 0
        seen.update({("iso", wl.dtype), ("T", T)})
    for c in range(N_ROWS):
        dtype, D, H, lens, qs = draw_prefix_rows(c)
        assert lens.sum() > 0
        seen.add(("rows", dtype))
    for c in range(N_FP8):
        wl, env = draw_fp8(c)
        assert wl.n_s.sum() > 0
        seen.add(("fp8", wl.D))
    for want in [("gqa", "bf16"), ("gqa", "f32"), ("iso", "bf16"), ("iso", "f32"), ("T", 1),
                 ("T", 2), ("T", 8), ("rows", "bf16"), ("rows", "f32"), ("fp8", 64),
                 ("fp8", 128)]:
        assert want in seen, want


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(N_GQA))
def test_random_gqa(gpu_ready, monkeypatch, case):
    from test_gqa import _compare as gqa_compare
    wl, H, env = draw_gqa(case)
    _set_env(monkeypatch, env)
    print(f"[sweep] gqa case {case}: env={env}", flush=True)
    gqa_compare(wl, H)


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(N_ISO))
def test_random_isolated(gpu_ready, monkeypatch, case):
    from test_isolated import _compare as iso_compare
    wl, T, env = draw_isolated(case)
    _set_env(monkeypatch, env)
    print(f"[sweep] isolated case {case}: env={env}", flush=True)
    iso_compare(wl, T)


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(N_ROWS))
def test_random_prefix_rows(gpu_ready, case):
    import oracle
    from test_prefix_rows import _inputs, _prefix_rows_gpu
    dtype, D, H, lens, q_scale = draw_prefix_rows(case)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    print(f"[sweep] prefix rows case {case}: {dtype} D={D} H={H} lens={lens.tolist()} "
          f"q_scale={q_scale}", flush=True)
    q, k, v = _inputs(9750 + case, int(cu[-1]), H, D, dtype, q_scale)
    got, got_lse, scale = _prefix_rows_gpu(q, k, v, cu, dtype)
    ref, ref_lse = oracle.prefix_rows(q, k, v, cu, scale)
    check_close(got, ref, dtype)
    tol = 1e-5 if dtype == "f32" else 1e-3
    assert np.abs(got_lse - ref_lse).max() <= tol


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(N_FP8))
def test_random_fp8(gpu_ready, monkeypatch, case):
    from test_fp8 import _fp8_reference, _run_fp8
    wl, env = draw_fp8(case)
    _set_env(monkeypatch, env)
    print(f"[sweep] fp8 case {case}: D={wl.D} bs={wl.user_block_size} n_s={wl.n_s.tolist()} "
          f"n_p={wl.n_p.tolist()} mode={wl.mode.tolist()} env={env}", flush=True)
    got, lse, _ = _run_fp8(wl)
    ref_o, ref_l = _fp8_reference(wl)
    check_close(got, ref_o, "bf16")
    assert np.abs(lse - ref_l).max() <= 1e-3


# ---- many small requests ---------------------------------------------------

N_WIDE = 6


def draw_wide(case):
    """Hundreds of short requests: the planner's item list, the per-request
    metadata and the block-table rows at batch sizes the other draws do not
    reach."""
    rng = np.random.default_rng(10100 + case)
    dtype = ("bf16", "f32")[case % 2]
    D = int(rng.choice([64, 128]))
    B = int(rng.integers(64, 513))
    mode = rng.integers(0, 2, size=B).astype(np.uint8)
    n_s = np.where(rng.random(B) < 0.25, 0, rng.integers(1, 48, size=B))
    n_s[rng.integers(B)] = rng.integers(1, 48)
    n_p = np.where(rng.random(B) < 0.2, 0, rng.integers(1, 320, size=B))
    n_p = np.where(mode == W.ITEM, (n_p // W.ITEM_TOKENS) * W.ITEM_TOKENS, n_p)
    wl = W.make_custom(dtype=dtype, H=int(rng.choice([1, 4, 8])), D=D, n_s=n_s, n_p=n_p,
                       mode=mode, seed=10200 + case, user_block_size=int(rng.choice([4, 16, 64])),
                       num_items=2000, name=f"sweep_wide{case}")
    return wl


def test_wide_draws_are_valid():
    """Host only: the wide draws reach both dtypes and more than 256 requests."""
    wls = [draw_wide(c) for c in range(N_WIDE)]
    assert {wl.dtype for wl in wls} == {"bf16", "f32"}
    assert max(wl.B for wl in wls) > 256 and all(wl.n_s.sum() > 0 for wl in wls)


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(N_WIDE))
def test_random_wide_batch(gpu_ready, monkeypatch, case):
    from prefix_reuse_attention_amd.device import DeviceWorkload, to_host
    import torch
    _set_env(monkeypatch, {})
    wl = draw_wide(case)
    print(f"[sweep] wide case {case}: dtype={wl.dtype} B={wl.B} H={wl.H} D={wl.D} "
          f"bs={wl.user_block_size} total_s={int(wl.n_s.sum())} max_p={int(wl.n_p.max())}",
          flush=True)
    dw = DeviceWorkload(wl)
    out, lse = dw.run()
    torch.cuda.synchronize()
    got = as_f64(to_host(out, wl.dtype), wl.dtype)
    lse = lse.cpu().numpy().astype(np.float64)
    ref_o, ref_l = oracle_full(wl)
    check_close(got, ref_o, wl.dtype)
    tol = 1e-5 if wl.dtype == "f32" else 1e-3
    assert np.abs(lse - ref_l).max() <= tol, f"lse max-abs {np.abs(lse - ref_l).max():.3e}"


# ---- long prefixes, few requests: the automatic prefix split ----------------

N_LONG = 6


def draw_long(case):
    """A few requests over prefixes of up to 16k keys: too few work items to
    fill the GPU, so the library splits the prefixes by itself (no forced
    chunk length) and merges the partials."""
    rng = np.random.default_rng(10300 + case)
    dtype = ("bf16", "bf16", "f32")[case % 3]
    D = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 4))
    mode = rng.integers(0, 2, size=B).astype(np.uint8)
    n_s = rng.integers(1, 600, size=B)
    n_p = rng.integers(2048, 16385, size=B)
    n_p = np.where(mode == W.ITEM, (n_p // W.ITEM_TOKENS) * W.ITEM_TOKENS, n_p)
    wl = W.make_custom(dtype=dtype, H=int(rng.choice([1, 2])), D=D, n_s=n_s, n_p=n_p, mode=mode,
                       seed=10400 + case, user_block_size=int(rng.choice([16, 64, 128])),
                       num_items=5000, name=f"sweep_long{case}")
    return wl


def test_long_draws_split():
    """Host only: the library's plan splits every long draw (its workspace
    holds chunk partials, which it does not with splitting switched off)."""
    import os
    from prefix_reuse_attention_amd import api
    for c in range(N_LONG):
        wl = draw_long(c)
        dt = api.BAT_BF16 if wl.dtype == "bf16" else api.BAT_F32
        args = (wl.B, wl.H, wl.D, dt, int(wl.total_s), int(wl.n_s.max()), int(wl.n_p.max()))
        split_ws = api.workspace_size(*args)
        os.environ["BAT_SPLIT_CHUNK"] = "100000000"
        try:
            whole_ws = api.workspace_size(*args)
        finally:
            del os.environ["BAT_SPLIT_CHUNK"]
        assert split_ws - whole_ws >= 2 * wl.total_s * wl.H * wl.D * 4, (c, split_ws, whole_ws)


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(N_LONG))
def test_random_long_prefixes(gpu_ready, monkeypatch, case):
    from prefix_reuse_attention_amd.device import DeviceWorkload, to_host
    import torch
    _set_env(monkeypatch, {})
    wl = draw_long(case)
    print(f"[sweep] long case {case}: dtype={wl.dtype} B={wl.B} H={wl.H} D={wl.D} "
          f"bs={wl.user_block_size} n_s={wl.n_s.tolist()} n_p={wl.n_p.tolist()} "
          f"mode={wl.mode.tolist()}", flush=True)
    dw = DeviceWorkload(wl)
    out, lse = dw.run()
    torch.cuda.synchronize()
    got = as_f64(to_host(out, wl.dtype), wl.dtype)
    lse = lse.cpu().numpy().astype(np.float64)
    ref_o, ref_l = oracle_full(wl)
    check_close(got, ref_o, wl.dtype)
    tol = 1e-5 if wl.dtype == "f32" else 1e-3
    assert np.abs(lse - ref_l).max() <= tol, f"lse max-abs {np.abs(lse - ref_l).max():.3e}"


# ---- grouped heads and fp8 pools over long prefixes (automatic split) ------

N_LONG_GQA, N_LONG_FP8 = 3, 3


def draw_long_gqa(case):
    rng = np.random.default_rng(10500 + case)
    D = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 4))
    mode = rng.integers(0, 2, size=B).astype(np.uint8)
    n_s = rng.integers(1, 600, size=B)
    n_p = rng.integers(4096, 16385, size=B)
    n_p = np.where(mode == W.ITEM, (n_p // W.ITEM_TOKENS) * W.ITEM_TOKENS, n_p)
    H_kv = int(rng.choice([1, 2]))
    wl = W.make_custom(dtype="bf16", H=H_kv, D=D, n_s=n_s, n_p=n_p, mode=mode,
                       seed=10600 + case, user_block_size=64, num_items=5000,
                       name=f"sweep_long_gqa{case}")
    return wl, H_kv * int(rng.choice([2, 4]))


def draw_long_fp8(case):
    rng = np.random.default_rng(10700 + case)
    D = (64, 128, 64)[case % 3]
    B = int(rng.integers(1, 4))
    mode = rng.integers(0, 2, size=B).astype(np.uint8)
    n_s = rng.integers(1, 600, size=B)
    n_p = rng.integers(4096, 16385, size=B)
    n_p = np.where(mode == W.ITEM, (n_p // W.ITEM_TOKENS) * W.ITEM_TOKENS, n_p)
    return W.make_custom(dtype="bf16", H=int(rng.choice([1, 2])), D=D, n_s=n_s, n_p=n_p,
                         mode=mode, seed=10800 + case, user_block_size=64, num_items=5000,
                         name=f"sweep_long_fp8_{case}")


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(N_LONG_GQA))
def test_random_long_gqa(gpu_ready, monkeypatch, case):
    from test_gqa import _compare as gqa_compare
    _set_env(monkeypatch, {})
    wl, H = draw_long_gqa(case)
    print(f"[sweep] long gqa case {case}: H={H} H_kv={wl.H} D={wl.D}", flush=True)
    gqa_compare(wl, H)


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(N_LONG_FP8))
def test_random_long_fp8(gpu_ready, monkeypatch, case):
    from test_fp8 import _fp8_reference, _run_fp8
    _set_env(monkeypatch, {})
    wl = draw_long_fp8(case)
    print(f"[sweep] long fp8 case {case}: D={wl.D} n_s={wl.n_s.tolist()} n_p={wl.n_p.tolist()} "
          f"mode={wl.mode.tolist()}", flush=True)
    got, lse, _ = _run_fp8(wl)
    ref_o, ref_l = _fp8_reference(wl)
    check_close(got, ref_o, "bf16")
    assert np.abs(lse - ref_l).max() <= 1e-3
