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
