"""GPU parity: candidate-isolated suffix rows (bat_attn_prefill_isolated)
against the oracle, through the C ABI.

Each suffix row sees its request's prefix and the T tokens of its own
candidate.  Cases: every supported T, both bf16 head dims and fp32, user and
item prefixes in one batch, empty prefixes and empty suffixes, the four- and
eight-wave kernels (the ping-pong kernel), the batch of single-token
candidates of the 1024-history configuration on sampled rows, and
single-token candidates on the ping-pong kernel, which folds each row's own
key into its prefix result in one launch (ragged rows, a request with no
prefix, user and item prefixes, and the 8k-history shape on sampled rows).
Every expected value comes from the oracle.
"""
import numpy as np
import pytest

import oracle
from helpers import as_f64, assemble_prefix, check_close
from prefix_reuse_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


def _run_isolated(wl, T):
    import torch
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd.device import DeviceWorkload, to_host
    dw = DeviceWorkload(wl)
    out, lse = api.attn_prefill_isolated(dw.q, dw.k, dw.v, dw.cu_s, dw.prefix_lens,
                                         dw.prefix_mode, dw.block_table, T, dw.user_pool,
                                         dw.item_pool, wl.scale, dw.max_s, dw.max_p,
                                         want_lse=True)
    torch.cuda.synchronize()
    return as_f64(to_host(out, wl.dtype), wl.dtype), lse.cpu().numpy().astype(np.float64)


def _compare(wl, T):
    print(f"[isolated] {wl.name} dtype={wl.dtype} D={wl.D} T={T} n_s={wl.n_s.tolist()} "
          f"n_p={wl.n_p.tolist()}", flush=True)
    got, lse = _run_isolated(wl, T)
    k_p, v_p, cu_p = assemble_prefix(wl)
    ref, ref_lse = oracle.prefill_isolated(wl.q, wl.k_s, wl.v_s, wl.cu_s, k_p, v_p, cu_p, T,
                                           wl.scale)
    check_close(got, ref, wl.dtype)
    tol = 1e-5 if wl.dtype == "f32" else 1e-3
    assert np.abs(lse - ref_lse).max() <= tol


@pytest.mark.parametrize("T", [1, 2, 4, 8])
@pytest.mark.parametrize("D", [64, 128])
def test_isolated_bf16_mixed(gpu_ready, T, D):
    wl = W.make_custom(dtype="bf16", H=2, D=D, n_s=[8, 136, 0, 64, 8 * 9],
                       n_p=[0, 200, 100, 4, 129], mode=[W.USER, W.USER, W.ITEM, W.ITEM, W.USER],
                       seed=90 + T + D, num_items=300, name=f"iso_bf16_T{T}_D{D}")
    _compare(wl, T)


@pytest.mark.parametrize("D", [32, 128])
def test_isolated_fp32(gpu_ready, D):
    wl = W.make_custom(dtype="f32", H=3, D=D, n_s=[2, 70, 128], n_p=[0, 33, 200],
                       mode=[W.USER, W.USER, W.ITEM], seed=110 + D, user_block_size=16,
                       num_items=80, name=f"iso_f32_D{D}")
    _compare(wl, 2)


@pytest.mark.parametrize("D", [64, 128])
def test_isolated_eight_wave_items(gpu_ready, D):
    """Long suffixes: 256-row items (eight waves, the ping-pong kernel)
    writing prefix partials, a ragged last row tile."""
    wl = W.make_custom(dtype="bf16", H=2, D=D, n_s=[512, 264], n_p=[700, 1031],
                       mode=[W.USER, W.USER], seed=120 + D, name=f"iso_w8_D{D}")
    _compare(wl, 4)


def test_isolated_single_token_candidates_1024_history(gpu_ready):
    """32 requests x 256 single-token candidates over a 1024-token history
    (H=8, D=64, bf16), on sampled (row, head) pairs."""
    wl = W.make_config(2)
    T = 1
    print("[isolated] config 2 shape, T=1, sampled", flush=True)
    got, lse = _run_isolated(wl, T)
    rng = np.random.default_rng(130)
    rows = np.concatenate([rng.integers(0, wl.total_s, 150), [0, wl.total_s - 1]])
    rows = rows.astype(np.int32)
    heads = rng.integers(0, wl.H, len(rows)).astype(np.int32)
    req = np.searchsorted(wl.cu_s, rows, side="right") - 1
    k_p, v_p, cu_p = assemble_prefix(wl, np.unique(req))
    ref, ref_lse = oracle.prefill_isolated(wl.q, wl.k_s, wl.v_s, wl.cu_s, k_p, v_p, cu_p, T,
                                           wl.scale, rows=rows, heads=heads)
    check_close(got[rows, heads], ref, "bf16")
    assert np.abs(lse[heads, rows] - ref_lse).max() <= 1e-3


def test_isolated_single_token_fused_ping_pong(gpu_ready):
    """T = 1 on the ping-pong kernel (bf16, D=128, 256-row items): the
    row's own key is merged in the attention kernel's epilogue.  A request
    with no prefix (its rows are their own token alone), an item prefix, a
    ragged last row tile, a one-row request."""
    wl = W.make_custom(dtype="bf16", H=2, D=128, n_s=[512, 264, 300, 8, 1],
                       n_p=[700, 0, 129 * 4, 33, 64],
                       mode=[W.USER, W.USER, W.ITEM, W.USER, W.USER], seed=170,
                       num_items=300, name="iso_fused_T1")
    assert wl.total_s > 128 * wl.B  # the eight-wave (ping-pong) plan
    _compare(wl, 1)


@pytest.mark.slow
def test_isolated_single_token_fused_8k_history_sampled(gpu_ready):
    """The 8k-history configuration's shape (16 x 8192 prefix, 512 single-
    token candidates each, H=16, D=128, bf16), on sampled (row, head) pairs."""
    wl = W.make_config(4)
    print("[isolated] config 4 shape, T=1, sampled", flush=True)
    got, lse = _run_isolated(wl, 1)
    rng = np.random.default_rng(171)
    rows = np.concatenate([rng.integers(0, wl.total_s, 120), [0, wl.total_s - 1]])
    rows = rows.astype(np.int32)
    heads = rng.integers(0, wl.H, len(rows)).astype(np.int32)
    req = np.searchsorted(wl.cu_s, rows, side="right") - 1
    k_p, v_p, cu_p = assemble_prefix(wl, np.unique(req))
    ref, ref_lse = oracle.prefill_isolated(wl.q, wl.k_s, wl.v_s, wl.cu_s, k_p, v_p, cu_p, 1,
                                           wl.scale, rows=rows, heads=heads)
    check_close(got[rows, heads], ref, "bf16")
    assert np.abs(lse[heads, rows] - ref_lse).max() <= 1e-3
