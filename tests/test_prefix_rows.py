"""GPU parity: prefix rows (bat_attn_prefix_rows) and per-item rows
(bat_attn_item_local) against the oracle, through the C ABI.

Prefix rows: each prefix token sees every prefix token of its own request
(ragged requests, empty requests, one-token requests, lengths around the
64/128-key tile and the 128/256-row item sizes), and, at the size of the
8k-history configuration, on sampled rows.  Per-item rows: each item's T
tokens see only their own item, for every supported T, head dim and dtype,
and on sampled rows of the 20000-item pool of the item-prefix configuration.
Inputs are seeded N(0, 1) in the storage dtype; every expected value comes
from the oracle.
"""
import numpy as np
import pytest

import oracle
from helpers import as_f64, check_close
from prefix_reuse_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


def _inputs(seed, n, H, D, dtype, q_scale=1.0):
    rng = np.random.default_rng(seed)
    q = W._normal(rng, (n, H, D), dtype, q_scale)
    k = W._normal(rng, (n, H, D), dtype)
    v = W._normal(rng, (n, H, D), dtype)
    return q, k, v


def _to_dev(dtype, *arrs):
    from prefix_reuse_attention_amd.device import to_device
    return [to_device(a, dtype) for a in arrs]


def _prefix_rows_gpu(q, k, v, cu, dtype):
    import torch
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd.device import to_host
    dq, dk, dv = _to_dev(dtype, q, k, v)
    dcu = torch.from_numpy(np.ascontiguousarray(cu, np.int32)).to("cuda")
    scale = oracle.default_scale(q.shape[2])
    out, lse = api.attn_prefix_rows(dq, dk, dv, dcu, softmax_scale=scale, want_lse=True)
    torch.cuda.synchronize()
    return as_f64(to_host(out, dtype), dtype), lse.cpu().numpy().astype(np.float64), scale


@pytest.mark.parametrize("dtype,D", [("f32", 32), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_prefix_rows_ragged(gpu_ready, dtype, D):
    lens = [1, 0, 63, 64, 65, 130, 257, 3]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    H = 2
    print(f"[prefix_rows] {dtype} D={D} lens={lens}", flush=True)
    q, k, v = _inputs(40 + D, int(cu[-1]), H, D, dtype)
    got, got_lse, scale = _prefix_rows_gpu(q, k, v, cu, dtype)
    ref, ref_lse = oracle.prefix_rows(q, k, v, cu, scale)
    check_close(got, ref, dtype)
    tol = 1e-5 if dtype == "f32" else 1e-3
    assert np.abs(got_lse - ref_lse).max() <= tol


@pytest.mark.parametrize("D", [64, 128])
def test_prefix_rows_eight_wave_items(gpu_ready, D):
    """Long prefixes: 256-row items of the eight-wave (ping-pong) kernel,
    several row tiles per request and a ragged last tile."""
    lens = [700, 512, 1031]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    H = 2
    print(f"[prefix_rows] bf16 D={D} lens={lens}", flush=True)
    q, k, v = _inputs(50 + D, int(cu[-1]), H, D, "bf16")
    got, got_lse, scale = _prefix_rows_gpu(q, k, v, cu, "bf16")
    ref, ref_lse = oracle.prefix_rows(q, k, v, cu, scale)
    check_close(got, ref, "bf16")
    assert np.abs(got_lse - ref_lse).max() <= 1e-3


@pytest.mark.slow
def test_prefix_rows_8k_history_sampled(gpu_ready):
    """The 8k-history configuration's prefixes (16 requests x 8192 tokens,
    H=16, D=128, bf16) as prefix rows, checked on sampled (row, head) pairs."""
    B, n_p, H, D = 16, 8192, 16, 128
    cu = (np.arange(B + 1) * n_p).astype(np.int32)
    print("[prefix_rows] 8k history, sampled", flush=True)
    q, k, v = _inputs(61, B * n_p, H, D, "bf16")
    got, got_lse, scale = _prefix_rows_gpu(q, k, v, cu, "bf16")
    rng = np.random.default_rng(62)
    rows = np.concatenate([rng.integers(0, B * n_p, 120), [0, n_p - 1, n_p, B * n_p - 1]])
    rows = rows.astype(np.int32)
    heads = rng.integers(0, H, len(rows)).astype(np.int32)
    ref, ref_lse = oracle.prefix_rows(q, k, v, cu, scale, rows=rows, heads=heads)
    check_close(got[rows, heads], ref, "bf16")
    assert np.abs(got_lse[heads, rows] - ref_lse).max() <= 1e-3


def _item_local_gpu(q, k, v, T, dtype):
    import torch
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd.device import to_host
    dq, dk, dv = _to_dev(dtype, q, k, v)
    scale = oracle.default_scale(q.shape[2])
    out, lse = api.attn_item_local(dq, dk, dv, T, softmax_scale=scale, want_lse=True)
    torch.cuda.synchronize()
    return as_f64(to_host(out, dtype), dtype), lse.cpu().numpy().astype(np.float64), scale


@pytest.mark.parametrize("T", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype,D", [("f32", 32), ("f32", 64), ("f32", 128), ("bf16", 64),
                                     ("bf16", 128)])
def test_item_local(gpu_ready, T, dtype, D):
    n_items, H = 37, 3
    print(f"[item_local] {dtype} D={D} T={T}", flush=True)
    q, k, v = _inputs(70 + T + D, n_items * T, H, D, dtype, q_scale=2.0)
    got, got_lse, scale = _item_local_gpu(q, k, v, T, dtype)
    ref, ref_lse = oracle.item_local(q, k, v, T, scale)
    check_close(got, ref, dtype)
    tol = 1e-5 if dtype == "f32" else 1e-3
    assert np.abs(got_lse - ref_lse).max() <= tol


def test_item_local_item_pool_sampled(gpu_ready):
    """The item-prefix configuration's pool (20000 items x 4 tokens, H=8,
    D=64, bf16), on sampled (row, head) pairs."""
    n_items, T, H, D = 20000, 4, 8, 64
    print("[item_local] 20000-item pool, sampled", flush=True)
    q, k, v = _inputs(81, n_items * T, H, D, "bf16")
    got, got_lse, scale = _item_local_gpu(q, k, v, T, "bf16")
    rng = np.random.default_rng(82)
    rows = np.concatenate([rng.integers(0, n_items * T, 200), [0, n_items * T - 1]])
    rows = rows.astype(np.int32)
    heads = rng.integers(0, H, len(rows)).astype(np.int32)
    ref, ref_lse = oracle.item_local(q, k, v, T, scale, rows=rows, heads=heads)
    check_close(got[rows, heads], ref, "bf16")
    assert np.abs(got_lse[heads, rows] - ref_lse).max() <= 1e-3
