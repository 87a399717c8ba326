"""GPU parity: grouped key/value heads (bat_attn_prefill_gqa) against the
oracle, through the C ABI.

H query heads share H_kv key/value heads; the pools are built with H_kv heads
by bat_kv_build and the fresh suffix keys/values carry H_kv heads.  Cases:
groups of 2, 4 and 8 query heads per key/value head, user and item prefixes,
empty prefixes, both bf16 head dims and fp32, the four- and eight-wave
kernels (the eight-wave one is the ping-pong kernel).  Every expected value comes from the
oracle.
"""
import numpy as np
import pytest

import oracle
from helpers import as_f64, assemble_prefix, check_close
from prefix_reuse_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


def _compare(wl, H):
    """wl is built with H_kv heads (pools, suffix keys/values); queries of H
    heads are drawn on top."""
    import torch
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd.device import DeviceWorkload, to_device, to_host
    rng = np.random.default_rng(wl.seed + 1000)
    q = W._normal(rng, (wl.total_s, H, wl.D), wl.dtype)
    print(f"[gqa] {wl.name} dtype={wl.dtype} D={wl.D} H={H} H_kv={wl.H} "
          f"n_s={wl.n_s.tolist()} n_p={wl.n_p.tolist()}", flush=True)
    dw = DeviceWorkload(wl)
    dq = to_device(q, wl.dtype)
    out, lse = api.attn_prefill_gqa(dq, dw.k, dw.v, dw.cu_s, dw.prefix_lens, dw.prefix_mode,
                                    dw.block_table, dw.user_pool, dw.item_pool, wl.scale,
                                    dw.max_s, dw.max_p, want_lse=True)
    torch.cuda.synchronize()
    got = as_f64(to_host(out, wl.dtype), wl.dtype)
    got_lse = lse.cpu().numpy().astype(np.float64)
    k_p, v_p, cu_p = assemble_prefix(wl)
    ref, ref_lse = oracle.prefill_suffix_gqa(q, wl.k_s, wl.v_s, wl.cu_s, k_p, v_p, cu_p,
                                             wl.scale)
    check_close(got, ref, wl.dtype)
    tol = 1e-5 if wl.dtype == "f32" else 1e-3
    assert np.abs(got_lse - ref_lse).max() <= tol


@pytest.mark.parametrize("H,H_kv", [(8, 4), (8, 2), (8, 1)])
@pytest.mark.parametrize("D", [64, 128])
def test_gqa_bf16_mixed(gpu_ready, H, H_kv, D):
    wl = W.make_custom(dtype="bf16", H=H_kv, D=D, n_s=[1, 130, 64, 5], n_p=[0, 200, 1000, 129],
                       mode=[W.USER, W.USER, W.ITEM, W.USER], seed=140 + H_kv + D,
                       num_items=400, name=f"gqa_bf16_{H}x{H_kv}_D{D}")
    _compare(wl, H)


def test_gqa_fp32(gpu_ready):
    wl = W.make_custom(dtype="f32", H=2, D=32, n_s=[3, 70], n_p=[0, 152],
                       mode=[W.USER, W.ITEM], seed=150, user_block_size=16, num_items=80,
                       name="gqa_f32")
    _compare(wl, 4)


@pytest.mark.parametrize("D", [64, 128])
def test_gqa_eight_wave_items(gpu_ready, D):
    wl = W.make_custom(dtype="bf16", H=2, D=D, n_s=[512, 264], n_p=[700, 1031],
                       mode=[W.USER, W.USER], seed=160 + D, name=f"gqa_w8_D{D}")
    _compare(wl, 8)
