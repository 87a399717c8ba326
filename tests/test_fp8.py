"""fp8 key/value pools: the build (bat_kv_build_fp8) bit-exact against the
oracle's pool, and the prefill over them (bat_attn_prefill_fp8) against the
oracle's attention over the read-back prefix (code value * scale), at the
bfloat16 bars.

The pool format is a reading (the pages prescribe no cache format): OCP
E4M3 codes with one power-of-two scale per block and head.  CPU tests cover
the binding's argument checks; GPU tests print their case before running.
"""
import numpy as np
import pytest

import oracle
from helpers import as_f64, check_close
from prefix_reuse_attention_amd import api
from prefix_reuse_attention_amd import workloads as W


def test_fp8_argument_errors():
    lib = api.load()
    fake = __import__("ctypes").c_void_p(0x1000)
    pool = api.KvPoolFp8(0x1000, 0x1000, 0x1000, None, 4, 64)
    ref = __import__("ctypes").byref
    # a pool without its V scales
    assert lib.bat_kv_build_fp8(fake, fake, fake, fake, 2, 1, 2, 64, 10, api.BAT_BF16, ref(pool),
                                None) == api.BAT_ERR_INVALID_ARG
    good = api.KvPoolFp8(0x1000, 0x1000, 0x1000, 0x1000, 4, 64)
    assert lib.bat_kv_build_fp8(fake, fake, fake, fake, 2, 1, 2, 48, 10, api.BAT_BF16, ref(good),
                                None) == api.BAT_ERR_UNSUPPORTED
    assert lib.bat_kv_build_fp8(fake, fake, fake, fake, 2, 1, 2, 64, 0, api.BAT_BF16, ref(good),
                                None) == api.BAT_OK
    # the prefill: bf16 only, D in {64, 128}, scales required
    args = lambda D, up: (fake, fake, fake, fake, fake, fake, fake, 2, ref(up), None, 1, 2, D,
                          0.1, 8, 8, 64, fake, None, fake, 1 << 20, None)
    assert lib.bat_attn_prefill_fp8(*args(32, good)) == api.BAT_ERR_UNSUPPORTED
    assert lib.bat_attn_prefill_fp8(*args(64, pool)) == api.BAT_ERR_INVALID_ARG
    assert api.fp8_workspace_size(2, 4, 128, 1024, 512, 4096) > 0
    assert api.fp8_workspace_size(2, 4, 96, 1024, 512, 4096) == 0


@pytest.mark.gpu
def test_kv_build_fp8_bit_exact(gpu_ready):
    """Codes and scales equal the oracle's pool, bit for bit: bf16 user pools
    (64-token blocks at D=128, 16-token blocks with partial last blocks at
    D=64), an item pool of 4-token blocks, fp32 input at D=32; blocks no token
    maps to keep their fill."""
    import torch
    from prefix_reuse_attention_amd.device import to_device, to_host
    cases = [("bf16", 128, 64, [130, 0, 64], 1.0), ("bf16", 64, 16, [33, 7, 100], 1.0),
             ("bf16", 64, 4, [8, 12], 30.0), ("f32", 32, 16, [40, 17], 0.01)]
    for dt, D, bs, lens, vscale in cases:
        wl = W.make_custom(dtype=dt, H=3, D=D, n_s=[1] * len(lens), n_p=lens,
                           mode=[W.USER] * len(lens), seed=501 + D, user_block_size=bs,
                           extra_user_blocks=2, value_scale=vscale)
        print(f"[fp8] build {dt} D={D} bs={bs} lens={lens}", flush=True)
        pool = api.new_pool_fp8(wl.user_num_blocks, wl.H, bs, D)
        pool.k.fill_(0xEE)
        pool.v.fill_(0xEE)
        pool.k_scale.fill_(-1.0)
        pool.v_scale.fill_(-1.0)
        api.kv_build_fp8(to_device(wl.user_k, dt), to_device(wl.user_v, dt),
                         torch.from_numpy(wl.cu_user).cuda(),
                         torch.from_numpy(wl.block_table).cuda(), pool)
        torch.cuda.synchronize()
        for codes, scales, src in ((pool.k, pool.k_scale, wl.user_k),
                                   (pool.v, pool.v_scale, wl.user_v)):
            ref_c, ref_s = oracle.kv_scatter_fp8(src, wl.cu_user, wl.block_table,
                                                 wl.user_num_blocks, bs, 0xEE, -1.0)
            np.testing.assert_array_equal(codes.cpu().numpy(), ref_c)
            np.testing.assert_array_equal(scales.cpu().numpy().astype(np.float64), ref_s)


def _fp8_reference(wl):
    """The oracle over the read-back prefix: each request's prefix keys and
    values as their codes read back, the suffix as stored (bfloat16)."""
    ks, vs, cu = [], [], [0]
    for r in range(wl.B):
        if wl.mode[r] == W.ITEM:
            # each item is one block of the item pool, quantised on its own
            T = W.ITEM_TOKENS
            ids = wl.block_table[r, : wl.n_p[r] // T]
            cu_i = np.arange(0, len(ids) * T + 1, T)
            _, _, kb = oracle.fp8_quantize_blocks(oracle.gather_item_prefix(wl.item_k, ids, T),
                                                  cu_i, T)
            _, _, vb = oracle.fp8_quantize_blocks(oracle.gather_item_prefix(wl.item_v, ids, T),
                                                  cu_i, T)
        else:
            p0, p1 = wl.cu_user[r], wl.cu_user[r + 1]
            _, _, kb = oracle.fp8_quantize_blocks(wl.user_k[p0:p1], [0, p1 - p0],
                                                  wl.user_block_size)
            _, _, vb = oracle.fp8_quantize_blocks(wl.user_v[p0:p1], [0, p1 - p0],
                                                  wl.user_block_size)
        ks.append(kb)
        vs.append(vb)
        cu.append(cu[-1] + len(kb))
    shape = (0, wl.H, wl.D)
    k_p = np.concatenate(ks) if ks else np.zeros(shape)
    v_p = np.concatenate(vs) if vs else np.zeros(shape)
    f = lambda a: as_f64(a, wl.dtype)
    return oracle.prefill_suffix(f(wl.q), f(wl.k_s), f(wl.v_s), wl.cu_s, k_p, v_p,
                                 np.array(cu, np.int32), wl.scale)


def _run_fp8(wl):
    import torch
    from prefix_reuse_attention_amd.device import DeviceWorkload, to_host
    dw = DeviceWorkload(wl, build=False)
    dw.build_pools_fp8()
    out, lse = dw.run_fp8()
    torch.cuda.synchronize()
    return as_f64(to_host(out, "bf16"), "bf16"), lse.cpu().numpy().astype(np.float64), dw


@pytest.mark.gpu
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_fp8_ragged_mixed(gpu_ready, D):
    """User and item prefixes from fp8 pools, ragged everything: suffixes
    off the row tile, prefixes ending mid-block and mid-tile, an empty
    prefix, a single-row suffix."""
    wl = W.make_custom(dtype="bf16", H=3, D=D, n_s=[1, 130, 257, 64, 5],
                       n_p=[0, 200, 1000, 4, 129], mode=[W.USER, W.USER, W.ITEM, W.ITEM, W.USER],
                       seed=510 + D, num_items=400, name=f"fp8_ragged_D{D}")
    print(f"[fp8] prefill ragged D={D}", flush=True)
    got, lse, _ = _run_fp8(wl)
    ref_o, ref_l = _fp8_reference(wl)
    check_close(got, ref_o, "bf16")
    assert np.abs(lse - ref_l).max() <= 1e-3


@pytest.mark.gpu
@pytest.mark.parametrize("waves", ["4", "8"])
def test_prefill_fp8_workgroup_shapes_and_split(gpu_ready, monkeypatch, waves):
    """Both workgroup shapes at D=64 (the head-dim-128 fp8 path always takes
    four waves), and split prefixes recombined by the merge."""
    monkeypatch.setenv("BAT_WAVES", waves)
    monkeypatch.setenv("BAT_SPLIT_CHUNK", "512")
    wl = W.make_custom(dtype="bf16", H=2, D=64, n_s=[300, 17, 256], n_p=[2000, 64, 777],
                       mode=[W.USER, W.ITEM, W.USER], seed=520, num_items=300,
                       name=f"fp8_w{waves}")
    print(f"[fp8] prefill waves={waves} split", flush=True)
    got, lse, _ = _run_fp8(wl)
    ref_o, ref_l = _fp8_reference(wl)
    check_close(got, ref_o, "bf16")
    assert np.abs(lse - ref_l).max() <= 1e-3


@pytest.mark.gpu
def test_prefill_fp8_layout_independence(gpu_ready):
    """The same prefixes behind a shuffled and an identity block table give
    bitwise the same rows from fp8 pools."""
    import torch
    from prefix_reuse_attention_amd.device import to_host
    kw = dict(dtype="bf16", H=2, D=128, n_s=[200, 64], n_p=[1000, 300], mode=[W.USER] * 2,
              seed=530, extra_user_blocks=3)
    wl, wl_id = W.make_custom(**kw), W.make_custom(**kw)
    nb = -(-np.asarray(wl.n_p) // 64)
    bt = np.full_like(wl.block_table, -1)
    bt[0, :nb[0]] = np.arange(nb[0])
    bt[1, :nb[1]] = np.arange(nb[0], nb[0] + nb[1])
    wl_id.block_table = bt
    print("[fp8] layout independence", flush=True)
    a, la, _ = _run_fp8(wl)
    b, lb, _ = _run_fp8(wl_id)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


@pytest.mark.gpu
@pytest.mark.slow
def test_prefill_fp8_config4_shape_every_row(gpu_ready):
    """Config 4's shape (16 requests, 8192-token prefixes in 64-token blocks,
    suffix 512, H=16, D=128) from an fp8 pool, every (row, head) against
    the oracle over the read-back prefixes."""
    wl = W.make_config(4)
    print("[fp8] config 4 shape, every row", flush=True)
    got, lse, _ = _run_fp8(wl)
    print("[fp8] config 4 shape: oracle", flush=True)
    ref_o, ref_l = _fp8_reference(wl)
    check_close(got, ref_o, "bf16", strict_abs=4e-3)
    assert np.abs(lse - ref_l).max() <= 1e-3
