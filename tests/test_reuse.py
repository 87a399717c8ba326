"""GPU: the paged prefix cache and its reuse.

* bat_kv_build is a bit-exact scatter (against the oracle's pool layout) and
  leaves unowned slots untouched;
* the result does not depend on where the blocks live (identity vs shuffled
  block table: bitwise equal) and is run-to-run deterministic;
* serving a prefix from the cache equals recomputing it as fresh tokens;
* BAT_VALIDATE reports out-of-range block ids.
"""
import numpy as np
import pytest

import oracle
from helpers import as_f64, check_close
from prefix_reuse_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


def test_kv_build_bit_exact(gpu_ready):
    import torch
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd.device import to_device, to_host
    for dtype, D, bs in (("bf16", 128, 64), ("bf16", 64, 4), ("f32", 32, 16), ("bf16", 64, 1)):
        wl = W.make_custom(dtype=dtype, H=3, D=D, n_s=[1, 1, 1], n_p=[130, 0, 67],
                           mode=[W.USER] * 3, seed=5, user_block_size=bs, extra_user_blocks=3)
        print(f"[kv_build] {dtype} D={D} bs={bs}", flush=True)
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        pool = api.new_pool(wl.user_num_blocks, wl.H, bs, D, tdt, fill=-7.0)
        api.kv_build(to_device(wl.user_k, dtype), to_device(wl.user_v, dtype),
                     torch.from_numpy(wl.cu_user).cuda(), torch.from_numpy(wl.block_table).cuda(),
                     pool)
        torch.cuda.synchronize()
        fill = W.f32_to_bf16(np.float32(-7.0)) if dtype == "bf16" else np.float32(-7.0)
        for got, src in ((pool.k, wl.user_k), (pool.v, wl.user_v)):
            ref = oracle.kv_scatter(src, wl.cu_user, wl.block_table, wl.user_num_blocks, bs, fill)
            np.testing.assert_array_equal(to_host(got, dtype), ref)


def _two_layouts(seed):
    """Config-2-shaped batch (smaller): the same logical prefixes behind an
    identity block table and behind a shuffled one."""
    wl = W.make_custom(dtype="bf16", H=4, D=64, n_s=[256] * 6, n_p=[1024] * 6,
                       mode=[W.USER] * 6, seed=seed, extra_user_blocks=5)
    wl_id = W.make_custom(dtype="bf16", H=4, D=64, n_s=[256] * 6, n_p=[1024] * 6,
                          mode=[W.USER] * 6, seed=seed, extra_user_blocks=5)
    nb = 1024 // 64
    wl_id.block_table = np.arange(6 * nb, dtype=np.int32).reshape(6, nb)
    return wl, wl_id


def test_layout_independence_and_determinism(gpu_ready):
    import torch
    from prefix_reuse_attention_amd.device import DeviceWorkload, to_host
    wl, wl_id = _two_layouts(11)
    assert not np.array_equal(wl.block_table, wl_id.block_table)
    a = DeviceWorkload(wl)
    b = DeviceWorkload(wl_id)
    o1, l1 = a.run()
    o2, l2 = a.run()
    o3, l3 = b.run()
    torch.cuda.synchronize()
    h1, h2, h3 = (to_host(o, "bf16") for o in (o1, o2, o3))
    np.testing.assert_array_equal(h1, h2)            # run to run
    np.testing.assert_array_equal(h1, h3)            # physical layout
    np.testing.assert_array_equal(l1.cpu().numpy(), l3.cpu().numpy())


def test_item_order_and_shared_items(gpu_ready):
    """Item prefixes share hot items across requests (one cached block read
    by many); permuting a request's item list leaves its rows unchanged up to
    rounding."""
    import torch
    from prefix_reuse_attention_amd.device import DeviceWorkload, to_host
    wl = W.make_custom(dtype="bf16", H=2, D=64, n_s=[100, 100, 100], n_p=[512, 512, 256],
                       mode=[W.ITEM] * 3, seed=12, num_items=300)
    ids = wl.block_table[:, :128]
    assert len(np.intersect1d(ids[0], ids[1])) > 0   # hot items shared
    a = DeviceWorkload(wl)
    o1, _ = a.run()
    rng = np.random.default_rng(1)
    bt = wl.block_table.copy()
    for r in range(3):
        n = wl.n_p[r] // 4
        bt[r, :n] = bt[r, rng.permutation(n)]
    o2, _ = a.run(block_table=torch.from_numpy(bt).cuda())
    torch.cuda.synchronize()
    check_close(as_f64(to_host(o2, "bf16"), "bf16"), as_f64(to_host(o1, "bf16"), "bf16"), "bf16",
                strict_abs=4e-3)


def test_cached_prefix_equals_recompute(gpu_ready):
    """Suffix rows with the prefix served from the paged cache equal the same
    rows when the prefix is recomputed as fresh tokens of the request."""
    import torch
    from prefix_reuse_attention_amd.device import DeviceWorkload, to_host
    wl = W.make_custom(dtype="bf16", H=4, D=128, n_s=[256, 40], n_p=[1000, 130],
                       mode=[W.USER, W.USER], seed=13)
    cached = DeviceWorkload(wl)
    oc, lc = cached.run()
    # recompute: every token fresh, no prefix: [P; U] as one suffix group
    segs_q, segs_k, segs_v, n_s = [], [], [], []
    for r in range(wl.B):
        p0, p1 = wl.cu_user[r], wl.cu_user[r + 1]
        s0, s1 = wl.cu_s[r], wl.cu_s[r + 1]
        segs_q += [np.zeros((p1 - p0, wl.H, wl.D), np.uint16), wl.q[s0:s1]]
        segs_k += [wl.user_k[p0:p1], wl.k_s[s0:s1]]
        segs_v += [wl.user_v[p0:p1], wl.v_s[s0:s1]]
        n_s.append(int(p1 - p0 + s1 - s0))
    fresh = W.make_custom(dtype="bf16", H=4, D=128, n_s=n_s, n_p=[0, 0], mode=[W.USER] * 2,
                          seed=13, materialize=False)
    fresh.q, fresh.k_s, fresh.v_s = (np.concatenate(x) for x in (segs_q, segs_k, segs_v))
    fresh.user_k = fresh.user_v = np.zeros((0, 4, 128), np.uint16)
    fresh.item_k = fresh.item_v = np.zeros((0, 4, 128), np.uint16)
    rec = DeviceWorkload(fresh)
    orc, lrc = rec.run()
    torch.cuda.synchronize()
    got_c = as_f64(to_host(oc, "bf16"), "bf16")
    got_r = as_f64(to_host(orc, "bf16"), "bf16")
    lc, lrc = lc.cpu().numpy(), lrc.cpu().numpy()
    for r in range(wl.B):
        s0, s1 = wl.cu_s[r], wl.cu_s[r + 1]
        f1 = fresh.cu_s[r + 1]
        rows_r = np.arange(f1 - (s1 - s0), f1)
        check_close(got_c[s0:s1], got_r[rows_r], "bf16", strict_abs=4e-3)
        assert np.abs(lc[:, s0:s1] - lrc[:, rows_r]).max() < 1e-3


def test_validate_reports_bad_block_ids(gpu_ready, monkeypatch):
    import torch
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd.device import DeviceWorkload
    monkeypatch.setenv("BAT_VALIDATE", "1")
    wl = W.make_custom(dtype="bf16", H=2, D=64, n_s=[10], n_p=[128], mode=[W.USER], seed=14)
    dw = DeviceWorkload(wl)
    dw.run()  # valid table: no error
    bad = dw.block_table.clone()
    bad[0, 1] = wl.user_num_blocks + 5
    with pytest.raises(api.BatError) as ei:
        dw.run(block_table=bad)
    assert ei.value.status == api.BAT_ERR_BLOCK_TABLE
    bad[0, 1] = -3
    with pytest.raises(api.BatError) as ei:
        api.kv_build(torch.zeros((128, 2, 64), dtype=torch.bfloat16, device="cuda"),
                     torch.zeros((128, 2, 64), dtype=torch.bfloat16, device="cuda"),
                     dw.prefix_lens.new_tensor([0, 128]), bad, dw.user_pool)
    assert ei.value.status == api.BAT_ERR_BLOCK_TABLE


def test_lse_merge_entry_point(gpu_ready):
    """bat_lse_merge against the oracle's merge definition, including an
    empty (-inf) part."""
    import torch
    from prefix_reuse_attention_amd import api
    rng = np.random.default_rng(15)
    n, rows, H, D = 3, 50, 2, 64
    o = rng.standard_normal((n, rows, H, D)).astype(np.float32)
    l = rng.standard_normal((n, H, rows)).astype(np.float32) * 3
    l[1, :, :10] = -np.inf
    out, lse = api.lse_merge(torch.from_numpy(o).cuda(), torch.from_numpy(l).cuda(), torch.float32)
    torch.cuda.synchronize()
    parts = [(o[i].astype(np.float64), l[i].T.astype(np.float64)) for i in range(n)]
    ref_o, ref_l = oracle.lse_merge(parts)
    assert np.abs(out.cpu().numpy() - ref_o).max() <= 1e-5
    assert np.abs(lse.cpu().numpy().T - ref_l).max() <= 1e-5
