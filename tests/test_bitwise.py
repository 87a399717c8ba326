"""GPU: bitwise properties of the kernels that serve the long-suffix shapes.

The result of a suffix row depends on its logical keys only: the blocks'
physical places in a pool, the run, and where the work item runs (which
workgroup slot, planner or no planner) must not change a single bit.  Bat
page, "Problem": a prefix's key/value cache is computed once and served
again, so the cached copy has to be as good as the original wherever it
sits.  Each case prints its name before it runs.

Shapes are chosen so that the eight-wave, head-dim-128 kernel (the one
config 4 runs) serves them: D=128 and suffixes averaging more than 128 rows.
"""
import numpy as np
import pytest

from helpers import as_f64, check_close, oracle_full
from prefix_reuse_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


def _host(t, dt="bf16"):
    from prefix_reuse_attention_amd.device import to_host
    return to_host(t, dt)


def _user_pair(seed, n_s, n_p, H=4, D=128):
    """The same logical prefixes behind the generator's shuffled block table
    and behind an identity table (each its own pool)."""
    kw = dict(dtype="bf16", H=H, D=D, n_s=n_s, n_p=n_p, mode=[W.USER] * len(n_s), seed=seed,
              extra_user_blocks=7, name=f"bitwise_user_{seed}")
    wl, wl_id = W.make_custom(**kw), W.make_custom(**kw)
    nb = wl.block_table.shape[1]
    bt = np.full_like(wl.block_table, -1)
    pos = 0
    for r in range(wl.B):
        n = -(-int(n_p[r]) // wl.user_block_size)
        bt[r, :n] = np.arange(pos, pos + n)
        pos += n
    wl_id.block_table = bt
    assert not np.array_equal(wl.block_table, wl_id.block_table)
    return wl, wl_id


def test_ping_pong_layout_independence_and_determinism(gpu_ready):
    import torch
    from prefix_reuse_attention_amd.device import DeviceWorkload
    n_s, n_p = [256, 200, 300, 256], [1000, 4096, 64, 777]
    assert sum(n_s) > 128 * len(n_s)
    wl, wl_id = _user_pair(201, n_s, n_p)
    print(f"[bitwise] user pool D=128 n_s={n_s} n_p={n_p}", flush=True)
    a, b = DeviceWorkload(wl), DeviceWorkload(wl_id)
    o1, l1 = a.run(want_lse=True)
    o2, l2 = a.run(want_lse=True)
    o3, l3 = b.run(want_lse=True)
    torch.cuda.synchronize()
    h1, h2, h3 = _host(o1), _host(o2), _host(o3)
    np.testing.assert_array_equal(h1, h2)                 # run to run
    np.testing.assert_array_equal(h1, h3)                 # physical placement
    np.testing.assert_array_equal(l1.cpu().numpy(), l2.cpu().numpy())
    np.testing.assert_array_equal(l1.cpu().numpy(), l3.cpu().numpy())
    ref_o, ref_l = oracle_full(wl)
    check_close(as_f64(h1, "bf16"), ref_o, "bf16", strict_abs=4e-3)
    assert np.abs(l1.cpu().numpy() - ref_l).max() <= 1e-3


def test_item_pool_permuted_slots_bitwise(gpu_ready):
    """An item pool whose items sit at permuted physical slots (built through
    a permuted slot table), read through block-table rows that list those
    slots, gives bitwise the rows of the pool with item i in slot i."""
    import torch
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd.device import DeviceWorkload, to_device
    n_s, n_p = [256, 224, 300], [512, 1024, 132]
    wl = W.make_custom(dtype="bf16", H=2, D=128, n_s=n_s, n_p=n_p, mode=[W.ITEM] * 3,
                       seed=202, num_items=700, name="bitwise_items")
    print(f"[bitwise] item pool D=128 n_s={n_s} n_p={n_p} permuted slots", flush=True)
    a = DeviceWorkload(wl)                                # item i in slot i
    o1, l1 = a.run(want_lse=True)
    rng = np.random.default_rng(203)
    slot = rng.permutation(wl.num_items).astype(np.int32)
    n = wl.num_items
    pool = api.new_pool(n, wl.H, W.ITEM_TOKENS, wl.D, torch.bfloat16)
    api.kv_build(to_device(wl.item_k, "bf16"), to_device(wl.item_v, "bf16"),
                 torch.arange(0, (n + 1) * W.ITEM_TOKENS, W.ITEM_TOKENS, dtype=torch.int32,
                              device="cuda"),
                 torch.from_numpy(slot.reshape(n, 1)).cuda(), pool)
    bt = wl.block_table.copy()
    bt[bt >= 0] = slot[bt[bt >= 0]]
    o2, l2 = api.attn_prefill(a.q, a.k, a.v, a.cu_s, a.prefix_lens, a.prefix_mode,
                              torch.from_numpy(bt).cuda(), None, pool, wl.scale, a.max_s, a.max_p,
                              want_lse=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_host(o1), _host(o2))
    np.testing.assert_array_equal(l1.cpu().numpy(), l2.cpu().numpy())
    ref_o, _ = oracle_full(wl)
    check_close(as_f64(_host(o2), "bf16"), ref_o, "bf16", strict_abs=4e-3)


def test_planner_and_in_kernel_placement_bitwise(gpu_ready, monkeypatch):
    """A batch of equal suffixes runs without the planner launch (the
    kernels derive their work item from the workgroup index); the same batch
    with the planner (forced by validation, which always plans) must give
    bitwise the same rows, at both head dims and with grouped heads."""
    import torch
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd.device import DeviceWorkload, to_device
    cases = [(128, [256] * 5, [1000, 4096, 64, 777, 0], 4),
             (64, [128] * 9, [1024] * 9, 3),
             (128, [100] * 3, [300, 0, 2000], 2)]
    for D, n_s, n_p, H in cases:
        wl = W.make_custom(dtype="bf16", H=H, D=D, n_s=n_s, n_p=n_p, mode=[W.USER] * len(n_s),
                           seed=204 + D, name=f"placement_D{D}")
        print(f"[bitwise] placement D={D} B={wl.B} n_s={n_s[0]}", flush=True)
        dw = DeviceWorkload(wl)
        monkeypatch.delenv("BAT_VALIDATE", raising=False)
        o1, l1 = dw.run(want_lse=True)
        monkeypatch.setenv("BAT_VALIDATE", "1")
        o2, l2 = dw.run(want_lse=True)
        monkeypatch.delenv("BAT_VALIDATE")
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_host(o1), _host(o2))
        np.testing.assert_array_equal(l1.cpu().numpy(), l2.cpu().numpy())
        ref_o, _ = oracle_full(wl)
        check_close(as_f64(_host(o1), "bf16"), ref_o, "bf16", strict_abs=4e-3)
    # grouped heads: 8 query heads over 2 key/value heads, equal suffixes
    wl = W.make_custom(dtype="bf16", H=2, D=128, n_s=[256] * 3, n_p=[512, 64, 1500],
                       mode=[W.USER] * 3, seed=210, name="placement_gqa")
    print("[bitwise] placement grouped heads", flush=True)
    dw = DeviceWorkload(wl)
    q = to_device(W._normal(np.random.default_rng(211), (wl.total_s, 8, 128), "bf16"), "bf16")
    run = lambda: api.attn_prefill_gqa(q, dw.k, dw.v, dw.cu_s, dw.prefix_lens, dw.prefix_mode,
                                       dw.block_table, dw.user_pool, None, wl.scale, dw.max_s,
                                       dw.max_p, want_lse=True)
    o1, l1 = run()
    monkeypatch.setenv("BAT_VALIDATE", "1")
    o2, l2 = run()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_host(o1), _host(o2))
    np.testing.assert_array_equal(l1.cpu().numpy(), l2.cpu().numpy())


def test_cached_equals_recompute_ping_pong(gpu_ready):
    """Suffix rows over the paged cache equal the same rows with the prefix
    recomputed as fresh tokens, both on the eight-wave head-dim-128 kernel."""
    import torch
    from prefix_reuse_attention_amd.device import DeviceWorkload
    n_s, n_p = [256, 200], [1000, 130]
    wl = W.make_custom(dtype="bf16", H=4, D=128, n_s=n_s, n_p=n_p, mode=[W.USER] * 2, seed=212)
    assert sum(n_s) > 128 * 2
    print("[bitwise] cached = recompute, eight waves", flush=True)
    cached = DeviceWorkload(wl)
    oc, lc = cached.run(want_lse=True)
    segs_q, segs_k, segs_v, lens = [], [], [], []
    for r in range(wl.B):
        p0, p1 = wl.cu_user[r], wl.cu_user[r + 1]
        s0, s1 = wl.cu_s[r], wl.cu_s[r + 1]
        segs_q += [np.zeros((p1 - p0, wl.H, wl.D), np.uint16), wl.q[s0:s1]]
        segs_k += [wl.user_k[p0:p1], wl.k_s[s0:s1]]
        segs_v += [wl.user_v[p0:p1], wl.v_s[s0:s1]]
        lens.append(int(p1 - p0 + s1 - s0))
    fresh = W.make_custom(dtype="bf16", H=4, D=128, n_s=lens, n_p=[0, 0], mode=[W.USER] * 2,
                          seed=212, materialize=False)
    fresh.q, fresh.k_s, fresh.v_s = (np.concatenate(x) for x in (segs_q, segs_k, segs_v))
    fresh.user_k = fresh.user_v = np.zeros((0, 4, 128), np.uint16)
    fresh.item_k = fresh.item_v = np.zeros((0, 4, 128), np.uint16)
    rec = DeviceWorkload(fresh)
    orc, lrc = rec.run(want_lse=True)
    torch.cuda.synchronize()
    got_c, got_r = as_f64(_host(oc), "bf16"), as_f64(_host(orc), "bf16")
    lc, lrc = lc.cpu().numpy(), lrc.cpu().numpy()
    for r in range(wl.B):
        s0, s1 = wl.cu_s[r], wl.cu_s[r + 1]
        f1 = fresh.cu_s[r + 1]
        rows_r = np.arange(f1 - (s1 - s0), f1)
        check_close(got_c[s0:s1], got_r[rows_r], "bf16", strict_abs=4e-3)
        assert np.abs(lc[:, s0:s1] - lrc[:, rows_r]).max() < 1e-3


def test_prepared_call_matches_the_plain_call(gpu_ready):
    """api.PreparedPrefill (arguments marshalled once, as the benchmark calls
    the library) enqueues the same call: bitwise the same rows, call after
    call."""
    import torch
    from prefix_reuse_attention_amd.device import DeviceWorkload
    wl = W.make_custom(dtype="bf16", H=2, D=64, n_s=[256] * 4, n_p=[1024, 64, 0, 777],
                       mode=[W.USER] * 4, seed=220, name="prepared")
    print("[bitwise] prepared call", flush=True)
    dw = DeviceWorkload(wl)
    o1, l1 = dw.run(want_lse=True)
    out, lse = torch.empty_like(o1), torch.empty_like(l1)
    call = dw.prepared(out, lse, dw.workspace())
    for _ in range(3):
        out.zero_()
        call()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_host(out), _host(o1))
        np.testing.assert_array_equal(lse.cpu().numpy(), l1.cpu().numpy())
