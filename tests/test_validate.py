"""GPU: BAT_VALIDATE=1 reports every length that breaks the call's bounds.

The checks run on the device (the planner compares each request's lengths
with the host bounds and its block-table row; the prefix build checks its
tokens against their rows), the call synchronises its stream and returns
BAT_ERR_BLOCK_TABLE.  No case here makes a kernel read out of bounds: the
kernels clamp a prefix to max_prefix_len and treat missing block ids as
empty whether or not validation is on; validation only reports.
"""
import threading

import numpy as np
import pytest

from prefix_reuse_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture
def validated(monkeypatch):
    monkeypatch.setenv("BAT_VALIDATE", "1")


def _wl(seed=300):
    return W.make_custom(dtype="bf16", H=2, D=64, n_s=[40, 17, 64], n_p=[300, 128, 0],
                         mode=[W.USER, W.USER, W.USER], seed=seed, user_block_size=64,
                         name="validate")


def _expect_status(fn, status):
    from prefix_reuse_attention_amd import api
    with pytest.raises(api.BatError) as ei:
        fn()
    assert ei.value.status == status, ei.value


def test_valid_call_passes(gpu_ready, validated):
    from prefix_reuse_attention_amd.device import DeviceWorkload
    dw = DeviceWorkload(_wl())
    dw.run()


def test_prefix_longer_than_its_bound(gpu_ready, validated):
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd.device import DeviceWorkload
    wl = _wl()
    dw = DeviceWorkload(wl)
    print("[validate] prefix_lens > max_prefix_len", flush=True)
    _expect_status(lambda: api.attn_prefill(dw.q, dw.k, dw.v, dw.cu_s, dw.prefix_lens,
                                            dw.prefix_mode, dw.block_table, dw.user_pool, None,
                                            wl.scale, dw.max_s, 200),
                   api.BAT_ERR_BLOCK_TABLE)


def test_prefix_longer_than_its_table_row(gpu_ready, validated):
    """300 prefix tokens need 5 blocks of 64; a table of 4 columns cannot
    hold them."""
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd.device import DeviceWorkload
    wl = _wl()
    dw = DeviceWorkload(wl)
    assert dw.block_table.shape[1] == 5
    short = dw.block_table[:, :4].contiguous()
    print("[validate] prefix_lens > bt_stride * block_size", flush=True)
    _expect_status(lambda: api.attn_prefill(dw.q, dw.k, dw.v, dw.cu_s, dw.prefix_lens,
                                            dw.prefix_mode, short, dw.user_pool, None, wl.scale,
                                            dw.max_s, dw.max_p),
                   api.BAT_ERR_BLOCK_TABLE)


def test_suffix_longer_than_its_bound(gpu_ready, validated):
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd.device import DeviceWorkload
    wl = _wl()
    dw = DeviceWorkload(wl)
    print("[validate] n_s > max_suffix_len", flush=True)
    _expect_status(lambda: api.attn_prefill(dw.q, dw.k, dw.v, dw.cu_s, dw.prefix_lens,
                                            dw.prefix_mode, dw.block_table, dw.user_pool, None,
                                            wl.scale, 50, dw.max_p),
                   api.BAT_ERR_BLOCK_TABLE)


def test_negative_prefix_length(gpu_ready, validated):
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd.device import DeviceWorkload
    wl = _wl()
    dw = DeviceWorkload(wl)
    bad = dw.prefix_lens.clone()
    bad[1] = -4
    print("[validate] negative prefix length", flush=True)
    _expect_status(lambda: api.attn_prefill(dw.q, dw.k, dw.v, dw.cu_s, bad, dw.prefix_mode,
                                            dw.block_table, dw.user_pool, None, wl.scale,
                                            dw.max_s, dw.max_p),
                   api.BAT_ERR_BLOCK_TABLE)


def test_prefix_rows_longer_than_bound(gpu_ready, validated):
    import torch
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd.device import to_device
    rng = np.random.default_rng(301)
    q = to_device(W._normal(rng, (300, 2, 64), "bf16"), "bf16")
    cu = torch.tensor([0, 100, 300], dtype=torch.int32, device="cuda")
    print("[validate] prefix rows longer than max_prefix_len", flush=True)
    api.attn_prefix_rows(q, q, q, cu, max_prefix_len=200)
    _expect_status(lambda: api.attn_prefix_rows(q, q, q, cu, max_prefix_len=150),
                   api.BAT_ERR_BLOCK_TABLE)


def test_kv_build_tokens_past_table_row(gpu_ready, validated):
    import torch
    from prefix_reuse_attention_amd import api
    z = torch.zeros((200, 2, 64), dtype=torch.bfloat16, device="cuda")
    pool = api.new_pool(8, 2, 64, 64, torch.bfloat16)
    bt = torch.tensor([[0, 1], [2, 3]], dtype=torch.int32, device="cuda")
    print("[validate] kv_build: 150 tokens in a 2 x 64 row", flush=True)
    api.kv_build(z, z, torch.tensor([0, 100, 200], dtype=torch.int32, device="cuda"), bt, pool)
    _expect_status(lambda: api.kv_build(z, z, torch.tensor([0, 150, 200], dtype=torch.int32,
                                                           device="cuda"), bt, pool),
                   api.BAT_ERR_BLOCK_TABLE)


def test_concurrent_validated_builds_report_their_own_errors(gpu_ready, validated):
    """Validated builds on two threads and two streams, one with a bad block
    id and one clean: each reports only its own violation."""
    import torch
    from prefix_reuse_attention_amd import api
    z = torch.zeros((128, 2, 64), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 128], dtype=torch.int32, device="cuda")
    good_bt = torch.tensor([[0, 1]], dtype=torch.int32, device="cuda")
    bad_bt = torch.tensor([[0, 99]], dtype=torch.int32, device="cuda")
    pools = [api.new_pool(4, 2, 64, 64, torch.bfloat16) for _ in range(2)]
    torch.cuda.synchronize()
    results = {"good": [], "bad": []}

    def worker(name, bt, pool):
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            for _ in range(40):
                try:
                    api.kv_build(z, z, cu, bt, pool)
                    results[name].append(api.BAT_OK)
                except api.BatError as e:
                    results[name].append(e.status)

    print("[validate] concurrent validated builds", flush=True)
    ts = [threading.Thread(target=worker, args=("good", good_bt, pools[0])),
          threading.Thread(target=worker, args=("bad", bad_bt, pools[1]))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert results["good"] == [api.BAT_OK] * 40
    assert results["bad"] == [api.BAT_ERR_BLOCK_TABLE] * 40


# Every copy path of the attention kernels meets a block id outside its pool:
# (name, dtype, head dim, user page size, BAT_WAVES, BAT_GATHER, prefix mode of
# the request whose row is corrupted)
BAD_ID_PATHS = [
    ("ping_pong_d128_pages", "bf16", 128, 64, "8", "", W.USER),
    ("ping_pong_d64_pages", "bf16", 64, 64, "8", "", W.USER),
    ("four_wave_pages", "bf16", 128, 64, "4", "", W.USER),
    ("four_wave_per_key", "bf16", 64, 16, "4", "", W.USER),
    ("ping_pong_per_key", "bf16", 128, 16, "8", "", W.USER),
    ("per_key_global_loads", "bf16", 64, 4, "4", "flat", W.USER),
    ("ping_pong_items", "bf16", 128, 64, "8", "", W.ITEM),
    ("fp32", "f32", 64, 16, "", "", W.USER),
]


@pytest.mark.parametrize("where", ["past_pool", "negative"])
@pytest.mark.parametrize("name,dtype,D,bs,waves,gather,mode", BAD_ID_PATHS)
def test_bad_block_id_every_copy_path(gpu_ready, monkeypatch, name, dtype, D, bs, waves, gather,
                                      mode, where):
    """One block id of request 0's row lies outside its pool (past the end,
    or negative).  With validation off the call succeeds: the kernels' bounds
    checks read that block as zeros, and request 1's rows still match the
    oracle.  With validation on the call returns BAT_ERR_BLOCK_TABLE."""
    import torch
    from helpers import as_f64, check_close, oracle_full
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd.device import DeviceWorkload, to_host
    for k, v in (("BAT_WAVES", waves), ("BAT_GATHER", gather)):
        if v:
            monkeypatch.setenv(k, v)
        else:
            monkeypatch.delenv(k, raising=False)
    monkeypatch.delenv("BAT_VALIDATE", raising=False)
    wl = W.make_custom(dtype=dtype, H=2, D=D, n_s=[300, 260], n_p=[700, 512],
                       mode=[mode, W.USER], seed=330 + D + bs, user_block_size=bs,
                       num_items=400, name=f"bad_id_{name}")
    dw = DeviceWorkload(wl)
    pool_blocks = 400 if mode == W.ITEM else wl.user_num_blocks
    bad = dw.block_table.clone()
    bad[0, 3] = pool_blocks + 7 if where == "past_pool" else -5
    print(f"[validate] bad block id, {name}, {where}", flush=True)
    out, lse = dw.run(block_table=bad)
    torch.cuda.synchronize()
    got = as_f64(to_host(out, wl.dtype), wl.dtype)
    got_lse = lse.cpu().numpy().astype(np.float64)
    ref_o, ref_l = oracle_full(wl)
    r0, r1 = int(wl.cu_s[1]), int(wl.cu_s[2])
    check_close(got[r0:r1], ref_o[r0:r1], wl.dtype)
    tol = 1e-5 if dtype == "f32" else 1e-3
    assert np.abs(got_lse[:, r0:r1] - ref_l[:, r0:r1]).max() <= tol
    monkeypatch.setenv("BAT_VALIDATE", "1")
    _expect_status(lambda: dw.run(block_table=bad), api.BAT_ERR_BLOCK_TABLE)
