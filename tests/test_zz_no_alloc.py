"""GPU: bat_attn_prefill_noalloc (the entry point with no workspace, for
callers that cannot allocate) against bat_attn_prefill on the same inputs.

Two calls in a row on one device, the second with a smaller batch, so the
second runs over the scratch the first left behind.  Each is compared with
bat_attn_prefill to the parity bar (bitwise where both take the same plan,
which they do here) and with the oracle.  A batch whose split partials
would not fit the scratch runs unsplit (same rows up to rounding), and the
out-of-range case returns BAT_ERR_WORKSPACE without launching anything.
"""
import numpy as np
import pytest

from helpers import as_f64, check_close, oracle_full
from prefix_reuse_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


def _noalloc(dw, out, lse):
    from prefix_reuse_attention_amd import api
    return api.attn_prefill_noalloc(dw.q, dw.k, dw.v, dw.cu_s, dw.prefix_lens, dw.prefix_mode,
                                    dw.block_table, dw.user_pool, dw.item_pool, dw.wl.scale,
                                    dw.max_s, dw.max_p, out, lse)


def test_noalloc_matches_prefill_twice(gpu_ready):
    import torch
    from prefix_reuse_attention_amd.device import DeviceWorkload, to_host
    big = W.make_custom(dtype="bf16", H=4, D=128, n_s=[256, 300, 17, 256],
                        n_p=[2000, 64, 700, 1000], mode=[W.USER, W.ITEM, W.USER, W.USER],
                        seed=401, num_items=300, name="noalloc_big")
    small = W.make_custom(dtype="bf16", H=2, D=64, n_s=[40, 40], n_p=[130, 0],
                          mode=[W.USER, W.USER], seed=402, name="noalloc_small")
    for wl in (big, small):
        print(f"[noalloc] {wl.name} B={wl.B} H={wl.H} D={wl.D}", flush=True)
        dw = DeviceWorkload(wl)
        ref_out, ref_lse = dw.run(want_lse=True)
        out = torch.empty_like(dw.q)
        lse = torch.empty((wl.H, wl.total_s), dtype=torch.float32, device="cuda")
        _noalloc(dw, out, lse)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host(out, "bf16"), to_host(ref_out, "bf16"))
        np.testing.assert_array_equal(lse.cpu().numpy(), ref_lse.cpu().numpy())
        o_ref, l_ref = oracle_full(wl)
        check_close(as_f64(to_host(out, "bf16"), "bf16"), o_ref, "bf16")
        assert np.abs(lse.cpu().numpy() - l_ref).max() <= 1e-3


def test_noalloc_split_partials_too_large_run_unsplit(gpu_ready):
    """Two 32768-token prefixes with short suffixes: bat_attn_prefill splits
    them (partials beyond the scratch); the allocation-free call computes the
    same rows unsplit."""
    import torch
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd.device import DeviceWorkload, to_host
    wl = W.make_custom(dtype="bf16", H=16, D=128, n_s=[512, 512], n_p=[32768, 32768],
                       mode=[W.USER] * 2, seed=403, name="noalloc_split")
    assert api.workspace_size(wl.B, wl.H, wl.D, api.BAT_BF16, wl.total_s, 512, 32768) > \
        api.noalloc_scratch_bytes()
    print("[noalloc] split partials beyond the scratch", flush=True)
    dw = DeviceWorkload(wl)
    ref_out, ref_lse = dw.run(want_lse=True)
    out = torch.empty_like(dw.q)
    lse = torch.empty((wl.H, wl.total_s), dtype=torch.float32, device="cuda")
    _noalloc(dw, out, lse)
    torch.cuda.synchronize()
    got = as_f64(to_host(out, "bf16"), "bf16")
    check_close(got, as_f64(to_host(ref_out, "bf16"), "bf16"), "bf16", strict_abs=4e-3)
    assert np.abs(lse.cpu().numpy() - ref_lse.cpu().numpy()).max() <= 1e-3


def test_noalloc_rejects_a_batch_beyond_the_scratch(gpu_ready):
    """A work list larger than the scratch is refused before any launch (the
    pointers are never read: the call returns during planning)."""
    import ctypes
    from prefix_reuse_attention_amd import api
    lib = api.load()
    fake = ctypes.c_void_p(0x1000)
    pool = api.KvPool(0x1000, 0x1000, 1 << 20, 64)
    # 2^20 requests x 64 heads of one row each: 2^26 work items of 16 bytes
    st = lib.bat_attn_prefill_noalloc(fake, fake, fake, fake, fake, fake, fake, 1,
                                      ctypes.byref(pool), None, 1 << 20, 64, 128, api.BAT_BF16,
                                      0.088, 1 << 20, 1, 64, fake, None, None)
    assert st == api.BAT_ERR_WORKSPACE
