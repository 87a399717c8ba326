"""GPU: the device planner's work decomposition (white-box).

The planner writes its work items into the workspace, right after the
256-byte header: one {request, head, row tile, chunk} record of four int32 per
slot, slot index = 8 * per-XCD slot + XCD, unused slots with request -1.  The
tests read that list back after bat_attn_prefill and check it against what
the decomposition must be:

* every (request, head, row tile) of a non-empty suffix exactly once, nothing
  else, and the header's item count equal to their number;
* all row tiles of one (request, head) on one XCD, in consecutive slots in
  row-tile order (they share that XCD's L2 copy of the prefix);
* on every XCD, requests in non-increasing order of keys per item (longest
  first), which bounds the tail.

Batches of up to 256 requests and larger ones take different planner paths;
both are covered.  Prefixes are never split here (BAT_SPLIT_CHUNK beyond the
longest prefix), so the chunk of every item is 0.
"""
import numpy as np
import pytest

from prefix_reuse_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

HDR_BYTES = 256
ITEMS_OFF = 256


def _run_plan(wl, monkeypatch):
    import torch
    from prefix_reuse_attention_amd.device import DeviceWorkload
    monkeypatch.setenv("BAT_SPLIT_CHUNK", "1000000")
    dw = DeviceWorkload(wl)
    ws = dw.workspace()
    ws.fill_(0xAB)
    dw.run(workspace=ws)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    hdr = raw[:HDR_BYTES].view(np.int32)
    return hdr, raw


def _check(wl, hdr, raw, H=None, hg=1):
    """H query heads (wl.H by default), hg of them per key/value head."""
    B, H = wl.B, (wl.H if H is None else H)
    total_s = int(wl.n_s.sum())
    # eight-wave (256-row) items when suffixes average more than 128 rows
    eight = total_s > 128 * B
    bm = 256 if eight else 128
    max_s = int(wl.n_s.max())
    t_max = -(-max_s // bm)
    grid = 8 * (-(-((H // hg) * B) // 8)) * hg * t_max
    items = raw[ITEMS_OFF:ITEMS_OFF + 16 * grid].view(np.int32).reshape(grid, 4)
    real = items[items[:, 0] >= 0]
    assert np.all(items[items[:, 0] < 0, 0] == -1), "unused slots must hold request -1"
    expect = set()
    for r in range(B):
        T = -(-int(wl.n_s[r]) // bm)
        for h in range(H):
            for t in range(T):
                expect.add((r, h, t, 0))
    got = [tuple(int(v) for v in row) for row in real]
    assert len(got) == len(set(got)), "an item appears twice"
    assert set(got) == expect
    assert int(hdr[1]) == len(expect)
    # row tiles of one (request, head) on one XCD, consecutive slots in order
    idx = np.nonzero(items[:, 0] >= 0)[0]
    pos = {}
    for i in idx:
        r, h, t, c = (int(v) for v in items[i])
        pos.setdefault((r, h), {})[t] = int(i)
    for (r, h), ts in pos.items():
        slots = [ts[t] for t in range(len(ts))]
        assert len({s % 8 for s in slots}) == 1, f"group {(r, h)} spans XCDs"
        assert all(b - a == 8 for a, b in zip(slots, slots[1:])), f"group {(r, h)} not consecutive"
    # with grouped heads: the hg query heads of one key/value head follow one
    # another on one XCD, head by head
    if hg > 1:
        for r in range(B):
            for hk in range(H // hg):
                seq = [pos[(r, h)][t] for h in range(hk * hg, (hk + 1) * hg)
                       if (r, h) in pos for t in range(len(pos[(r, h)]))]
                if not seq:
                    continue
                assert len({s % 8 for s in seq}) == 1, f"kv group {(r, hk)} spans XCDs"
                assert all(b - a == 8 for a, b in zip(seq, seq[1:])), \
                    f"kv group {(r, hk)} not consecutive"
    # longest first on every XCD
    key = wl.n_s.astype(np.int64) + np.minimum(wl.n_p, int(wl.n_p.max())).astype(np.int64)
    for x in range(8):
        seq = [key[int(items[i, 0])] for i in idx if i % 8 == x]
        assert all(a >= b for a, b in zip(seq, seq[1:])), f"XCD {x} not longest first"


@pytest.mark.parametrize("B,seed,D", [(3, 1, 64), (16, 2, 64), (100, 3, 64), (256, 4, 64),
                                      (300, 5, 64), (100, 8, 128), (300, 9, 128)])
def test_plan_items(gpu_ready, monkeypatch, B, seed, D):
    """Head dim 64 plans 128-row items here (short prefixes), head dim 128
    256-row items: both item sizes on both planner paths."""
    rng = np.random.default_rng(1000 + seed)
    n_s = rng.integers(1, 600, size=B)
    n_s[rng.random(B) < 0.1] = 0        # some empty suffixes
    n_p = rng.integers(0, 700, size=B)
    wl = W.make_custom(dtype="bf16", H=2, D=D, n_s=n_s.tolist(), n_p=n_p.tolist(),
                       mode=[W.USER] * B, seed=seed, user_block_size=64,
                       name=f"plan_B{B}")
    print(f"[planner] B={B} total_s={int(n_s.sum())}", flush=True)
    hdr, raw = _run_plan(wl, monkeypatch)
    _check(wl, hdr, raw)


@pytest.mark.parametrize("B,hg,seed", [(16, 4, 6), (300, 2, 7)])
def test_plan_items_grouped_heads(gpu_ready, monkeypatch, B, hg, seed):
    """Grouped key/value heads (8 query heads over 8 / hg key/value heads),
    through bat_attn_prefill_gqa; both planner paths."""
    import torch
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd.device import DeviceWorkload, to_device
    monkeypatch.setenv("BAT_SPLIT_CHUNK", "1000000")
    rng = np.random.default_rng(2000 + seed)
    n_s = rng.integers(1, 600, size=B)
    n_s[rng.random(B) < 0.1] = 0
    n_p = rng.integers(0, 700, size=B)
    H = 8
    wl = W.make_custom(dtype="bf16", H=H // hg, D=64, n_s=n_s.tolist(), n_p=n_p.tolist(),
                       mode=[W.USER] * B, seed=seed, user_block_size=64,
                       name=f"plan_gqa_B{B}")
    print(f"[planner] gqa B={B} hg={hg} total_s={int(n_s.sum())}", flush=True)
    dw = DeviceWorkload(wl)
    q = to_device(W._normal(rng, (wl.total_s, H, wl.D), "bf16"), "bf16")
    n = api.load().bat_attn_gqa_workspace_size(B, H, H // hg, wl.D, api.BAT_BF16, wl.total_s,
                                               dw.max_s, dw.max_p)
    ws = torch.full((max(int(n), 1),), 0xAB, dtype=torch.uint8, device="cuda")
    api.attn_prefill_gqa(q, dw.k, dw.v, dw.cu_s, dw.prefix_lens, dw.prefix_mode, dw.block_table,
                         dw.user_pool, dw.item_pool, wl.scale, dw.max_s, dw.max_p, workspace=ws)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    _check(wl, raw[:HDR_BYTES].view(np.int32), raw, H=H, hg=hg)
