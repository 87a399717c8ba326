"""C ABI of libbat without a GPU: the library loads, exports every entry
point include/bat.h declares, and rejects host-detectable argument errors
with the right status before enqueueing anything."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

from prefix_reuse_attention_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bat.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below returns early


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(api.LIB_PATH):
        from prefix_reuse_attention_amd import build
        build.build()
    return api.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[a-z_0-9 \*]*\b(bat_[a-z_0-9]+)\s*\(", text, re.M)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(api.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (bat_[a-z_0-9]+)$", out, re.M))
    assert set(declared_functions()) <= exported


def test_one_hip_runtime_in_the_process():
    """Loading the library through the binding maps exactly one HIP runtime:
    torch's (the one its tensors and streams belong to).  A second runtime
    loaded from the ROCm install beside torch's sees no device of its own."""
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from prefix_reuse_attention_amd import api\n"
            "api.load()\n"
            "maps = open('/proc/self/maps').read()\n"
            "print(len({l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}))\n"
            % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True)
    assert out.stdout.strip() == "1", out.stdout + out.stderr


def test_status_strings_and_version(lib):
    for s in range(6):
        assert api.status_string(s).startswith("BAT_")
    assert "unknown" in api.status_string(99)
    assert api.version() >= 100
    assert lib.bat_last_hip_error() == b"hipSuccess"  # no HIP call has failed in this thread


def _pool(num_blocks=4, block_size=64, k=FAKE, v=FAKE):
    return api.KvPool(k.value if k else None, v.value if v else None, num_blocks, block_size)


def kv_build(lib, **over):
    a = dict(k=FAKE, v=FAKE, cu=FAKE, bt=FAKE, bt_stride=4, B=2, H=8, D=64, total=100,
             dt=api.BAT_BF16, pool=_pool(), stream=None)
    a.update(over)
    pool = ctypes.byref(a["pool"]) if a["pool"] is not None else None
    return lib.bat_kv_build(a["k"], a["v"], a["cu"], a["bt"], a["bt_stride"], a["B"], a["H"],
                            a["D"], a["total"], a["dt"], pool, a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(pool=None), api.BAT_ERR_INVALID_ARG),
    (dict(k=None), api.BAT_ERR_INVALID_ARG),
    (dict(cu=None), api.BAT_ERR_INVALID_ARG),
    (dict(bt=None), api.BAT_ERR_INVALID_ARG),
    (dict(H=0), api.BAT_ERR_INVALID_ARG),
    (dict(B=-1), api.BAT_ERR_INVALID_ARG),
    (dict(total=-5), api.BAT_ERR_INVALID_ARG),
    (dict(D=48), api.BAT_ERR_UNSUPPORTED),
    (dict(dt=7), api.BAT_ERR_INVALID_ARG),
    (dict(pool=_pool(block_size=3)), api.BAT_ERR_INVALID_ARG),
    (dict(pool=_pool(block_size=512)), api.BAT_ERR_INVALID_ARG),
    (dict(pool=_pool(num_blocks=-1)), api.BAT_ERR_INVALID_ARG),
    (dict(pool=_pool(k=None)), api.BAT_ERR_INVALID_ARG),
    (dict(total=0), api.BAT_OK),                      # nothing to do, nothing launched
])
def test_kv_build_argument_errors(lib, over, status):
    assert kv_build(lib, **over) == status


def prefill(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, plen=FAKE, mode=FAKE, bt=FAKE, bt_stride=16,
             up=_pool(), ip=None, B=2, H=8, D=128, dt=api.BAT_BF16, scale=0.088, total=1024,
             max_s=512, max_p=1024, out=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(over)
    up = ctypes.byref(a["up"]) if a["up"] is not None else None
    ip = ctypes.byref(a["ip"]) if a["ip"] is not None else None
    if a["ws_bytes"] == "exact-1":
        a["ws_bytes"] = lib.bat_attn_workspace_size(a["B"], a["H"], a["D"], a["dt"], a["total"],
                                                    a["max_s"], a["max_p"]) - 1
        # the only remaining error is the workspace size: make every other
        # argument valid so that the call would otherwise launch
    return lib.bat_attn_prefill(a["q"], a["k"], a["v"], a["cu"], a["plen"], a["mode"], a["bt"],
                                a["bt_stride"], up, ip, a["B"], a["H"], a["D"], a["dt"],
                                a["scale"], a["total"], a["max_s"], a["max_p"], a["out"],
                                a["lse"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(q=None), api.BAT_ERR_INVALID_ARG),
    (dict(out=None), api.BAT_ERR_INVALID_ARG),
    (dict(cu=None), api.BAT_ERR_INVALID_ARG),
    (dict(plen=None), api.BAT_ERR_INVALID_ARG),
    (dict(mode=None), api.BAT_ERR_INVALID_ARG),
    (dict(bt=None), api.BAT_ERR_INVALID_ARG),          # prefixes but no block table
    (dict(up=None), api.BAT_ERR_INVALID_ARG),          # prefixes but no pool
    (dict(scale=0.0), api.BAT_ERR_INVALID_ARG),
    (dict(scale=-1.0), api.BAT_ERR_INVALID_ARG),
    (dict(scale=float("nan")), api.BAT_ERR_INVALID_ARG),
    (dict(H=0), api.BAT_ERR_INVALID_ARG),
    (dict(B=-2), api.BAT_ERR_INVALID_ARG),
    (dict(max_s=0), api.BAT_ERR_INVALID_ARG),
    (dict(max_p=-1), api.BAT_ERR_INVALID_ARG),
    (dict(D=32), api.BAT_ERR_UNSUPPORTED),             # bf16 kernels: D in {64, 128}
    (dict(D=96), api.BAT_ERR_UNSUPPORTED),
    (dict(D=256, dt=api.BAT_F32), api.BAT_ERR_UNSUPPORTED),
    (dict(dt=3), api.BAT_ERR_INVALID_ARG),
    (dict(up=_pool(block_size=6)), api.BAT_ERR_INVALID_ARG),
    (dict(ws=None), api.BAT_ERR_WORKSPACE),
    (dict(ws_bytes="exact-1"), api.BAT_ERR_WORKSPACE),
    (dict(total=0), api.BAT_OK),                       # no suffix rows: nothing to write
])
def test_prefill_argument_errors(lib, over, status):
    assert prefill(lib, **over) == status


def test_workspace_size(lib):
    f = lib.bat_attn_workspace_size
    assert f(2, 8, 128, api.BAT_BF16, 1024, 512, 1024) > 0
    assert f(2, 8, 128, api.BAT_BF16, 1024, 512, 1024) <= f(4, 8, 128, api.BAT_BF16, 2048, 512, 1024)
    assert f(-1, 8, 128, api.BAT_BF16, 1024, 512, 1024) == 0
    assert f(2, 8, 96, api.BAT_BF16, 1024, 512, 1024) == 0
    # a batch too small to fill the GPU with a long prefix gets split partials
    assert f(1, 2, 128, api.BAT_BF16, 64, 64, 16384) > f(1, 2, 128, api.BAT_BF16, 64, 64, 1024)


def _partial_rows(lib, B, H, D, total_s, max_s, max_p, monkeypatch):
    """Split-partial copies of every row in the plan: (workspace with the
    library's policy - workspace with splitting off) / bytes of one copy."""
    f = lib.bat_attn_workspace_size
    split = f(B, H, D, api.BAT_BF16, total_s, max_s, max_p)
    monkeypatch.setenv("BAT_SPLIT_CHUNK", "100000000")
    whole = f(B, H, D, api.BAT_BF16, total_s, max_s, max_p)
    monkeypatch.delenv("BAT_SPLIT_CHUNK")
    return (split - whole) / (total_s * H * (D + 1) * 4)


@pytest.mark.parametrize("B,H,n_s,n_p,chunks", [
    (64, 8, 32, 4096, 0),     # 512 four-wave items, one per request and head: full
    (32, 8, 128, 2048, 0),    # 256 four-wave items: a split would need 1024-key chunks
    (16, 16, 512, 8192, 0),   # 512 eight-wave items (the 8k-history shape): full
    (32, 8, 64, 8192, 2),     # 256 four-wave items over 8k prefixes: 4096-key chunks
    (16, 8, 96, 8192, 4),     # 128 items: 2048-key chunks
    (2, 16, 512, 32768, 4),   # 64 eight-wave items: 8192-key chunks, one item per CU
    (1, 2, 64, 16384, 32),    # 2 items: 512-key chunks, the most the GPU can use
])
def test_split_policy(lib, monkeypatch, B, H, n_s, n_p, chunks):
    """The automatic prefix split (D=128, equal suffixes): none when the
    unsplit items already fill the CUs (one per request and head at least),
    chunks of 2048 keys or more once every CU has an item, shorter ones only
    while CUs would stay idle."""
    got = _partial_rows(lib, B, H, 128, B * n_s, n_s, n_p, monkeypatch)
    assert abs(got - chunks) < 0.1, (B, H, n_s, n_p, got)


def test_prefill_workspace_size_bounds_every_call(lib):
    """The bound with the surveyed signature (no dtype, no suffix bound)
    covers the exact size for both dtypes and every suffix bound up to
    total_suffix, and is rejected where the exact size is."""
    f, g = lib.bat_attn_prefill_workspace_size, lib.bat_attn_workspace_size
    for B, H, D, total, max_p in [(2, 8, 128, 1024, 1024), (16, 16, 128, 8192, 8192),
                                  (1, 2, 64, 64, 16384), (32, 8, 64, 8192, 1024),
                                  (128, 8, 128, 70000, 16384), (3, 4, 32, 24, 64)]:
        bound = f(B, H, D, total, max_p)
        assert bound > 0
        for dt in (api.BAT_F32, api.BAT_BF16):
            for max_s in sorted({1, total // B, total // 2, total}):
                n = g(B, H, D, dt, total, max_s, max_p)
                if n:
                    assert n <= bound, (B, H, D, dt, total, max_s, max_p)
    assert f(2, 8, 96, 1024, 1024) == 0
    assert f(-1, 8, 128, 1024, 1024) == 0
    assert f(2, 0, 128, 1024, 1024) == 0
    # head dim 32 has only the fp32 kernel: the bound is the fp32 size
    assert f(1, 4, 32, 8, 64) == max(g(1, 4, 32, api.BAT_F32, 8, s, 64) for s in range(1, 9))


def prefix_rows(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, B=2, H=8, D=128, dt=api.BAT_BF16, scale=0.088,
             total=1024, max_p=512, out=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(over)
    if a["ws_bytes"] == "exact-1":
        a["ws_bytes"] = lib.bat_attn_workspace_size(a["B"], a["H"], a["D"], a["dt"], a["total"],
                                                    a["max_p"], 0) - 1
    return lib.bat_attn_prefix_rows(a["q"], a["k"], a["v"], a["cu"], a["B"], a["H"], a["D"],
                                    a["dt"], a["scale"], a["total"], a["max_p"], a["out"],
                                    a["lse"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(q=None), api.BAT_ERR_INVALID_ARG),
    (dict(k=None), api.BAT_ERR_INVALID_ARG),
    (dict(out=None), api.BAT_ERR_INVALID_ARG),
    (dict(cu=None), api.BAT_ERR_INVALID_ARG),
    (dict(scale=0.0), api.BAT_ERR_INVALID_ARG),
    (dict(H=0), api.BAT_ERR_INVALID_ARG),
    (dict(B=-1), api.BAT_ERR_INVALID_ARG),
    (dict(max_p=0), api.BAT_ERR_INVALID_ARG),
    (dict(D=32), api.BAT_ERR_UNSUPPORTED),
    (dict(dt=7), api.BAT_ERR_INVALID_ARG),
    (dict(ws=None), api.BAT_ERR_WORKSPACE),
    (dict(ws_bytes="exact-1"), api.BAT_ERR_WORKSPACE),
    (dict(total=0), api.BAT_OK),                       # no prefix rows: nothing to write
])
def test_prefix_rows_argument_errors(lib, over, status):
    assert prefix_rows(lib, **over) == status


def item_local(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, n=100, T=4, H=8, D=64, dt=api.BAT_BF16, scale=0.125,
             out=FAKE, lse=None, stream=None)
    a.update(over)
    return lib.bat_attn_item_local(a["q"], a["k"], a["v"], a["n"], a["T"], a["H"], a["D"],
                                   a["dt"], a["scale"], a["out"], a["lse"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(q=None), api.BAT_ERR_INVALID_ARG),
    (dict(v=None), api.BAT_ERR_INVALID_ARG),
    (dict(out=None), api.BAT_ERR_INVALID_ARG),
    (dict(n=-1), api.BAT_ERR_INVALID_ARG),
    (dict(H=0), api.BAT_ERR_INVALID_ARG),
    (dict(scale=float("inf")), api.BAT_ERR_INVALID_ARG),
    (dict(T=3), api.BAT_ERR_UNSUPPORTED),              # T in {1, 2, 4, 8}
    (dict(T=16), api.BAT_ERR_UNSUPPORTED),
    (dict(D=32), api.BAT_ERR_UNSUPPORTED),
    (dict(dt=5), api.BAT_ERR_INVALID_ARG),
    (dict(n=1 << 29, T=8), api.BAT_ERR_INVALID_ARG),   # rows beyond int32
    (dict(n=0), api.BAT_OK),
])
def test_item_local_argument_errors(lib, over, status):
    assert item_local(lib, **over) == status


def isolated(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, plen=FAKE, mode=FAKE, bt=FAKE, bt_stride=16,
             up=_pool(), ip=None, B=2, H=8, D=64, dt=api.BAT_BF16, scale=0.125, T=4, total=1024,
             max_s=512, max_p=1024, out=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(over)
    up = ctypes.byref(a["up"]) if a["up"] is not None else None
    ip = ctypes.byref(a["ip"]) if a["ip"] is not None else None
    if a["ws_bytes"] == "exact-1":
        a["ws_bytes"] = lib.bat_attn_isolated_workspace_size(a["B"], a["H"], a["D"], a["dt"],
                                                             a["total"], a["max_s"],
                                                             a["max_p"]) - 1
    return lib.bat_attn_prefill_isolated(a["q"], a["k"], a["v"], a["cu"], a["plen"], a["mode"],
                                         a["bt"], a["bt_stride"], up, ip, a["B"], a["H"], a["D"],
                                         a["dt"], a["scale"], a["T"], a["total"], a["max_s"],
                                         a["max_p"], a["out"], a["lse"], a["ws"], a["ws_bytes"],
                                         a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(q=None), api.BAT_ERR_INVALID_ARG),
    (dict(plen=None), api.BAT_ERR_INVALID_ARG),
    (dict(bt=None), api.BAT_ERR_INVALID_ARG),          # prefixes but no block table
    (dict(up=None), api.BAT_ERR_INVALID_ARG),          # prefixes but no pool
    (dict(scale=0.0), api.BAT_ERR_INVALID_ARG),
    (dict(T=3), api.BAT_ERR_UNSUPPORTED),
    (dict(T=16), api.BAT_ERR_UNSUPPORTED),
    (dict(total=1022), api.BAT_ERR_INVALID_ARG),       # not whole candidates
    (dict(D=32), api.BAT_ERR_UNSUPPORTED),
    (dict(ws=None), api.BAT_ERR_WORKSPACE),
    (dict(ws_bytes="exact-1"), api.BAT_ERR_WORKSPACE),
    (dict(total=0), api.BAT_OK),
])
def test_isolated_argument_errors(lib, over, status):
    assert isolated(lib, **over) == status


def test_isolated_workspace_holds_a_partial_per_row(lib):
    f, g = lib.bat_attn_isolated_workspace_size, lib.bat_attn_workspace_size
    # one fp32 output row and lse per (suffix row, head) beyond the work list
    assert f(2, 8, 64, api.BAT_BF16, 1024, 512, 1024) >= \
        g(2, 8, 64, api.BAT_BF16, 1024, 512, 1024) + 1024 * 8 * (64 + 1) * 4
    assert f(2, 8, 96, api.BAT_BF16, 1024, 512, 1024) == 0


def gqa(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, plen=FAKE, mode=FAKE, bt=FAKE, bt_stride=16,
             up=_pool(), ip=None, B=2, H=8, H_kv=2, D=128, dt=api.BAT_BF16, scale=0.088,
             total=1024, max_s=512, max_p=1024, out=FAKE, lse=None, ws=None, ws_bytes=0,
             stream=None)
    a.update(over)
    up = ctypes.byref(a["up"]) if a["up"] is not None else None
    ip = ctypes.byref(a["ip"]) if a["ip"] is not None else None
    return lib.bat_attn_prefill_gqa(a["q"], a["k"], a["v"], a["cu"], a["plen"], a["mode"],
                                    a["bt"], a["bt_stride"], up, ip, a["B"], a["H"], a["H_kv"],
                                    a["D"], a["dt"], a["scale"], a["total"], a["max_s"],
                                    a["max_p"], a["out"], a["lse"], a["ws"], a["ws_bytes"],
                                    a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(H_kv=3), api.BAT_ERR_INVALID_ARG),           # 8 query heads, 3 key/value heads
    (dict(H_kv=0), api.BAT_ERR_INVALID_ARG),
    (dict(H_kv=16), api.BAT_ERR_INVALID_ARG),          # more key/value heads than query heads
    (dict(k=None), api.BAT_ERR_INVALID_ARG),
    (dict(D=96), api.BAT_ERR_UNSUPPORTED),
    (dict(), api.BAT_ERR_WORKSPACE),                   # valid otherwise: no workspace
    (dict(total=0), api.BAT_OK),
])
def test_gqa_argument_errors(lib, over, status):
    assert gqa(lib, **over) == status


def test_lse_merge_argument_errors(lib):
    m = lib.bat_lse_merge
    assert m(FAKE, FAKE, 0, 10, 2, 64, api.BAT_F32, FAKE, None, None) == api.BAT_ERR_INVALID_ARG
    assert m(FAKE, FAKE, 2, 10, 2, 62, api.BAT_F32, FAKE, None, None) == api.BAT_ERR_INVALID_ARG
    assert m(None, FAKE, 2, 10, 2, 64, api.BAT_F32, FAKE, None, None) == api.BAT_ERR_INVALID_ARG
    assert m(FAKE, FAKE, 2, 10, 2, 64, 9, FAKE, None, None) == api.BAT_ERR_INVALID_ARG
    assert m(FAKE, FAKE, 2, 0, 2, 64, api.BAT_F32, FAKE, None, None) == api.BAT_OK
