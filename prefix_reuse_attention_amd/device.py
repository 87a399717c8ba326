"""Put a seeded workload on the GPU: upload tensors, build the paged pools with
bat_kv_build, and run bat_attn_prefill over it.  Used by the tests, the smoke
check and the benchmark."""
import numpy as np

from . import api
from . import workloads as W


def to_device(a, dtype_name):
    """numpy float32 / uint16-bf16-bits array -> device tensor of the same values."""
    import torch
    a = np.ascontiguousarray(a)
    if dtype_name == "bf16":
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to("cuda")
    return torch.from_numpy(a).to("cuda")


def to_host(t, dtype_name):
    """Device tensor -> numpy (float32, or uint16 bf16 bits)."""
    import torch
    if dtype_name == "bf16":
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


class DeviceWorkload:
    """Device copy of a Workload with its user and item pools built."""

    def __init__(self, wl: W.Workload, pool_fill=None, build=True):
        import torch
        self.wl = wl
        self.tdtype = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        self.q = to_device(wl.q, wl.dtype)
        self.k = to_device(wl.k_s, wl.dtype)
        self.v = to_device(wl.v_s, wl.dtype)
        self.cu_s = torch.from_numpy(wl.cu_s).to("cuda")
        self.prefix_lens = torch.from_numpy(np.ascontiguousarray(wl.n_p)).to("cuda")
        self.prefix_mode = torch.from_numpy(np.ascontiguousarray(wl.mode)).to("cuda")
        self.block_table = torch.from_numpy(wl.block_table).to("cuda")
        self.max_s = int(wl.n_s.max()) if wl.B else 0
        self.max_p = int(wl.n_p.max()) if wl.B else 0
        self.user_pool = None
        self.item_pool = None
        if build:
            self.build_pools(pool_fill)

    def upload_prefix(self):
        """Copy the logical prefix tokens (and the item pool's source) to the device."""
        import torch
        wl = self.wl
        self._src = {}
        if np.any(wl.mode == W.USER) and wl.cu_user[-1] > 0:
            self._src["user"] = (to_device(wl.user_k, wl.dtype), to_device(wl.user_v, wl.dtype),
                                 torch.from_numpy(wl.cu_user).to("cuda"), self.block_table)
        if np.any(wl.mode == W.ITEM):
            n = wl.num_items
            cu = torch.arange(0, (n + 1) * W.ITEM_TOKENS, W.ITEM_TOKENS, dtype=torch.int32,
                              device="cuda")
            bt = torch.arange(n, dtype=torch.int32, device="cuda").reshape(n, 1)
            self._src["item"] = (to_device(wl.item_k, wl.dtype), to_device(wl.item_v, wl.dtype),
                                 cu, bt)

    def build_pools_fp8(self):
        """fp8 copies of the pools (E4M3 codes with a power-of-two scale per
        block and head), built by bat_kv_build_fp8 from the same tokens and
        block tables; they replace the bf16 pools for run_fp8."""
        wl = self.wl
        self.upload_prefix()
        self.user_pool8 = self.item_pool8 = None
        if "user" in self._src:
            self.user_pool8 = api.new_pool_fp8(wl.user_num_blocks, wl.H, wl.user_block_size, wl.D)
            api.kv_build_fp8(*self._src["user"], self.user_pool8)
        if "item" in self._src:
            self.item_pool8 = api.new_pool_fp8(wl.num_items, wl.H, W.ITEM_TOKENS, wl.D)
            api.kv_build_fp8(*self._src["item"], self.item_pool8)
        self.drop_prefix_source()

    def run_fp8(self, out=None, lse=None, workspace=None, want_lse=True, block_table=None):
        return api.attn_prefill_fp8(self.q, self.k, self.v, self.cu_s, self.prefix_lens,
                                    self.prefix_mode,
                                    self.block_table if block_table is None else block_table,
                                    self.user_pool8, self.item_pool8, self.wl.scale, self.max_s,
                                    self.max_p, out=out, lse=lse, workspace=workspace,
                                    want_lse=want_lse)

    def alloc_pools(self, fill=None):
        wl = self.wl
        if "user" in self._src:
            self.user_pool = api.new_pool(wl.user_num_blocks, wl.H, wl.user_block_size, wl.D,
                                          self.tdtype, fill)
        if "item" in self._src:
            self.item_pool = api.new_pool(wl.num_items, wl.H, W.ITEM_TOKENS, wl.D, self.tdtype,
                                          fill)

    def build_kv(self):
        """bat_kv_build of every pool from the uploaded prefix tokens."""
        if "user" in self._src:
            api.kv_build(*self._src["user"], self.user_pool)
        if "item" in self._src:
            api.kv_build(*self._src["item"], self.item_pool)

    def prefix_bytes(self):
        """Bytes of K+V the build copies (each read once and written once)."""
        return sum(2 * s[0].numel() * s[0].element_size() for s in self._src.values())

    def drop_prefix_source(self):
        self._src = {k: () for k in self._src}

    def build_pools(self, fill=None):
        self.upload_prefix()
        self.alloc_pools(fill)
        self.build_kv()
        self.drop_prefix_source()

    def workspace(self):
        import torch
        n = api.workspace_size(self.wl.B, self.wl.H, self.wl.D,
                               api.BAT_BF16 if self.wl.dtype == "bf16" else api.BAT_F32,
                               self.wl.total_s, self.max_s, self.max_p)
        return torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")

    def prepared(self, out, lse, workspace):
        """bat_attn_prefill over this workload with its arguments marshalled
        once (api.PreparedPrefill)."""
        return api.PreparedPrefill(self.q, self.k, self.v, self.cu_s, self.prefix_lens,
                                   self.prefix_mode, self.block_table, self.user_pool,
                                   self.item_pool, self.wl.scale, self.max_s, self.max_p, out,
                                   lse, workspace)

    def run(self, out=None, lse=None, workspace=None, want_lse=True, block_table=None):
        return api.attn_prefill(self.q, self.k, self.v, self.cu_s, self.prefix_lens,
                                self.prefix_mode,
                                self.block_table if block_table is None else block_table,
                                self.user_pool, self.item_pool, self.wl.scale, self.max_s,
                                self.max_p, out=out, lse=lse, workspace=workspace,
                                want_lse=want_lse)
