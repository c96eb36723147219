"""A paged KV cache over the C ABI: slabs for owning layers only.

Every layer that owns KV gets its own K/V slab (and scales for the int8
per-token-head format); a KV-shared layer gets none and reads its source's slab
through the library's layer map (unsloth commit dee9371, "scripts": shared
layers reference the store layer's cache; FreeToken PR #898, description: the
pool allocates slabs only for layers that own KV).  PyTorch provides the device
memory and the stream; all computation is in libpakv.so.
"""

import torch

from . import pakv

SLIDING, FULL = 0, 1


class PagedKVCache:
    """layers: sequence of objects or dicts with head_dim, num_q_heads,
    num_kv_heads, window (0 = full), kv_dtype ("bf16" / "int8") and sm_scale.
    first_shared: index of the first KV-shared layer, or None."""

    DTYPES = {"bf16": pakv.KV_BF16, "int8": pakv.KV_INT8_PTH, "fp8": pakv.KV_FP8_PTH}

    def __init__(self, layers, first_shared, num_pages, device="cuda", sentinel=True, k_eq_v_storage=True,
                 v_norm_eps=1e-6):
        """k_eq_v_storage: layers whose spec says k_eq_v keep one slab (values
        derived from the keys in-kernel); False keeps two slabs and the caller
        stores the value rows itself."""
        def get(l, k, default=None):
            if isinstance(l, dict):
                return l.get(k, default)
            return getattr(l, k, default)
        self.specs = [{k: get(l, k) for k in ("head_dim", "num_q_heads", "num_kv_heads", "window",
                                              "kv_dtype", "sm_scale")} for l in layers]
        for s, l in zip(self.specs, layers):
            s["k_eq_v"] = bool(get(l, "k_eq_v", False)) and k_eq_v_storage
            s["v_norm_eps"] = float(v_norm_eps)
        n = len(self.specs)
        types = [SLIDING if s["window"] > 0 else FULL for s in self.specs]
        fs = n if first_shared is None else first_shared
        self.sources = pakv.resolve_kv_sources(types, fs)
        descs = []
        for l, s in enumerate(self.specs):
            descs.append(pakv.LayerDesc(s["head_dim"], s["num_q_heads"], s["num_kv_heads"], s["window"],
                                        -1 if self.sources[l] == l else self.sources[l],
                                        self.DTYPES[s["kv_dtype"]], float(s["sm_scale"]),
                                        1 if s["k_eq_v"] else 0, s["v_norm_eps"]))
        self.map = pakv.LayerMap(descs)
        # num_pages: one pool size for every slab, or {"sliding": n, "full": m}
        # when each group has its own pool (a window pool for the sliding group)
        self.num_pages = num_pages
        self.device = torch.device(device)
        self.slabs = {}
        for l, s in enumerate(self.specs):
            if self.sources[l] != l:
                continue
            hkv, d = s["num_kv_heads"], s["head_dim"]
            if isinstance(num_pages, dict):
                num_pages_l = num_pages["sliding" if s["window"] > 0 else "full"]
            else:
                num_pages_l = num_pages
            self._fill_slab(l, s, hkv, d, num_pages_l, sentinel)
        self.pages = None
        self.page_table = None
        self._group_pages = {}     # "sliding" / "full" -> (table tensor, pakv_pages) of that group
        self._workspace = None
        self._stage_ws = None

    def _fill_slab(self, l, s, hkv, d, num_pages, sentinel):
        """Allocates and binds owner layer l's slab, filled with a sentinel
        (a NaN, or a code the encoders never make) where nothing is stored."""
        if s["kv_dtype"] == "bf16":
            fill = 0x7FC0 if sentinel else 0            # bf16 quiet NaN
            k = torch.full((num_pages, hkv, 16, d), fill, dtype=torch.int16, device=self.device)
            v = None if s["k_eq_v"] else torch.full((num_pages, hkv, d, 16), fill, dtype=torch.int16,
                                                    device=self.device)
            ks = vs = None
        else:
            # int8: -128, a code the encoder never makes; fp8: 0xFF, an E4M3 NaN
            fill = (-128 if s["kv_dtype"] == "int8" else -1) if sentinel else 0
            k = torch.full((num_pages, hkv, 16, d), fill, dtype=torch.int8, device=self.device)
            v = torch.full((num_pages, hkv, d, 16), fill, dtype=torch.int8, device=self.device)
            sfill = float("nan") if sentinel else 0.0
            ks = torch.full((num_pages, hkv, 16), sfill, dtype=torch.float32, device=self.device)
            vs = torch.full((num_pages, hkv, 16), sfill, dtype=torch.float32, device=self.device)
        self.map.bind_slab(l, k, v, num_pages, ks, vs)
        self.slabs[l] = (k, v, ks, vs)

    def slab_of(self, layer):
        return self.slabs[self.sources[layer]]

    def set_page_table(self, page_table, group=None):
        """page_table: int32 [B, max_pages] (host or device).  group None: one
        table for every layer; "sliding" or "full": that group's own table (a
        window pool's, for the sliding group), used by its layers in place of
        the shared one."""
        t = torch.as_tensor(page_table, dtype=torch.int32).to(self.device).contiguous()
        if group is None:
            self.page_table = t
            self.pages = pakv.make_pages(self.page_table)
        else:
            assert group in ("sliding", "full")
            self._group_pages[group] = (t, pakv.make_pages(t))

    def pages_of(self, layer):
        group = "sliding" if self.specs[layer]["window"] > 0 else "full"
        if group in self._group_pages:
            return self._group_pages[group][1]
        return self.pages

    def store(self, layer, cu_tokens, start_pos, k, v=None, stream=None):
        total = k.shape[0]
        nseq = cu_tokens.shape[0] - 1
        pakv.paged_kv_store(self.map, layer, self.pages_of(layer), cu_tokens, start_pos, k, v, nseq, total, stream)

    def workspace(self, layer, num_seqs, max_kv_len):
        need = pakv.decode_workspace_bytes(self.map, layer, num_seqs, max_kv_len)
        if self._workspace is None or self._workspace.numel() < need:
            # zero-filled before first use; the library leaves it zeroed
            self._workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=self.device)
        return self._workspace, need

    def status(self):
        """The decode workspace's status word (pakv.DECODE_* bits), read after
        the stream's work is done; 0 if no decode ran yet."""
        if self._workspace is None:
            return 0
        torch.cuda.current_stream().synchronize()
        return int(self._workspace[:4].view(torch.int32).item()) & 0xffffffff

    def clear_status(self):
        if self._workspace is not None:
            self._workspace[:4].zero_()

    def plan_key(self, layer):
        """Layers with equal keys can share a decode plan (same window and Hkv)."""
        s = self.specs[layer]
        return (s["window"], s["num_kv_heads"])

    def decode_plan(self, layer, kv_lens, max_kv_len, stream=None):
        """The split of a decode call's keys for layer's window and Hkv, as a
        device buffer; valid for every layer with the same plan_key while
        kv_lens and the page table stay unchanged."""
        nseq = kv_lens.shape[0]
        nbytes = pakv.decode_plan_bytes(self.map, layer, nseq, max_kv_len)
        plan = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        pakv.decode_plan(self.map, layer, self.pages_of(layer), kv_lens, nseq, max_kv_len, plan, plan.numel(), stream)
        return plan

    def decode(self, layer, kv_lens, q, max_kv_len, out=None, stream=None, plan=None):
        """plan: a buffer from decode_plan for a layer with the same plan_key
        (kv_lens is then not read), or None."""
        nseq = q.shape[0]
        if out is None:
            out = torch.empty_like(q)
        ws, need = self.workspace(layer, nseq, max_kv_len)
        if plan is None:
            pakv.paged_attn_decode(self.map, layer, self.pages_of(layer), kv_lens, q, out, nseq, max_kv_len,
                                   ws, ws.numel(), stream)
        else:
            pakv.paged_attn_decode_planned(self.map, layer, self.pages_of(layer), plan, plan.numel(), q, out, nseq,
                                           max_kv_len, ws, ws.numel(), stream)
        return out

    def decode_append(self, layer, plan, k_new, v_new, q, max_kv_len, out=None, stream=None):
        """Stores this step's K/V row of every sequence (at kv_len - 1, where
        kv_len is what `plan` was made from) and decodes, in one launch; the
        same as store() then decode(plan=plan).  A shared layer only decodes."""
        nseq = q.shape[0]
        if out is None:
            out = torch.empty_like(q)
        ws, need = self.workspace(layer, nseq, max_kv_len)
        pakv.paged_attn_decode_append(self.map, layer, self.pages_of(layer), plan, plan.numel(), k_new, v_new, q, out, nseq,
                                      max_kv_len, ws, ws.numel(), stream)
        return out

    def extend(self, layer, cu_q, prefix_lens, q, max_q_len, max_kv_len, out=None, stream=None):
        nseq = cu_q.shape[0] - 1
        if out is None:
            out = torch.empty_like(q)
        pakv.paged_attn_extend(self.map, layer, self.pages_of(layer), cu_q, prefix_lens, q, out, nseq, q.shape[0],
                               max_q_len, max_kv_len, stream)
        return out

    def extend_packed(self, layer, cu_q, prefix_lens, q, k_ext, v_ext, max_q_len, max_kv_len, out=None,
                      stream=None):
        """Extend with the chunk's own rows given as packed tensors (v_ext None
        for a K=V layer); only the prefix is read from the slab."""
        nseq = cu_q.shape[0] - 1
        if out is None:
            out = torch.empty_like(q)
        pakv.paged_attn_extend_packed(self.map, layer, self.pages_of(layer), cu_q, prefix_lens, q, k_ext, v_ext, out, nseq,
                                      q.shape[0], max_q_len, max_kv_len, stream)
        return out

    def extend_staged(self, layer, cu_q, prefix_lens, q, max_q_len, max_kv_len, k_ext=None, v_ext=None, out=None,
                      stream=None, workspace=None, stage=True):
        """Extend on the bf16 MFMA kernel for every format (8-bit slabs, K=V
        layers and packed chunks staged first into a workspace); k_ext / v_ext
        as in extend_packed, or None.  workspace: a uint8 device tensor of at
        least staging_bytes(...) bytes, or None for one the cache keeps and
        grows.  stage=False reuses what an earlier call with the same source
        layer and arguments staged into that workspace (a KV-shared layer
        after its source)."""
        nseq = cu_q.shape[0] - 1
        if out is None:
            out = torch.empty_like(q)
        need = self.staging_bytes(layer, nseq, max_q_len, max_kv_len, k_ext is not None)
        if workspace is None:
            if need and (self._stage_ws is None or self._stage_ws.numel() < need):
                if not stage:
                    raise ValueError("stage=False needs the workspace an earlier call staged")
                self._stage_ws = torch.empty(need, dtype=torch.uint8, device=self.device)
            workspace = self._stage_ws
        ws = workspace if need else None
        pakv.paged_attn_extend_staged(self.map, layer, self.pages_of(layer), cu_q, prefix_lens, q, k_ext, v_ext, out,
                                      nseq, q.shape[0], max_q_len, max_kv_len, ws,
                                      workspace.numel() if ws is not None else 0, stage, stream)
        return out

    def staging_bytes(self, layer, num_seqs, max_q_len, max_kv_len, packed=False):
        """Workspace bytes a staged extend call of this layer needs (0: none)."""
        return pakv.extend_staging_bytes(self.map, layer, num_seqs, max_q_len, max_kv_len, packed)

    def capture_decode_step(self, kv_lens, max_kv_len, layers_io, buckets, max_batch=None):
        """A decode step of the given layers captured into one HIP graph per
        batch-size bucket (pakv_decode_step).  layers_io: (layer, q, out, k_new,
        v_new) per step layer, tensors sized for max_batch (k_new / v_new None
        where the rows are stored beforehand); kv_lens: device int32
        [max_batch], read at every replay.  Run it with step.run(batch)."""
        if max_batch is None:
            max_batch = kv_lens.shape[0]
        need = pakv.DecodeStep.workspace_bytes(self.map, layers_io, max_batch, max_kv_len)
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=self.device)
        full = self._group_pages["full"][1] if "full" in self._group_pages else self.pages
        sliding = self._group_pages["sliding"][1] if "sliding" in self._group_pages else None
        return pakv.DecodeStep(self.map, full, kv_lens, max_batch, max_kv_len, layers_io, buckets, ws,
                               pages_sliding=sliding)
