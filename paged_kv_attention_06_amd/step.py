"""Drives one serving step through the C ABI: builds a paged cache on the GPU
with the library's host allocator and kernels, then runs the step's block
copies, KV writes and attention.

The order of operations follows the pages: prompts and histories are
appended through allocate_slots-style block allocation and written to their
slots; forks share their prompt's blocks (ref counts); the step appends each
sequence's new tokens, copying a shared partly-filled last block first
(copy-on-write), writes the new K/V and runs attention over the cache.
Torch provides device memory and the stream only.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as L

_CODE_TORCH = {1: torch.uint8, 2: torch.int16, 4: torch.int32}
_CODE_NP = {1: np.uint8, 2: np.int16, 4: np.int32}
_DTYPE = {"f32": L.PKV_F32, "bf16": L.PKV_BF16, "fp8": L.PKV_FP8_E4M3}


def _dev_codes(a: np.ndarray, es: int, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(_CODE_NP[es])).to(device)


class PagedStep:
    """GPU state of one workload step.  ``w`` has the fields of
    ``workloads.Workload`` (sizes, lengths, free order, drawn values)."""

    def __init__(self, w, device: str = "cuda"):
        self.w = w
        self.device = torch.device(device)
        kv_dtype = getattr(w, "kv_dtype", w.dtype)
        self.es = {"f32": 4, "bf16": 2, "fp8": 1}[kv_dtype]   # cache element bytes
        self.in_es = w.dtype_bytes                           # new rows and queries
        self.dtype = _DTYPE[kv_dtype]
        self.block_bytes = 2 * 16 * w.num_kv_heads * w.head_size * self.es
        nbytes = w.num_blocks * self.block_bytes
        self.kv = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        fill = int(w.pool_fill)
        if self.es == 1:
            self.kv.fill_(fill)
        elif self.es == 2:
            self.kv.view(torch.int16).fill_(fill - (1 << 16) if fill >= 1 << 15 else fill)
        else:
            self.kv.view(torch.int32).fill_(fill - (1 << 32) if fill >= 1 << 31 else fill)
        self.cache = L.Cache(self.kv, w.num_blocks, w.num_kv_heads, w.head_size, self.dtype,
                             k_scale=getattr(w, "k_scale", 1.0), v_scale=getattr(w, "v_scale", 1.0))
        assert L.pkv_block_bytes(self.cache.desc) == self.block_bytes
        self.pool = L.Pool(w.num_blocks, w.free_order)
        self.max_blocks = max(1, int(-(-int(w.seq_lens.max()) // 16)))
        self.tables = np.zeros((w.batch, self.max_blocks), np.int32)
        self.prompt_tables = []

    # -------------------------------------------------------------- history
    def build_history(self) -> None:
        """Allocate and write every prompt and every independent history."""
        w = self.w
        slots_all, k_parts, v_parts = [], [], []
        for p in range(len(w.prompt_len)):
            n = int(w.prompt_len[p])
            t = np.zeros(self.max_blocks, np.int32)
            slots, _ = self.pool.append(t, 0, n)
            a, b = int(w.prompt_start[p]), int(w.prompt_start[p + 1])
            slots_all.append(slots)
            k_parts.append(w.prompt_k[a:b])
            v_parts.append(w.prompt_v[a:b])
            self.prompt_tables.append(t)
        for s in range(w.batch):
            if w.fork_of[s] >= 0:
                continue
            slots, _ = self.pool.append(self.tables[s], 0, int(w.hist_len[s]))
            slots_all.append(slots)
        if w.hist_k.shape[0]:
            k_parts.append(w.hist_k)
            v_parts.append(w.hist_v)
        for s in range(w.batch):
            if w.fork_of[s] >= 0:
                p = int(w.fork_of[s])
                nb = -(-int(w.prompt_len[p]) // 16)
                self.tables[s, :nb] = self.pool.fork(self.prompt_tables[p], nb)[:nb]
        if not w.prompt_owner_keeps_ref:
            for p, t in enumerate(self.prompt_tables):
                self.pool.release(t, -(-int(w.prompt_len[p]) // 16))
        slots = np.concatenate(slots_all) if slots_all else np.zeros(0, np.int64)
        if slots.size:
            k = _dev_codes(np.concatenate(k_parts), self.in_es, self.device)
            v = _dev_codes(np.concatenate(v_parts), self.in_es, self.device)
            s_dev = torch.from_numpy(slots).to(self.device)
            L.paged_kv_write(self.cache, k, v, s_dev)

    # -------------------------------------------------------------- the step
    def prepare_step(self) -> None:
        """Host metadata of the step: append slots (with COW), tables,
        lengths; uploads them and the step's new K/V and queries."""
        w = self.w
        slots, cow = [], []
        for s in range(w.batch):
            sl, c = self.pool.append(self.tables[s], int(w.hist_len[s]), int(w.q_len[s]))
            slots.append(sl)
            if c is not None:
                cow.append(c)
        self.h_slots = np.concatenate(slots) if slots else np.zeros(0, np.int64)
        self.h_cow = np.asarray(cow, np.int64).reshape(-1, 2)
        self.h_seq_lens = w.seq_lens.astype(np.int32)
        self.h_qsl = w.query_start_loc.astype(np.int32)
        d = self.device
        self.slots = torch.from_numpy(self.h_slots).to(d)
        self.cow = torch.from_numpy(self.h_cow).to(d)
        self.block_tables = torch.from_numpy(self.tables).to(d)
        self.seq_lens = torch.from_numpy(self.h_seq_lens).to(d)
        self.qsl = torch.from_numpy(self.h_qsl).to(d)
        self.k_new = _dev_codes(w.new_k, self.in_es, d)
        self.v_new = _dev_codes(w.new_v, self.in_es, d)
        self.q = _dev_codes(w.q, self.in_es, d)
        self.out = torch.zeros((w.num_tokens, w.num_q_heads, w.head_size), dtype=torch.float32,
                               device=d)
        self.decode_only = bool(np.all(w.q_len == 1))
        ws = L.pkv_attention_workspace_bytes(self.cache, w.num_q_heads, self.h_seq_lens,
                                             None if self.decode_only else self.h_qsl)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=d)

    def copy_and_write(self, stream=None) -> None:
        if self.h_cow.shape[0]:
            L.block_copy(self.cache, self.cow, stream)
        if self.h_slots.shape[0]:
            L.paged_kv_write(self.cache, self.k_new, self.v_new, self.slots, stream)

    def attend(self, stream=None) -> None:
        w = self.w
        if self.decode_only:
            L.paged_attention_decode(self.cache, self.out, self.q, self.block_tables, self.seq_lens,
                                     self.h_seq_lens, w.scale, self.workspace, stream)
        else:
            L.paged_attention_mixed(self.cache, self.out, self.q, self.qsl, self.seq_lens,
                                    self.h_qsl, self.h_seq_lens, self.block_tables, w.scale,
                                    self.workspace, stream)

    def run(self, stream=None) -> torch.Tensor:
        self.copy_and_write(stream)
        self.attend(stream)
        return self.out

    def pool_codes(self) -> np.ndarray:
        """The whole pool as codes [num_blocks][Hkv][2][16*D] on the host."""
        w = self.w
        a = self.kv.cpu().numpy().view({1: np.uint8, 2: np.uint16, 4: np.uint32}[self.es])
        return a.reshape(w.num_blocks, w.num_kv_heads, 2, 16 * w.head_size)


def run_workload(w, device: str = "cuda") -> PagedStep:
    st = PagedStep(w, device)
    st.build_history()
    st.prepare_step()
    st.run()
    torch.cuda.synchronize()
    return st
