"""Drive one decode step of the library from torch tensors.

``DeviceBatch`` takes a paged pool that is already in device memory plus the
host page table, lowers the table with the library's ``pkv_lower_page_table``
(host), uploads the token-flat indices once, and then runs plans against it.
All attention arithmetic happens in the library's kernels.
"""
import math

import numpy as np
import torch

from . import (Plan, make_pool, pkv_cascade_prefix_attn, pkv_decode_step, pkv_decode_step_grouped,
               pkv_lower_page_table, pkv_merge_states, pkv_paged_decode_attn, pkv_paged_decode_attn_pages,
               pkv_plan_create, pkv_plan_create_grouped, pkv_plan_metadata, workspace_for)

_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}
_NAME = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float8_e4m3fn: "fp8"}


class DeviceBatch:
    def __init__(self, q, k_pool, v_pool, page_size, page_indptr, page_indices, seq_lens, k_scale=None,
                 v_scale=None, device="cuda"):
        dev = torch.device(device)
        self.device = dev
        self.q = q.to(dev).contiguous()
        self.k_pool = k_pool.to(dev).contiguous()
        self.v_pool = v_pool.to(dev).contiguous()
        self.page_size = int(page_size)
        self.B, self.H_q, self.d = self.q.shape
        self.H_kv = self.k_pool.shape[1]
        self.q_dtype = _NAME[self.q.dtype]
        self.kv_dtype = _NAME[self.k_pool.dtype]
        self.k_scale = None if k_scale is None else torch.as_tensor(k_scale, dtype=torch.float32).to(dev)
        self.v_scale = None if v_scale is None else torch.as_tensor(v_scale, dtype=torch.float32).to(dev)
        self.kv_indptr_host, kv_indices_host = pkv_lower_page_table(self.page_size, page_indptr, page_indices,
                                                                    seq_lens)
        self.kv_indices_host = kv_indices_host
        self.kv_indptr = torch.from_numpy(self.kv_indptr_host).to(dev)
        self.kv_indices = torch.from_numpy(kv_indices_host if len(kv_indices_host) else np.zeros(1, np.int32)).to(dev)
        self.page_indptr_host = np.asarray(page_indptr, np.int32)
        self.page_indices_host = np.asarray(page_indices, np.int32)
        self.seq_lens_host = np.asarray(seq_lens, np.int32)
        self.page_indptr = torch.from_numpy(self.page_indptr_host).to(dev)
        pages = self.page_indices_host
        self.page_indices = torch.from_numpy(pages if len(pages) else np.zeros(1, np.int32)).to(dev)
        self.pool = make_pool(self.k_pool, self.v_pool, self.page_size, self.k_scale, self.v_scale)
        self.sm_scale = 1.0 / math.sqrt(self.d)

    @classmethod
    def from_batch(cls, batch, device="cuda"):
        """From a synthetic batch object with q, k_pool, v_pool, page table fields."""
        return cls(batch.q, batch.k_pool, batch.v_pool, batch.page_size, batch.page_indptr, batch.page_indices,
                   batch.seq_lens, batch.k_scale, batch.v_scale, device)

    def plan(self, shared_prefix_len=0, force_path=-1, tuning=None, host_indices=True) -> Plan:
        """host_indices: hand the planner the host kv_indices as well, so that a
        contiguously placed prefix is found (and read as base + offset)."""
        return pkv_plan_create(batch=self.B, num_q_heads=self.H_q, num_kv_heads=self.H_kv, head_dim=self.d,
                               q_dtype=self.q_dtype, kv_dtype=self.kv_dtype, page_size=self.page_size,
                               kv_indptr=self.kv_indptr_host, shared_prefix_len=shared_prefix_len,
                               force_path=force_path, tuning=tuning,
                               kv_indices=self.kv_indices_host if host_indices else None)

    def plan_grouped(self, force_path=-1, tuning=None) -> Plan:
        """Plan with the prefix groups found in the page table."""
        return pkv_plan_create_grouped(batch=self.B, num_q_heads=self.H_q, num_kv_heads=self.H_kv, head_dim=self.d,
                                       q_dtype=self.q_dtype, kv_dtype=self.kv_dtype, page_size=self.page_size,
                                       page_indptr=self.page_indptr_host, page_indices=self.page_indices_host,
                                       seq_lens=self.seq_lens_host, force_path=force_path, tuning=tuning)

    def metadata(self, plan):
        """Device copy of a grouped plan's metadata block."""
        m = pkv_plan_metadata(plan)
        return torch.from_numpy(m if len(m) else np.zeros(1, np.int32)).to(self.device)

    def step_grouped(self, plan, meta, o=None, lse=None, ws=None, sm_scale=None, stream=None):
        o = self.new_out() if o is None else o
        lse = self.new_lse() if lse is None else lse
        pkv_decode_step_grouped(plan, self.q, self.pool, meta, self.sm_scale if sm_scale is None else sm_scale, o,
                                lse, self.workspace(plan) if ws is None else ws, stream)
        return o, lse

    def workspace(self, plan):
        return workspace_for(plan, self.device)

    def new_out(self, dtype=None):
        return torch.empty((self.B, self.H_q, self.d), dtype=dtype or self.q.dtype, device=self.device)

    def new_lse(self):
        return torch.empty((self.B, self.H_q), dtype=torch.float32, device=self.device)

    def step(self, plan, o=None, lse=None, ws=None, sm_scale=None, stream=None):
        o = self.new_out() if o is None else o
        lse = self.new_lse() if lse is None else lse
        pkv_decode_step(plan, self.q, self.pool, self.kv_indptr, self.kv_indices,
                        self.sm_scale if sm_scale is None else sm_scale, o, lse,
                        self.workspace(plan) if ws is None else ws, stream)
        return o, lse

    def paged(self, plan, o=None, o_f32=None, lse=None, ws=None, sm_scale=None, stream=None, want_f32=False):
        if o is None and o_f32 is None:
            if want_f32:
                o_f32 = self.new_out(torch.float32)
            else:
                o = self.new_out()
        lse = self.new_lse() if lse is None else lse
        pkv_paged_decode_attn(plan, self.q, self.pool, self.kv_indptr, self.kv_indices,
                              self.sm_scale if sm_scale is None else sm_scale, o, o_f32, lse,
                              self.workspace(plan) if ws is None else ws, stream)
        return (o if o is not None else o_f32), lse

    def paged_pages(self, plan, o=None, o_f32=None, lse=None, ws=None, sm_scale=None, stream=None, want_f32=False):
        """As paged(), with the kernel reading the page table instead of kv_indices."""
        if o is None and o_f32 is None:
            if want_f32:
                o_f32 = self.new_out(torch.float32)
            else:
                o = self.new_out()
        lse = self.new_lse() if lse is None else lse
        pkv_paged_decode_attn_pages(plan, self.q, self.pool, self.kv_indptr, self.page_indptr, self.page_indices,
                                    self.sm_scale if sm_scale is None else sm_scale, o, o_f32, lse,
                                    self.workspace(plan) if ws is None else ws, stream)
        return (o if o is not None else o_f32), lse

    def prefix_indices(self, plan):
        n = plan.info["prefix_tokens"]
        start = int(self.kv_indptr_host[0])
        return self.kv_indices[start:start + n]

    def prefix(self, plan, o_p=None, lse_p=None, ws=None, sm_scale=None, stream=None):
        o_p = self.new_out(torch.float32) if o_p is None else o_p
        lse_p = self.new_lse() if lse_p is None else lse_p
        pkv_cascade_prefix_attn(plan, self.q, self.pool, self.prefix_indices(plan), plan.info["prefix_tokens"],
                                self.sm_scale if sm_scale is None else sm_scale, o_p, lse_p,
                                self.workspace(plan) if ws is None else ws, stream)
        return o_p, lse_p

    @staticmethod
    def merge(o_a, lse_a, o_b, lse_b, out_dtype=torch.float32, lse_out=None, stream=None):
        o = torch.empty(o_a.shape, dtype=out_dtype, device=o_a.device)
        pkv_merge_states(o_a, lse_a, o_b, lse_b, o, lse_out, stream)
        return o
