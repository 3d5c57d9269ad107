"""One layer's retrieval-sparse decode step over a batch of paged sequences.

`DecodeSession` owns the device buffers the C ABI writes (representations,
selections, merged tables, workspaces, output) and issues the per-step call
sequence on the current stream:

    rkv_append_kv   write the decoded token's K/V (and a just-completed
                    block's representation)
    rkv_select      inner-product scores, per-(sequence, KV head) top-k and
                    the merged block table
    rkv_decode_attn split-K paged attention and the log-sum-exp combine

A step issues them as rkv_decode_step (the append folded into the scoring
launch; for a batch of one the top-k and merge folded into the attention
launch).  PyTorch only allocates memory and provides the stream here.
"""

from __future__ import annotations

import torch

from . import binding as B


class DecodeSession:
    def __init__(self, prm: B.Params, k_pages: torch.Tensor, v_pages: torch.Tensor,
                 block_table: torch.Tensor, prompt_lens: torch.Tensor | None = None):
        dev = k_pages.device
        self.p = prm
        self.k_pages, self.v_pages = k_pages, v_pages
        self.block_table = block_table
        self.batch, self.max_blocks = block_table.shape
        self.prompt_lens = prompt_lens
        hkv, hq = prm.n_kv_heads, prm.n_q_heads
        self.k_cap = max(1, B.topk_capacity(prm, self.max_blocks))
        self.m_cap = self.max_blocks
        self.reps = torch.zeros((self.batch, hkv, self.max_blocks, B.HEAD_DIM),
                                dtype=torch.float32, device=dev)
        self.sel_ids = torch.zeros((self.batch, hkv, self.k_cap), dtype=torch.int32,
                                   device=dev)
        self.n_sel = torch.zeros((self.batch, hkv), dtype=torch.int32, device=dev)
        self.merged = torch.zeros((self.batch, hkv, self.m_cap), dtype=torch.int32,
                                  device=dev)
        self.n_merged = torch.zeros((self.batch, hkv), dtype=torch.int32, device=dev)
        self.out = torch.zeros((self.batch, hq, B.HEAD_DIM), dtype=torch.float32,
                               device=dev)
        ws = B.select_workspace_size(prm, self.batch, self.max_blocks)
        self.ws_select = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev) \
            if ws else None
        wa = B.attn_workspace_size(prm, self.batch, self.m_cap)
        self.ws_attn = torch.empty(max(wa, 16), dtype=torch.uint8, device=dev)
        self.ws_cascade = None  # sized on the first cascade call
        self._fast = None  # per-step calls with the session buffers bound once

    def _prepared(self) -> B.PreparedStep:
        if self._fast is None:
            self._fast = B.PreparedStep(self.p, self.k_pages, self.v_pages, self.reps,
                                        self.block_table, self.sel_ids, self.n_sel,
                                        self.merged, self.n_merged, self.prompt_lens,
                                        self.ws_select, self.out, self.ws_attn)
        return self._fast

    def build_reps(self, lens: torch.Tensor, block_begin: torch.Tensor | None = None):
        B.build_reps(self.p, self.k_pages, self.block_table, lens, self.reps,
                     block_begin)

    def append(self, k_new, v_new, lens):
        B.append_kv(self.p, k_new, v_new, self.k_pages, self.v_pages,
                    self.block_table, lens, self.reps)

    def select(self, q, lens):
        B.select(self.p, q, self.reps, self.block_table, lens, self.sel_ids,
                 self.n_sel, self.merged, self.n_merged, self.prompt_lens,
                 self.ws_select)

    def attend(self, q, lens):
        self._prepared().decode_attn(q, lens)
        return self.out

    def append_select(self, q, k_new, v_new, lens):
        """The append folded into the selection's launches."""
        self._prepared().append_select(q, k_new, v_new, lens)

    def select_attend(self, q, lens):
        """Selection from the scores the last selection left in the select
        workspace, then attention (rkv_select_attend)."""
        self._prepared().select_attend(q, lens)
        return self.out

    def step(self, q, k_new, v_new, lens):
        """One decode step (rkv_decode_step: append + scores, then selection
        and attention; for a batch of one the selection runs inside the
        attention launch); returns `out`."""
        self._prepared().decode_step(q, k_new, v_new, lens)
        return self.out

    def step_separate(self, q, k_new, v_new, lens):
        """The same step as rkv_append_select + rkv_decode_attn."""
        self.append_select(q, k_new, v_new, lens)
        return self.attend(q, lens)

    def attend_cascade(self, q, lens, shared_blocks: int):
        """Attention with the shared-prefix cascade (rkv_decode_attn_cascade):
        the first `shared_blocks` blocks of every sequence sit on sequence
        0's pages, and each attended tile of that prefix is read once per
        group of sequences.  Uses the merged tables and kept ids of the last
        selection."""
        need = B.attn_cascade_workspace_size(self.p, self.batch, self.m_cap,
                                             shared_blocks)
        if self.ws_cascade is None or self.ws_cascade.numel() < need:
            self.ws_cascade = torch.empty(max(need, 16), dtype=torch.uint8,
                                          device=self.k_pages.device)
        B.decode_attn_cascade(self.p, q, self.k_pages, self.v_pages, self.merged,
                              self.n_merged, self.sel_ids, self.n_sel,
                              self.block_table, shared_blocks, lens, self.out,
                              self.ws_cascade)
        return self.out

    def step_cascade(self, q, k_new, v_new, lens, shared_blocks: int):
        """rkv_append_select, then the cascade attention."""
        self.append_select(q, k_new, v_new, lens)
        return self.attend_cascade(q, lens, shared_blocks)


class HostTierSession(DecodeSession):
    """Decode step with the offload region in pinned host memory: the kept
    offload blocks are staged into HBM staging pages (the last
    batch * k_cap pages of the device pools) before attention, on a side
    stream that the main stream waits for.  With `resident` (the default) a
    kept block already held by a staging slot from an earlier step is not
    copied again (rkv_stage_resident); otherwise every kept block is copied
    each step (rkv_stage_blocks + rkv_merge_table).

    With `copy_mode="memcpy"` the copies go through the copy engines
    (rkv_stage_resident_async / rkv_stage_blocks_async: the kept ids or the
    residency planner's copy list go to the host, which issues coalesced
    hipMemcpy2DAsync / hipMemcpyAsync calls on the side stream, or spread
    over `prm.copy_lanes` streams of the library forked from it, and records
    an event the main stream waits for); the default "kernel" mode copies
    with a gather kernel that reads the pinned host pools directly.

    Representations are built while every block is still in HBM (after
    prefill); `attach_host` then hands over the host pools that hold the
    offload blocks from then on."""

    def __init__(self, prm: B.Params, k_pages, v_pages, block_table,
                 prompt_lens=None, side_stream=True, resident=True, slot_cap=None,
                 copy_mode="kernel"):
        super().__init__(prm, k_pages, v_pages, block_table, prompt_lens)
        self.host_k = self.host_v = self.host_table = None
        # staging slots per (sequence, KV head): k_cap by default (always
        # enough); a caller that knows its largest kept count (no prompt
        # below the dense boundary) may size them from that.  The last
        # batch * max(slot_cap, k_cap) pages of the device pools are the
        # staging area and must not hold any page the block table uses.
        self.slot_cap = self.k_cap if slot_cap is None else int(slot_cap)
        if self.slot_cap < 1:
            raise ValueError("slot_cap must be >= 1")
        area = self.batch * max(self.slot_cap, self.k_cap)
        self.stage_page0 = k_pages.shape[0] - area
        if self.stage_page0 < 0:
            raise ValueError("the device pools have no room for staging pages")
        used = int(block_table.max().item()) if block_table.numel() else -1
        if used >= self.stage_page0:
            raise ValueError(f"staging pages [{self.stage_page0}, {k_pages.shape[0]}) "
                             f"overlap page {used} of the block table")
        self.side = torch.cuda.Stream(device=k_pages.device) if side_stream else None
        # residency across steps: the block each staging slot holds
        self.resident = resident
        dev = k_pages.device
        n_kv = prm.n_kv_heads
        self.slot_ids = torch.full((self.batch, n_kv, self.slot_cap), -1,
                                   dtype=torch.int32, device=dev)
        self.slot_cursor = torch.zeros((self.batch, n_kv), dtype=torch.int32, device=dev)
        self.n_staged = torch.zeros((self.batch, n_kv), dtype=torch.int32, device=dev)
        ws = B.stage_workspace_size(prm, self.batch, self.k_cap)
        self.ws_stage = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
        self.host_table_host = None
        self.host_list = self.done = None
        self.copy_mode = copy_mode
        self._check_copy_mode()

    def _check_copy_mode(self):
        if self.copy_mode not in ("kernel", "memcpy"):
            raise ValueError("copy_mode must be 'kernel' or 'memcpy'")
        if self.copy_mode == "memcpy" and self.host_list is None:
            if self.side is None:
                raise ValueError("the memcpy staging mode needs the side stream")
            n = B.stage_host_list_size(self.p, self.batch, self.k_cap)
            self.host_list = torch.empty(max(n, 16), dtype=torch.uint8, pin_memory=True)
            self.done = torch.cuda.Event()
            self.done.record(self.side)  # creates the event the library records

    def attach_host(self, host_k, host_v, host_table):
        self.host_k, self.host_v, self.host_table = host_k, host_v, host_table
        # the copy-engine mode issues its copies from a host copy of the table
        self.host_table_host = host_table.to("cpu").contiguous()
        self.reset_residency()

    def offload_prefill(self, host_k, host_v, host_table, lens, concurrent=False):
        """Hand a prefilled batch over to the host tier: the representations
        of the complete blocks are built, then the offload-region pages go to
        the pinned pools (rkv_offload_blocks).  `lens` = tokens prefilled per
        sequence.  With `concurrent`, the copies run on the side stream while
        the representations are built; that is slower on MI355X (a kernel
        writing host memory over the bus holds up the HBM reads of the
        other compute units), so it is off by default."""
        dev = self.k_pages.device
        main = torch.cuda.current_stream(dev)
        if concurrent and self.side is not None:
            self.side.wait_stream(main)
            with torch.cuda.stream(self.side):
                B.offload_blocks(self.p, self.k_pages, self.v_pages, self.block_table,
                                 lens, host_table, host_k, host_v)
            self.build_reps(lens)
            main.wait_stream(self.side)
        else:
            self.build_reps(lens)
            B.offload_blocks(self.p, self.k_pages, self.v_pages, self.block_table,
                             lens, host_table, host_k, host_v)
        self.attach_host(host_k, host_v, host_table)

    def reset_residency(self):
        """Forget what the staging slots hold (new sequences or host pools)."""
        self.slot_ids.fill_(-1)
        self.slot_cursor.zero_()

    def select(self, q, lens):
        # the selection only: the merged table is built after staging
        B.select(self.p, q, self.reps, self.block_table, lens, self.sel_ids,
                 self.n_sel, None, None, self.prompt_lens, self.ws_select)

    def stage(self, lens):
        self._check_copy_mode()
        if self.copy_mode == "memcpy":
            # the planner (or the kept ids) on the current stream, the copies
            # on the side stream; the current stream then waits for them
            main = torch.cuda.current_stream(self.k_pages.device)
            if self.resident:
                B.stage_resident_async(self.p, self.host_k, self.host_v, self.host_table,
                                       self.host_table_host, self.block_table, lens,
                                       self.sel_ids, self.n_sel, self.slot_ids,
                                       self.slot_cursor, self.k_pages, self.v_pages,
                                       self.stage_page0, self.merged, self.n_merged,
                                       self.ws_stage, self.host_list, self.side, self.done,
                                       self.n_staged)
            else:
                B.stage_blocks_async(self.p, self.host_k, self.host_v, self.host_table_host,
                                     self.sel_ids, self.n_sel, self.k_pages, self.v_pages,
                                     self.stage_page0, self.host_list, self.side, self.done)
                B.merge_table(self.p, self.block_table, lens, self.sel_ids, self.n_sel,
                              self.merged, self.n_merged, self.host_table,
                              self.stage_page0)
            main.wait_event(self.done)
            return
        if self.resident:
            B.stage_resident(self.p, self.host_k, self.host_v, self.host_table,
                             self.block_table, lens, self.sel_ids, self.n_sel,
                             self.slot_ids, self.slot_cursor, self.k_pages, self.v_pages,
                             self.stage_page0, self.merged, self.n_merged,
                             self.ws_stage, self.n_staged)
            return
        B.stage_blocks(self.p, self.host_k, self.host_v, self.host_table,
                       self.sel_ids, self.n_sel, self.k_pages, self.v_pages,
                       self.stage_page0)
        B.merge_table(self.p, self.block_table, lens, self.sel_ids, self.n_sel,
                      self.merged, self.n_merged, self.host_table, self.stage_page0)

    def append_select(self, q, k_new, v_new, lens):
        B.append_select(self.p, k_new, v_new, self.k_pages, self.v_pages, q,
                        self.reps, self.block_table, lens, self.sel_ids,
                        self.n_sel, None, None, self.prompt_lens, self.ws_select)

    def step_overlapped(self, q, k_new, v_new, lens):
        """One decode step whose copies overlap the attention over the blocks
        already in HBM: the residency planner in split mode on the current
        stream, the copies of the blocks new to the kept set on the side
        stream while the current stream attends the rest
        (rkv_decode_attn_lse), then the newly staged blocks folded in by
        log-sum-exp.  The same result as step() up to rounding (the softmax
        partials are merged in another grouping); the same slot state.
        Gather-kernel staging with residency only."""
        if self.side is None or not self.resident or self.copy_mode != "kernel":
            raise ValueError("the overlapped step needs the side stream, residency "
                             "and the gather-kernel staging")
        dev = self.k_pages.device
        if getattr(self, "merged_new", None) is None:
            hkv = self.p.n_kv_heads
            self.merged_new = torch.zeros((self.batch, hkv, self.k_cap),
                                          dtype=torch.int32, device=dev)
            self.n_new = torch.zeros((self.batch, hkv), dtype=torch.int32, device=dev)
            self.out_res = torch.zeros_like(self.out)
            self.lse_res = torch.zeros(self.out.shape[:2], dtype=torch.float32,
                                       device=dev)
            # every newly staged entry is a whole block
            self.lens_whole = torch.full((self.batch,), 128 * self.k_cap,
                                         dtype=torch.int32, device=dev)
        self.append_select(q, k_new, v_new, lens)
        B.stage_plan(self.p, self.host_table, self.block_table, lens, self.sel_ids,
                     self.n_sel, self.slot_ids, self.slot_cursor, self.k_pages.shape[0],
                     self.stage_page0, self.merged, self.n_merged, self.ws_stage,
                     self.merged_new, self.n_new, self.n_staged)
        main = torch.cuda.current_stream(dev)
        self.side.wait_stream(main)
        with torch.cuda.stream(self.side):
            B.stage_copy(self.p, self.host_k, self.host_v, self.host_table, self.k_cap,
                         self.slot_cap, self.k_pages, self.v_pages, self.stage_page0,
                         self.ws_stage)
        B.decode_attn_lse(self.p, q, self.k_pages, self.v_pages, self.merged,
                          self.n_merged, lens, self.out_res, self.ws_attn,
                          lse=self.lse_res)
        main.wait_stream(self.side)
        B.decode_attn_lse(self.p, q, self.k_pages, self.v_pages, self.merged_new,
                          self.n_new, self.lens_whole, self.out, self.ws_attn,
                          prev_out=self.out_res, prev_lse=self.lse_res)
        return self.out

    def step(self, q, k_new, v_new, lens):
        self.append_select(q, k_new, v_new, lens)
        if self.side is None or self.copy_mode == "memcpy":
            self.stage(lens)
        else:
            main = torch.cuda.current_stream(self.k_pages.device)
            self.side.wait_stream(main)
            with torch.cuda.stream(self.side):
                self.stage(lens)
            main.wait_stream(self.side)
        return self.attend(q, lens)
