"""Device-memory plumbing around the C ABI: holds torch tensors for the
inputs, the page table, the plan, the partial workspace and the output, and
calls the libcap entry points on the current torch stream.  PyTorch provides
memory and streams only; all attention arithmetic happens in libcap."""
from __future__ import annotations

import numpy as np

from . import cap


def _dev_u16(torch, a, device):
    """Device int16 tensor of bf16 bits: numpy arrays are copied over, device
    tensors (int16 or bfloat16, contiguous) are used as they are."""
    if isinstance(a, torch.Tensor):
        if a.device != device or not a.is_contiguous() or a.element_size() != 2:
            raise ValueError("device arrays must be contiguous 2-byte tensors on the decoder's device")
        return a.view(torch.int16)
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


class TreeDecoder:
    """One radix tree resident on the GPU, ready to plan and decode steps.

    tree: a ``workloads.Tree`` (or any object with the same attributes);
    q, k_pool, v_pool: uint16 bf16-bit arrays in the layouts of include/cap.h,
    or device tensors already holding them.
    """

    def __init__(self, tree, q, k_pool, v_pool, device="cuda", **plan_opts):
        import torch
        self.torch = torch
        self.device = torch.device(device)
        if self.device.type != "cuda" or not torch.cuda.is_available():
            raise RuntimeError("TreeDecoder needs a GPU (ROCm) device")
        if self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.tree_host = tree
        self.R, self.Hq, self.D = int(tree.num_requests), int(tree.num_q_heads), int(tree.head_dim)
        self.q = _dev_u16(torch, q, self.device)
        self.k = _dev_u16(torch, k_pool, self.device)
        self.v = _dev_u16(torch, v_pool, self.device)
        self.out = torch.empty((self.R, self.Hq, self.D), dtype=torch.int16, device=self.device)
        nbytes = cap.cap_tree_device_bytes(tree)
        self.tree_buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.tree = cap.cap_tree_upload(tree, self.tree_buf.data_ptr(), nbytes, self.stream())
        self.plan_h = 0
        self.plan_buf = None
        self.ws = None
        self.stats = None
        self.plan_opts = dict(plan_opts)
        self._grow_bufs = None
        # second plan slot for replan(): handle, device buffer, and the event
        # recorded after its last upload (the host image is that copy's source)
        self._spare_h, self._spare_buf, self._spare_ev = 0, None, None
        self._cur_ev = None
        self.plan(**plan_opts)

    def stream(self) -> int:
        return self.torch.cuda.current_stream(self.device).cuda_stream

    def plan(self, **opts):
        torch = self.torch
        self.plan_opts = dict(opts)
        if self.plan_h:
            torch.cuda.current_stream(self.device).synchronize()
            cap.cap_plan_free(self.plan_h)
            self.plan_h = 0
        self.plan_h = cap.cap_plan_step(self.tree, **opts)
        self.stats = cap.cap_plan_get_stats(self.plan_h)
        pb = int(self.stats["plan_device_bytes"])
        wb = int(self.stats["workspace_bytes"])
        if self.plan_buf is None or self.plan_buf.numel() < pb:
            self.plan_buf = torch.empty(pb, dtype=torch.uint8, device=self.device)
        if self.ws is None or self.ws.numel() * 4 < wb:
            self.ws = torch.empty(max(wb // 4, 64), dtype=torch.float32, device=self.device)
        cap.cap_plan_upload(self.plan_h, self.plan_buf.data_ptr(), self.plan_buf.numel(), self.stream())
        self._cur_ev = self._record()
        return self.stats

    def _record(self):
        """Event after the copies just queued from the current plan's host
        memory (an upload or a refresh patch): a rebuild of that handle waits
        for it."""
        ev = self.torch.cuda.Event()
        ev.record(self.torch.cuda.current_stream(self.device))
        return ev

    def replan(self, **opts):
        """Plan the tree as it stands for the next step without waiting for
        the steps in flight: cap_plan_rebuild into the second plan slot (its
        host memory reused), cap_plan_upload into that slot's own device
        buffer on the stream, then the slots swap.  Steps already queued keep
        their plan buffer; the only wait is for the spare slot's previous
        upload, long done in a loop that plans every step."""
        torch = self.torch
        self.plan_opts = dict(opts)
        if self._spare_h:
            if self._spare_ev is not None:
                self._spare_ev.synchronize()
            cap.cap_plan_rebuild(self._spare_h, self.tree, **opts)
        else:
            self._spare_h = cap.cap_plan_step(self.tree, **opts)
        st = cap.cap_plan_get_stats(self._spare_h)
        pb, wb = int(st["plan_device_bytes"]), int(st["workspace_bytes"])
        if self._spare_buf is None or self._spare_buf.numel() < pb:
            self._spare_buf = torch.empty(pb, dtype=torch.uint8, device=self.device)
        if self.ws.numel() * 4 < wb:
            # stream-ordered: the old workspace is reused only after the steps queued on it
            self.ws = torch.empty(max(wb // 4, 64), dtype=torch.float32, device=self.device)
        cap.cap_plan_upload(self._spare_h, self._spare_buf.data_ptr(), self._spare_buf.numel(), self.stream())
        ev = self._record()
        self.plan_h, self._spare_h = self._spare_h, self.plan_h
        self.plan_buf, self._spare_buf = self._spare_buf, self.plan_buf
        self._cur_ev, self._spare_ev = ev, self._cur_ev
        self.stats = st
        return st

    def set_q(self, q: np.ndarray):
        """Next step's queries (uint16 bf16 bits [R][Hq][D])."""
        self.q.copy_(_dev_u16(self.torch, q, self.device))

    def grow(self, k_new: np.ndarray, v_new: np.ndarray, new_pages=None, active=None, rebuild=False):
        """One decode step's new tokens (uint16 bf16 bits [R][Hkv][D]): extend
        the tree on the host (cap_tree_append), write their K/V into the pools
        (cap_append_kv) and bring the plan up to date (cap_plan_refresh, or a
        new plan with the same options when it answers CAP_ERR_REPLAN; with
        rebuild=True, always a new plan through replan(), as a loop that
        plans every step does).  Returns (dest, replanned)."""
        torch = self.torch
        dest = cap.cap_tree_append(self.tree, self.R, active, new_pages)
        d = torch.from_numpy(dest).to(self.device)
        k = _dev_u16(torch, k_new, self.device)
        v = _dev_u16(torch, v_new, self.device)
        self._grow_bufs = (d, k, v)
        cap.cap_append_kv(self.tree, d.data_ptr(), self.R, k.data_ptr(), v.data_ptr(), self.k.data_ptr(),
                          self.v.data_ptr(), self.stream())
        if rebuild:
            self.replan(**self.plan_opts)
            return dest, True
        try:
            cap.cap_plan_refresh(self.plan_h, self.stream())
            self._cur_ev = self._record()
            replanned = False
        except cap.CapError as e:
            if e.status != cap.CAP_ERR_REPLAN:
                raise
            self.plan(**self.plan_opts)
            replanned = True
        self.stats = cap.cap_plan_get_stats(self.plan_h)
        return dest, replanned

    def poison_workspace(self):
        """Fill the partial workspace with all-ones bytes, a NaN in fp32 and in
        fp16 alike (tests: unwritten slots show up)."""
        self.ws.view(self.torch.int32).fill_(-1)

    def decode(self):
        cap.cap_decode_attention(self.plan_h, self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(),
                                 self.ws.data_ptr(), self.ws.numel() * 4, self.stream())

    def decode_timed(self) -> float:
        """decode(), timed by events bound to the kernel's dispatch (blocks);
        returns the kernel's execution time in microseconds."""
        return cap.cap_bench_decode_timed(self.plan_h, self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(),
                                          self.ws.data_ptr(), self.ws.numel() * 4, self.stream())

    def merge(self):
        cap.cap_merge_partials(self.plan_h, self.ws.data_ptr(), self.ws.numel() * 4,
                               self.out.data_ptr(), self.stream())

    def fused_step(self):
        cap.cap_decode_step(self.plan_h, self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(),
                            self.ws.data_ptr(), self.ws.numel() * 4, self.out.data_ptr(), self.stream())

    def step(self, fused: bool = True):
        if fused:
            self.fused_step()
        else:
            self.decode()
            self.merge()

    def capture_step(self, fused: bool = False):
        """Record one step (decode + merge, or the fused launch) into a HIP
        graph through torch's stream capture and return it; replay() runs the
        same kernels with the same buffers.  The graph holds no memset (the
        kernels clear their own counters), and the plan buffer must stay
        uploaded and unchanged while it is used."""
        torch = self.torch
        torch.cuda.synchronize(self.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(fused=fused)
        torch.cuda.synchronize(self.device)
        return g

    def output_bits(self) -> np.ndarray:
        self.torch.cuda.current_stream(self.device).synchronize()
        return self.out.cpu().numpy().view(np.uint16)

    def output(self) -> np.ndarray:
        b = self.output_bits().astype(np.uint32) << 16
        return b.view(np.float32)

    def close(self):
        if self.plan_h or self._spare_h or self.tree:
            self.torch.cuda.synchronize(self.device)
        if self.plan_h:
            cap.cap_plan_free(self.plan_h)
            self.plan_h = 0
        if self._spare_h:
            cap.cap_plan_free(self._spare_h)
            self._spare_h = 0
        if self.tree:
            cap.cap_tree_free(self.tree)
            self.tree = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
