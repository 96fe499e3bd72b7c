"""Torch-facing wrapper around one libkvq cache layer.

PyTorch only provides device memory and the current HIP stream; every step of
append, flush and decode attention runs in libkvq's HIP kernels. Shapes, dtypes
and devices are checked here before a pointer crosses the C ABI, so a mismatch
raises instead of reaching a kernel.
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import binding as B

_DTYPES = {torch.float16: B.KVQ_F16, torch.bfloat16: B.KVQ_BF16}


def _stream_handle():
    """The current torch stream as the C ABI's void* stream."""
    return ctypes.c_void_p(int(torch.cuda.current_stream().cuda_stream))


class QuantizedKVCache:
    """One layer of a KIVI-style quantized KV cache living in device memory.

    Dense store: max_tokens bounds every sequence. Paged store: pass
    `page_table` (int32 [B][max_blocks], page of each G-token block) and
    `num_pages`; one page holds one block of every kv head. `sink` > 0 keeps
    the first `sink` tokens of every sequence in full precision (attention
    sink); the quantized blocks and the ring then hold the tokens after them.
    `fp8_blocks` > 0 keeps the most recent `fp8_blocks` quantized blocks of
    every (sequence, kv head) also as FP8 records, which decode reads instead.
    `rotate` (binding.KVQ_ROTATE_KEYS | KVQ_ROTATE_VALUES) rotates key and/or
    value rows by a Walsh-Hadamard transform before they are quantized.
    """

    def __init__(self, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int, *,
                 k_bits: int, v_bits: int, k_group: int, v_group: int, residual: int,
                 dtype=torch.float16, max_tokens: int | None = None, res_capacity: int | None = None,
                 page_table: torch.Tensor | None = None, num_pages: int = 0, sink: int = 0, fp8_blocks: int = 0,
                 rotate: int = 0, device="cuda"):
        if dtype not in _DTYPES:
            raise TypeError(f"dtype must be float16 or bfloat16, got {dtype}")
        self.device = torch.device(device)
        self.dtype = dtype
        res_capacity = res_capacity or (residual + k_group)
        if page_table is not None:
            if page_table.dtype != torch.int32 or page_table.dim() != 2 or page_table.shape[0] != batch:
                raise ValueError("page_table must be int32 [batch][max_blocks]")
            max_blocks = page_table.shape[1]
            if num_pages <= 0:
                raise ValueError("a paged cache needs num_pages > 0")
        else:
            if max_tokens is None:
                raise ValueError("a dense cache needs max_tokens")
            max_blocks = math.ceil(max_tokens / k_group)
            num_pages = 0
        self.cfg = B.kvq_config(batch=batch, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                                head_dim=head_dim, k_bits=k_bits, v_bits=v_bits, k_group=k_group,
                                v_group=v_group, residual=residual, res_capacity=res_capacity,
                                max_blocks=max_blocks, num_pages=num_pages, dtype=_DTYPES[dtype], sink=sink,
                                fp8_blocks=fp8_blocks, rotate=rotate)
        self.layout = B.kvq_layout_bytes(self.cfg)
        dev = self.device
        self.blocks = torch.zeros(self.layout.blocks, dtype=torch.uint8, device=dev)
        self.page_table = page_table.to(dev).contiguous() if page_table is not None else None
        ring_shape = (batch, num_kv_heads, res_capacity, head_dim)
        self.k_ring = torch.zeros(ring_shape, dtype=dtype, device=dev)
        self.v_ring = torch.zeros(ring_shape, dtype=dtype, device=dev)
        self.state = torch.zeros(self.layout.state // 4, dtype=torch.int32, device=dev)
        self.k_sink = self.v_sink = None
        self.fp8 = torch.zeros(self.layout.fp8, dtype=torch.uint8, device=dev) if fp8_blocks > 0 else None
        if sink > 0:
            sink_shape = (batch, num_kv_heads, sink, head_dim)
            self.k_sink = torch.zeros(sink_shape, dtype=dtype, device=dev)
            self.v_sink = torch.zeros(sink_shape, dtype=dtype, device=dev)
        self.cache = B.kvq_cache(
            blocks=self.blocks.data_ptr(),
            block_table=self.page_table.data_ptr() if self.page_table is not None else None,
            k_ring=self.k_ring.data_ptr(), v_ring=self.v_ring.data_ptr(), state=self.state.data_ptr(),
            k_sink=self.k_sink.data_ptr() if self.k_sink is not None else None,
            v_sink=self.v_sink.data_ptr() if self.v_sink is not None else None,
            fp8=self.fp8.data_ptr() if self.fp8 is not None else None)
        self.max_len_bound = 0          # host-side upper bound on every S_b
        self._ws = None

    # --- shapes --------------------------------------------------------------------
    @property
    def batch(self):
        return self.cfg.batch

    @property
    def record_bytes(self) -> int:
        return self.layout.record

    def _check(self, t: torch.Tensor, shape, dtype, name):
        if not isinstance(t, torch.Tensor) or t.device.type != self.device.type:
            raise ValueError(f"{name} must be a tensor on {self.device}")
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    # --- the three calls -----------------------------------------------------------
    def append(self, k_new: torch.Tensor, v_new: torch.Tensor, n_new: torch.Tensor | None = None):
        c = self.cfg
        n_max = k_new.shape[2] if k_new.dim() == 4 else -1
        shape = (c.batch, c.num_kv_heads, n_max, c.head_dim)
        self._check(k_new, shape, self.dtype, "k_new")
        self._check(v_new, shape, self.dtype, "v_new")
        n_ptr = None
        if n_new is not None:
            self._check(n_new, (c.batch,), torch.int32, "n_new")
            n_ptr = n_new.data_ptr()
        B.kvq_append(c, self.cache, k_new.data_ptr(), v_new.data_ptr(), n_ptr, n_max, _stream_handle())
        self.max_len_bound += n_max

    def append_flush(self, k_new: torch.Tensor, v_new: torch.Tensor, n_new: torch.Tensor | None = None):
        """append() then flush(), fused into one launch for small appends."""
        c = self.cfg
        n_max = k_new.shape[2] if k_new.dim() == 4 else -1
        shape = (c.batch, c.num_kv_heads, n_max, c.head_dim)
        self._check(k_new, shape, self.dtype, "k_new")
        self._check(v_new, shape, self.dtype, "v_new")
        n_ptr = None
        if n_new is not None:
            self._check(n_new, (c.batch,), torch.int32, "n_new")
            n_ptr = n_new.data_ptr()
        B.kvq_append_flush(c, self.cache, k_new.data_ptr(), v_new.data_ptr(), n_ptr, n_max, _stream_handle())
        self.max_len_bound += n_max

    def flush(self):
        B.kvq_flush_residual(self.cfg, self.cache, _stream_handle())

    def workspace_bytes(self, max_seq_tokens: int | None = None) -> int:
        return B.kvq_workspace_size(self.cfg, self.max_len_bound if max_seq_tokens is None else max_seq_tokens)

    def decode(self, q: torch.Tensor, out: torch.Tensor | None = None, softmax_scale: float = 0.0,
               max_seq_tokens: int | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
        c = self.cfg
        self._check(q, (c.batch, c.num_q_heads, c.head_dim), self.dtype, "q")
        if out is None:
            out = torch.empty(c.batch, c.num_q_heads, c.head_dim, dtype=torch.float32, device=self.device)
        self._check(out, (c.batch, c.num_q_heads, c.head_dim), torch.float32, "out")
        msl = self.max_len_bound if max_seq_tokens is None else int(max_seq_tokens)
        need = B.kvq_workspace_size(c, msl)
        if workspace is None:
            if self._ws is None or self._ws.numel() < need:
                self._ws = torch.empty(max(need, 16), dtype=torch.uint8, device=self.device)
            workspace = self._ws
        B.kvq_decode_attention(c, self.cache, q.data_ptr(), out.data_ptr(), softmax_scale, msl,
                               workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                               _stream_handle())
        return out

    def decode_multi(self, q: torch.Tensor, out: torch.Tensor | None = None, softmax_scale: float = 0.0,
                     max_seq_tokens: int | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
        """Attention of the T newest tokens of every sequence, causal within the
        block (q, out: [B][H_q][T][d]); the T tokens must already be appended."""
        c = self.cfg
        if not isinstance(q, torch.Tensor) or q.dim() != 4:
            raise ValueError("q must be a [B][H_q][T][d] tensor")
        T = q.shape[2]
        self._check(q, (c.batch, c.num_q_heads, T, c.head_dim), self.dtype, "q")
        if out is None:
            out = torch.empty(c.batch, c.num_q_heads, T, c.head_dim, dtype=torch.float32, device=self.device)
        self._check(out, (c.batch, c.num_q_heads, T, c.head_dim), torch.float32, "out")
        msl = self.max_len_bound if max_seq_tokens is None else int(max_seq_tokens)
        need = B.kvq_workspace_size_multi(c, msl, T)
        if workspace is None:
            if self._ws is None or self._ws.numel() < need:
                self._ws = torch.empty(max(need, 16), dtype=torch.uint8, device=self.device)
            workspace = self._ws
        B.kvq_decode_attention_multi(c, self.cache, q.data_ptr(), T, out.data_ptr(), softmax_scale, msl,
                                     workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                     _stream_handle())
        return out

    def _workspace(self, msl: int, workspace: torch.Tensor | None) -> torch.Tensor:
        need = B.kvq_workspace_size(self.cfg, msl)
        if workspace is not None:
            return workspace
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 16), dtype=torch.uint8, device=self.device)
        return self._ws

    def decode_partials(self, q: torch.Tensor, softmax_scale: float = 0.0, max_seq_tokens: int | None = None,
                        workspace: torch.Tensor | None = None) -> torch.Tensor:
        """First launch of decode(): the units' partial softmax states into the workspace (returned)."""
        c = self.cfg
        self._check(q, (c.batch, c.num_q_heads, c.head_dim), self.dtype, "q")
        msl = self.max_len_bound if max_seq_tokens is None else int(max_seq_tokens)
        ws = self._workspace(msl, workspace)
        B.kvq_decode_partials(c, self.cache, q.data_ptr(), softmax_scale, msl, ws.data_ptr(),
                              ws.numel() * ws.element_size(), _stream_handle())
        return ws

    def decode_combine(self, out: torch.Tensor | None = None, max_seq_tokens: int | None = None,
                       workspace: torch.Tensor | None = None) -> torch.Tensor:
        """Second launch of decode(): merge the partial states left by decode_partials()."""
        c = self.cfg
        if out is None:
            out = torch.empty(c.batch, c.num_q_heads, c.head_dim, dtype=torch.float32, device=self.device)
        self._check(out, (c.batch, c.num_q_heads, c.head_dim), torch.float32, "out")
        msl = self.max_len_bound if max_seq_tokens is None else int(max_seq_tokens)
        ws = self._workspace(msl, workspace)
        B.kvq_decode_combine(c, self.cache, out.data_ptr(), msl, ws.data_ptr(), ws.numel() * ws.element_size(),
                             _stream_handle())
        return out

    def prefill(self, k: torch.Tensor, v: torch.Tensor, lengths, chunk: int):
        """Append every sequence's first lengths[b] tokens of k, v ([B][H_kv][>=S][d])
        in chunks of `chunk` (ragged counts per sequence), flushing after each chunk.
        `chunk` must not exceed res_capacity - (R + G - 1)."""
        c = self.cfg
        if chunk <= 0 or chunk > c.res_capacity - (c.residual + c.k_group - 1):
            raise ValueError("chunk must be in [1, res_capacity - (R + G - 1)]")
        S_max = max(lengths)
        lens = torch.tensor(list(lengths), dtype=torch.int64)
        for t0 in range(0, S_max, chunk):
            n = min(chunk, S_max - t0)
            counts = torch.clamp(lens - t0, 0, n).to(torch.int32).to(self.device)
            self.append(k[:, :, t0:t0 + n].contiguous(), v[:, :, t0:t0 + n].contiguous(), counts)
            self.flush()
        return self

    # --- inspection (tests) --------------------------------------------------------
    def read_device_error(self) -> int:
        return B.kvq_get_device_error(self.cfg, self.cache, _stream_handle())

    def lengths(self):
        """(Q_b, S_b) per sequence, copied to the host."""
        st = self.state[:4 * self.cfg.batch].view(self.cfg.batch, 4).cpu()
        return st[:, 0].tolist(), st[:, 1].tolist()

    def fp8_record(self, b: int, h: int, blk: int) -> torch.Tensor:
        """Bytes of the FP8 record of one block of the FP8 tier (slot blk mod W)."""
        c, rb = self.cfg, self.layout.fp8_record
        off = ((b * c.num_kv_heads + h) * c.fp8_blocks + blk % c.fp8_blocks) * rb
        return self.fp8[off:off + rb]

    def record(self, b: int, h: int, blk: int) -> torch.Tensor:
        """Bytes of one block record (a view into the device store)."""
        c, rb = self.cfg, self.layout.record
        if self.page_table is None:
            off = ((b * c.num_kv_heads + h) * c.max_blocks + blk) * rb
        else:
            page = int(self.page_table[b, blk].item())
            off = (page * c.num_kv_heads + h) * rb
        return self.blocks[off:off + rb]


def cache_for_workload(w, lengths, chunk: int, extra_tokens: int = 0, device="cuda", seed: int = 0, sink: int = 0,
                       fp8_blocks: int = 0, rotate: int = 0):
    """An empty cache for a `workloads.Workload`, sized for `lengths` plus
    `extra_tokens` of decode growth, whose ring takes `chunk` tokens per append
    on top of R + G - 1, with a sink of `sink` tokens. Paged workloads get a
    random page table."""
    from . import workloads as W
    res_capacity = w.residual + w.k_group - 1 + max(chunk, 1)
    common = dict(k_bits=w.k_bits, v_bits=w.v_bits, k_group=w.k_group, v_group=w.v_group,
                  residual=w.residual, dtype=w.torch_dtype, res_capacity=res_capacity, sink=sink,
                  fp8_blocks=fp8_blocks, rotate=rotate, device=device)
    if w.paged:
        table, num_pages = W.random_page_table(w, lengths, extra_tokens=extra_tokens, seed=seed)
        return QuantizedKVCache(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                page_table=table, num_pages=num_pages, **common)
    return QuantizedKVCache(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                            max_tokens=max(lengths) + extra_tokens, **common)
