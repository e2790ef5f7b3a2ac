"""Rolling sink + window block KV cache, simulated as a plain list of logical tokens.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's CPU
baseline, never by the product path.

Source: WorldFoundry "Core 注意力" page, section "Block KV cache 的调用顺序" (block KV
cache call order) and the sentence after its example:
  * every chunk goes through before_update -> update -> cached_k/cached_v -> after_update;
  * repeating the current chunk_idx overwrites the same logical chunk, the next index
    appends (or rolls the window), a skipped index is an error;
  * sink_size keeps a prefix that is never evicted, window_size is the rolling region;
    their sum equals the cache's sequence length and is divisible by chunk_size;
  * the worked example (k_shape (1,1,4,2), v_shape (1,1,4,3), chunk 2, window 4, chunks
    filled with their own index) sees 2, then 4, then 4 rolled tokens.

This simulation holds no slots and no ring: it keeps a dict from token id to that token's
newest K/V rows and evicts by the sink/window rule. The visible view is the tokens

    [0, min(T, sink))  ++  [max(sink, T - window), T),    T = (last_chunk + 1) * chunk

in chronological order. Readings (listed in the design notes): the first chunk must be 0;
an update carries exactly chunk_size tokens; sink_size defaults to 0; window >= chunk so a
chunk always sees itself; the view is chronological (sink, then the window oldest to
newest).

Parity pins (tests/test_oracle.py): the page's worked example (visible counts 2, 4, 4;
values equal to chunk indices; tests/golden/block_kv_cache_example.json) and invariants of
the rule (sink tokens never leave, the newest chunk is always visible, visible count =
min(T, sink + window), every visible row equals the last write of its token).
"""
from __future__ import annotations

import numpy as np


class CacheOrderError(ValueError):
    """A chunk index that is neither the current one nor the next one."""


class CacheConfigError(ValueError):
    """sink/window/chunk sizes that break the page's rule."""


class BlockKVCacheOracle:
    def __init__(self, k_shape, v_shape, seq_dim, chunk_size, window_size, sink_size=0):
        k_shape, v_shape = tuple(int(x) for x in k_shape), tuple(int(x) for x in v_shape)
        if len(k_shape) != len(v_shape) or not (0 <= seq_dim < len(k_shape)):
            raise CacheConfigError("k_shape/v_shape/seq_dim disagree")
        length = k_shape[seq_dim]
        if v_shape[seq_dim] != length:
            raise CacheConfigError("k and v caches differ in sequence length")
        if chunk_size <= 0 or window_size <= 0 or sink_size < 0:
            raise CacheConfigError("sizes must be positive (sink may be 0)")
        if sink_size + window_size != length:
            raise CacheConfigError("sink_size + window_size must equal the cache length")
        if length % chunk_size != 0:
            raise CacheConfigError("sink_size + window_size must be divisible by chunk_size")
        if window_size < chunk_size:
            raise CacheConfigError("window_size must hold at least one chunk")
        self.k_shape, self.v_shape, self.seq_dim = k_shape, v_shape, seq_dim
        self.chunk, self.window, self.sink = int(chunk_size), int(window_size), int(sink_size)
        self.last_chunk = -1
        self.tokens = {}  # token id -> (k row, v row), rows taken along seq_dim

    # -- protocol ---------------------------------------------------------------------
    def update(self, chunk_idx, k, v):
        """before_update(chunk_idx) + update(k, v) + after_update(chunk_idx) in one call."""
        chunk_idx = int(chunk_idx)
        if chunk_idx not in (self.last_chunk, self.last_chunk + 1):
            raise CacheOrderError(f"chunk {chunk_idx} after {self.last_chunk}")
        k, v = np.asarray(k), np.asarray(v)
        if k.shape[self.seq_dim] != self.chunk or v.shape[self.seq_dim] != self.chunk:
            raise ValueError("an update must carry exactly chunk_size tokens")
        for r in range(self.chunk):
            t = chunk_idx * self.chunk + r
            self.tokens[t] = (np.take(k, r, axis=self.seq_dim).copy(),
                              np.take(v, r, axis=self.seq_dim).copy())
        self.last_chunk = chunk_idx
        keep = set(self.visible_tokens())
        for t in list(self.tokens):
            if t not in keep:
                del self.tokens[t]

    # -- views ------------------------------------------------------------------------
    def total_tokens(self):
        return (self.last_chunk + 1) * self.chunk

    def visible_tokens(self):
        T = self.total_tokens()
        head = list(range(0, min(T, self.sink)))
        tail = list(range(max(self.sink, T - self.window), T))
        return head + tail

    def _stack(self, which):
        rows = [self.tokens[t][which] for t in self.visible_tokens()]
        if not rows:
            shape = list(self.k_shape if which == 0 else self.v_shape)
            shape[self.seq_dim] = 0
            return np.zeros(shape)
        return np.stack(rows, axis=self.seq_dim)

    def cached_k(self):
        return self._stack(0)

    def cached_v(self):
        return self._stack(1)
