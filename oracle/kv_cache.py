"""Plain model of the paged K/V cache operations (test infrastructure only).

Only ``tests/`` may use this module; the product path never does.

What it follows: "Architecture", "Serving boundary" -- a request owns a logical
page table, physical pages are leased from shared per-layer pools, and each new
token's K/V is appended before attention reads it through the table;
"Execution Backends and the Python ABI", "Incremental attention" -- the pools are
[physical_page, H, page_offset, d_h].  The pages do not fix a leasing order; the
reading used here (and stated for the library) is a stack of free pages: the
sequences whose next position starts a page take pages from the top in sequence
index order, and released pages are pushed in the order they are listed.

Everything is numpy, one sequence at a time, in the order the definition reads:
no vectorised tricks, so a reader can check each step against the text.
"""
import numpy as np

KV_OK = 0
KV_POOL_EXHAUSTED = 1
KV_SEQUENCE_FULL = 2
KV_STACK_OVERFLOW = 3


class KvCacheModel:
    """State of one layer's cache, exactly as the library lays it out."""

    def __init__(self, S, Hkv, D, page_size, max_pages, num_pages):
        self.S, self.Hkv, self.D = S, Hkv, D
        self.page_size, self.max_pages, self.num_pages = page_size, max_pages, num_pages
        self.k_pool = np.zeros((num_pages, Hkv, page_size, D), dtype=np.float32)
        self.v_pool = np.zeros((num_pages, Hkv, page_size, D), dtype=np.float32)
        self.block_table = np.zeros((S, max_pages), dtype=np.int32)
        self.context_lens = np.zeros((S,), dtype=np.int32)
        # free stack: entries 0 .. free_count-1, top at free_count-1; page 0 on top at the start
        self.free_pages = np.arange(num_pages - 1, -1, -1, dtype=np.int32)
        self.free_count = num_pages
        self.status = KV_OK

    def append(self, k_new, v_new):
        """Append k_new[s], v_new[s] ([Hkv, D] each) to every sequence s."""
        capacity = self.page_size * self.max_pages
        lengths = [int(t) for t in self.context_lens]
        if any(t >= capacity for t in lengths):
            self.status = KV_SEQUENCE_FULL
            return self.status
        starting = [s for s in range(self.S) if lengths[s] % self.page_size == 0]
        if len(starting) > self.free_count:
            self.status = KV_POOL_EXHAUSTED
            return self.status
        # lease: the r-th sequence (index order) that starts a page takes the r-th page from the top
        for r, s in enumerate(starting):
            page = int(self.free_pages[self.free_count - 1 - r])
            self.block_table[s, lengths[s] // self.page_size] = page
        self.free_count -= len(starting)
        # write each sequence's new row into its page slot, then advance its length
        for s in range(self.S):
            t = lengths[s]
            page = int(self.block_table[s, t // self.page_size])
            self.k_pool[page, :, t % self.page_size, :] = k_new[s]
            self.v_pool[page, :, t % self.page_size, :] = v_new[s]
            self.context_lens[s] = t + 1
        self.status = KV_OK
        return self.status

    def append_tokens(self, k_new, v_new, token_start):
        """Append rows token_start[s] .. token_start[s+1]-1 of k_new, v_new ([N, Hkv, D])
        to sequence s, for every s.  The pages the new positions start are leased from
        the top of the stack: sequences in index order, each one's pages in logical
        order."""
        capacity = self.page_size * self.max_pages
        lengths = [int(t) for t in self.context_lens]
        counts = [int(token_start[s + 1]) - int(token_start[s]) for s in range(self.S)]
        if any(lengths[s] + counts[s] > capacity for s in range(self.S)):
            self.status = KV_SEQUENCE_FULL
            return self.status
        # logical pages that do not exist yet: ceil(t / page) .. ceil((t + n) / page) - 1
        new_pages = []
        for s in range(self.S):
            first = -(-lengths[s] // self.page_size)
            last = -(-(lengths[s] + counts[s]) // self.page_size)
            new_pages.extend((s, p) for p in range(first, last))
        if len(new_pages) > self.free_count:
            self.status = KV_POOL_EXHAUSTED
            return self.status
        for r, (s, p) in enumerate(new_pages):
            self.block_table[s, p] = int(self.free_pages[self.free_count - 1 - r])
        self.free_count -= len(new_pages)
        for s in range(self.S):
            for j in range(counts[s]):
                t = lengths[s] + j
                page = int(self.block_table[s, t // self.page_size])
                self.k_pool[page, :, t % self.page_size, :] = k_new[int(token_start[s]) + j]
                self.v_pool[page, :, t % self.page_size, :] = v_new[int(token_start[s]) + j]
            self.context_lens[s] = lengths[s] + counts[s]
        self.status = KV_OK
        return self.status

    def release(self, seq_ids):
        """Push the pages of seq_ids back (in list order, each sequence's pages in
        logical order) and zero their lengths."""
        pages = []
        for s in seq_ids:
            n = -(-int(self.context_lens[s]) // self.page_size)
            pages.extend(int(self.block_table[s, p]) for p in range(n))
        if self.free_count + len(pages) > self.num_pages:
            self.status = KV_STACK_OVERFLOW
            return self.status
        for page in pages:
            self.free_pages[self.free_count] = page
            self.free_count += 1
        for s in seq_ids:
            self.context_lens[s] = 0
        self.status = KV_OK
        return self.status

    def gather(self, s):
        """Sequence s's cached keys and values [ctx, Hkv, D] in logical order,
        read through its page table."""
        t = int(self.context_lens[s])
        ks = np.zeros((t, self.Hkv, self.D), dtype=np.float32)
        vs = np.zeros((t, self.Hkv, self.D), dtype=np.float32)
        for pos in range(t):
            page = int(self.block_table[s, pos // self.page_size])
            ks[pos] = self.k_pool[page, :, pos % self.page_size, :]
            vs[pos] = self.v_pool[page, :, pos % self.page_size, :]
        return ks, vs

    def live_pages(self):
        """Pages held by the sequences, as a list of (sequence, logical page, physical page)."""
        out = []
        for s in range(self.S):
            for p in range(-(-int(self.context_lens[s]) // self.page_size)):
                out.append((s, p, int(self.block_table[s, p])))
        return out
