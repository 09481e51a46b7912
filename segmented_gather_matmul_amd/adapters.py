"""Adapters held in host memory and placed into a paged pool's slots on demand, ahead of
their use (S-LoRA summary, "Adapter Loading, Prefetching, and Overlapping I/O with
Computation"; Punica summary, "On-Demand LoRA Weight Loading").

Host-side orchestration over the C library's free-page list and loader; no arithmetic of
the path happens here.

- PagedModel: one paged weight descriptor per adapted projection of a model (layer x
  projection), all sharing one pool of pages and one rank and scale array over the slots.
- HostAdapter: one adapter's rank-rows for every target, packed once into a page-locked
  blob laid out for the loader's direct route (job table, page ids, then all rank-rows),
  so that loading it again rewrites only its page ids.
- AdapterCache: which adapter sits in which slot.  ensure(keys) loads the adapters a batch
  needs that are not resident, on a side stream, evicting least recently used adapters
  that the batch does not need; the compute stream waits on the returned event.  A slot is
  reloaded (and its pages handed to another adapter) only after the last batch that read
  it has finished: every load waits on the events mark_used recorded.  prefetch(keys) is
  ensure for the next batch, issued while the current one runs.
"""
from __future__ import annotations

import collections
import ctypes

import numpy as np

from . import binding as B


class PagedModel:
    """Paged descriptors of one model's adapted projections over num_slots slots."""

    def __init__(self, shapes, num_slots, r_max, page_elems, num_pages, device="cuda"):
        import torch
        self.shapes = [(int(di), int(do)) for di, do in shapes]
        self.num_slots, self.r_max, self.P = int(num_slots), int(r_max), int(page_elems)
        self.pool = torch.empty((int(num_pages), self.P), dtype=torch.float16, device=device)
        self.rank = torch.zeros(self.num_slots, dtype=torch.int32, device=device)
        self.scale = torch.zeros(self.num_slots, dtype=torch.float32, device=device)
        self.state = B.PoolState(int(num_pages))
        self.targets, self.caps = [], []
        for di, do in self.shapes:
            if di % self.P or do % self.P:
                raise ValueError(f"page_elems {self.P} must divide d_in {di} and d_out {do}")
            cap = self.r_max * (di // self.P + do // self.P)   # page-table entries per slot
            self.caps.append(cap)
            self.targets.append(B.Weights(
                num_slots=self.num_slots, d_in=di, d_out=do, r_max=self.r_max, rank=self.rank, scale=self.scale,
                pool=self.pool, page_elems=self.P,
                page_table=torch.full((self.num_slots * cap,), -1, dtype=torch.int32, device=device),
                a_pt_off=torch.zeros(self.num_slots, dtype=torch.int64, device=device),
                b_pt_off=torch.zeros(self.num_slots, dtype=torch.int64, device=device)))

    def pages_for(self, rank):
        """Pages one adapter of this rank takes, per target."""
        return [B.lora_pool_pages_for(int(rank), di, do, self.P) for di, do in self.shapes]


class HostAdapter:
    """One adapter (rank, scale, A^T and B per target) packed into a page-locked blob."""

    def __init__(self, model: PagedModel, rank, scale, a_t, b):
        import torch
        self.rank, self.scale = int(rank), float(scale)
        if not 1 <= self.rank <= model.r_max:
            raise ValueError(f"rank {self.rank} outside 1..{model.r_max}")
        if len(a_t) != len(model.shapes) or len(b) != len(model.shapes):
            raise ValueError("one A^T and one B per target")
        n = len(model.shapes)
        self.n_pages = model.pages_for(self.rank)
        off = int(B.lib().lora_pool_load_header_bytes(n))
        self.pages_off = []
        for np_t in self.n_pages:
            self.pages_off.append(off)
            off = -(-(off + 4 * np_t) // 16) * 16
        self.data_off, datas = [], []
        for (di, do), a, bb in zip(model.shapes, a_t, b):
            a = np.ascontiguousarray(a, dtype=np.float16)
            bb = np.ascontiguousarray(bb, dtype=np.float16)
            if a.shape != (self.rank, di) or bb.shape != (self.rank, do):
                raise ValueError(f"target {di}->{do}: A^T {a.shape} and B {bb.shape} for rank {self.rank}")
            self.data_off.append(off)
            datas.append((off, a, bb))
            off += 2 * self.rank * (di + do)   # a multiple of 16: P divides d_in and d_out, P % 8 == 0
        self.blob = torch.zeros(off, dtype=torch.uint8, pin_memory=True)
        view = self.blob.numpy()
        for o, a, bb in datas:
            na = a.size * 2
            view[o:o + na] = a.view(np.uint8).ravel()
            view[o + na:o + na + bb.size * 2] = bb.view(np.uint8).ravel()
        self.load_done = None   # event of the last load that read the blob

    def jobs(self, model: PagedModel, slot, pages):
        """Load jobs placing this adapter into `slot` on the given pages (one id array per
        target), with the page ids written into the blob."""
        if self.load_done is not None:
            self.load_done.synchronize()   # a load still reading the blob's page ids
        view = self.blob.numpy()
        jobs = (B.CLoadJob * len(model.targets))()
        for t, (w, cap) in enumerate(zip(model.targets, model.caps)):
            ids = np.ascontiguousarray(pages[t], dtype=np.int32)
            if len(ids) != self.n_pages[t]:
                raise ValueError(f"target {t}: {len(ids)} pages for {self.n_pages[t]}")
            o = self.pages_off[t]
            view[o:o + 4 * len(ids)] = ids.view(np.uint8)
            j = jobs[t]
            j.w = ctypes.addressof(w.c)
            j.slot, j.rank, j.scale, j.reserved = int(slot), self.rank, self.scale, 0
            j.pt_off = int(slot) * cap
            j.data_off, j.pages_off = self.data_off[t], o
        return jobs


class AdapterCache:
    """Slots of a PagedModel holding adapters from a host store (key -> HostAdapter)."""

    def __init__(self, model: PagedModel, store, stream=None):
        import torch
        self.model, self.store = model, store
        self.side = stream if stream is not None else torch.cuda.Stream()
        self.slot_of = {}                                   # resident key -> slot
        self.key_in = [None] * model.num_slots              # slot -> key
        self.lru = collections.OrderedDict()                # resident keys, least recently used first
        self.pages = {}                                      # resident key -> page ids per target
        self.last_use = [None] * model.num_slots            # event after the last batch that read the slot
        self.loaded = {}                                     # resident key -> (load number, event after its load)
        self.staging = None
        self.loads = 0

    # -------------------------------------------------------------- host policy
    def plan(self, keys):
        """Where to put the batch's missing adapters and whom to evict, without changing
        anything: [(key, slot, [evicted keys])] in batch order.  Keys the batch needs are
        never evicted; free slots go first, then the least recently used residents, which
        are also evicted while the pool lacks pages.  ValueError when the batch cannot fit
        (more distinct adapters than slots, or too few pages even after every eviction);
        KeyError for a key the host store lacks."""
        need = [k for k in dict.fromkeys(k for k in keys if k is not None)]
        if len(need) > self.model.num_slots:
            raise ValueError(f"{len(need)} distinct adapters in one batch, {self.model.num_slots} slots")
        needed = set(need)
        free_slots = [s for s, k in enumerate(self.key_in) if k is None]
        victims = [k for k in self.lru if k not in needed]
        free_pages = self.model.state.free
        out = []
        for k in need:
            if k in self.slot_of:
                continue
            if k not in self.store:
                raise KeyError(f"adapter {k!r} is not in the host store")
            want = sum(self.store[k].n_pages)
            evicted = []
            slot = free_slots.pop(0) if free_slots else None
            while slot is None or free_pages < want:
                if not victims:
                    raise ValueError(f"no room for adapter {k!r}: {free_pages} free pages, {want} needed")
                v = victims.pop(0)
                evicted.append(v)
                free_pages += sum(len(p) for p in self.pages[v])
                if slot is None:
                    slot = self.slot_of[v]
                else:
                    free_slots.append(self.slot_of[v])
            free_pages -= want
            out.append((k, slot, evicted))
        return out

    # -------------------------------------------------------------- GPU work
    def ensure(self, keys):
        """Makes every adapter named in keys (None = no adapter) resident; returns the device
        slot per key as a numpy int32 array (-1 for None) and the event the compute stream
        must wait on before reading those slots: the side stream's event after the latest
        load of any of these adapters, issued now or by an earlier prefetch (the side stream
        runs its loads in order), or None when none was ever loaded through this cache."""
        import torch
        for k, slot, evicted in self.plan(keys):
            pages, waits = self.take(k, slot, evicted)
            ad = self.store[k]
            jobs = ad.jobs(self.model, slot, pages)
            if self.staging is None or self.staging.numel() < ad.blob.numel():
                self.side.synchronize()   # the previous staging may still be read
                self.staging = torch.empty(ad.blob.numel(), dtype=torch.uint8, device=self.model.pool.device)
            for e in waits:
                self.side.wait_event(e)
            B.lora_pool_load(jobs, ad.blob, self.staging, stream=self.side)
            ad.load_done = torch.cuda.Event()
            ad.load_done.record(self.side)
            self.loaded[k] = (self.loads, ad.load_done)
        latest = None
        for k in keys:
            if k is not None:
                self.lru.move_to_end(k)
                if latest is None or self.loaded[k][0] > latest[0]:
                    latest = self.loaded[k]
        slots = np.array([self.slot_of[k] if k is not None else -1 for k in keys], dtype=np.int32)
        return slots, (latest[1] if latest is not None else None)

    prefetch = ensure

    def take(self, k, slot, evicted):
        """The host side of one step of a plan: evicts (their pages back to the free list),
        gives `slot` and fresh pages to k; returns k's page ids per target and the events
        the load must wait for (the last batches that read the evicted slots and `slot`,
        whose pages the free list may hand out again at once)."""
        waits = []
        for v in evicted:
            s = self.slot_of.pop(v)
            self.key_in[s] = None
            del self.lru[v]
            self.loaded.pop(v, None)
            self.model.state.release(np.concatenate(self.pages.pop(v)))
            if self.last_use[s] is not None:
                waits.append(self.last_use[s])
        if self.last_use[slot] is not None and self.last_use[slot] not in waits:
            waits.append(self.last_use[slot])
        pages = [self.model.state.alloc(n) for n in self.store[k].n_pages]
        self.slot_of[k], self.key_in[slot], self.pages[k] = slot, k, pages
        self.lru[k] = None
        self.loads += 1
        self.loaded[k] = (self.loads, None)
        return pages, waits

    def mark_used(self, keys, stream=None):
        """Records, on `stream` (default: the current one), that the work enqueued so far
        reads the slots of these keys."""
        import torch
        e = torch.cuda.Event()
        e.record(stream if stream is not None else torch.cuda.current_stream())
        for k in set(k for k in keys if k is not None):
            self.last_use[self.slot_of[k]] = e
        return e
