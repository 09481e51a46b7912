"""Adapters held in host memory and placed into a paged pool's slots on demand, ahead of
their use (S-LoRA summary, "Adapter Loading, Prefetching, and Overlapping I/O with
Computation"; Punica summary, "On-Demand LoRA Weight Loading").

Host-side orchestration over the C library's free-page list and loader; no arithmetic of
the path happens here.

- PagedModel: one paged weight descriptor per adapted projection of a model (layer x
  projection), all sharing one pool of pages and one rank and scale array over the slots.
- HostAdapter: one adapter's rank-rows for every target, packed once into a page-locked
  blob laid out for the loader's direct route (job table, the page ids of all targets
  back to back, then all rank-rows), so that loading it again rewrites only its page ids
  (one array) and two fields of its prepared job records.
- AdapterCache: which adapter sits in which slot.  ensure(keys) loads the adapters a batch
  needs that are not resident, each on a side stream with nothing in flight, evicting
  least recently used adapters that the batch does not need (nor those of batches
  prefetched but not yet run).  A slot is reloaded (and its pages handed to another
  adapter) only after the last batch that read it has finished (the events mark_used
  recorded).  prefetch(keys, keep) is ensure for a later batch, issued while the current
  ones run.
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
        self.ids_off = off                       # every target's page ids, back to back
        self.pages_off = []
        for np_t in self.n_pages:
            self.pages_off.append(off)
            off += 4 * np_t
        off = -(-off // 16) * 16
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
        self.last_load = (0, 0)  # (number, side stream) of the last load of this blob (AdapterCache)
        self._jobs = None       # job records for `model`, all but slot and pt_off filled in

    def jobs(self, model: PagedModel, slot, pages):
        """Load jobs placing this adapter into `slot` on the given pages (the ids of all
        targets back to back, target by target), with the page ids written into the blob.
        The caller makes sure no earlier load still reads the blob."""
        ids = np.ascontiguousarray(pages, dtype=np.int32)
        if len(ids) != sum(self.n_pages):
            raise ValueError(f"{len(ids)} pages for {sum(self.n_pages)}")
        self.blob.numpy()[self.ids_off:self.ids_off + 4 * len(ids)] = ids.view(np.uint8)
        if self._jobs is None:
            self._jobs = (B.CLoadJob * len(model.targets))()
            for t, w in enumerate(model.targets):
                j = self._jobs[t]
                j.w = ctypes.addressof(w.c)
                j.rank, j.scale, j.reserved = self.rank, self.scale, 0
                j.data_off, j.pages_off = self.data_off[t], self.pages_off[t]
        for j, cap in zip(self._jobs, model.caps):
            j.slot, j.pt_off = int(slot), int(slot) * cap
        return self._jobs


class AdapterCache:
    """Slots of a PagedModel holding adapters from a host store (key -> HostAdapter).

    Anything queued on a stream behind a host-to-device copy still in flight (a kernel, an
    event, a wait) holds back the kernels of the other streams until the copy ends: a 7B
    decode step ran a fifth slower with one event recorded behind each load's copies, and
    2 % slower with the copies alone.  So each load (lora_pool_load: a small copy, a small
    kernel, then the long copies of the rank-rows) goes to a side stream with nothing in
    flight (up to `max_side` of them; past that the host waits for the oldest), and
    nothing is queued behind its copies: what a load must wait for is waited for on the
    host (normally long finished), and whether it has landed is asked on the host of its
    side stream, which has finished every earlier load once it has taken a later one.
    Only a batch whose load is still in flight gets an event behind it to wait on."""

    def __init__(self, model: PagedModel, store, streams=None, max_side=4):
        import torch
        self.model, self.store = model, store
        self.sides = list(streams) if streams is not None else [torch.cuda.Stream()]
        self.max_side = max(max_side, len(self.sides))
        self.side_load = [0] * len(self.sides)          # the last load each side stream took
        self.side = self.sides[0]
        self.slot_of = {}                                   # resident key -> slot
        self.key_in = [None] * model.num_slots              # slot -> key
        self.lru = collections.OrderedDict()                # resident keys, least recently used first
        self.pages = {}                                      # resident key -> its page ids (all targets)
        self.last_use = [None] * model.num_slots            # event after the last batch that read the slot
        self.loaded = {}                                     # resident key -> (its load's number, side stream)
        self.staging = [None] * len(self.sides)             # per side stream (the staged route's copy)
        self.loads = 0                                       # loads issued; number of the latest
        self.late = 0                                        # batches that had to wait for a load in flight

    # -------------------------------------------------------------- host policy
    def plan(self, keys, keep=()):
        """Where to put the batch's missing adapters and whom to evict, without changing
        anything: [(key, slot, [evicted keys])] in batch order.  Keys the batch needs, and
        keys in `keep` (batches prefetched but not yet run), are never evicted; free slots
        go first, then the least recently used residents, which are also evicted while the
        pool lacks pages.  ValueError when the batch cannot fit (more distinct adapters than
        slots, or too few pages even after every eviction); KeyError for a key the host
        store lacks."""
        need = [k for k in dict.fromkeys(k for k in keys if k is not None)]
        if len(need) > self.model.num_slots:
            raise ValueError(f"{len(need)} distinct adapters in one batch, {self.model.num_slots} slots")
        needed = set(need) | set(k for k in keep if k is not None)
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
                free_pages += len(self.pages[v])
                if slot is None:
                    slot = self.slot_of[v]
                else:
                    free_slots.append(self.slot_of[v])
            free_pages -= want
            out.append((k, slot, evicted))
        return out

    # -------------------------------------------------------------- GPU work
    def has_landed(self, load):
        """True when `load` (number, side stream) has finished: its side stream has taken a
        later load (it only takes one when idle) or has nothing in flight (asked on the host)."""
        n, si = load
        return n <= 0 or self.side_load[si] != n or self.sides[si].query()

    def free_side(self):
        """A side stream with nothing in flight: an idle one, a new one, or (at max_side
        streams) the one with the oldest load, once the host has waited for it."""
        import torch
        for si, side in enumerate(self.sides):
            if side.query():
                return si
        if len(self.sides) < self.max_side:
            self.sides.append(torch.cuda.Stream())
            self.side_load.append(0)
            self.staging.append(None)   # allocated at the stream's first load, which waits for nothing
            return len(self.sides) - 1
        si = min(range(len(self.sides)), key=lambda i: self.side_load[i])
        self.sides[si].synchronize()
        return si

    def ensure(self, keys, keep=()):
        """Makes every adapter named in keys (None = no adapter) resident, keeping the keys
        in `keep`; returns the device slot per key as a numpy int32 array (-1 for None) and
        the events the stream that reads those slots must wait on first: none when their
        loads (issued now or by an earlier prefetch) have landed, else one event after the
        side stream's copies."""
        import torch
        self.prefetch(keys, keep)
        slots = np.array([self.slot_of[k] if k is not None else -1 for k in keys], dtype=np.int32)
        if all(self.has_landed(self.loaded[k]) for k in keys if k is not None):
            return slots, []
        self.late += 1
        waits = []
        for si in sorted(set(self.loaded[k][1] for k in keys if k is not None and not self.has_landed(self.loaded[k]))):
            e = torch.cuda.Event()        # an event behind the copies of each load in flight
            e.record(self.sides[si])
            waits.append(e)
        return slots, waits

    def prefetch(self, keys, keep=()):
        """The loads of ensure(keys, keep) without waiting for them: for a batch that runs
        later, issued while earlier ones run."""
        import torch
        for k, slot, evicted in self.plan(keys, keep):
            for v in evicted:              # pages still being written by an unfinished load
                if not self.has_landed(self.loaded[v]):
                    self.sides[self.loaded[v][1]].synchronize()
            pages, waits = self.take(k, slot, evicted)
            ad = self.store[k]
            if not self.has_landed(ad.last_load):
                self.sides[ad.last_load[1]].synchronize()    # its blob is still being read
            jobs = ad.jobs(self.model, slot, pages)
            n = self.loads + 1
            si = self.free_side()
            side = self.sides[si]
            if self.staging[si] is None or self.staging[si].numel() < ad.blob.numel():
                if self.staging[si] is not None:
                    torch.cuda.synchronize()   # the previous staging may still be read
                size = max(ad.blob.numel(), max((a.blob.numel() for a in self.store.values()), default=0))
                self.staging[si] = torch.empty(size, dtype=torch.uint8, device=self.model.pool.device)
            for e in waits:               # the last readers of the slot and pages, normally done
                if not e.query():
                    e.synchronize()
            B.lora_pool_load(jobs, ad.blob, self.staging[si], stream=side)
            self.loads = n
            self.side_load[si] = n
            self.loaded[k] = ad.last_load = (n, si)
        for k in keys:
            if k is not None:
                self.lru.move_to_end(k)

    def take(self, k, slot, evicted):
        """The host side of one step of a plan: evicts (their pages back to the free list),
        gives `slot` and fresh pages to k; returns k's page ids (all targets back to back,
        one allocation) and the events the load must wait for (the last batches that read
        the evicted slots and `slot`, whose pages the free list may hand out again at
        once)."""
        waits = []
        for v in evicted:
            s = self.slot_of.pop(v)
            self.key_in[s] = None
            del self.lru[v]
            self.loaded.pop(v, None)
            self.model.state.release(self.pages.pop(v))
            if self.last_use[s] is not None:
                waits.append(self.last_use[s])
        if self.last_use[slot] is not None and self.last_use[slot] not in waits:
            waits.append(self.last_use[slot])
        pages = self.model.state.alloc(sum(self.store[k].n_pages))
        self.slot_of[k], self.key_in[slot], self.pages[k] = slot, k, pages
        self.lru[k] = None
        self.loaded[k] = (0, 0)          # set once its load is issued
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
