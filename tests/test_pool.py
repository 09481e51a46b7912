"""Adapter pool, host side: the free-page list and every check lora_pool_load makes
before it issues anything (device pointers here are stand-ins that are never used)."""
import ctypes

import numpy as np
import pytest

from segmented_gather_matmul_amd import binding as B

FAKE = 0x7f0000000000


def test_free_list_order_and_counts():
    st = B.PoolState(8)
    assert st.free == 8
    a = st.alloc(5)
    assert a.tolist() == [0, 1, 2, 3, 4] and st.free == 3
    st.release([3, 1])
    assert st.free == 5
    assert st.alloc(3).tolist() == [3, 1, 5]          # the last release first, in its order
    assert st.alloc(2).tolist() == [6, 7] and st.free == 0


def test_free_list_errors_change_nothing():
    st = B.PoolState(4)
    taken = st.alloc(3)
    with pytest.raises(B.LoraError) as e:
        st.alloc(2)
    assert e.value.code == B.LORA_E_CAPACITY and st.free == 1
    for bad in ([3], [0, 0], [-1], [4], [0, 3]):           # not taken, twice, out of range
        with pytest.raises(B.LoraError) as e:
            st.release(bad)
        assert e.value.code == B.LORA_E_INDEX
        assert st.free == 1
    st.release(taken)
    assert st.free == 4 and sorted(st.alloc(4).tolist()) == [0, 1, 2, 3]


def test_free_list_state_checks():
    L = B.lib()
    assert L.lora_pool_state_bytes(0) == 0 and L.lora_pool_state_bytes(1 << 31) == 0
    n = L.lora_pool_state_bytes(100)
    assert n % 16 == 0 and n >= 100 * 5
    buf = np.zeros(n, dtype=np.uint8)
    assert L.lora_pool_init(buf.ctypes.data, n - 16, 100) == B.LORA_E_CAPACITY
    assert L.lora_pool_init(None, n, 100) == B.LORA_E_NULL
    assert L.lora_pool_init(buf.ctypes.data, n, 0) == B.LORA_E_SHAPE
    assert L.lora_pool_free_count(buf.ctypes.data) == -1             # not initialised
    out = np.zeros(1, np.int32)
    assert L.lora_pool_alloc(buf.ctypes.data, 1, out.ctypes.data) == B.LORA_E_NULL
    assert L.lora_pool_init(buf.ctypes.data, n, 100) == B.LORA_OK
    assert L.lora_pool_alloc(buf.ctypes.data, -1, out.ctypes.data) == B.LORA_E_SHAPE
    assert L.lora_pool_alloc(buf.ctypes.data, 1, None) == B.LORA_E_NULL


def test_pages_for():
    assert B.lora_pool_pages_for(16, 4096, 4096, 1024) == 16 * 8
    assert B.lora_pool_pages_for(0, 4096, 4096, 1024) == 0
    with pytest.raises(B.LoraError):
        B.lora_pool_pages_for(16, 4096, 1000, 1024)


# ------------------------------------------------------------------ loader argument checks
P, D_IN, D_OUT, R_MAX, S, NP, PT = 8, 16, 24, 4, 3, 40, 64


def _target(**kw):
    c = B.CWeights()
    c.layout, c.num_slots, c.d_in, c.d_out, c.r_max = B.LAYOUT_PAGED, S, D_IN, D_OUT, R_MAX
    c.rank = c.scale = c.pool = c.page_table = c.a_pt_off = c.b_pt_off = FAKE
    c.page_elems, c.num_pages, c.pt_entries = P, NP, PT
    for k, v in kw.items():
        setattr(c, k, v)
    return c


class _W:
    def __init__(self, c):
        self.c = c


def _job(w, slot, rank, pt_off, first_page, scale=1.0):
    n = rank * (D_IN // P + D_OUT // P)
    return dict(w=w, slot=slot, rank=rank, scale=scale, pt_off=pt_off,
                a_t=np.zeros((rank, D_IN), np.float16), b=np.zeros((rank, D_OUT), np.float16),
                pages=np.arange(first_page, first_page + n, dtype=np.int32))


def _load(adapters, staging_bytes=None, mutate=None):
    blob, jobs = B.pack_adapters(adapters, pinned=False)
    if mutate:
        mutate(jobs, blob)
    n = blob.numel()
    return B.lib().lora_pool_load(None, len(jobs), jobs, B._ptr(blob), n, FAKE,
                                  n if staging_bytes is None else staging_bytes)


def test_load_rejects_before_issuing_anything():
    L = B.lib()
    w, w2 = _W(_target()), _W(_target(a_pt_off=FAKE + 64, page_table=FAKE + 128))
    ok = [_job(w, 0, 2, 0, 0), _job(w, 1, 1, 10, 10)]
    assert L.lora_pool_load(None, 0, None, None, 0, None, 0) == B.LORA_OK         # nothing to do
    assert L.lora_pool_load(None, -1, None, None, 0, None, 0) == B.LORA_E_SHAPE
    assert _load(ok, staging_bytes=16) == B.LORA_E_CAPACITY                          # staging smaller than blob
    dense = _W(_target(layout=B.LAYOUT_DENSE, a_t=FAKE, b=FAKE))
    assert _load([_job(dense, 0, 1, 0, 0)]) == B.LORA_E_UNSUPPORTED                  # target not paged
    assert _load([_job(w, S, 1, 0, 0)]) == B.LORA_E_INDEX                            # slot out of range
    assert _load([_job(w, 0, R_MAX + 1, 0, 0)]) == B.LORA_E_SHAPE                    # rank above r_max
    assert _load([_job(w, 0, 2, PT - 5, 0)]) == B.LORA_E_INDEX                       # page-table range past the end
    assert _load([_job(w, 0, 2, 0, NP - 3)]) == B.LORA_E_INDEX                       # page id past the pool
    assert _load([_job(w, 0, 2, 0, 0), _job(w, 1, 1, 10, 4)]) == B.LORA_E_INDEX      # page named twice
    assert _load([_job(w, 0, 2, 0, 0), _job(w, 1, 1, 5, 10)]) == B.LORA_E_INDEX      # page-table ranges overlap
    assert _load([_job(w, 0, 2, 0, 0), _job(w, 0, 1, 10, 10)]) == B.LORA_E_INDEX     # one slot loaded twice
    # two targets sharing rank/scale: the same slot must get the same rank and scale
    assert _load([_job(w, 0, 2, 0, 0), _job(w2, 0, 1, 10, 10)]) == B.LORA_E_INDEX
    assert _load([_job(w, 0, 2, 0, 0), _job(w2, 0, 2, 10, 10, scale=2.0)]) == B.LORA_E_INDEX

    def misalign(jobs, blob):
        jobs[0].data_off += 8
    assert _load(ok, mutate=misalign) == B.LORA_E_ALIGN

    def into_header(jobs, blob):
        jobs[0].data_off = 0
    assert _load(ok, mutate=into_header) == B.LORA_E_SHAPE

    def past_end(jobs, blob):
        jobs[1].pages_off = blob.numel() - 4
    assert _load(ok, mutate=past_end) == B.LORA_E_SHAPE

    def reserved(jobs, blob):
        jobs[0].reserved = 1
    assert _load(ok, mutate=reserved) == B.LORA_E_SHAPE
    assert "reserved" in B.last_error()


def test_load_job_layout_and_header():
    assert ctypes.sizeof(B.CLoadJob) == 48
    hb = B.lib().lora_pool_load_header_bytes
    assert hb(0) == 0 and hb(1) % 16 == 0 and hb(10) == 10 * hb(1)
