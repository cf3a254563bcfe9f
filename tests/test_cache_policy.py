"""The expert cache's replacement policy on the CPU (k3moe_cache_plan plans
a batch without copying anything): hits keep their slot and are refreshed,
misses take a free slot or the least recently used one that the batch does
not need, and a batch never evicts its own experts."""
import ctypes

import numpy as np
import pytest

k3 = pytest.importorskip("mxfp4_routed_expert_gemv_amd")

FAKE = 0x10000


def _cache(slots, E=16, k=2):
    shape = k3.make_shape(1, 256, 128, E, k, 0, 0, k3.F32, k3.F32)
    host = k3.make_bank(k3.FMT_MXFP4, E, 256, 128, FAKE, FAKE, FAKE, FAKE)
    dev = k3.make_bank(k3.FMT_MXFP4, slots, 256, 128, FAKE, FAKE, FAKE, FAKE)
    return k3.ExpertCache(shape, host, dev)


def test_lru_sequence():
    c = _cache(4)
    assert c.plan([1, 2]).tolist() == [0, 1]          # free slots in order
    assert c.plan([3, 4]).tolist() == [2, 3]
    assert c.plan([1, 5]).tolist() == [0, 1]          # 1 hits; 5 evicts 2 (oldest unpinned)
    # 3 hits and is pinned before 2 misses: 2 evicts 4 (slot 3, older than 1 and 5)
    assert c.plan([2, 3]).tolist() == [3, 2]
    st = c.stats()
    assert (st["lookups"], st["hits"], st["misses"], st["evictions"]) == (8, 2, 6, 2)
    # a batch's own experts are never evicted, even when its misses come first
    assert c.plan([9, 10, 3, 2]).tolist()[2:] == [2, 3]


def test_more_experts_than_slots():
    c = _cache(3, E=16, k=2)
    with pytest.raises(k3.K3moeError, match="ESHAPE"):
        c.plan([0, 1, 2, 3])
    with pytest.raises(k3.K3moeError, match="EINVAL"):
        c.plan([0, 16])
    with pytest.raises(k3.K3moeError, match="EINVAL"):
        c.plan([4, 4])


def test_full_cache_holds_everything():
    """With as many slots as experts nothing is ever evicted: after one pass
    every lookup hits."""
    c = _cache(16)
    rng = np.random.default_rng(0)
    for _ in range(50):
        c.plan(rng.choice(16, size=4, replace=False))
    st = c.stats()
    assert st["evictions"] == 0 and st["misses"] <= 16


def test_create_validation():
    shape = k3.make_shape(1, 256, 128, 16, 2, 0, 0, k3.F32, k3.F32)
    host = k3.make_bank(k3.FMT_MXFP4, 16, 256, 128, FAKE, FAKE, FAKE, FAKE)
    h = ctypes.c_void_p()
    for dev, code in [(k3.make_bank(k3.FMT_MXFP4, 1, 256, 128, FAKE, FAKE, FAKE, FAKE), 2),
                      (k3.make_bank(k3.FMT_MXFP4, 4, 256, 128, FAKE + 4, FAKE, FAKE, FAKE), 3),
                      (k3.make_bank(k3.FMT_BF16, 4, 256, 128, FAKE, FAKE, FAKE, FAKE), 5),
                      (k3.make_bank(k3.FMT_MXFP4, 4, 512, 128, FAKE, FAKE, FAKE, FAKE), 1)]:
        assert k3.lib.k3moe_cache_create(ctypes.byref(shape), ctypes.byref(host),
                                         ctypes.byref(dev), ctypes.byref(h)) == code
    assert k3.lib.k3moe_cache_workspace_bytes(ctypes.byref(shape), 1) == 0
