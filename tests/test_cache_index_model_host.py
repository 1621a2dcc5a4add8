"""CPU model of the whole-tile phase of reshape_and_cache_kernel (pa_cache.hip):
a workgroup writes the K and V tiles of up to HPW KV heads of one block with
256 threads, thread t taking items t, t + 256, ...  The kernel drops the
per-item bound check when every item exists (all HPW heads present and the
item count a multiple of 256), so the model checks, for every pool / input
dtype pair, head dim, heads per workgroup and KV head count the launcher can
produce, that each item the loops visit lies inside the workgroup's heads,
that every 16-byte unit of every tile is written exactly once, and that the
input elements each item reads lie inside one token row of one head.

The index formulas are restated from the kernel; nothing here runs it.
"""
import pytest

THREADS = 256
BLOCK = 16
ELEM = {0: 4, 1: 2, 2: 1}      # pool dtype -> bytes (fp32, bf16, fp8)
IN_ELEM = {0: 4, 1: 2}         # input dtype -> bytes (fp32, bf16)


def visit(pool, inp, D, hpw, hkv):
    eb, ib = ELEM[pool], IN_ELEM[inp]
    x = 16 // eb                      # K: elements per 16-byte run
    w = 4 // eb                       # V: head dims per 16-byte cell
    k_units = BLOCK * D * eb // 16    # 16-byte units of one tile
    cpi = 2 if pool == 1 else 1       # V cells per work item
    vu = k_units // cpi               # V work items per tile
    ki = (hpw * k_units + THREADS - 1) // THREADS
    vi = (hpw * vu + THREADS - 1) // THREADS
    for gy in range((hkv + hpw - 1) // hpw):
        g0 = gy * hpw
        nh = min(hpw, hkv - g0)
        full = nh == hpw
        kfull = full and (hpw * k_units) % THREADS == 0
        vfull = full and (hpw * vu) % THREADS == 0
        k_written, v_written = set(), set()
        for t in range(THREADS):
            for j in range(ki):
                i = t + j * THREADS
                if not kfull and i >= nh * k_units:
                    break
                assert i < nh * k_units
                hh, u = divmod(i, k_units)
                # input: token u % 16, elements (u / 16) x .. + x - 1 of head g0 + hh
                e0 = (u // BLOCK) * x
                assert 0 <= e0 and e0 + x <= D and (x * ib) % 16 == 0
                key = (g0 + hh, u)
                assert key not in k_written
                k_written.add(key)
            for j in range(vi):
                i = t + j * THREADS
                if not vfull and i >= nh * vu:
                    break
                assert i < nh * vu
                hh, u = divmod(i, vu)
                tg, q = divmod(u, D // w // cpi)
                # input: tokens 4 tg .. 4 tg + 3, elements w cpi q .. + w cpi - 1
                assert 4 * tg + 3 < BLOCK
                assert w * cpi * (q + 1) <= D
                for cc in range(cpi):
                    key = (g0 + hh, u * cpi + cc)
                    assert key[1] < k_units and key not in v_written
                    v_written.add(key)
        every = {(g0 + h, u) for h in range(nh) for u in range(k_units)}
        assert k_written == every and v_written == every


@pytest.mark.parametrize("pool,inp", [(0, 0), (1, 1), (2, 1), (2, 0)])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("hpw", [1, 2, 4, 8])
def test_whole_tile_items_cover_each_unit_once(pool, inp, D, hpw):
    for hkv in (1, 2, 3, 5, 8, 12, 40):
        visit(pool, inp, D, hpw, hkv)

