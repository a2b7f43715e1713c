"""Host-side model of the decode kernel's work partition (CPU only).

The persistent decode gives wave w of NW the items [w*W/NW, (w+1)*W/NW) of
the (request, kv-head, page) list; a piece that is not a whole segment goes to
slot w + segment, and the merge pass collects, for each segment, the slots of
the waves between the waves holding its first and last item (none of them has
an empty slice).  This
checks, in integers, that every slot is written once and that each segment's
pieces tile its pages exactly -- for empty requests, more waves than pages and
fewer waves than segments alike.  Slices hold at least 4 pages: with less work
than that per workgroup, only ceil(W / 4) workgroups take slices.
"""
import random


MIN_SLICE = 4  # pages per slice at least: the slice count is min(grid, ceil(W / 4))


def _check(pages, Hkv, grid):
    pre = [0]
    for n in pages:
        pre.append(pre[-1] + n)
    B = len(pages)
    W = Hkv * pre[-1]
    if W == 0:
        return
    NW = max(1, min(grid, -(-W // MIN_SLICE)))
    assert NW == grid or W < grid * MIN_SLICE
    slots = {}
    for w in range(NW):
        x0, x1 = w * W // NW, (w + 1) * W // NW
        x = x0
        while x < x1:
            b = max(i for i in range(B) if Hkv * pre[i] <= x)
            n = pre[b + 1] - pre[b]
            off = x - Hkv * pre[b]
            g, page = off // n, off % n
            seg = b * Hkv + g
            seg_end = Hkv * pre[b] + g * n + n
            end = min(x1, seg_end)
            if not (page == 0 and end == seg_end):
                assert w + seg not in slots
                slots[w + seg] = (seg, x, end)
            x = end
    for b in range(B):
        n = pre[b + 1] - pre[b]
        if n == 0:
            continue
        for g in range(Hkv):
            seg = b * Hkv + g
            first = Hkv * pre[b] + g * n
            last = first + n - 1
            wf = ((first + 1) * NW - 1) // W
            wl = ((last + 1) * NW - 1) // W
            if wf == wl:
                assert all(v[0] != seg for v in slots.values())
                continue
            # the merge pass reads every workgroup between them: with at least one
            # page per workgroup no slice is empty
            assert all(w * W // NW != (w + 1) * W // NW for w in range(wf, wl + 1))
            got = [slots[w + seg] for w in range(wf, wl + 1)]
            assert all(p[0] == seg for p in got)
            cov = sorted((p[1], p[2]) for p in got)
            assert cov[0][0] == first and cov[-1][1] == last + 1
            assert all(cov[i][1] == cov[i + 1][0] for i in range(len(cov) - 1))


def test_partition_random():
    rng = random.Random(0)
    for _ in range(300):
        B = rng.randint(1, 7)
        Hkv = rng.randint(1, 4)
        pages = [rng.choice([0, 0, 1, 2, 3, 5, 17, 40]) for _ in range(B)]
        for grid in (4, 8, 12, 64, 4096):
            _check(pages, Hkv, grid)


def test_partition_workload_shapes():
    import workloads
    for cfg in (1, 3):
        w = workloads.make(cfg)
        for grid in (64, 768, 4096):
            _check([int(n) for n in w.n_pages], w.Hkv, grid)
