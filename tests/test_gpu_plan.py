"""The segment decode (h3attn_plan) read back from the workspace and compared with a decode written
here in plain Python: the header's counts, the segment table (start, length), the work items
(segment, 256-query tile, segment start, length) grouped by the cost class of their segment, most
expensive first (a segment's tiles together and in order; the segments of a class in any order),
the class table, and every token's segment index.  Packed layouts ("ws1_one_h3_block" page, Summary: several sequences share one token axis)
reach the library as one id per token; a segment is a maximal run of equal ids and ids never
decrease.  The sizes sit
on both sides of the decode's two paths: the ids staged in LDS for 2048 < T <= 16384, read from
global memory otherwise."""
import numpy as np
import pytest
import torch

import deterministic_invariant_attention_amd as h3
from gpu_util import say

pytestmark = pytest.mark.gpu

BQ, HD = 256, 128
STATUS_SEG_BIT = 1
SCHED_BYTES = 2048


def _a256(x):
    return (x + 255) & ~255


def _offsets(T, H):
    """Byte offsets of the forward workspace's tables (256-byte header, then each region 256-aligned)."""
    max_items = T + (T + BQ - 1) // BQ
    segtab = 256
    items = segtab + _a256(T * 8)
    khat = items + _a256(max_items * 16)
    tok2seg = khat + 3 * _a256(T * H * HD * 2)
    sched = tok2seg + 2 * _a256(T * 4)
    bkt = sched + SCHED_BYTES
    return segtab, items, tok2seg, bkt


def _cost_class(L):
    """floor(log2(ceil(L / 64))): the segment's cost class."""
    return int(np.floor(np.log2((L + 63) // 64)))


def _decode(ids):
    """Segments as (start, length) runs of equal ids, the (segment, tile, start, length) items and
    tok2seg."""
    T = len(ids)
    starts = [t for t in range(T) if t == 0 or ids[t] != ids[t - 1]]
    bounds = starts + [T]
    segtab = [(bounds[i], bounds[i + 1] - bounds[i]) for i in range(len(starts))]
    tok2seg = np.repeat(np.arange(len(segtab)), [L for _, L in segtab])
    return segtab, tok2seg


def _ids_from_lengths(lens, first=0, step=1):
    return np.repeat(first + step * np.arange(len(lens)), lens).astype(np.int32)


def _run_plan(ids, H=2):
    T = len(ids)
    dev = torch.device("cuda:0")
    ws = h3.workspace(T, H, dev)
    ws.fill_(0xA5)  # every table the plan owns must be rewritten
    h3.h3attn_plan(torch.from_numpy(ids).to(dev), H, ws)
    torch.cuda.synchronize()
    w = ws.cpu()
    hdr = w[:256].view(torch.int32).numpy()
    return hdr, w, _offsets(T, H)


def _check(ids, H=2):
    T = len(ids)
    hdr, w, (so, io, to, bo) = _run_plan(ids, H)
    segtab, tok2seg = _decode(ids)
    ntiles = [(L + BQ - 1) // BQ for _, L in segtab]
    assert hdr[0] == 0, f"status {hdr[0]}"
    assert hdr[1] == len(segtab) and hdr[2] == sum(ntiles), (hdr[1], hdr[2], len(segtab), sum(ntiles))
    got_seg = w[so:so + 8 * len(segtab)].view(torch.int32).numpy().reshape(-1, 2)
    assert np.array_equal(got_seg, np.array(segtab, dtype=np.int32).reshape(-1, 2))
    got_t2s = w[to:to + 4 * T].view(torch.int32).numpy()
    assert np.array_equal(got_t2s, tok2seg.astype(np.int32))
    # the class table: non-empty classes, most expensive first
    cls = [_cost_class(L) for _, L in segtab]
    order = sorted(set(cls), reverse=True)
    want_bkt, first = [], 0
    for c in order:
        n = sum(nt for nt, cc in zip(ntiles, cls) if cc == c)
        want_bkt.append((first, n))
        first += n
    assert hdr[3] == len(order)
    got_bkt = w[bo:bo + 8 * len(order)].view(torch.int32).numpy().reshape(-1, 2)
    assert np.array_equal(got_bkt, np.array(want_bkt, dtype=np.int32).reshape(-1, 2))
    # the items: within each class, every segment of that class once, its tiles together and in order
    got = w[io:io + 16 * sum(ntiles)].view(torch.int32).numpy().reshape(-1, 4)
    for c, (f, n) in zip(order, want_bkt):
        rows, seen, r = got[f:f + n], set(), 0
        while r < n:
            sg = int(rows[r, 0])
            assert 0 <= sg < len(segtab) and cls[sg] == c and sg not in seen, (c, r, sg)
            seen.add(sg)
            st, L = segtab[sg]
            want = np.array([(sg, j, st, L) for j in range(ntiles[sg])], dtype=np.int32)
            assert np.array_equal(rows[r:r + ntiles[sg]], want), (c, sg)
            r += ntiles[sg]
        assert seen == {s for s in range(len(segtab)) if cls[s] == c}


def _random_lengths(rng, T, lo, hi):
    lens = []
    while sum(lens) < T:
        lens.append(int(rng.integers(lo, hi + 1)))
    lens[-1] -= sum(lens) - T
    return [n for n in lens if n > 0]


@pytest.mark.parametrize("T", [925, 2048, 2049, 3072, 8349, 16383, 16384, 16385, 20100])
def test_plan_matches_host_decode_random_segments(T):
    rng = np.random.default_rng(T)
    lens = _random_lengths(rng, T, 1, 700)
    say(f"[plan] T={T}: {len(lens)} segments of 1..700 tokens")
    _check(_ids_from_lengths(lens, first=-5, step=3))


@pytest.mark.parametrize("T", [2047, 2049, 16384, 16385])
def test_plan_one_segment_and_all_singletons(T):
    say(f"[plan] T={T}: one segment, then {T} one-token segments")
    _check(np.full(T, 7, dtype=np.int32))
    _check(np.arange(T, dtype=np.int32) * 2 - 3)  # more segments than threads: several per thread


@pytest.mark.parametrize("T", [2049, 8349, 16384])
def test_plan_segment_starts_on_thread_run_edges(T):
    """Segments that start exactly at, just before and just after the first token of a thread's
    run (runs of ceil(T / 1024) tokens), where a run's first id is compared with the previous run's
    last."""
    per = (T + 1023) // 1024
    starts = sorted({0} | {k * per + d for k in range(1, 1024) for d in (-1, 0, 1) if 0 < k * per + d < T})
    starts = starts[::3]
    ids = np.zeros(T, dtype=np.int32)
    ids[starts[1:]] = 1
    ids = np.cumsum(ids).astype(np.int32)
    say(f"[plan] T={T}: {len(starts)} segments starting on run edges (run {per})")
    _check(ids)


@pytest.mark.parametrize("T", [1500, 8349, 16385])
def test_plan_decreasing_ids_set_the_segment_error(T):
    """Ids that decrease inside a run and across two runs: the status word names the error and no
    segment or item is planned."""
    per = (T + 1023) // 1024
    for where in (T // 2 + 1, per * 517):
        ids = np.repeat(np.arange(T // 64 + 1, dtype=np.int32), 64)[:T].copy()
        ids[where] = ids[where - 1] - 1
        hdr, *_ = _run_plan(ids)
        say(f"[plan] T={T}: id decreases at {where}: status {hdr[0]}")
        assert hdr[0] & STATUS_SEG_BIT and hdr[1] == 0 and hdr[2] == 0
