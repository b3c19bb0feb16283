"""Reference work-map builder (oracle; test infrastructure only).

What the method does before every inference step, as the pages describe it
([P3] §3.1 "方案", steps 1-5; [P4] §二.1; [P1] §3.1):

1. cut every request's KV range into tiles of one uniform size;
2. concatenate all requests' tiles into one task stream;
3. give every worker (a CTA on the pages' GPU, a workgroup here) the same, or
   nearly the same, budget of tiles from the global tile count;
4. fill each worker greedily from the stream up to its budget, so that a long
   request may span several workers; the resulting task map is built once per
   step and read by the attention kernel of every layer;
5. (kernel side) each split writes a partial result and a combine merges them.

The budget arithmetic is the one in [P2] §二.1 ``dynamic_tile_scheduler``:
``base = total // workers`` and the first ``total % workers`` workers get one
extra tile.  [P3]'s worked example: lengths 1024, 5120 and 2048 with 512-token
tiles give 2, 10 and 4 tiles, and 4 workers receive 4 tiles each.

Readings where the pages are silent:

* tile count is a ceiling (a partial last tile is still a tile; a floor, as in
  [P2]'s pseudocode, would drop tokens and make attention wrong);
* the task stream is in batch order, tiles in ascending KV order;
* "greedy bin-packing" is a contiguous fill: worker w takes the next budget_w
  tiles of the stream ([P3]'s "long request spans CTAs" and "4 tiles each"
  hold under it);
* consecutive tiles of one request inside one worker form one split
  ("segment"), which owns one partial slot;
* every tile costs one budget unit, a partial last tile included.

Work-map layout (int32 words, one flat buffer; the GPU planner must produce
exactly these words)::

    [0] version (=1)     [1] B (requests)   [2] W (workers)   [3] kv_tile
    [4] S (segments)     [5] T (tiles)      [6] q_tile (1 for decode)
    [7] U (query units)
    worker_ptr[W + 1]               segments of worker w: [worker_ptr[w], worker_ptr[w+1])
    unit_ptr[U + 1]                 segments of unit u:   [unit_ptr[u],  unit_ptr[u+1])
    unit[U][2]   = (b, q_tile_index)
    seg[S][4]    = (b, q_tile_index, kv_begin, kv_end)   (KV token range, end exclusive)

A decode unit is one request (q_tile_index 0).  A prefill unit is one
q_tile-row block of one request's query chunk.

Version 2 (the LPT comparison planner below): a worker's segments need not be
contiguous in unit-major order, so the segments stay unit-major (segment i owns
partial slot i) and an extra ``order[S]`` follows ``seg``: worker w runs the
segments ``order[worker_ptr[w] .. worker_ptr[w+1])``.

Version 3 (the rate-proportional planner below): the words of version 1; the
version only tells the split-KV launch to run worker w's list for every head
group on workgroups b with b mod W = w (list-major order), so that a list's
workgroups share one placement on the device.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np

MAP_VERSION = 1
MAP_VERSION_ORDERED = 2   # version 1 plus order[S]: the segments each worker runs, by slot index
MAP_VERSION_PLACED = 3    # version 1's words, list-major workgroup order in the split-KV launch
RATE_MAX = 1 << 20        # largest per-worker rate the rate-proportional planner accepts
HEADER_WORDS = 8


@dataclass
class Unit:
    b: int            # request index
    qt: int           # q-tile index inside the request (0 for decode)
    extent: int       # number of KV tokens this unit attends to (its KV range is [0, extent))


@dataclass
class Segment:
    b: int
    qt: int
    kv_begin: int
    kv_end: int


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def tiles_of(extent: int, tile: int) -> int:
    """Step 1, tile cut: number of uniform tiles covering ``extent`` tokens (ceiling)."""
    return ceil_div(extent, tile) if extent > 0 else 0


def budgets(total_tiles: int, workers: int) -> List[int]:
    """Step 3, equal budgets: ``base = T // W``; the first ``T % W`` workers get one more."""
    base, rem = divmod(total_tiles, workers)
    return [base + (1 if w < rem else 0) for w in range(workers)]


def _check_common(num_workers: int, tile: int) -> None:
    if num_workers < 1:
        raise ValueError("num_workers must be >= 1")
    if tile < 1:
        raise ValueError("tile must be >= 1")


def _greedy_fill(units: Sequence[Unit], num_workers: int, tile: int) -> Tuple[List[List[Segment]], int]:
    """Steps 2-4: one stream of (unit, tile) in unit order; contiguous fill per worker budget."""
    # step 2: the task stream, unit (batch) order, ascending tile index inside a unit
    stream = []
    for ui, u in enumerate(units):
        for t in range(tiles_of(u.extent, tile)):
            stream.append((ui, t))
    total = len(stream)
    # step 3
    budget = budgets(total, num_workers)
    # step 4: worker w takes the next budget[w] tiles; runs of one unit become one segment
    lists: List[List[Segment]] = []
    cursor = 0
    for w in range(num_workers):
        taken = stream[cursor:cursor + budget[w]]
        cursor += budget[w]
        lists.append(_runs(units, taken, tile))
    assert cursor == total
    return lists, total


def _runs(units: Sequence[Unit], taken: Sequence[Tuple[int, int]], tile: int) -> List[Segment]:
    """A worker's consecutive stretch of the stream, (unit, tile) pairs in stream order, as segments:
    each maximal run of one unit's tiles is one segment."""
    segs: List[Segment] = []
    run_start = 0
    for i in range(1, len(taken) + 1):
        if i == len(taken) or taken[i][0] != taken[run_start][0]:
            ui, t_first = taken[run_start]
            t_last = taken[i - 1][1]
            u = units[ui]
            segs.append(Segment(u.b, u.qt, t_first * tile, min(u.extent, (t_last + 1) * tile)))
            run_start = i
    return segs


def _serialise(B: int, units: Sequence[Unit], lists: Sequence[Sequence[Segment]],
               kv_tile: int, q_tile: int, total_tiles: int, version: int = MAP_VERSION) -> np.ndarray:
    W = len(lists)
    U = len(units)
    segs = [s for lst in lists for s in lst]
    S = len(segs)
    worker_ptr = [0]
    for lst in lists:
        worker_ptr.append(worker_ptr[-1] + len(lst))
    # segments are in stream order, which is unit-major, so each unit's segments are contiguous
    unit_index = {(u.b, u.qt): i for i, u in enumerate(units)}
    counts = [0] * U
    last = -1
    for s in segs:
        ui = unit_index[(s.b, s.qt)]
        if ui < last:
            raise AssertionError("segments are not unit-major")
        last = ui
        counts[ui] += 1
    unit_ptr = [0]
    for c in counts:
        unit_ptr.append(unit_ptr[-1] + c)
    words = [version, B, W, kv_tile, S, total_tiles, q_tile, U]
    words += worker_ptr
    words += unit_ptr
    for u in units:
        words += [u.b, u.qt]
    for s in segs:
        words += [s.b, s.qt, s.kv_begin, s.kv_end]
    return np.asarray(words, dtype=np.int32)


def decode_units(seq_lens: Sequence[int]) -> List[Unit]:
    """Decode: one unit per request; a single query token at position L_b - 1 sees keys [0, L_b)."""
    for L in seq_lens:
        if L < 0:
            raise ValueError("negative sequence length")
    return [Unit(b, 0, int(L)) for b, L in enumerate(seq_lens)]


def ref_plan(seq_lens: Sequence[int], num_workers: int, tile: int) -> np.ndarray:
    """Dynamic (load-balanced) decode work map, [P3] §3.1 方案 steps 1-4, [P2] budget formula."""
    _check_common(num_workers, tile)
    units = decode_units(seq_lens)
    lists, total = _greedy_fill(units, num_workers, tile)
    return _serialise(len(seq_lens), units, lists, tile, 1, total)


def ref_plan_static(seq_lens: Sequence[int], num_splits: int, tile: int) -> np.ndarray:
    """Static split-KV baseline ([P3] §3.1 问题; [P4] §二.1): one fixed split count for the batch.

    Request b is cut into k_b = min(num_splits, n_b) tile-aligned chunks whose tile counts
    differ by at most one (the larger chunks first); every chunk is a worker of its own with one
    segment, so the worker count is sum(k_b) and depends on the batch.
    """
    if num_splits < 1:
        raise ValueError("num_splits must be >= 1")
    _check_common(1, tile)
    units = decode_units(seq_lens)
    lists: List[List[Segment]] = []
    total = 0
    for u in units:
        n = tiles_of(u.extent, tile)
        total += n
        k = min(num_splits, n)
        if k == 0:
            continue
        small, big_count = divmod(n, k)
        t0 = 0
        for c in range(k):
            size = small + (1 if c < big_count else 0)
            lists.append([Segment(u.b, 0, t0 * tile, min(u.extent, (t0 + size) * tile))])
            t0 += size
        assert t0 == n
    return _serialise(len(seq_lens), units, lists, tile, 1, total)


def prefill_units(q_lens: Sequence[int], kv_lens: Sequence[int], q_tile: int, causal: bool) -> List[Unit]:
    """Chunked prefill over a cached prefix: units are q_tile-row blocks of each request's chunk.

    Query row j of request b sits at absolute position kv_len_b - q_len_b + j (the chunk is the
    last q_len_b tokens of the context); under the causal mask it sees keys [0, that position].
    A unit's KV extent is therefore set by its last row.
    """
    if len(q_lens) != len(kv_lens):
        raise ValueError("q_lens and kv_lens differ in length")
    if q_tile < 1:
        raise ValueError("q_tile must be >= 1")
    units = []
    for b, (ql, kl) in enumerate(zip(q_lens, kv_lens)):
        if ql < 0 or kl < 0 or ql > kl:
            raise ValueError("need 0 <= q_len <= kv_len")
        for i in range(tiles_of(ql, q_tile)):
            if causal:
                extent = kl - ql + min(ql, (i + 1) * q_tile)
            else:
                extent = kl
            units.append(Unit(b, i, extent))
    return units


def ref_plan_prefill(q_lens: Sequence[int], kv_lens: Sequence[int], num_workers: int,
                     q_tile: int, kv_tile: int, causal: bool) -> np.ndarray:
    """Same greedy equal-budget fill, over (request, q-tile) units instead of requests."""
    _check_common(num_workers, kv_tile)
    units = prefill_units(q_lens, kv_lens, q_tile, causal)
    lists, total = _greedy_fill(units, num_workers, kv_tile)
    return _serialise(len(q_lens), units, lists, kv_tile, q_tile, total)


def ref_plan_lpt(seq_lens: Sequence[int], num_workers: int, tile: int) -> np.ndarray:
    """LPT bucket packing, the assignment of [P5] "大模型推理性能优化揭秘" §五(一): every request is
    cut into tiles, the tiles are taken in decreasing size, and each goes to the worker with the
    smallest load so far; a tile's size (and a worker's load) is counted in KV tokens.

    Readings: equal sizes keep stream order (batch order, ascending tile); equal loads go to the
    lowest worker index; inside a worker the tiles are run in stream order and consecutive tiles of
    one request merge into one segment.  Serialised as a version-2 map (see the module header).
    """
    _check_common(num_workers, tile)
    units = decode_units(seq_lens)
    pieces = []                                   # (size, unit index, tile index)
    for ui, u in enumerate(units):
        for t in range(tiles_of(u.extent, tile)):
            pieces.append((min(tile, u.extent - t * tile), ui, t))
    total = len(pieces)
    pieces.sort(key=lambda x: (-x[0], x[1], x[2]))
    load = [0] * num_workers
    mine: List[List[Tuple[int, int]]] = [[] for _ in range(num_workers)]
    for size, ui, t in pieces:
        w = min(range(num_workers), key=lambda i: (load[i], i))
        load[w] += size
        mine[w].append((ui, t))
    # per worker: runs of consecutive tiles of one unit, in stream order
    runs: List[List[Tuple[int, int, int]]] = []   # (unit index, first tile, last tile)
    for w in range(num_workers):
        got = sorted(mine[w])
        lst: List[Tuple[int, int, int]] = []
        for ui, t in got:
            if lst and lst[-1][0] == ui and lst[-1][2] == t - 1:
                lst[-1] = (ui, lst[-1][1], t)
            else:
                lst.append((ui, t, t))
        runs.append(lst)
    # slots: all segments in unit-major order (by unit, then KV start)
    all_runs = sorted({r for lst in runs for r in lst})
    slot = {r: i for i, r in enumerate(all_runs)}
    segs = []
    for ui, t0, t1 in all_runs:
        u = units[ui]
        segs.append(Segment(u.b, u.qt, t0 * tile, min(u.extent, (t1 + 1) * tile)))
    counts = [0] * len(units)
    for ui, _, _ in all_runs:
        counts[ui] += 1
    unit_ptr = [0]
    for c in counts:
        unit_ptr.append(unit_ptr[-1] + c)
    worker_ptr = [0]
    order = []
    for lst in runs:
        order += [slot[r] for r in lst]
        worker_ptr.append(len(order))
    S = len(segs)
    words = [MAP_VERSION_ORDERED, len(seq_lens), num_workers, tile, S, total, 1, len(units)]
    words += worker_ptr + unit_ptr
    for u in units:
        words += [u.b, u.qt]
    for sg in segs:
        words += [sg.b, sg.qt, sg.kv_begin, sg.kv_end]
    words += order
    return np.asarray(words, dtype=np.int32)


def ref_plan_weighted(seq_lens: Sequence[int], num_workers: int, tile: int, split_cost: int) -> np.ndarray:
    """Cost-weighted contiguous fill: steps 1, 2 and 4 as in ``ref_plan``, with step 3's equal
    budgets counted in cost instead of tiles.  A variant of the pages' scheduler ([P3] §3.1 方案
    steps 3-4 count uniform tiles; [P5] §五(一) counts a tile's size in tokens) for comparison.

    Readings: a tile costs its KV tokens (a partial last tile costs less than a full one), and the
    first tile of a request costs ``split_cost`` more — every request opens at least one split
    (query load, pipeline start, a partial to write and combine); the splits a worker boundary adds
    fall one per boundary whatever the placement, so they are not charged.  With C the total cost and
    P_i the cost of the stream before tile i, tile i goes to worker
        floor(W (2 P_i + c_i) / (2 C))
    — the worker whose equal share [w C / W, (w + 1) C / W) of the cost holds the tile's midpoint —
    which keeps every worker's stretch of the stream contiguous and its cost within one tile's cost
    of C / W.  Serialised as a version-1 map, so the decode and combine kernels take it unchanged.
    """
    _check_common(num_workers, tile)
    if split_cost < 0:
        raise ValueError("split_cost must be >= 0")
    units = decode_units(seq_lens)
    stream = []                                   # (unit index, tile index, cost)
    for ui, u in enumerate(units):
        for t in range(tiles_of(u.extent, tile)):
            stream.append((ui, t, min(tile, u.extent - t * tile) + (split_cost if t == 0 else 0)))
    total_cost = sum(c for _, _, c in stream)
    mine: List[List[Tuple[int, int]]] = [[] for _ in range(num_workers)]
    before = 0
    for ui, t, c in stream:
        w = (num_workers * (2 * before + c)) // (2 * total_cost)
        mine[w].append((ui, t))
        before += c
    lists = [_runs(units, taken, tile) for taken in mine]
    return _serialise(len(seq_lens), units, lists, tile, 1, len(stream))


def ref_plan_rated(seq_lens: Sequence[int], num_workers: int, tile: int, split_cost: int,
                   rates: Sequence[int]) -> np.ndarray:
    """Rate-proportional contiguous fill: ``ref_plan_weighted`` with worker w's share of the cost
    line proportional to ``rates[w]`` instead of equal.  The pages' scheduler gives every worker the
    same budget ([P3] §3.1 方案 step 3), which balances finish times when every worker streams at
    the same rate; here the workers' rates may differ (on the device they depend on where a
    worker's workgroups run), and the aim, equal finish times, is kept by giving each worker the cost
    it can stream in the same time.

    With R_w = rates[0] + ... + rates[w - 1] and R = R_W, worker w's share of the cost line is
    [C R_w / R, C R_(w+1) / R).  Tile i (cost c_i, P_i the cost before it; costs as in
    ``ref_plan_weighted``: KV tokens, plus ``split_cost`` on a request's first tile) goes to the
    worker whose share holds its midpoint P_i + c_i / 2: the last worker w with
    C R_w / R <= P_i + c_i / 2, i.e. 2 C R_w <= R (2 P_i + c_i) in integers.  A worker of rate 0
    holds an empty share and gets nothing.  With equal rates the rule is ``ref_plan_weighted``'s
    floor(W (2 P_i + c_i) / (2 C)).  Every worker's stretch of the stream stays contiguous and its
    cost within one tile's cost of C rates[w] / R.  Serialised as a version-3 map.
    """
    _check_common(num_workers, tile)
    if split_cost < 0:
        raise ValueError("split_cost must be >= 0")
    rates = [int(r) for r in rates]
    if len(rates) != num_workers or any(r < 0 or r > RATE_MAX for r in rates) or sum(rates) == 0:
        raise ValueError(f"need num_workers rates in [0, {RATE_MAX}], not all zero")
    units = decode_units(seq_lens)
    tiles = []                                    # (unit index, tile index, cost)
    for ui, u in enumerate(units):
        for t in range(tiles_of(u.extent, tile)):
            tokens = min(tile, u.extent - t * tile)
            tiles.append((ui, t, tokens + split_cost * (t == 0)))
    C = sum(c for _, _, c in tiles)
    R = sum(rates)
    share_start = [0]                             # R_w for w = 0 .. W
    for r in rates:
        share_start.append(share_start[-1] + r)
    mine: List[List[Tuple[int, int]]] = [[] for _ in range(num_workers)]
    P = 0
    for ui, t, c in tiles:
        w = max(v for v in range(num_workers) if 2 * C * share_start[v] <= R * (2 * P + c))
        mine[w].append((ui, t))
        P += c
    lists = [_runs(units, taken, tile) for taken in mine]
    return _serialise(len(seq_lens), units, lists, tile, 1, len(tiles), version=MAP_VERSION_PLACED)


# ----------------------------------------------------------------------------------------------
# Reading a map back (used by tests and by the attention oracle's split helpers)

@dataclass
class WorkMap:
    version: int
    B: int
    W: int
    kv_tile: int
    S: int
    T: int
    q_tile: int
    U: int
    worker_ptr: np.ndarray
    unit_ptr: np.ndarray
    units: np.ndarray      # [U, 2]
    segs: np.ndarray       # [S, 4]
    order: np.ndarray = None   # version 2: slot indices, worker-major

    def worker_slots(self, w: int) -> np.ndarray:
        idx = np.arange(self.worker_ptr[w], self.worker_ptr[w + 1])
        return idx if self.order is None else self.order[idx]

    def worker_segments(self, w: int) -> np.ndarray:
        return self.segs[self.worker_slots(w)]

    def unit_segments(self, u: int) -> np.ndarray:
        return self.segs[self.unit_ptr[u]:self.unit_ptr[u + 1]]


def parse_map(words: np.ndarray) -> WorkMap:
    words = np.asarray(words, dtype=np.int64)
    version, B, W, kv_tile, S, T, q_tile, U = (int(x) for x in words[:HEADER_WORDS])
    o = HEADER_WORDS
    worker_ptr = words[o:o + W + 1]; o += W + 1
    unit_ptr = words[o:o + U + 1]; o += U + 1
    units = words[o:o + 2 * U].reshape(U, 2); o += 2 * U
    segs = words[o:o + 4 * S].reshape(S, 4); o += 4 * S
    order = None
    if version == MAP_VERSION_ORDERED:
        order = words[o:o + S]; o += S
    elif version not in (MAP_VERSION, MAP_VERSION_PLACED):
        raise ValueError(f"unknown map version {version}")
    if o != len(words):
        raise ValueError(f"map has {len(words)} words, layout implies {o}")
    return WorkMap(version, B, W, kv_tile, S, T, q_tile, U, worker_ptr, unit_ptr, units, segs, order)


def map_words(num_units: int, num_workers: int, num_segments: int) -> int:
    """Exact word count of a map with the given counts."""
    return HEADER_WORDS + (num_workers + 1) + (num_units + 1) + 2 * num_units + 4 * num_segments
