"""a0: the integer work plan of the in-place block attention (oracle side).

H-Spec's attention modules read every request's target KV in place (Abstract;
review page, "Key claims under review": concurrent serving at C = 8-128, with
ragged contexts).  The pages give no work decomposition; the reading here
spreads the whole batch's keys evenly over a fixed number of work ranges, so
that long and short requests cost the same wall time:

  * Request b's key sequence is its context, in slabs of 16 tokens
    (n_b = ceil(ctx_b / 16)), followed by its K block keys (nbk =
    ceil(K / 16) slabs): L_b = n_b + nbk slabs.
  * Slabs are grouped into granules of g = max(2, P/16) slabs (P = tokens per
    page), counted from each request's start, so every granule boundary
    starts a page and an even slab.  Request b holds G_b = ceil(L_b / g)
    granules; the batch holds T = sum_b G_b, request b starting at granule
    S_b = sum_{b' < b} G_b' of the concatenation.
  * Automatic ranges also charge every request a fixed cost of sigma =
    ceil(12 / g) virtual granules (12 slabs' worth) placed before its keys:
    the work a request costs its range however short it is (its query rows
    and page-table window, the first stages' round trip, the partial last
    page and the block's own slabs on the general path, the output store).
    With more than 64 query rows per kv head (rows = (Hq / Hkv) * K) that
    work is twice as large and the charge is ceil(24 / g).
    Request b then spans V_b = sigma + G_b units of the concatenation and its
    keys start at unit S_b = sum_{b' < b} V_b' + sigma; T = sum_b V_b.  Fixed
    ranges take sigma = 0 (V_b = G_b, S_b the plain prefix sum).
  * The concatenation is cut into W ranges, range w holding units
    [B_w, B_{w+1}):
      - automatic (range_pages = 0): W = min(w_max, max(1, floor(T / r_min))),
        r_min = ceil(16 / g) granules (every range holds >= 16 slabs' worth
        when the batch has them), and B_w = floor(w * T / W): ranges of
        nearly equal cost;
      - fixed (range_pages > 0): ranges of exactly R = max(1,
        ceil(range_pages * (P/16) / g)) granules, the last one shorter:
        W = ceil(T / R), B_w = min(w * R, T).
    In both cases W <= T, so no range is empty (a range may still hold only
    the fixed cost of a request, and then no keys).
  * Request b's pieces are the ranges its keys overlap: w_first_b (the range
    holding unit S_b) through the range holding unit S_b + G_b - 1.
    A request inside one range (one piece) is finished by that range; the
    pieces of a longer request are merged by log-sum-exp (E5).
  * A piece's partial result goes to slot 2*w + k of its range w: k = 0 for
    the segment that starts at the range's first granule, k = 1 for a segment
    that starts later in the range (which, when it is a piece, must run to
    the range's end).  Piece i of request b therefore sits in slot
    2*(w_first_b + i) + (1 if i == 0 and B_{w_first_b} < S_b else 0).

The plan is one int32 array, laid out as the library writes it at the start
of its attention workspace (so the two can be compared bit for bit):

    [0] W     [1] g     [2] C     [3] w_max
    [4 : 4+C]            S_b        (unit of request b's first key granule)
    [4+C : 4+2C]         w_first_b  (range holding request b's first granule)
    [4+2C : 4+3C]        pieces_b   (ranges request b overlaps)
    [4+3C : 4+3C+w_max+1]  B_w for w = 0..W (B_W = T), then -1 up to the capacity

w_max (the capacity) is the caller's bound on W: the library sizes its grid
and workspace by it.
"""
import numpy as np

SLAB = 16
SEG_SLABS = 12   # a request's fixed cost in automatic ranges, in slabs
SEG_SLABS_TWO_TILES = 24   # the same with more than 64 query rows per kv head


def granule_slabs(page_size: int) -> int:
    if page_size < SLAB or page_size % SLAB or (page_size // SLAB) & (page_size // SLAB - 1):
        raise ValueError("page size must be 16 tokens times a power of two")
    return max(2, page_size // SLAB)


def request_granules(ctx_lens, K: int, page_size: int = 16) -> np.ndarray:
    """G_b: granules of request b's key sequence (context slabs, then block slabs)."""
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    if (ctx < 0).any():
        raise ValueError("negative context length")
    if K < 1:
        raise ValueError("the draft block holds at least one key")
    g = granule_slabs(page_size)
    L = (ctx + SLAB - 1) // SLAB + (K + SLAB - 1) // SLAB
    return (L + g - 1) // g


def segment_granules(page_size: int = 16, range_pages: int = 0, rows: int = 64) -> int:
    """sigma: a request's fixed cost in units (0 for fixed ranges); rows =
    query rows per kv head, (Hq / Hkv) * K."""
    if range_pages:
        return 0
    slabs = SEG_SLABS_TWO_TILES if rows > 64 else SEG_SLABS
    return -(-slabs // granule_slabs(page_size))


def range_count(T: int, *, w_max: int, page_size: int = 16, range_pages: int = 0) -> int:
    g = granule_slabs(page_size)
    if range_pages < 0 or w_max < 1:
        raise ValueError("range_pages >= 0 and w_max >= 1")
    if range_pages == 0:
        r_min = -(-SLAB // g)
        return int(min(w_max, max(1, T // r_min)))
    R = max(1, -(-(range_pages * (page_size // SLAB)) // g))
    W = -(-T // R)
    if W > w_max:
        raise ValueError("fixed ranges exceed the capacity w_max")
    return int(W)


def plan_len(C: int, w_max: int) -> int:
    return 4 + 3 * int(C) + int(w_max) + 1


def range_plan(ctx_lens, *, K: int, w_max: int, page_size: int = 16, range_pages: int = 0,
               rows: int = 64) -> np.ndarray:
    """The int32 plan laid out as in the module docstring (rows = query rows
    per kv head, which sets the fixed cost of automatic ranges)."""
    G = request_granules(ctx_lens, K, page_size)
    C = len(G)
    if C < 1:
        raise ValueError("at least one request")
    sigma = segment_granules(page_size, range_pages, rows)
    T = int((G + sigma).sum())
    W = range_count(T, w_max=w_max, page_size=page_size, range_pages=range_pages)
    assert 1 <= W <= T
    if range_pages == 0:
        B = [w * T // W for w in range(W + 1)]
    else:
        R = max(1, -(-(range_pages * (page_size // SLAB)) // granule_slabs(page_size)))
        B = [min(w * R, T) for w in range(W + 1)]
    S = np.cumsum(G + sigma) - G   # each request's keys start after its fixed cost
    w_first = np.zeros(C, np.int64)
    pieces = np.zeros(C, np.int64)
    for b in range(C):
        first, last = int(S[b]), int(S[b] + G[b] - 1)
        wf = max(w for w in range(W) if B[w] <= first)
        wl = max(w for w in range(W) if B[w] <= last)
        w_first[b], pieces[b] = wf, wl - wf + 1
    bounds = np.full(w_max + 1, -1, np.int64)
    bounds[:W + 1] = B
    out = np.concatenate([[W, granule_slabs(page_size), C, w_max], S, w_first, pieces, bounds])
    return out.astype(np.int32)


def unpack(plan, C: int) -> dict:
    """The fields of a plan array (by name)."""
    p = np.asarray(plan, np.int64)
    W = int(p[0])
    B = p[4 + 3 * C:4 + 3 * C + W + 1]
    return dict(W=W, g=int(p[1]), C=int(p[2]), w_max=int(p[3]), T=int(B[-1]), S=p[4:4 + C],
                w_first=p[4 + C:4 + 2 * C], pieces=p[4 + 2 * C:4 + 3 * C], B=B)


def request_pieces(plan, C: int, b: int, L_b: int):
    """Request b's pieces as (range w, slot, first slab, end slab) of its key
    sequence (L_b slabs), in order."""
    f = unpack(plan, C)
    g, S, B = f["g"], int(f["S"][b]), f["B"]
    out = []
    for i in range(int(f["pieces"][b])):
        w = int(f["w_first"][b]) + i
        lo = max(int(B[w]) - S, 0) * g
        hi = min((int(B[w + 1]) - S) * g, L_b)
        k = 1 if (i == 0 and int(B[w]) < S) else 0
        out.append((w, 2 * w + k, lo, hi))
    return out
