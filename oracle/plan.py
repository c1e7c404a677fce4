"""a0: the integer split plan for split-KV attention (oracle side).

The target context of request b spans n_b = ceil(ctx_b / 16) pages.  Its
pages are cut into splits of a fixed number of pages `pps`; the draft block's
own K keys belong to the last split.  A request with no context still has one
split (block keys only):

    n_splits_b = max(1, ceil(n_b / pps))

Work items are the (request, split) pairs, request-major.  The plan is laid
out as one int32 array (the same layout the library writes at the start of
its attention workspace, so the two can be compared bit for bit):

    [0] total items      [1] pps      [2] C      [3] capacity M
    [4 : 4+C]            n_splits_b
    [4+C : 4+2C]         index of request b's first item (exclusive prefix sum)
    [4+2C : 4+2C+M]      request of item i, or -1 for i >= total
    [4+2C+M : 4+2C+2M]   split of item i,   or -1 for i >= total

Capacity M = C * max(1, ceil(ceil(max_ctx / 16) / pps)), where max_ctx is the
caller's upper bound on the context lengths.
"""
import numpy as np

PAGE = 16


def max_items_for(C: int, max_ctx: int, pps: int) -> int:
    max_pages = -(-int(max_ctx) // PAGE)
    return int(C) * max(1, -(-max_pages // int(pps)))


def plan_len(C: int, max_items: int) -> int:
    return 4 + 2 * int(C) + 2 * int(max_items)


def split_plan(ctx_lens, pps: int, max_ctx: int | None = None) -> np.ndarray:
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    if pps <= 0:
        raise ValueError("pages per split must be positive")
    if max_ctx is None:
        max_ctx = int(ctx.max()) if len(ctx) else 0
    if len(ctx) and int(ctx.max()) > max_ctx:
        raise ValueError("a context length exceeds max_ctx")
    if (ctx < 0).any():
        raise ValueError("negative context length")
    C = len(ctx)
    M = max_items_for(C, max_ctx, pps)
    n_pages = (ctx + PAGE - 1) // PAGE
    n_splits = np.maximum(1, (n_pages + pps - 1) // pps)
    first = np.concatenate([[0], np.cumsum(n_splits)[:-1]]) if C else np.zeros(0, np.int64)
    total = int(n_splits.sum())
    item_req = np.full(M, -1, dtype=np.int64)
    item_split = np.full(M, -1, dtype=np.int64)
    i = 0
    for b in range(C):
        for s in range(int(n_splits[b])):
            item_req[i] = b
            item_split[i] = s
            i += 1
    assert i == total <= M
    out = np.concatenate([[total, pps, C, M], n_splits, first, item_req, item_split])
    return out.astype(np.int32)
