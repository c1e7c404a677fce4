"""hspec_draft_layer_noalloc (the layer on the library's static scratch, for
callers that cannot allocate) against hspec_draft_layer (a caller-provided
workspace): bit-identical outputs on two calls in a row, the second with a
smaller input, and a call whose workspace would exceed the static scratch is
refused before anything is launched."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from hybrid_mamba_attention_amd import ops
from hybrid_mamba_attention_amd import workloads as wl

from helpers import flush, layer_from_inputs

pytestmark = pytest.mark.gpu

OUTS = ("h0", "y", "h_final", "out")


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _compare_entry_points(w, kv_split_pages=0):
    inp = wl.make_inputs(w)
    layer = layer_from_inputs(inp, kv_split_pages=kv_split_pages)   # hspec_draft_layer
    ref = {k: getattr(layer, k).clone() for k in OUTS}
    for k in OUTS:
        getattr(layer, k).fill_(float("nan"))
    layer.noalloc()
    torch.cuda.synchronize()
    for k in OUTS:
        assert torch.equal(_bits(getattr(layer, k)), _bits(ref[k])), f"{w.name}: {k} differs"
    C = w.C
    return int(layer.plan()[4 + 2 * C:4 + 3 * C].max())   # most pieces of one request


def test_noalloc_matches_the_workspace_entry_point_twice():
    """A ragged case whose requests take several splits (partials and the
    merge in the scratch), then a smaller one: the second call runs on what
    the first left in the scratch and must not be disturbed by it."""
    big = replace(wl.sweep_workload(4), name="noalloc-big", ctx=("uniform", 3000, 8192), seed=9001)
    small = replace(wl.sweep_workload(2), name="noalloc-small", ctx=("uniform", 1, 600), seed=9002)
    flush("[noalloc] big call")
    pieces = _compare_entry_points(big)
    assert pieces > 1, "the first call must cut requests into pieces (partials in the scratch)"
    flush("[noalloc] smaller call")
    _compare_entry_points(small)


def test_noalloc_refuses_more_than_the_scratch():
    """One-page ranges of 8192-token contexts need ~0.28 GB of partial slots."""
    w = replace(wl.sweep_workload(4), name="noalloc-too-big", seed=9003)
    inp = wl.make_inputs(w, parts=("attn", "mamba"))
    layer = layer_from_inputs(inp, kv_split_pages=1)
    assert layer.workspace.numel() > 128 << 20
    out_before = layer.out.clone()
    with pytest.raises(ops.HspecError) as e:
        layer.noalloc()
    assert e.value.code == -5
    torch.cuda.synchronize()
    assert torch.equal(_bits(layer.out), _bits(out_before)), "a refused call must launch nothing"
