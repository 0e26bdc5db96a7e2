"""The grouped call without a workspace (mxq_group_rht_quant_nvfp4_noalloc), through
the C ABI: two calls in a row, the second on a smaller input, each equal byte for
byte to the workspace call on the same input (which the other tests hold against
the oracle)."""
import pytest
import torch

import nvfp4_quantization_amd as mxq
from nvfp4_quantization_amd import synth
from tests.gpu_util import announce, assert_same, device, host

pytestmark = pytest.mark.gpu

NAMES = ("row_global", "row_scales", "row_codes", "col_global", "col_scales", "col_codes", "fp8_scales", "fp8_codes")


def _both(x, sections, mask, flags, seed=None, ro=None, co=None):
    want = mxq.mxq_group_rht_quant_nvfp4(x, sections, mask, flags, seed, ro, co)
    out = mxq.alloc_nvfp4_outputs(x.shape[0], x.shape[1], len(sections), flags, x.device)
    for name in NAMES:                                  # poison: every byte must be written
        t = getattr(out, name)
        if t is not None:
            t.view(torch.uint8).fill_(0xA5)
    got = mxq.mxq_group_rht_quant_nvfp4_noalloc(x, sections, mask, flags, seed, ro, co, out=out)
    torch.cuda.synchronize()
    for name in NAMES:
        g = getattr(got, name)
        if g is not None:
            assert_same(name, host(g), host(getattr(want, name)))


@pytest.mark.parametrize("first,second", [
    # (rows, k, parts, empties, flags, sr) of the first and the smaller second call
    ((4096, 2048, 9, 2, 7, True), (1024, 512, 3, 1, 3, False)),      # SR + FP8, then RNE row + col
    ((2048, 1024, 5, 1, 3, False), (512, 384, 2, 0, 7, True)),       # single-read form, then k / 128 odd
])
def test_noalloc_matches_workspace_call(first, second):
    dev = device()
    for i, (rows, k, parts, empties, flags, sr) in enumerate((first, second)):
        announce(f"noalloc call {i}: {rows}x{k} parts={parts} flags={flags} sr={sr}")
        w = synth.grouped_nvfp4_sr(total_rows=rows, k=k, parts=parts, forced_empty=empties, seed=60 + i)
        p = w.params
        seed, ro, co = (p["seed"], p["row_offsets"], p["col_offsets"]) if sr else (None, None, None)
        _both(w.tensors["x"].to(dev), p["split_sections"], p["sign_mask"], flags, seed, ro, co)
