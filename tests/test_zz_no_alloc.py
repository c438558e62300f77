"""kda_prefill_noalloc (the prefill for callers that cannot allocate: its
workspace is the library's fixed device scratch) against kda_prefill,
through the C ABI.

Two calls in a row, the second with smaller sizes, so that it runs over what
the first left in the scratch.  The first is one long sequence that the
automatic rule splits into segments, so the segment transitions and incoming
states live in the scratch as well.  Both must equal kda_prefill on the same
inputs bit for bit (the same kernels run) and meet the oracle's bars."""
import pytest
import torch

import gated_delta_rule_21_amd as kda
from gated_delta_rule_21_amd import workloads as W
from gpu_util import compare_prefill, oracle_prefill, to_gpu

pytestmark = pytest.mark.gpu


def noalloc(g, io):
    T, H, d = g["q"].shape
    N = g["cu_seqlens"].numel() - 1
    o = torch.empty((T, H, d), dtype=g["q"].dtype, device="cuda")
    hT = torch.empty((N, H, d, d), dtype=torch.float32, device="cuda")
    code = kda.KDA_F32 if io == "f32" else kda.KDA_BF16
    st = kda.kda_prefill_noalloc(code, g["q"].data_ptr(), g["k"].data_ptr(), g["v"].data_ptr(),
                                 g["z"].data_ptr(), g["A"].data_ptr(), g["beta"].data_ptr(), g["h0"].data_ptr(),
                                 g["cu_seqlens"].data_ptr(), N, T, H, d, d, o.data_ptr(), hT.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
    assert st == 0, kda.kda_status_string(st)
    return o, hT


@pytest.mark.parametrize("io,d", [("bf16", 128), ("f32", 64)])
def test_noalloc_matches_prefill_on_two_calls(io, d):
    big = W.random_prefill([8192], 2, d, io, h0_std=0.05, seed=900 + d)
    small = W.random_prefill([300, 0, 77], 3, d, io, h0_std=0.05, seed=901 + d)
    assert kda.kda_prefill_segments(1, 8192, 2, d, d, kda.KDA_BF16) > 1
    for inp in (big, small):
        assert kda.kda_prefill_workspace_size(inp["cu_seqlens"].numel() - 1, inp["q"].shape[0], inp["q"].shape[1],
                                              d, d, 0) <= kda.NOALLOC_SCRATCH_BYTES
    print("case noalloc %s d=%d" % (io, d), flush=True)
    gs = [to_gpu(big), to_gpu(small)]
    outs = [noalloc(g, io) for g in gs]          # the second call runs over the first's scratch contents
    torch.cuda.synchronize()
    for inp, g, (o, hT) in zip((big, small), gs, outs):
        o_ref, h_ref = kda.prefill(g["q"], g["k"], g["v"], g["z"], g["A"], g["beta"], g["cu_seqlens"], h0=g["h0"])
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(hT, h_ref)
        ro, rh = oracle_prefill(inp)
        compare_prefill(o, hT, ro, rh, inp["cu_seqlens"], io, label="noalloc %s d=%d" % (io, d))


def test_noalloc_refuses_sizes_beyond_the_scratch():
    g = to_gpu(W.random_prefill([64], 1, 128, "bf16", seed=902))
    o = torch.full((64, 1, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    # claim a K3-sized call: refused on the host, nothing launched, o untouched
    st = kda.kda_prefill_noalloc(kda.KDA_BF16, g["q"].data_ptr(), g["k"].data_ptr(), g["v"].data_ptr(),
                                 g["z"].data_ptr(), g["A"].data_ptr(), g["beta"].data_ptr(), None,
                                 g["cu_seqlens"].data_ptr(), 1, 65536, 96, 128, 128, o.data_ptr(), None,
                                 torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == -9
    assert bool((o == 7.0).all())
