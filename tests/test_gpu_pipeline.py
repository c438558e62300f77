"""The chunk-block pipeline of the bf16 prefill (kda_prefill_options.blocks).

The intra kernel of one run of chunks runs beside the inter kernel of the
run before it, and a sequence's state crosses run boundaries through the
workspace.  Every value is computed exactly as without the pipeline, so the
outputs must be bit-identical to blocks = 1, for sequences that start, end
or lie wholly inside a run, empty ones at any position (the last run takes
those past the end of the table), and hT aliasing h0; and they are compared
with the oracle by every measure of gpu_util.  Where the pipeline does not
apply (fp32 path) the option changes nothing; forced segments and forced
blocks together are rejected."""
import pytest
import torch

import gated_delta_rule_21_amd as kda
from gated_delta_rule_21_amd import workloads as W
from gpu_util import compare_prefill, oracle_prefill, to_gpu

pytestmark = pytest.mark.gpu

LENS = [700, 0, 1, 129, 64, 0, 333, 1500, 2, 0]


def run(g, blocks, segments=0, h0="same", hT=None):
    o, hT_ = kda.prefill(g["q"], g["k"], g["v"], g["z"], g["A"], g["beta"], g["cu_seqlens"],
                         h0=g["h0"] if h0 == "same" else h0, hT=hT, segments=segments, blocks=blocks)
    torch.cuda.synchronize()
    return o, hT_


@pytest.mark.parametrize("d,blocks,h0", [(128, 2, 0.05), (128, 3, None), (64, 5, 0.05), (32, 16, 0.05)])
def test_blocks_bit_identical_and_oracle(d, blocks, h0):
    print("case pipeline d=%d blocks=%d h0=%s" % (d, blocks, h0), flush=True)
    inp = W.random_prefill(LENS, 3, d, "bf16", h0_std=h0, seed=9000 + d + blocks)
    g = to_gpu(inp)
    o1, h1 = run(g, 1)
    ob, hb = run(g, blocks)
    assert torch.equal(ob, o1), "o differs from blocks = 1"
    assert torch.equal(hb, h1), "hT differs from blocks = 1"
    ro, rh = oracle_prefill(inp)
    compare_prefill(ob, hb, ro, rh, inp["cu_seqlens"], "bf16", label="blocks %d" % blocks)


@pytest.mark.parametrize("lens", [[0, 0, 0], [1], [5, 0, 64]])
def test_blocks_degenerate_batches(lens):
    """More runs than chunks, every sequence empty, one token: each run may
    hold no chunk at all; the outputs are still bit-identical to one run and
    an empty sequence's final state is its h0."""
    print("case pipeline degenerate lens=%s" % lens, flush=True)
    inp = W.random_prefill(lens, 2, 64, "bf16", h0_std=0.05, seed=9050 + len(lens) + sum(lens))
    g = to_gpu(inp)
    o1, h1 = run(g, 1)
    ob, hb = run(g, 16)
    assert torch.equal(ob, o1) and torch.equal(hb, h1)
    for n, L in enumerate(lens):
        if L == 0:
            assert torch.equal(hb[n], g["h0"][n])
    if sum(lens) > 0:
        ro, rh = oracle_prefill(inp)
        compare_prefill(ob, hb, ro, rh, inp["cu_seqlens"], "bf16", label="degenerate %s" % lens)


def test_blocks_chained_calls_equal_one_call():
    """A long sequence prefilled in two pipelined calls, cut at a chunk
    boundary and carried through hT -> h0, equals one call bit for bit: the
    chunks are the same, and so is every value computed on them."""
    print("case pipeline chained calls", flush=True)
    inp = W.random_prefill([64 * 40], 3, 128, "bf16", h0_std=0.05, seed=9300)
    g = to_gpu(inp)
    o1, h1 = run(g, 1)
    cut = 64 * 17
    parts = []
    for lo, hi, h0 in ((0, cut, g["h0"]), (cut, 64 * 40, None)):
        sub = {n: g[n][lo:hi].contiguous() for n in ("q", "k", "v", "z", "beta")}
        sub["A"] = g["A"]
        sub["cu_seqlens"] = W.cu_from_lengths([hi - lo]).cuda()
        sub["h0"] = h0 if h0 is not None else parts[-1][1]
        parts.append(run(sub, 3))
    assert torch.equal(torch.cat([parts[0][0], parts[1][0]]), o1)
    assert torch.equal(parts[1][1], h1)


def test_blocks_hT_may_alias_h0():
    print("case pipeline hT aliasing h0", flush=True)
    inp = W.random_prefill(LENS, 2, 128, "bf16", h0_std=0.05, seed=9100)
    g = to_gpu(inp)
    o1, h1 = run(g, 1)
    S = g["h0"].clone()
    ob, hb = run(g, 4, h0=S, hT=S)
    assert hb.data_ptr() == S.data_ptr()
    assert torch.equal(ob, o1) and torch.equal(S, h1)


def test_blocks_k3_shape_automatic():
    """The K3 shape pipelines by default; it matches blocks = 1 bit for bit."""
    print("case pipeline K3 automatic", flush=True)
    pre = W.make("k3_prefill", device="cuda")
    ws_auto = kda.kda_prefill_workspace_size(1, 65536, 96, 128, 128, kda.KDA_BF16)
    ws_off = kda.kda_prefill_ex_workspace_size(1, 65536, 96, 128, 128, kda.KDA_BF16, kda.options(blocks=1))
    assert ws_auto > ws_off          # the carried state: the automatic choice pipelines
    oa, ha = run(pre, 0)
    o1, h1 = run(pre, 1)
    assert torch.equal(oa, o1) and torch.equal(ha, h1)


def test_blocks_ignored_on_fp32_and_rejected_with_segments():
    print("case pipeline fp32 / segments", flush=True)
    inp = W.random_prefill([300, 77], 2, 64, "f32", h0_std=0.05, seed=9200)
    g = to_gpu(inp)
    o1, h1 = run(g, 1)
    o3, h3 = run(g, 3)
    assert torch.equal(o3, o1) and torch.equal(h3, h1)
    gb = to_gpu(W.random_prefill([300, 77], 2, 64, "bf16", seed=9201))
    with pytest.raises((kda.KdaError, ValueError)):
        run(gb, 3, segments=2)
