"""C-ABI checks that need no GPU: the library loads, exports every function
include/kda.h declares, sizes the workspace, and rejects bad arguments with
the documented status before touching the device."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_21_amd as kda

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "kda.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(["kda_build_info", "kda_decode", "kda_decode_fused", "kda_decode_window",
                                           "kda_prefill",
                                           "kda_prefill_ex", "kda_prefill_ex_workspace_size",
                                           "kda_prefill_noalloc", "kda_prefill_fused", "kda_prefill_fused_ex",
                                           "kda_prefill_fused_workspace_size",
                                           "kda_qkv_shortconv", "kda_output_gate",
                                           "kda_prefill_segments", "kda_prefill_workspace_size",
                                           "kda_prefill_backward", "kda_prefill_backward_workspace_size",
                                           "kda_status_string"])


def test_library_exports_every_declared_symbol():
    L = kda.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = os.popen("nm -D --defined-only %s" % kda.LIB_PATH).read()
    for name in declared_functions():
        assert re.search(r"\bT %s\b" % name, out), name


def test_status_strings():
    assert kda.kda_status_string(0) == "ok"
    for s in range(-9, 0):
        assert kda.kda_status_string(s) != "unknown kda status"
    assert kda.kda_status_string(-99) == "unknown kda status"


def test_workspace_size():
    # slabs: H * (ceil(T/64) + N) chunks, one slab each
    n1 = kda.kda_prefill_workspace_size(1, 65536, 96, 128, 128, kda.KDA_BF16)
    n2 = kda.kda_prefill_workspace_size(1, 65536 + 64, 96, 128, 128, kda.KDA_BF16)
    per = (n2 - n1) // 96
    assert per > 0 and per % 256 == 0
    assert n1 >= 96 * 1025 * per
    assert kda.kda_prefill_workspace_size(1, 100, 2, 32, 64, kda.KDA_BF16) == 0   # dk != dv
    assert kda.kda_prefill_workspace_size(1, 100, 2, 96, 96, kda.KDA_BF16) == 0   # d unsupported
    assert kda.kda_prefill_workspace_size(1, 100, 2, 32, 32, 7) == 0              # dtype
    assert kda.kda_prefill_workspace_size(0, 0, 2, 32, 32, kda.KDA_F32) > 0


FAKE = 1 << 20   # an aligned address that is never dereferenced: every call below fails its checks first


def _prefill(**over):
    a = dict(io_dtype=kda.KDA_BF16, q=FAKE, k=FAKE + 4096, v=FAKE + 8192, z=FAKE + 16384,
             A=FAKE + 32768, beta=FAKE + 40960, h0=None, cu=FAKE + 49152, N=1, T=16, H=2,
             dk=32, dv=32, o=FAKE + 65536, hT=None, ws=1 << 24, ws_bytes=0, stream=None)
    a.update(over)
    if a["ws_bytes"] == 0 and "ws_bytes" not in over:
        a["ws_bytes"] = kda.kda_prefill_workspace_size(a["N"], a["T"], a["H"], a["dk"], a["dv"], 0) - 1
    return kda.kda_prefill(a["io_dtype"], a["q"], a["k"], a["v"], a["z"], a["A"], a["beta"], a["h0"],
                           a["cu"], a["N"], a["T"], a["H"], a["dk"], a["dv"], a["o"], a["hT"], a["ws"],
                           a["ws_bytes"], a["stream"])


def test_prefill_rejects_bad_arguments():
    assert _prefill(io_dtype=5) == -4
    assert _prefill(N=-1) == -1
    assert _prefill(H=0) == -1
    assert _prefill(dk=64) == -3
    assert _prefill(dk=48, dv=48) == -3
    assert _prefill(q=None) == -2
    assert _prefill(cu=None) == -2
    assert _prefill(ws=None) == -2
    assert _prefill(q=FAKE + 2) == -5
    assert _prefill(ws=(1 << 24) + 16) == -5
    assert _prefill() == -6                       # workspace one byte short
    big = 1 << 40
    assert _prefill(ws_bytes=big, o=FAKE) == -8   # o on top of q


def test_prefill_noalloc_rejects_before_touching_the_device():
    """Argument errors are kda_prefill's; sizes beyond the fixed scratch are
    refused with their own status.  All of this is decided on the host."""
    n = lambda **o: kda.kda_prefill_noalloc(o.get("io", 0), FAKE, FAKE + 4096, FAKE + 8192, FAKE + 16384,
                                            FAKE + 32768, FAKE + 40960, None, FAKE + 49152, o.get("N", 1),
                                            o.get("T", 65536), o.get("H", 96), o.get("d", 128), o.get("d", 128),
                                            1 << 40, None, None)
    assert n(io=5) == -4 and n(N=-1) == -1 and n(d=48) == -3
    assert kda.kda_prefill_workspace_size(1, 65536, 96, 128, 128, 0) > kda.NOALLOC_SCRATCH_BYTES
    assert n() == -9                                   # the K3 prefill does not fit 256 MiB
    assert kda.kda_status_string(-9) != "unknown kda status"
    # what does fit: a 1024-token chunk of the 96-head prefill, 8 heads x 16384 tokens
    assert kda.kda_prefill_workspace_size(1, 1024, 96, 128, 128, 0) <= kda.NOALLOC_SCRATCH_BYTES
    assert kda.kda_prefill_workspace_size(2, 16384, 8, 128, 128, 0) <= kda.NOALLOC_SCRATCH_BYTES


def test_decode_rejects_bad_arguments():
    d = lambda **o: kda.kda_decode(o.get("io", 0), o.get("q", FAKE), FAKE + 4096, FAKE + 8192,
                                   FAKE + 16384, FAKE + 32768, FAKE + 40960, o.get("S", FAKE + 65536),
                                   o.get("N", 2), 2, o.get("d", 32), o.get("d", 32),
                                   o.get("o", 1 << 22), None)
    assert d(io=3) == -4
    assert d(N=-2) == -1
    assert d(d=16) == -3
    assert d(q=None) == -2
    assert d(S=FAKE + 8) == -5
    assert d(o=FAKE + 4096) == -8                 # o on top of k


def test_decode_fused_rejects_bad_arguments():
    """bf16 only, dk == dv in {32, 64, 128}, eps >= 0, the pointers a step
    needs, 16-byte alignment, and outputs (y, S, the new window) that overlap
    an input or each other; the window in place is allowed."""
    base = dict(io=0, xq=FAKE, xk=FAKE + 4096, xv=FAKE + 8192, wq=FAKE + 12288, wk=FAKE + 16384,
                wv=FAKE + 20480, win_in=None, win_out=None, z=FAKE + 24576, A=FAKE + 32768, beta=FAKE + 36864,
                S=FAKE + 40960, gate=FAKE + 57344, w=FAKE + 61440, eps=1e-6, N=2, H=2, dk=32, dv=32,
                y=FAKE + 65536)

    def d(**o):
        a = dict(base)
        a.update(o)
        return kda.kda_decode_fused(a["io"], a["xq"], a["xk"], a["xv"], a["wq"], a["wk"], a["wv"], a["win_in"],
                                    a["win_out"], a["z"], a["A"], a["beta"], a["S"], a["gate"], a["w"], a["eps"],
                                    a["N"], a["H"], a["dk"], a["dv"], a["y"], None)
    assert d(io=1) == -4                          # fp32 io
    assert d(N=-1) == -1 and d(H=0) == -1 and d(eps=-1.0) == -1
    assert d(dk=64) == -3 and d(dk=48, dv=48) == -3
    assert d(xq=None) == -2 and d(S=None) == -2 and d(gate=None) == -2 and d(w=None) == -2
    assert d(A=None) == -2 and d(wv=None) == -2
    assert d(xk=FAKE + 4098) == -5 and d(y=FAKE + 65538) == -5
    assert d(y=FAKE + 4096) == -8                 # y on top of xk
    assert d(S=FAKE + 24576) == -8                # the state on top of z
    assert d(y=FAKE + 40960) == -8                # y on top of the state
    assert d(win_in=1 << 22, win_out=(1 << 22) + 512) == -8   # two windows that overlap
    assert d(win_out=FAKE + 57344) == -8          # the new window on top of the gate


def test_block_option():
    """The chunk-block pipeline option: range checks, the conflict with forced
    segments, and the workspace growing by the carried state (N H dk dv fp32)
    and the block counters wherever the pipeline applies (bf16 path, one
    segment, no checkpoints; never in the backward)."""
    assert ctypes.sizeof(kda.PrefillOptions) == 32
    big = lambda **kw: kda.kda_prefill_ex_workspace_size(1, 65536, 96, 128, 128, kda.KDA_BF16, kda.options(**kw))
    assert big(blocks=-1) == 0 and big(blocks=17) == 0
    assert big(segments=3, blocks=3) == 0
    carry = 96 * 128 * 128 * 4 + 256
    assert big(blocks=3) - big(blocks=1) == carry
    assert big(blocks=16) - big(blocks=1) == carry
    # the K3 shape pipelines by default (the chain leaves CUs free, the sequence is long)
    assert big() == big(blocks=3) == kda.kda_prefill_workspace_size(1, 65536, 96, 128, 128, kda.KDA_BF16)
    # not applicable: fp32 io, checkpoints
    f32 = lambda **kw: kda.kda_prefill_ex_workspace_size(1, 65536, 8, 64, 64, kda.KDA_F32, kda.options(**kw))
    assert f32(blocks=3) == f32(blocks=1) > 0
    assert big(blocks=3, interval=512, checkpoints=FAKE) == big(blocks=1, interval=512, checkpoints=FAKE) > 0
    # forced blocks with automatic segments mean one segment: the small-head
    # shape, split by default, then needs no segment transitions
    small = lambda **kw: kda.kda_prefill_ex_workspace_size(2, 16384, 8, 128, 128, kda.KDA_BF16, kda.options(**kw))
    assert small(blocks=3) == small(segments=1) + 2 * 8 * 128 * 128 * 4 + 256
    # a chain that fills the device: four runs from 16 sequences of 128 chunks on average
    # (the varlen batch), none for fewer or shorter sequences
    vw = lambda N, T, **kw: kda.kda_prefill_ex_workspace_size(N, T, 96, 128, 128, kda.KDA_BF16, kda.options(**kw))
    assert vw(32, 262144) == vw(32, 262144, blocks=4) == vw(32, 262144, blocks=1) + 32 * 96 * 128 * 128 * 4 + 256
    assert vw(8, 131072) == vw(8, 131072, blocks=1)
    assert vw(16, 98304) == vw(16, 98304, blocks=1)
    assert vw(64, 262144) == vw(64, 262144, blocks=1)
    # the backward ignores the option
    bw = lambda o: kda.kda_prefill_backward_workspace_size(1, 65536, 8, 128, 128, kda.KDA_BF16, o)
    assert bw(kda.options(blocks=3)) == bw(kda.options(blocks=1)) > 0


def test_prefill_fused_ex_options():
    """The fused prefill's options: checkpoints are refused (the gated output
    pass stores no states), out-of-range blocks and forced segments with
    forced blocks likewise; all decided on the host, before any launch.  With
    NULL options it is kda_prefill_fused.  Its workspace is the plain call's,
    plus the staged q, k, v (3 T H d bf16) where the call is pipelined."""
    def f(opts, io=0, ws_bytes=1 << 40):
        return kda.kda_prefill_fused_ex(io, FAKE, FAKE + 4096, FAKE + 8192, FAKE + 12288, FAKE + 16384,
                                        FAKE + 20480, None, None, FAKE + 24576, FAKE + 32768, FAKE + 36864, None,
                                        FAKE + 40960, 1, 64, 2, 32, 32, FAKE + 45056, FAKE + 49152, 1e-6,
                                        1 << 41, None, opts, FAKE + (1 << 24), ws_bytes, None)
    assert f(kda.options(interval=512, checkpoints=FAKE)) == -1
    assert f(kda.options(interval=64)) == -1
    assert f(kda.options(blocks=17)) == -1 and f(kda.options(blocks=-1)) == -1
    assert f(kda.options(segments=2, blocks=2)) == -1
    assert f(kda.options(blocks=2), io=1) == -4
    assert f(kda.options(blocks=2), ws_bytes=16) == -6     # workspace too small, reported before any launch
    fws = lambda N, T, H, **kw: kda.kda_prefill_fused_workspace_size(N, T, H, 128, 128, kda.KDA_BF16,
                                                                     kda.options(**kw) if kw else None)
    pws = lambda N, T, H, **kw: kda.kda_prefill_ex_workspace_size(N, T, H, 128, 128, kda.KDA_BF16,
                                                                  kda.options(**kw) if kw else None)
    staged = lambda T, H: 3 * ((T * H * 128 * 2 + 255) // 256 * 256)
    # the K3 shape pipelines by default: q, k, v staged
    assert fws(1, 65536, 96) == pws(1, 65536, 96) + staged(65536, 96)
    assert fws(1, 65536, 96, blocks=1) == pws(1, 65536, 96, blocks=1)
    assert fws(2, 1000, 3, blocks=4) == pws(2, 1000, 3, blocks=4) + staged(1000, 3)
    # not pipelined (segmented small-head shape, a chain of few sequences that fills the device): no staging
    assert fws(2, 16384, 8) == pws(2, 16384, 8) == kda.kda_prefill_workspace_size(2, 16384, 8, 128, 128, 0)
    assert fws(32, 262144, 96) == pws(32, 262144, 96) + staged(262144, 96)
    assert fws(8, 131072, 96) == pws(8, 131072, 96)
    # fp32 io and checkpoints are refused
    assert kda.kda_prefill_fused_workspace_size(1, 1000, 2, 64, 64, kda.KDA_F32, None) == 0
    assert fws(1, 1000, 2, interval=512) == 0


def test_segment_option():
    """The per-call segment count: range checks, and the workspace growing by
    the transitions (2 d^2) and incoming states (d^2) in fp32 per (segment,
    head).  The size is a function of the arguments alone: asking with other
    options in between changes nothing."""
    ws = lambda P, **kw: kda.kda_prefill_ex_workspace_size(2, 16384, 8, 128, 128, kda.KDA_BF16,
                                                          kda.options(P, **kw))
    assert ws(-1) == 0 and ws(17) == 0
    base = ws(1)
    assert base > 0
    for P in (2, 7, 16):
        extra = 2 * P * 8 * 3 * 128 * 128 * 4
        assert ws(P) - base == extra + (256 if 2 * P * 16 > 256 else 0), (P, ws(P) - base)
    assert ws(1) == base
    # options NULL and zero-initialised options are the automatic choice
    auto = kda.kda_prefill_segments(2, 16384, 8, 128, 128, kda.KDA_BF16)
    assert auto > 1
    assert kda.kda_prefill_ex_workspace_size(2, 16384, 8, 128, 128, kda.KDA_BF16, None) == ws(auto)
    assert kda.kda_prefill_workspace_size(2, 16384, 8, 128, 128, kda.KDA_BF16) == ws(0) == ws(auto)
    assert kda.kda_prefill_segments(2, 16384, 8, 96, 96, kda.KDA_BF16) == 0
    # checkpoint options: the interval must be a positive multiple of 64 when a buffer is given
    assert ws(0, interval=100, checkpoints=FAKE) == 0
    assert ws(0, interval=0, checkpoint_offsets=FAKE) == 0
    assert ws(0, interval=512, checkpoints=FAKE) == ws(0)
    # the backward takes the segment option only
    bw = lambda o: kda.kda_prefill_backward_workspace_size(2, 16384, 8, 128, 128, kda.KDA_BF16, o)
    assert bw(kda.options(3)) > bw(kda.options(1)) > 0
    assert bw(kda.options(0, 512, FAKE)) == 0 and bw(kda.options(0, 64)) == 0 and bw(kda.options(99)) == 0
    # automatic choice: one segment when one pass fills half the device or
    # the sequences are short
    assert kda.kda_prefill_segments(1, 65536, 96, 128, 128, kda.KDA_BF16) == 1
    assert kda.kda_prefill_segments(1, 256, 2, 32, 32, kda.KDA_F32) == 1
    assert kda.kda_prefill_segments(0, 0, 2, 32, 32, kda.KDA_F32) == 1


def test_prefill_ex_rejects_bad_options():
    e = lambda opts, ws_bytes=1 << 40: kda.kda_prefill_ex(0, FAKE, FAKE + 4096, FAKE + 8192, FAKE + 16384,
                                                          FAKE + 32768, FAKE + 40960, None, FAKE + 49152, 1, 16,
                                                          2, 32, 32, FAKE + 65536, None, opts, 1 << 24,
                                                          ws_bytes, None)
    assert e(kda.options(-1)) == -1
    assert e(kda.options(17)) == -1
    assert e(kda.options(0, 100, 1 << 26)) == -1
    assert e(kda.options(0, 0, None, 1 << 26)) == -1
    assert e(None, ws_bytes=0) == -6
    assert e(kda.options(4), ws_bytes=kda.kda_prefill_ex_workspace_size(1, 16, 2, 32, 32, 0, kda.options(4)) - 1) == -6


def test_decode_window_rejects_bad_arguments():
    def w(**o):
        a = dict(io=0, rk=FAKE, rv=FAKE + 4096, rz=FAKE + 8192, rb=FAKE + 12288, acc=FAKE + 16384, Lr=2,
                 q=FAKE + 20480, k=FAKE + 24576, v=FAKE + 28672, z=FAKE + 32768, b=FAKE + 36864, L=3,
                 A=FAKE + 40960, S=1 << 22, N=2, H=2, d=32, o=1 << 23, commit=0)
        a.update(o)
        return kda.kda_decode_window(a["io"], a["rk"], a["rv"], a["rz"], a["rb"], a["acc"], a["Lr"], a["q"],
                                     a["k"], a["v"], a["z"], a["b"], a["L"], a["A"], a["S"], a["N"], a["H"],
                                     a["d"], a["d"], a["o"], a["commit"], None)
    assert w(io=4) == -4
    assert w(Lr=17) == -1 and w(L=17) == -1 and w(L=-1) == -1 and w(N=-1) == -1
    assert w(commit=2) == -1
    assert w(d=48) == -3
    assert w(acc=None) == -2 and w(rk=None) == -2 and w(q=None) == -2 and w(S=None) == -2
    assert w(rk=None, rv=None, rz=None, rb=None, acc=None, Lr=0, o=FAKE + 8) == -5   # misaligned o
    assert w(o=FAKE + 24576) == -8                # o on top of k
    assert w(S=FAKE) == -8                        # state on top of the replay keys


def test_prefill_checkpoints_rejects_bad_arguments():
    def c(**o):
        a = dict(interval=512, ck=1 << 26, off=(1 << 26) - 4096, T=4096, ws_bytes=1 << 40)
        a.update(o)
        return kda.kda_prefill_ex(0, FAKE, FAKE + 4096 * 64, FAKE + 2 * 4096 * 64, FAKE + 3 * 4096 * 64,
                                  FAKE + 4 * 4096 * 64, FAKE + 6 * 4096 * 64, None, FAKE + 7 * 4096 * 64,
                                  1, a["T"], 2, 32, 32, 1 << 25, None,
                                  kda.options(0, a["interval"], a["ck"], a["off"]), 1 << 30, a["ws_bytes"], None)
    assert c(interval=0) == -1
    assert c(interval=100) == -1
    assert c(interval=-64) == -1
    assert c(ck=(1 << 26) + 8) == -5
    assert c(ck=1 << 25) == -8                       # checkpoints on top of o
    assert c(ck=FAKE) == -8                          # checkpoints on top of q
    assert c(off=1 << 30) == -8                      # offsets inside the workspace
    assert c(ck=None, off=None, interval=0, ws_bytes=0) == -6   # no checkpoints: plain prefill checks


def test_feature_path_and_gate_reject_bad_arguments():
    def f(**o):
        a = dict(io=0, xq=FAKE, xk=FAKE + 65536, xv=FAKE + 2 * 65536, w=1 << 24, cu=(1 << 24) + 65536, N=1, T=64,
                 H=2, dk=128, dv=128, win_in=None, win_out=None, q=1 << 26, k=(1 << 26) + 65536,
                 v=(1 << 26) + 2 * 65536)
        a.update(o)
        w2 = None if a["w"] is None else a["w"] + 4096
        w3 = None if a["w"] is None else a["w"] + 8192
        return kda.kda_qkv_shortconv(a["io"], a["xq"], a["xk"], a["xv"], a["w"], w2, w3,
                                     a["cu"], a["N"], a["T"], a["H"], a["dk"], a["dv"], a["win_in"], a["win_out"],
                                     a["q"], a["k"], a["v"], None)
    assert f(io=3) == -4
    assert f(T=64, N=0) == -1 and f(H=0) == -1
    assert f(dk=64) == -3 and f(dk=48, dv=48) == -3
    assert f(cu=None) == -2 and f(xq=None) == -2 and f(w=None) == -2
    assert f(q=(1 << 26) + 4) == -5
    assert f(q=FAKE) == -8                                   # q on top of xq
    assert f(k=1 << 26) == -8                                # k on top of q
    assert f(win_in=1 << 28, win_out=(1 << 28) + 256) == -8  # windows partly overlapping
    # the gate
    g = lambda **o: kda.kda_output_gate(o.get("io", 0), o.get("o", FAKE), o.get("g", FAKE + 65536),
                                        o.get("w", 1 << 24), o.get("eps", 1e-6), 64, 2, o.get("dv", 128),
                                        o.get("y", 1 << 26), None)
    assert g(io=2) == -4 and g(eps=-1.0) == -1 and g(eps=float("nan")) == -1
    assert g(dv=48) == -3 and g(w=None) == -2 and g(y=(1 << 26) + 2) == -5
    assert g(y=FAKE + 256) == -8                             # y partly over o


def test_backward_workspace_size():
    # per (chunk, head) fp32 record + chunk-boundary states + the forward's own workspace
    n1 = kda.kda_prefill_backward_workspace_size(1, 4096, 4, 128, 128, kda.KDA_BF16)
    f1 = kda.kda_prefill_workspace_size(1, 4096, 4, 128, 128, kda.KDA_BF16)
    assert n1 > f1 + (4096 // 64) * 4 * 128 * 128 * 4
    n2 = kda.kda_prefill_backward_workspace_size(1, 4096 + 64, 4, 128, 128, kda.KDA_BF16)
    assert n2 > n1
    assert kda.kda_prefill_backward_workspace_size(1, 100, 2, 32, 64, kda.KDA_BF16) == 0
    assert kda.kda_prefill_backward_workspace_size(1, 100, 2, 32, 32, 5) == 0
    assert kda.kda_prefill_backward_workspace_size(0, 0, 2, 32, 32, kda.KDA_F32) > 0


def test_prefill_backward_rejects_bad_arguments():
    T, H, d = 128, 2, 32
    span = T * H * d * 4

    def b(**o):
        base = 1 << 24
        a = dict(io=0, q=base, k=base + span, v=base + 2 * span, z=base + 3 * span, A=base + 4 * span,
                 beta=base + 4 * span + 256, cu=base + 5 * span, dO=base + 6 * span, dhT=None,
                 gq=1 << 26, gk=(1 << 26) + span, gv=(1 << 26) + 2 * span, gz=(1 << 26) + 3 * span,
                 gb=(1 << 26) + 4 * span, gA=(1 << 26) + 5 * span, gh0=None, d=d, N=1, ws=1 << 30,
                 ws_bytes=1 << 40)
        a.update(o)
        return kda.kda_prefill_backward(a["io"], a["q"], a["k"], a["v"], a["z"], a["A"], a["beta"], None, a["cu"],
                                        a["N"], T, H, a["d"], a["d"], a["dO"], a["dhT"], a["gq"], a["gk"], a["gv"],
                                        a["gz"], a["gb"], a["gA"], a["gh0"], a.get("opts"), a["ws"],
                                        a["ws_bytes"], None)
    assert b(io=3) == -4
    assert b(N=-1) == -1
    assert b(d=48) == -3
    assert b(gA=None) == -2 and b(dO=None) == -2 and b(gq=None) == -2 and b(ws=None) == -2
    assert b(gq=(1 << 26) + 4) == -5 and b(ws=(1 << 30) + 16) == -5
    assert b(ws_bytes=16) == -6
    assert b(gq=1 << 24) == -8                    # grad_q on top of q
    assert b(gk=(1 << 26) + 64) == -8             # grad_k over grad_q
    assert b(gh0=(1 << 30) + 256) == -8           # grad_h0 inside the workspace
    assert b(opts=kda.options(17)) == -1          # segment count out of range
    assert b(opts=kda.options(0, 512, 1 << 28)) == -1   # checkpoints are a prefill option only


# ---------------------------------------------------------------------------
# The torch wrappers check every tensor's dtype and shape before passing its
# pointer (the C ABI cannot see either).  CPU tensors get through those checks
# and are then refused as not being on a GPU; these tests run on the CPU.
# ---------------------------------------------------------------------------
import torch  # noqa: E402


def _prefill_tensors(T=70, H=2, d=32, N=2, io=torch.bfloat16):
    return dict(q=torch.zeros(T, H, d, dtype=io), k=torch.zeros(T, H, d, dtype=io),
                v=torch.zeros(T, H, d, dtype=io), z=torch.zeros(T, H, d), A=torch.zeros(H),
                beta=torch.zeros(T, H), cu_seqlens=torch.tensor([0, 30, T], dtype=torch.int32)[: N + 1],
                h0=torch.zeros(N, H, d, d))


PREFILL_BAD = [
    ("k", lambda t: t["k"].float(), TypeError),
    ("v", lambda t: t["v"].to(torch.float16), TypeError),
    ("z", lambda t: t["z"].bfloat16(), TypeError),
    ("z", lambda t: t["z"][:-1].clone(), ValueError),                    # a short z
    ("A", lambda t: t["A"].double(), TypeError),
    ("A", lambda t: torch.zeros(3), ValueError),
    ("beta", lambda t: t["beta"].bfloat16(), TypeError),
    ("beta", lambda t: torch.zeros(70, 3), ValueError),
    ("cu_seqlens", lambda t: t["cu_seqlens"].long(), TypeError),        # int64 offsets
    ("h0", lambda t: t["h0"].bfloat16(), TypeError),
    ("h0", lambda t: torch.zeros(1, 2, 32, 32), ValueError),
    ("k", lambda t: t["k"].transpose(0, 1).contiguous().transpose(0, 1), ValueError),   # not contiguous
]


@pytest.mark.parametrize("name,bad,err", PREFILL_BAD)
def test_prefill_wrapper_rejects(name, bad, err):
    t = _prefill_tensors()
    t[name] = bad(t)
    with pytest.raises(err, match=name):
        kda.prefill(**t)
    with pytest.raises(err, match=name):
        kda.prefill_checkpoints(**t, interval=64)
    with pytest.raises(err, match=name):
        kda.prefill_backward(**t, grad_o=torch.zeros(70, 2, 32, dtype=torch.bfloat16))


def test_prefill_wrapper_rejects_outputs_and_then_the_device():
    t = _prefill_tensors()
    with pytest.raises(TypeError, match="o"):
        kda.prefill(**t, o=torch.zeros(70, 2, 32))                         # fp32 o with bf16 q
    with pytest.raises(ValueError, match="hT"):
        kda.prefill(**t, hT=torch.zeros(2, 2, 32, 16))
    with pytest.raises(TypeError, match="workspace"):
        kda.prefill(**t, workspace=torch.zeros(16, dtype=torch.int32))
    with pytest.raises(ValueError, match="checkpoints"):
        kda.prefill_checkpoints(**t, interval=64, checkpoints=torch.zeros(2, 2, 32, 32))
    with pytest.raises(TypeError, match="offsets"):
        kda.prefill_checkpoints(**t, interval=64, offsets=torch.zeros(3, dtype=torch.int64))
    with pytest.raises(ValueError, match="interval"):
        kda.prefill_checkpoints(**t, interval=100)
    with pytest.raises(TypeError, match="grad_o"):
        kda.prefill_backward(**t, grad_o=torch.zeros(70, 2, 32))
    with pytest.raises(ValueError, match="dq"):
        kda.prefill_backward(**t, grad_o=torch.zeros(70, 2, 32, dtype=torch.bfloat16),
                             grads=dict(dq=torch.zeros(70, 2, 31)))
    # every check passed: a CPU tensor is refused, nothing is launched
    with pytest.raises(ValueError, match="GPU"):
        kda.prefill(**t)


def test_decode_wrappers_reject():
    N, H, d = 3, 2, 32
    base = dict(q=torch.zeros(N, H, d, dtype=torch.bfloat16), k=torch.zeros(N, H, d, dtype=torch.bfloat16),
                v=torch.zeros(N, H, d, dtype=torch.bfloat16), z=torch.zeros(N, H, d), A=torch.zeros(H),
                beta=torch.zeros(N, H), S=torch.zeros(N, H, d, d))
    for name, val, err in (("z", torch.zeros(N, H, d, dtype=torch.bfloat16), TypeError),
                           ("S", torch.zeros(N, H, d, 16), ValueError),
                           ("S", torch.zeros(N, H, d, d, dtype=torch.float64), TypeError),
                           ("beta", torch.zeros(N, H + 1), ValueError),
                           ("k", torch.zeros(N, H, d), TypeError)):
        with pytest.raises(err, match=name):
            kda.decode(**dict(base, **{name: val}))
    with pytest.raises(ValueError, match="GPU"):
        kda.decode(**base)
    # the decode window
    win = dict(q=torch.zeros(N, 2, H, d, dtype=torch.bfloat16), k=torch.zeros(N, 2, H, d, dtype=torch.bfloat16),
               v=torch.zeros(N, 2, H, d, dtype=torch.bfloat16), z=torch.zeros(N, 2, H, d), beta=torch.zeros(N, 2, H))
    rep = dict(k=torch.zeros(N, 3, H, d, dtype=torch.bfloat16), v=torch.zeros(N, 3, H, d, dtype=torch.bfloat16),
               z=torch.zeros(N, 3, H, d), beta=torch.zeros(N, 3, H))
    acc = torch.zeros(N, dtype=torch.int32)
    with pytest.raises(ValueError, match="window z"):
        kda.decode_window(base["A"], base["S"], window=dict(win, z=torch.zeros(N, 3, H, d)))
    with pytest.raises(TypeError, match="replay v"):
        kda.decode_window(base["A"], base["S"], replay=dict(rep, v=rep["v"].float()), n_accept=acc)
    with pytest.raises(TypeError, match="n_accept"):
        kda.decode_window(base["A"], base["S"], replay=rep, n_accept=acc.long())
    with pytest.raises(ValueError, match="n_accept"):
        kda.decode_window(base["A"], base["S"], replay=rep)
    with pytest.raises(TypeError, match="bfloat16 or float32"):
        kda.decode_window(base["A"], base["S"], window={n: (t.half() if n == "q" else t) for n, t in win.items()})
    with pytest.raises(ValueError, match="GPU"):
        kda.decode_window(base["A"], base["S"], window=win, replay=rep, n_accept=acc)


def test_feature_wrappers_reject():
    T, H, d = 20, 2, 32
    x = lambda: torch.zeros(T, H, d, dtype=torch.bfloat16)
    w = lambda: torch.zeros(H, d, 4)
    cu = torch.tensor([0, T], dtype=torch.int32)
    with pytest.raises(TypeError, match="wk"):
        kda.qkv_shortconv(x(), x(), x(), w(), w().bfloat16(), w(), cu)
    with pytest.raises(ValueError, match="conv_state_in"):
        kda.qkv_shortconv(x(), x(), x(), w(), w(), w(), cu, conv_state_in=torch.zeros(1, 3, H, d, dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="cu_seqlens"):
        kda.qkv_shortconv(x(), x(), x(), w(), w(), w(), cu.long())
    with pytest.raises(ValueError, match="GPU"):
        kda.qkv_shortconv(x(), x(), x(), w(), w(), w(), cu)
    with pytest.raises(TypeError, match="g"):
        kda.output_gate(x(), x().float(), torch.ones(d), 1e-6)
    with pytest.raises(ValueError, match="w"):
        kda.output_gate(x(), x(), torch.ones(d + 1), 1e-6)
    with pytest.raises(ValueError, match="GPU"):
        kda.output_gate(x(), x(), torch.ones(d), 1e-6)


def test_decode_fused_wrapper_rejects():
    N, H, d = 3, 2, 32
    bf = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)
    t = dict(xq=bf(N, H, d), xk=bf(N, H, d), xv=bf(N, H, d), wq=torch.zeros(H, d, 4), wk=torch.zeros(H, d, 4),
             wv=torch.zeros(H, d, 4), z=torch.zeros(N, H, d), A=torch.zeros(H), beta=torch.zeros(N, H),
             S=torch.zeros(N, H, d, d), gate=bf(N, H, d), norm_weight=torch.ones(d), eps=1e-6)
    bad = [("xv", bf(N, H, d + 1), ValueError), ("wk", torch.zeros(H, d, 4).bfloat16(), TypeError),
           ("z", torch.zeros(N, H, d).bfloat16(), TypeError), ("S", torch.zeros(N, H, d, d - 1), ValueError),
           ("gate", torch.zeros(N, H, d), TypeError), ("norm_weight", torch.ones(d + 1), ValueError)]
    for name, val, err in bad:
        with pytest.raises(err, match=name):
            kda.decode_fused(**dict(t, **{name: val}))
    with pytest.raises(ValueError, match="conv_state_in"):
        kda.decode_fused(**t, conv_state_in=bf(N, 3, H, d))
    with pytest.raises(TypeError, match="y"):
        kda.decode_fused(**t, y=torch.zeros(N, H, d))
    with pytest.raises(ValueError, match="GPU"):
        kda.decode_fused(**t)
