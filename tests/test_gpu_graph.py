"""The verification step captured in a HIP graph: every replay must equal the eager result.

Replays are interleaved with eager work and synchronizations; outputs are
cleared before each replay so a stale buffer cannot pass.
"""
import numpy as np
import pytest
import torch

import mx_fp4_weight_amd as mxs
import synth
from oracle import mx as omx
from tests.gpu_util import dev, dev_bf16, host, say

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    say("graph: capture GEMM + spec_accept, replay x4")
    n, k = 4096, 4096
    codes, scales, _ = omx.quantize(synth.weights(2, 77, n, k))
    dc, ds = dev(codes), dev(scales)
    x = dev_bf16(synth.activations(2, 77, 5, k))
    tgt, dft, tok, u = synth.accept_batch(2, 3, 4, 128256, 3.0, 1.0, seq0=900)
    dt, dd, dk, du = dev(tgt), dev(dft), dev(tok), dev(u)
    y = torch.empty((5, n), dtype=torch.float32, device="cuda")
    out = torch.empty((3, 5), dtype=torch.int32, device="cuda")
    num = torch.empty((3,), dtype=torch.int32, device="cuda")
    ws = torch.empty((mxs.spec_accept_workspace_bytes(3, 4, 128256),), dtype=torch.uint8, device="cuda")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")

    def step():
        mxs.mxfp4_verify_gemm(dc, ds, x, y=y)
        mxs.spec_accept(dt, dd, dk, du, out_tokens=out, out_num=num, workspace=ws, dev_flags=flags)

    step()
    torch.cuda.synchronize()
    y_ref, out_ref, num_ref = host(y).copy(), host(out).copy(), host(num).copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        y.fill_(float("nan"))
        out.fill_(-7)
        num.fill_(-7)
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(y), y_ref), rep
        assert np.array_equal(host(out), out_ref) and np.array_equal(host(num), num_ref), rep
        # eager work between replays
        mxs.mxfp4_verify_gemm(dc, ds, dev_bf16(synth.activations(2, 78, 3, k)))
        torch.cuda.synchronize()
    assert int(flags.item()) == 0


def test_multistream_graph_replays_match_eager():
    """Three independent GEMMs on three streams joined back, as the bench captures a layer."""
    say("graph: three streams, replay x3")
    shapes = [(4096, 4096), (1024, 4096), (1024, 4096)]
    mats = []
    for i, (n, k) in enumerate(shapes):
        c, s_, _ = omx.quantize(synth.weights(2, 300 + i, n, k))
        mats.append((dev(c), dev(s_), dev_bf16(synth.activations(2, 300 + i, 5, k)),
                     torch.empty((5, n), dtype=torch.float32, device="cuda")))
    side = [torch.cuda.Stream(), torch.cuda.Stream()]

    def step():
        st = torch.cuda.current_stream()
        for sd in side:
            sd.wait_stream(st)
        for (c, s_, x, y), where in zip(mats, [st, side[0], side[1]]):
            mxs.mxfp4_verify_gemm(c, s_, x, y=y, stream=where)
        for sd in side:
            st.wait_stream(sd)

    step()
    torch.cuda.synchronize()
    ref = [host(y).copy() for (_, _, _, y) in mats]
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for (_, _, _, y) in mats:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (_, _, _, y), r in zip(mats, ref):
            assert np.array_equal(host(y), r), rep
        step()
        torch.cuda.synchronize()
