"""GPU properties of the forward that hold at any size, checked on the HIP path through the C ABI
(the oracle pins the same properties on the CPU: tests/test_oracle.py P-8 and P-9).

  state passing   a sequence split in two, the second part started from the first part's final
                  state, gives the whole sequence's o and final state: compared with the fp64
                  oracle of the whole sequence at the parity bars (tests/parity_check.py)
  grouped heads   HV = G H value heads give bit for bit what H' = HV heads give with q and k
                  repeated per value head (the value heads of a group only share their q/k
                  reads)
  packed          packed sequences (cu_seqlens) give bit for bit what each sequence gives as
                  a batch of its own (chunk slots, workgroup maps and launch shapes differ; the
                  arithmetic of a (sequence, head) unit does not)
  slice grouping  a launch large enough for several V-slices per workgroup gives bit for bit
                  what one slice per workgroup gives (each sequence run alone)
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from errlog import report_named
from oracle.native import kda_oracle_c
from parity_check import check_outputs

import chunked_kimi_delta_amd as kda

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ORACLE_THREADS = 16


def dev(x):
    return None if x is None else x.to(DEV).contiguous()


def run(q, k, v, g, beta, scale, h0=None, cu=None, chunk=0):
    plan = kda.KdaFwdPlan(dev(q), dev(k), dev(v), dev(g), dev(beta), scale=scale,
                          cu_seqlens=dev(cu), initial_state=dev(h0), chunk=chunk)
    o, fin = plan()
    torch.cuda.synchronize()
    return o.float().cpu(), fin.cpu()


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_state_passing_full_size(chunk):
    # 16 heads x 4096 tokens, split after 2,065 tokens (a ragged first part)
    inp = W.make_inputs(W.WORKLOADS["h16_t4096"], seed=5)
    T1 = 2065
    part = lambda x, a, b: x[:, a:b].contiguous()
    args = lambda a, b: [part(x, a, b) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta)]
    o1, f1 = run(*args(0, T1), inp.scale, chunk=chunk)
    o2, f2 = run(*args(T1, inp.q.shape[1]), inp.scale, h0=f1, chunk=chunk)
    o = torch.cat([o1, o2], dim=1).numpy()
    f = W.as_f32_numpy
    o_ref, f_ref = kda_oracle_c(f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta), inp.scale,
                                n_threads=ORACLE_THREADS)
    worst = check_outputs(o, f2.numpy().astype(np.float64), o_ref, f_ref, inp.seq_bounds(),
                          "bf16", what=f"state passing, chunk {chunk}")
    report_named(**worst)


@pytest.mark.parametrize("chunk", [1, 16, 32, 64])
def test_grouped_heads_equal_repeated_qk(chunk):
    w = W.custom(B=2, T=1000, H=4, HV=8, K=128, V=128, h0_std=0.1)
    inp = W.make_inputs(w, seed=6)
    o_g, f_g = run(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, h0=inp.h0, chunk=chunk)
    rep = lambda x: x.repeat_interleave(w.G, dim=2)
    o_r, f_r = run(rep(inp.q), rep(inp.k), inp.v, inp.g, inp.beta, inp.scale, h0=inp.h0,
                   chunk=chunk)
    assert torch.equal(o_g, o_r), "o differs between grouped and repeated q/k"
    assert torch.equal(f_g, f_r), "final state differs between grouped and repeated q/k"


@pytest.mark.parametrize("chunk", [1, 16, 32, 64])
def test_packed_equals_per_sequence(chunk):
    # eight packed sequences of 0 to 4,112 tokens, ragged, 8 heads
    w = W.custom(H=8, HV=8, K=128, V=128, h0_std=0.1,
                 lengths=(256, 4112, 16, 1040, 0, 7, 2000, 33))
    inp = W.make_inputs(w, seed=8)
    o, f = run(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, h0=inp.h0,
               cu=inp.cu_seqlens, chunk=chunk)
    for s, (a, b) in enumerate(inp.seq_bounds()):
        if a == b:                    # an empty sequence passes its initial state through
            assert torch.equal(f[s], inp.h0[s]), f"empty sequence {s} changed its state"
            continue
        seq = lambda x: x[:, a:b].contiguous()
        # the sequence alone, also packed (cu_seqlens of one sequence), so that both runs take
        # the one-segment state pass (a dense batch this small runs as two segments at chunk
        # 32, with other rounding; that path is compared with the oracle on its own)
        one = torch.tensor([0, b - a], dtype=torch.int64)
        o_s, f_s = run(seq(inp.q), seq(inp.k), seq(inp.v), seq(inp.g), seq(inp.beta),
                       inp.scale, h0=inp.h0[s:s + 1], cu=one, chunk=chunk)
        assert torch.equal(o[:, a:b], o_s), f"o of sequence {s} differs from its own run"
        assert torch.equal(f[s:s + 1], f_s), f"final state of sequence {s} differs"


@pytest.mark.parametrize("chunk", [1, 16, 32, 64])
@pytest.mark.parametrize("case", ["dense_t1000", "packed"])
def test_state_update_in_place(case, chunk):
    # initial_state and final_state as one buffer (a state carried in place from call to
    # call): the same o and final state, bit for bit, as with separate buffers. At chunk 32 the
    # dense case runs as two segments, whose final state is written only by the correction.
    w = (W.custom(B=1, T=1000, H=2, HV=2, K=128, V=128, h0_std=0.1) if case == "dense_t1000"
         else W.custom(H=2, HV=4, K=128, V=128, h0_std=0.1, lengths=(600, 0, 77, 1100)))
    inp = W.make_inputs(w, seed=12)
    o_ref, f_ref = run(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, h0=inp.h0,
                       cu=inp.cu_seqlens, chunk=chunk)
    h = inp.h0.to(DEV).contiguous()
    plan = kda.KdaFwdPlan(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                          scale=inp.scale, cu_seqlens=dev(inp.cu_seqlens), initial_state=h,
                          final_state=h, chunk=chunk)
    o, fin = plan()
    torch.cuda.synchronize()
    assert fin.data_ptr() == h.data_ptr()
    assert torch.equal(o.float().cpu(), o_ref), "o differs with the state updated in place"
    assert torch.equal(h.cpu(), f_ref), "final state differs with the state updated in place"


@pytest.mark.parametrize("chunk", [32, 64])
def test_slice_grouping_bitwise(chunk):
    # 4 sequences x 32 value heads: 1,024 16-column slices, so the state kernel puts four slices
    # of a unit in one workgroup (chain and output waves serving two slices each at chunk 32);
    # each sequence alone (256 slices) runs one slice per workgroup. The arithmetic of a slice
    # is the same either way, so the results agree bit for bit.
    w = W.custom(B=4, T=300, H=16, HV=32, K=128, V=128, h0_std=0.1)
    inp = W.make_inputs(w, seed=9)
    o, f = run(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, h0=inp.h0, chunk=chunk)
    for b in range(w.B):
        one = lambda x: x[b:b + 1].contiguous()
        o_b, f_b = run(one(inp.q), one(inp.k), one(inp.v), one(inp.g), one(inp.beta),
                       inp.scale, h0=inp.h0[b:b + 1], chunk=chunk)
        assert torch.equal(o[b:b + 1], o_b), f"o of sequence {b} differs from its own run"
        assert torch.equal(f[b:b + 1], f_b), f"final state of sequence {b} differs"


@pytest.mark.parametrize("case", ["dense_split", "packed"])
def test_forward_replays_in_a_hip_graph(case):
    # The forward captured in a HIP graph (the library records kernel launches only: no memset,
    # copy or allocation) and replayed three times, with new inputs copied into the captured
    # buffers and eager work in between: every replay equals an eager run bit for bit. The
    # dense case runs the two-segment state pass (two kernels after the prepare).
    w = (W.custom(B=1, T=1000, H=2, HV=2, K=128, V=128, h0_std=0.1) if case == "dense_split"
         else W.custom(H=2, HV=4, K=128, V=128, h0_std=0.1, lengths=(300, 77, 700)))
    inp = W.make_inputs(w, seed=50)
    bufs = [dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0)]
    cu = dev(inp.cu_seqlens)
    plan = kda.KdaFwdPlan(*bufs[:5], scale=inp.scale, cu_seqlens=cu, initial_state=bufs[5])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan()
    for seed in (51, 52, 53):
        new = W.make_inputs(w, seed=seed)
        for b, x in zip(bufs, (new.q, new.k, new.v, new.g, new.beta, new.h0)):
            b.copy_(x.to(DEV))
        graph.replay()
        torch.cuda.synchronize()
        o_g, f_g = plan.o.float().cpu(), plan.final_state.cpu()
        o_e, f_e = run(new.q, new.k, new.v, new.g, new.beta, new.scale, h0=new.h0,
                       cu=new.cu_seqlens)
        assert torch.equal(o_g, o_e), f"o of replay (seed {seed}) differs from the eager run"
        assert torch.equal(f_g, f_e), f"final state of replay (seed {seed}) differs"
