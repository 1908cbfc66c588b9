"""kda_fwd_noalloc (the forward with its workspace in the library's static device array),
called through the C ABI: its outputs equal those of kda_fwd with a caller-allocated workspace
bit for bit, and meet the oracle's parity bars, on calls in a row that reuse the array with a
smaller input after a larger one."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import workloads as W
import chunked_kimi_delta_amd as kda
from chunked_kimi_delta_amd import _lib
from oracle.native import kda_oracle_c
from parity_check import check_outputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(x):
    return None if x is None else x.to(DEV).contiguous()


def plans(inp, chunk):
    """Two plans over the same inputs with separate outputs: one for kda_fwd (its own
    workspace), one whose argument struct kda_fwd_noalloc gets."""
    mk = lambda: kda.KdaFwdPlan(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                                cu_seqlens=dev(inp.cu_seqlens), initial_state=dev(inp.h0),
                                chunk=chunk)
    return mk(), mk()


def noalloc(plan):
    lib = _lib.load()
    stream = torch.cuda.current_stream(torch.device(DEV))
    st = lib.kda_fwd_noalloc(ctypes.byref(plan.args), ctypes.c_void_p(stream.cuda_stream))
    assert st == _lib.KDA_OK, _lib.strerror(st)
    return plan.o, plan.final_state


def oracle(inp):
    f = W.as_f32_numpy
    return kda_oracle_c(f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta), inp.scale,
                        None if inp.h0 is None else inp.h0.numpy(),
                        None if inp.cu_seqlens is None else inp.cu_seqlens.numpy(),
                        n_threads=16)


@pytest.mark.parametrize("chunk", [64, 32, 16, 1])
def test_noalloc_matches_kda_fwd_on_consecutive_calls(chunk):
    cases = [W.WORKLOADS["h16_t4096"],                                  # 72 MB of records
             W.custom(B=2, T=100, H=2, HV=4, K=128, V=128, h0_std=0.1),  # then a smaller one
             W.custom(H=1, HV=2, K=64, V=128, h0_std=0.1, lengths=(0, 17, 40))]
    for i, w in enumerate(cases):
        inp = W.make_inputs(w, seed=40 + i)
        ref_plan, na_plan = plans(inp, chunk)
        o_ref, f_ref = ref_plan()
        o_na, f_na = noalloc(na_plan)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ref) and torch.equal(f_na, f_ref), f"case {i}"
        o64, f64 = oracle(inp)
        check_outputs(o_na.float().cpu().numpy(), f_na.cpu().numpy().astype(np.float64),
                      o64, f64, inp.seq_bounds(), w.dtype, what=f"noalloc case {i}")


def test_noalloc_rejects_shapes_beyond_its_array():
    lib = _lib.load()
    a = _lib.KdaFwdArgs()
    # 32 value heads of 131,072 tokens need about 4.6 GB of chunk records
    for k, v in dict(B=1, T=131072, N=1, H=32, HV=32, K=128, V=128, io=0, chunk=32).items():
        setattr(a, k, v)
    assert lib.kda_fwd_workspace_bytes(ctypes.byref(a)) > _lib.KDA_NOALLOC_WORKSPACE_BYTES
    st = lib.kda_fwd_noalloc(ctypes.byref(a), None)
    assert st == _lib.KDA_ERR_NOALLOC_TOO_LARGE
    assert "128 MiB" in _lib.strerror(st)
