"""GPU parity of the backward (kda_bwd through the C ABI) against the fp64 oracle of
oracle/backward.py, element by element.

Bar: relative L2 error ||x_gpu - x_ref|| / ||x_ref|| of each gradient tensor (dq, dk, dv, dg,
dbeta, dh0), computed in fp64, <= 1e-4 for bf16 and fp32 io alike: the kernels compute in fp32
from exactly the values the oracle reads (bf16 -> fp32 is exact), so the only error is fp32
rounding, as for the forward's fp32 io. Small cases compare every element. The full-size
workloads compare every unit against the C backward oracle (oracle/kda_oracle_bwd.c), with the
bar applied per (sequence, head) unit and per token row of every tensor (tests/parity_check.py).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import workloads as W
from errlog import report_named
from oracle.backward import kda_backward_recurrent

import chunked_kimi_delta_amd as kda

pytestmark = pytest.mark.gpu
TOL = 1e-4
DEV = "cuda:0"
ORACLE_THREADS = 16             # the CPU share of a one-GPU machine
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def dev(x):
    return None if x is None else x.to(DEV).contiguous()


def f64(x):
    return None if x is None else x.float().cpu().numpy().astype(np.float64)


def gpu_bwd(inp: W.Inputs, gr: W.Grads):
    plan = kda.KdaBwdPlan(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                          dev(gr.d_o), dev(gr.dht), scale=inp.scale,
                          cu_seqlens=dev(inp.cu_seqlens), initial_state=dev(inp.h0))
    out = plan()
    torch.cuda.synchronize()
    return tuple(f64(x) for x in out)


def oracle_bwd(inp: W.Inputs, gr: W.Grads):
    f = W.as_f32_numpy
    return kda_backward_recurrent(
        f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta), inp.scale,
        None if inp.h0 is None else inp.h0.numpy(),
        None if inp.cu_seqlens is None else inp.cu_seqlens.numpy(),
        f(gr.d_o), None if gr.dht is None else gr.dht.numpy())


def rel_l2(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def check_grads(got, ref, tol=TOL):
    errs = {}
    for name, a, b in zip(NAMES, got, ref):
        b = np.asarray(b).reshape(a.shape)
        assert np.isfinite(a).all(), name
        errs[name] = rel_l2(a, b)
    report_named(**errs)
    bad = {k: v for k, v in errs.items() if v > tol}
    assert not bad, f"rel L2 above {tol}: {bad}"


SMALL = {
    "fp32_t64": W.WORKLOADS["tiny_fp32"],
    "fp32_t45_h0": W.custom(B=1, T=45, H=1, HV=1, K=64, V=64, dtype="fp32", h0_std=0.5),
    "bf16_b2_t100_gva_h0": W.custom(B=2, T=100, H=2, HV=4, K=128, V=128, h0_std=0.1),
    "bf16_k64v128_t50": W.custom(B=1, T=50, H=1, HV=2, K=64, V=128),
    "bf16_k128v64_t50_h0": W.custom(B=1, T=50, H=2, HV=2, K=128, V=64, h0_std=0.1),
    "bf16_varlen_edges": W.custom(H=1, HV=2, K=128, V=128, h0_std=0.1,
                                  lengths=(0, 1, 15, 16, 17, 100, 33, 0)),
    "fp32_varlen_gva": W.custom(H=2, HV=4, K=128, V=128, dtype="fp32", h0_std=0.1,
                                lengths=(5, 40, 0, 16)),
    "bf16_strong_decay": W.custom(B=1, T=200, H=2, HV=2, K=128, V=128, g_lo=0.5, g_hi=0.9999,
                                  beta_std=2.0),
    "bf16_t1": W.custom(B=3, T=1, H=1, HV=1, K=128, V=128, h0_std=0.1),
    "bf16_g4_varlen": W.custom(H=1, HV=4, K=128, V=64, h0_std=0.2, lengths=(3, 0, 40, 17)),
    "fp32_k64v128_b3_t31": W.custom(B=3, T=31, H=2, HV=2, K=64, V=128, dtype="fp32"),
}


@pytest.mark.parametrize("with_dht", [True, False])
@pytest.mark.parametrize("name", list(SMALL))
def test_backward_small_parity(name, with_dht):
    inp = W.make_inputs(SMALL[name], seed=0)
    gr = W.make_grads(inp, seed=0, dht_std=1.0 if with_dht else None)
    check_grads(gpu_bwd(inp, gr), oracle_bwd(inp, gr))


def test_backward_is_deterministic():
    inp = W.make_inputs(SMALL["bf16_b2_t100_gva_h0"], seed=2)
    gr = W.make_grads(inp, seed=2)
    a, b = gpu_bwd(inp, gr), gpu_bwd(inp, gr)
    for name, x, y in zip(NAMES, a, b):
        assert np.array_equal(x, y), name


@pytest.mark.parametrize("io", ["bf16", "fp32"])
def test_backward_empty_sequences_pass_dht_through(io):
    w = W.custom(B=2, T=0, H=1, HV=2, K=128, V=64, dtype=io, h0_std=1.0)
    inp = W.make_inputs(w, seed=3)
    gr = W.make_grads(inp, seed=3)
    out = gpu_bwd(inp, gr)
    assert all(x.size == 0 for x in out[:5])
    assert np.array_equal(out[5], gr.dht.numpy().astype(np.float64))


def test_backward_beta0_gives_zero_dk_dv():
    # with beta = 0 nothing is written to the state: k and v reach no output, so their
    # gradients are exactly zero; the rest must still match the oracle
    w = W.custom(B=1, T=90, H=2, HV=2, K=128, V=128, h0_std=0.5)
    inp = W.make_inputs(w, seed=5, beta_override=0.0)
    gr = W.make_grads(inp, seed=5)
    got = gpu_bwd(inp, gr)
    assert not got[1].any() and not got[2].any()
    check_grads(got, oracle_bwd(inp, gr))


def test_backward_g0_matches_oracle():
    w = W.custom(B=1, T=90, H=2, HV=2, K=128, V=128, h0_std=0.5)
    inp = W.make_inputs(w, seed=6, g_override=0.0)
    gr = W.make_grads(inp, seed=6)
    check_grads(gpu_bwd(inp, gr), oracle_bwd(inp, gr))


def gpu_bwd_f32(inp: W.Inputs, gr: W.Grads):
    """The GPU gradients as float32 numpy arrays (full-size workloads: half the memory of
    float64 copies; the checks convert one head at a time)."""
    plan = kda.KdaBwdPlan(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                          dev(gr.d_o), dev(gr.dht), scale=inp.scale,
                          cu_seqlens=dev(inp.cu_seqlens), initial_state=dev(inp.h0))
    out = plan()
    torch.cuda.synchronize()
    res = tuple(None if x is None else x.float().cpu().numpy() for x in out[:6])
    del plan, out
    return res


@pytest.mark.parametrize("name", ["h16_t4096", "varlen8_h32", "gva_b4_t8192", "long_t131072"])
def test_backward_full_size_every_unit(name):
    # every unit of the workload against the C backward oracle, both bars on every tensor
    from oracle.native import kda_oracle_bwd_c
    from parity_check import check_grads as check_every_unit
    w = W.WORKLOADS[name]
    inp = W.make_inputs(w, seed=0)
    gr = W.make_grads(inp, seed=0)
    print(f"[bwd full] {name}: GPU backward", file=sys.stderr, flush=True)
    got = gpu_bwd_f32(inp, gr)
    print(f"[bwd full] {name}: oracle over every unit", file=sys.stderr, flush=True)
    f = W.as_f32_numpy
    ref = kda_oracle_bwd_c(f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta), inp.scale,
                           None if inp.h0 is None else inp.h0.numpy(),
                           None if inp.cu_seqlens is None else inp.cu_seqlens.numpy(),
                           f(gr.d_o), None if gr.dht is None else gr.dht.numpy(),
                           n_threads=ORACLE_THREADS)
    print(f"[bwd full] {name}: compare", file=sys.stderr, flush=True)
    worst = check_every_unit(got, ref, inp.seq_bounds(), what=name)
    report_named(**worst)


# --------------------------------------------------------------------------- with the pre-stage

PRE_SHAPES = {
    "bf16_gva_b2_t100_h0": W.custom(B=2, T=100, H=2, HV=4, K=128, V=128, h0_std=0.1),
    "bf16_varlen_edges": W.custom(H=1, HV=2, K=128, V=128, h0_std=0.1,
                                  lengths=(0, 1, 17, 33, 64)),
    "bf16_k64v64_t50": W.custom(B=1, T=50, H=2, HV=2, K=64, V=64),
    "fp32_k128v64_t70": W.custom(B=1, T=70, H=1, HV=2, K=128, V=64, dtype="fp32"),
    "bf16_k64v128_g4_varlen": W.custom(H=1, HV=4, K=64, V=128, h0_std=0.1,
                                       lengths=(20, 0, 49)),
}
PNAMES = NAMES + ("dA_log", "ddt_bias")


def gpu_bwd_raw(raw: W.RawInputs, gr: W.Grads, pre):
    inp = raw.inp
    plan = kda.KdaBwdPlan(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                          dev(gr.d_o), dev(gr.dht), scale=inp.scale,
                          cu_seqlens=dev(inp.cu_seqlens), initial_state=dev(inp.h0),
                          use_qk_l2norm=pre.get("l2", False),
                          use_beta_sigmoid=pre.get("sig", False), gate=pre.get("gate"),
                          A_log=dev(raw.A_log), dt_bias=dev(pre.get("dt", raw.dt_bias)),
                          gate_lower_bound=pre.get("lb", -5.0))
    out = plan()
    torch.cuda.synchronize()
    return tuple(f64(x) for x in out)


def oracle_bwd_raw(raw: W.RawInputs, gr: W.Grads, pre):
    from oracle.backward import kda_backward_raw
    inp = raw.inp
    f = W.as_f32_numpy
    dt = pre.get("dt", raw.dt_bias)
    return kda_backward_raw(
        f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta), inp.scale,
        None if inp.h0 is None else inp.h0.numpy(),
        None if inp.cu_seqlens is None else inp.cu_seqlens.numpy(),
        f(gr.d_o), None if gr.dht is None else gr.dht.numpy(),
        pre.get("l2", False), pre.get("sig", False), pre.get("gate"), raw.A_log.numpy(),
        None if dt is None else dt.numpy(), pre.get("lb", -5.0))


def check_raw(got, ref, pre):
    check_grads(got[:6], ref[:6])
    if pre.get("gate"):
        errs = {n: rel_l2(a, b) for n, a, b in zip(PNAMES[6:], got[6:], ref[6:])}
        report_named(**errs)
        assert all(e <= TOL for e in errs.values()), errs
    else:
        assert got[6] is None and got[7] is None


@pytest.mark.parametrize("gate", ["softplus", "bounded"])
@pytest.mark.parametrize("name", list(PRE_SHAPES))
def test_backward_prestage_parity(name, gate):
    raw = W.make_raw_inputs(PRE_SHAPES[name], seed=31)
    gr = W.make_grads(raw.inp, seed=31)
    pre = {"l2": True, "sig": True, "gate": gate, "lb": -4.0}
    check_raw(gpu_bwd_raw(raw, gr, pre), oracle_bwd_raw(raw, gr, pre), pre)


@pytest.mark.parametrize("step", ["l2", "sig", "softplus_no_bias", "bounded"])
def test_backward_prestage_steps_one_at_a_time(step):
    pre = {"l2": {"l2": True}, "sig": {"sig": True},
           "softplus_no_bias": {"gate": "softplus", "dt": None},
           "bounded": {"gate": "bounded", "lb": -6.0}}[step]
    # the ordinary inputs (unit q, k rows, log decays, beta in (0, 1)) with the raw form of the
    # one input the step activates: unnormalised q, k would make the recurrence diverge
    raw = W.make_raw_inputs(W.custom(B=1, T=45, H=2, HV=4, K=128, V=128, h0_std=0.2), seed=7)
    base = W.make_inputs(raw.inp.w, seed=7)
    if "l2" in pre:
        base.q, base.k = raw.inp.q, raw.inp.k
    if "sig" in pre:
        base.beta = base.beta * 4 - 2
    if "gate" in pre:
        base.g = raw.inp.g
    raw = W.RawInputs(base, raw.A_log, raw.dt_bias)
    gr = W.make_grads(raw.inp, seed=7)
    check_raw(gpu_bwd_raw(raw, gr, pre), oracle_bwd_raw(raw, gr, pre), pre)


def test_backward_prestage_full_size_bounded_gate():
    # every unit of h16_t4096 (dA_log and dt_bias sum over all of them)
    raw = W.make_raw_inputs(W.WORKLOADS["h16_t4096"], seed=3)
    gr = W.make_grads(raw.inp, seed=3)
    pre = {"l2": True, "sig": True, "gate": "bounded", "lb": -5.0}
    print("[bwd pre full] GPU backward", file=sys.stderr, flush=True)
    got = gpu_bwd_raw(raw, gr, pre)
    print("[bwd pre full] oracle", file=sys.stderr, flush=True)
    ref = oracle_bwd_raw(raw, gr, pre)
    check_raw(got, ref, pre)
    # and per unit / per row on the six input gradients, per value head on the parameters
    from parity_check import check_grads as check_every_unit
    worst = check_every_unit(got[:6], ref[:6], raw.inp.seq_bounds(), what="prestage h16_t4096")
    report_named(**worst)
    # each head's parameter gradient within TOL x (its norm + the rms over heads), the row
    # bar's form: a sum over every token can cancel to a small value in one head
    dA, dA_ref = got[6], np.asarray(ref[6]).reshape(got[6].shape)
    rms = np.sqrt(np.mean(dA_ref ** 2))
    assert np.all(np.abs(dA - dA_ref) <= TOL * (np.abs(dA_ref) + rms)), "dA_log off in a head"
    ddt, ddt_ref = got[7], np.asarray(ref[7]).reshape(got[7].shape)
    nrm = np.linalg.norm(ddt_ref, axis=-1)
    bad = np.linalg.norm(ddt - ddt_ref, axis=-1) > TOL * (nrm + np.sqrt(np.mean(nrm ** 2)))
    assert not bad.any(), f"ddt_bias off in head {int(np.argmax(bad))}"


# --------------------------------------------------------------------------- torch.autograd

@pytest.mark.parametrize("pre", [{}, {"l2": True, "sig": True, "gate": "bounded", "lb": -4.0}],
                         ids=["plain", "prestage"])
def test_chunk_kda_autograd_matches_oracle(pre):
    # loss = sum(o * d_o) + sum(final * dht) through chunk_kda: torch.autograd drives kda_fwd
    # and kda_bwd; the gradients (cast to the inputs' dtypes) against the fp64 oracle
    from oracle.backward import kda_backward_raw
    w = W.custom(B=1, T=50, H=2, HV=4, K=64, V=64, dtype="fp32", h0_std=0.3)
    raw = W.make_raw_inputs(w, seed=11) if pre else None
    inp = raw.inp if pre else W.make_inputs(w, seed=11)
    gr = W.make_grads(inp, seed=11)
    leaf = lambda x: None if x is None else dev(x).requires_grad_(True)
    q, k, v, g, beta, h0 = map(leaf, (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0))
    A_log = leaf(raw.A_log) if pre else None
    dt_bias = leaf(raw.dt_bias) if pre else None
    o, fin = kda.chunk_kda(q, k, v, g, beta, scale=inp.scale, initial_state=h0,
                           use_qk_l2norm=pre.get("l2", False),
                           use_beta_sigmoid=pre.get("sig", False), gate=pre.get("gate"),
                           A_log=A_log, dt_bias=dt_bias,
                           gate_lower_bound=pre.get("lb", -5.0))
    loss = (o * dev(gr.d_o)).sum() + (fin * dev(gr.dht)).sum()
    leaves = [q, k, v, g, beta, h0] + ([A_log, dt_bias] if pre else [])
    got = torch.autograd.grad(loss, leaves)
    f = W.as_f32_numpy
    ref = kda_backward_raw(f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta), inp.scale,
                           inp.h0.numpy(), None, f(gr.d_o), gr.dht.numpy(),
                           pre.get("l2", False), pre.get("sig", False), pre.get("gate"),
                           raw.A_log.numpy() if pre else None,
                           raw.dt_bias.numpy() if pre else None, pre.get("lb", -5.0))
    for name, a, b in zip(PNAMES, got, ref):
        assert a.dtype == torch.float32, name
        e = rel_l2(a.detach().cpu().numpy(), np.asarray(b).reshape(a.shape))
        assert e <= TOL, (name, e)
