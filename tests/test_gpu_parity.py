"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by element.

Bars (tests/parity_check.py states and derives them): for o and final_state, the relative L2
error over every (sequence, value head) unit, computed in fp64, is
    bf16 io  <= 5e-3        fp32 io  <= 1e-4
and every row (one token of o, one key row of the final state) satisfies
||x_row - ref_row|| <= tol_row (||ref_row|| + rms row norm of its unit)  (bf16 5e-3, fp32 1e-4).
Every case compares every unit, including the full-size workloads in the launch configuration
bench.py times; the oracle of a full-size workload is computed once per module and shared by
its chunk variants.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle.chunked import chunk_prepare
from oracle.native import kda_oracle_c
from errlog import report_named
from parity_check import TOL, check_outputs, rel_l2
from ws_decode import (chunk_bytes, chunk_bytes32, decode_chunk, decode_chunk32,
                       decode_pair, pair_bytes)

import chunked_kimi_delta_amd as kda

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
# host threads for the oracle: the CPU share of a one-GPU machine
ORACLE_THREADS = 16


def dev(x):
    return None if x is None else x.to(DEV).contiguous()


def gpu_plan(inp: W.Inputs, scale=None, output_final_state=True, chunk=0):
    return kda.KdaFwdPlan(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                          scale=scale, cu_seqlens=dev(inp.cu_seqlens),
                          initial_state=dev(inp.h0), output_final_state=output_final_state,
                          chunk=chunk)


def gpu_run(inp: W.Inputs, **kw):
    """Run the forward through the C ABI (kwargs go to KdaFwdPlan); o as fp32 numpy (exact for
    bf16 values), the final state as fp64 numpy."""
    plan = gpu_plan(inp, **kw)
    o, fin = plan()
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    fin = None if fin is None else fin.cpu().numpy().astype(np.float64)
    return o, fin


def oracle_run(inp: W.Inputs, units=None, scale=None):
    f = W.as_f32_numpy
    return kda_oracle_c(f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta),
                        inp.scale if scale is None else scale,
                        None if inp.h0 is None else inp.h0.numpy(),
                        None if inp.cu_seqlens is None else inp.cu_seqlens.numpy(),
                        units=units, n_threads=ORACLE_THREADS)


def check_all(inp, o, fin, o_ref, f_ref, dtype, units=None, what=""):
    """Both bars of parity_check on o and (when present) the final state; the worst unit and
    row errors go to the error log."""
    worst = check_outputs(o, fin, o_ref, f_ref, inp.seq_bounds(), dtype, units=units,
                          what=what)
    report_named(**worst)
    return worst


SMALL = {
    "tiny_fp32": W.WORKLOADS["tiny_fp32"],
    "bf16_b2_t100_gva_h0": W.custom(B=2, T=100, H=2, HV=4, K=128, V=128, h0_std=0.1),
    "bf16_k64v64_t77": W.custom(B=1, T=77, H=3, HV=3, K=64, V=64),
    "bf16_k64v128_t50": W.custom(B=1, T=50, H=1, HV=2, K=64, V=128),
    "bf16_k128v64_t50_h0": W.custom(B=1, T=50, H=2, HV=2, K=128, V=64, h0_std=0.1),
    "bf16_varlen_edges": W.custom(H=1, HV=2, K=128, V=128, h0_std=0.1,
                                  lengths=(0, 1, 15, 16, 17, 100, 33, 0)),
    "bf16_strong_decay": W.custom(B=1, T=200, H=2, HV=2, K=128, V=128, g_lo=0.5, g_hi=0.9999,
                                  beta_std=2.0),
    "bf16_t1": W.custom(B=3, T=1, H=1, HV=1, K=128, V=128, h0_std=0.1),
    "fp32_varlen_gva": W.custom(H=2, HV=4, K=128, V=128, dtype="fp32", h0_std=0.1,
                                lengths=(5, 40, 0, 16)),
    "fp32_k64v128_t70": W.custom(B=2, T=70, H=1, HV=1, K=64, V=128, dtype="fp32"),
    # enough (sequence, head, 16-column slice) units that the 32-token state kernel groups 2
    # and 4 slices per workgroup (512 and 1024 slice units on a 256-CU part)
    "bf16_b4_h16_t70_slices2": W.custom(B=4, T=70, H=8, HV=16, K=128, V=128, h0_std=0.1),
    "bf16_b8_h16_t45_slices4": W.custom(B=8, T=45, H=16, HV=16, K=128, V=128),
    "bf16_b16_h16_k64v64_slices4": W.custom(B=16, T=40, H=16, HV=16, K=64, V=64, h0_std=0.1),
    # packed sequences run longest first: tied and empty lengths (ties keep the input order),
    # uneven lengths with enough units for four slices per workgroup, exactly 64 sequences
    # (every lane of the ranking wave holds one) and more than 64 (input order)
    "bf16_varlen_ties_h0": W.custom(H=1, HV=2, K=128, V=128, h0_std=0.1,
                                    lengths=(40, 100, 40, 0, 100, 0, 7)),
    "bf16_varlen_gva_slices4": W.custom(H=8, HV=16, K=128, V=128, h0_std=0.1,
                                        lengths=(3, 70, 150, 64, 33, 0, 97, 12)),
    "bf16_varlen_n64": W.custom(H=1, HV=2, K=64, V=64,
                                lengths=tuple((5 * i) % 37 for i in range(64))),
    "bf16_varlen_n70": W.custom(H=1, HV=1, K=64, V=64,
                                lengths=tuple((7 * i) % 23 for i in range(70))),
    # dense batches of at least 16 chunks whose value slices fill at most half of a 256-CU part:
    # at chunk 32 the state pass runs as two segments (the second from a zero state next to
    # its transition, then the correction); ragged last chunks, an initial state, grouped value
    # heads, K = V = 64 and strong decays
    "bf16_split_t600_h0": W.custom(B=1, T=600, H=2, HV=2, K=128, V=128, h0_std=0.1),
    "bf16_split_gva_k64_t1000": W.custom(B=2, T=1000, H=1, HV=2, K=64, V=64, h0_std=0.1),
    "bf16_split_strong_t700": W.custom(B=1, T=700, H=1, HV=1, K=128, V=128, g_lo=0.5,
                                       g_hi=0.9999, beta_std=2.0),
    # exactly 16 chunks (the smallest split: 9 + 7), three heads (padded workgroups)
    "bf16_split_t512_h3": W.custom(B=1, T=512, H=3, HV=3, K=128, V=128),
}


# chunk lengths the library offers per io dtype (0 = its default)
CHUNKS = {"bf16": [1, 16, 32, 64], "fp32": [1, 16]}
SMALL_CASES = [(n, c) for n in SMALL for c in CHUNKS[SMALL[n].dtype]]


@pytest.mark.parametrize("name,chunk", SMALL_CASES)
def test_small_parity(name, chunk):
    w = SMALL[name]
    inp = W.make_inputs(w, seed=0)
    o, fin = gpu_run(inp, chunk=chunk)
    o_ref, f_ref = oracle_run(inp)
    check_all(inp, o, fin, o_ref, f_ref, w.dtype, what=f"{name} chunk {chunk}")


@pytest.mark.parametrize("io,chunk", [("bf16", 1), ("bf16", 16), ("bf16", 32), ("bf16", 64),
                                      ("fp32", 1), ("fp32", 16)])
def test_empty_sequences_carry_initial_state(io, chunk):
    w = W.custom(B=2, T=0, H=1, HV=2, K=128, V=64, dtype=io, h0_std=1.0)
    inp = W.make_inputs(w, seed=3)
    o, fin = gpu_run(inp, chunk=chunk)
    assert o.size == 0
    assert np.array_equal(fin, inp.h0.numpy().astype(np.float64))


@pytest.mark.parametrize("chunk", [1, 16, 32, 64])
@pytest.mark.parametrize("case", ["beta0", "g0"])
def test_degenerate_gates(case, chunk):
    w = W.custom(B=1, T=90, H=2, HV=2, K=128, V=128, h0_std=0.5)
    kw = {"beta_override": 0.0} if case == "beta0" else {"g_override": 0.0}
    inp = W.make_inputs(w, seed=5, **kw)
    o, fin = gpu_run(inp, chunk=chunk)
    o_ref, f_ref = oracle_run(inp)
    check_all(inp, o, fin, o_ref, f_ref, "bf16")
    if case == "beta0":   # pure decay: the state never receives a write
        S0 = inp.h0.numpy().astype(np.float64)
        cum = np.cumsum(W.as_f32_numpy(inp.g)[0].astype(np.float64), axis=0)[-1]
        assert rel_l2(fin[0], np.exp(cum)[:, :, None] * S0[0]) <= 1e-3


@pytest.mark.parametrize("chunk", [1, 16, 32, 64])
def test_deltanet_retrieval_property(chunk):
    # g = 0, beta = 1 and one fixed unit key shared by all tokens with q = k: each output
    # returns scale * v_t (the plain delta rule overwrites the memory slot every token)
    T, K, V = 64, 128, 128
    gen = torch.Generator().manual_seed(11)
    kv = torch.randn(K, generator=gen)
    kv = (kv / kv.norm()).to(torch.bfloat16)
    kvf = kv.float()
    kv = (kvf / kvf.norm()).to(torch.bfloat16)   # unit to bf16 precision
    k = kv.expand(1, T, 1, K).contiguous()
    inp = W.Inputs(W.custom(B=1, T=T, H=1, HV=1, K=K, V=V), k.clone(), k,
                   torch.randn(1, T, 1, V, generator=gen).to(torch.bfloat16),
                   torch.zeros(1, T, 1, K, dtype=torch.bfloat16),
                   torch.ones(1, T, 1, dtype=torch.bfloat16), None, None, scale=0.5)
    o, fin = gpu_run(inp, scale=0.5, chunk=chunk)
    o_ref, f_ref = oracle_run(inp)
    check_all(inp, o, fin, o_ref, f_ref, "bf16")
    nk2 = float((kv.float() ** 2).sum())
    assert rel_l2(o[0, :, 0], 0.5 * nk2 * inp.v.float().numpy()[0, :, 0]) <= 2e-2


@pytest.mark.parametrize("chunk", [1, 16, 32, 64])
@pytest.mark.parametrize("T", [64, 1000])      # 1000 tokens at chunk 32: the two-segment pass
def test_no_final_state_and_explicit_scale(chunk, T):
    w = W.custom(B=1, T=T, H=1, HV=2, K=128, V=128)
    inp = W.make_inputs(w, seed=2)
    o, fin = gpu_run(inp, scale=0.3, output_final_state=False, chunk=chunk)
    assert fin is None
    o_ref, _ = oracle_run(inp, scale=0.3)
    check_all(inp, o, None, o_ref, None, "bf16", what=f"no final state, T {T}")


@pytest.mark.parametrize("chunk", [1, 16, 32, 64])
def test_deterministic_and_repeatable(chunk):
    w = W.custom(B=1, T=300, H=2, HV=2, K=128, V=128, h0_std=0.1)
    inp = W.make_inputs(w, seed=4)
    plan = gpu_plan(inp, chunk=chunk)
    o1, f1 = [x.clone() for x in plan()]
    o2, f2 = plan()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_prepare_workspace_matches_chunk_oracle():
    # stage-1 diagnostics: decode w, qd, kr, u, Mqk, exp(gam) of sampled chunks (including a
    # tail chunk) and compare with the fp64 chunked-form intermediates
    w = W.custom(B=1, T=37, H=1, HV=2, K=128, V=128)
    inp = W.make_inputs(w, seed=6)
    plan = gpu_plan(inp, chunk=16)
    plan()
    torch.cuda.synchronize()
    ws = plan.workspace.cpu().numpy()
    cb = chunk_bytes(128, 128)
    n_slots = 37 // 16 + 1
    f = W.as_f32_numpy
    for j in range(2):
        prep = chunk_prepare(f(inp.q)[0, :, 0], f(inp.k)[0, :, 0], f(inp.v)[0, :, j],
                             f(inp.g)[0, :, j], f(inp.beta)[0, :, j], inp.scale, 16)
        for c in range(3):
            off = (j * n_slots + c) * cb
            got = decode_chunk(ws[off:off + cb], 128, 128)
            for key in ("w", "qd", "kr", "u", "Mqk", "eg"):
                ref = prep[key][c]
                err = rel_l2(got[key], ref)
                assert err <= 1e-2, f"head {j} chunk {c} {key}: rel L2 {err:.2e}"


def test_prepare32_workspace_matches_chunk_oracle():
    # stage-1 diagnostics of the 32-token record (two blocks joined by block substitution)
    w = W.custom(B=1, T=77, H=1, HV=2, K=128, V=128)
    inp = W.make_inputs(w, seed=8)
    plan = gpu_plan(inp, chunk=32)
    plan()
    torch.cuda.synchronize()
    ws = plan.workspace.cpu().numpy()
    cb = chunk_bytes32(128, 128)
    n_slots = 77 // 32 + 1
    f = W.as_f32_numpy
    for j in range(2):
        prep = chunk_prepare(f(inp.q)[0, :, 0], f(inp.k)[0, :, 0], f(inp.v)[0, :, j],
                             f(inp.g)[0, :, j], f(inp.beta)[0, :, j], inp.scale, 32)
        for c in range(3):
            off = (j * n_slots + c) * cb
            got = decode_chunk32(ws[off:off + cb], 128, 128)
            for key in ("w", "qd", "kr", "u", "Mqk", "eg"):
                err = rel_l2(got[key], prep[key][c])
                assert err <= 1e-2, f"head {j} chunk {c} {key}: rel L2 {err:.2e}"


def test_prepare64_workspace_matches_chunk_oracle():
    # stage-1 diagnostics of the 64-token pair records: the first record of each pair is the
    # 32-token record of its chunk; the second holds its chunk's record with W scaled by the
    # first chunk's e^{gam} per key dim and P = W_second KR_first^T; a pair whose second chunk
    # is empty carries the identity step there
    w = W.custom(B=1, T=150, H=1, HV=2, K=128, V=128)
    inp = W.make_inputs(w, seed=9)
    plan = gpu_plan(inp, chunk=64)
    plan()
    torch.cuda.synchronize()
    ws = plan.workspace.cpu().numpy()
    pb = pair_bytes(128, 128)
    n_pairs = 150 // 64 + 1
    f = W.as_f32_numpy
    for j in range(2):
        prep = chunk_prepare(f(inp.q)[0, :, 0], f(inp.k)[0, :, 0], f(inp.v)[0, :, j],
                             f(inp.g)[0, :, j], f(inp.beta)[0, :, j], inp.scale, 32)
        nch = len(prep["w"])                       # 5 chunks of 32 tokens, the last ragged
        for m in range(n_pairs):
            off = (j * n_pairs + m) * 2 * pb
            first, second = decode_pair(ws[off:off + 2 * pb], 128, 128)
            c0, c1 = 2 * m, 2 * m + 1
            for key in ("w", "qd", "kr", "u", "Mqk", "eg"):
                err = rel_l2(first[key], prep[key][c0])
                assert err <= 1e-2, f"head {j} chunk {c0} {key}: rel L2 {err:.2e}"
            if c1 >= nch:                          # empty second chunk: the identity step
                for key in ("w", "qd", "kr", "u", "Mqk", "P"):
                    assert not np.any(second[key]), key
                assert np.all(second["eg"] == 1.0)
                continue
            ref = {k: prep[k][c1] for k in prep}
            ref["w"] = prep["w"][c1] * prep["eg"][c0][None, :]
            ref["P"] = prep["w"][c1] @ prep["kr"][c0].T
            for key in ("w", "qd", "kr", "u", "Mqk", "eg", "P"):
                err = rel_l2(second[key], ref[key])
                assert err <= 1e-2, f"head {j} chunk {c1} {key}: rel L2 {err:.2e}"


FULL = ["h16_t4096", "varlen8_h32", "gva_b4_t8192", "long_t131072"]
_FULL_CACHE: dict = {}


def full_case(name):
    """Inputs and the oracle's outputs of a full-size workload, computed once per module (every
    unit of every sequence and head)."""
    if name not in _FULL_CACHE:
        _FULL_CACHE.clear()              # one workload at a time in memory
        inp = W.make_inputs(W.WORKLOADS[name], seed=0)
        print(f"[full] {name}: oracle over every unit", file=sys.stderr, flush=True)
        _FULL_CACHE[name] = (inp, oracle_run(inp))
    return _FULL_CACHE[name]


@pytest.mark.parametrize("chunk", [64, 32, 16, 1])
@pytest.mark.parametrize("name", FULL)          # outermost: one oracle run per workload
def test_full_size_every_unit(name, chunk):
    inp, (o_ref, f_ref) = full_case(name)
    print(f"[full] {name}: GPU forward, chunk {chunk}", file=sys.stderr, flush=True)
    o, fin = gpu_run(inp, chunk=chunk)
    check_all(inp, o, fin, o_ref, f_ref, inp.w.dtype, what=f"{name} chunk {chunk}")


@pytest.mark.parametrize("chunk", [1, 16])
def test_full_size_fp32_every_unit(chunk):
    # the fp32 mode at the benchmark's size: every (sequence, head) against the oracle
    w = W.WORKLOADS["h16_t4096_fp32"]
    inp = W.make_inputs(w, seed=0)
    o, fin = gpu_run(inp, chunk=chunk)
    o_ref, f_ref = oracle_run(inp)
    check_all(inp, o, fin, o_ref, f_ref, "fp32", what=f"h16_t4096_fp32 chunk {chunk}")


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_prepare_records_repeat_bitwise_full_size(chunk):
    # every chunk record of the h16_t4096 workload, written twice into a zeroed workspace, is
    # the same bits both times (a lost or torn record store shows up as a difference)
    w = W.WORKLOADS["h16_t4096"]
    inp = W.make_inputs(w, seed=0)
    plan = gpu_plan(inp, chunk=chunk)
    runs = []
    for _ in range(3):
        plan.workspace.zero_()
        plan.prepare()
        torch.cuda.synchronize()
        runs.append(plan.workspace.clone())
    for r in runs[1:]:
        assert torch.equal(runs[0], r)


@pytest.mark.parametrize("T", [1, 16, 17])
def test_default_chunk_short_dense_batches(T):
    # chunk 0: the token recurrence for T <= 16 (decode steps), 32-token chunks above
    w = W.custom(B=4, T=T, H=2, HV=4, K=128, V=128, h0_std=0.1)
    inp = W.make_inputs(w, seed=13)
    o, fin = gpu_run(inp, chunk=0)
    o_ref, f_ref = oracle_run(inp)
    check_all(inp, o, fin, o_ref, f_ref, "bf16")


# --------------------------------------------------------------------------- fused pre-stage

def raw_plan(raw, chunk, pre, output_final_state=True):
    inp = raw.inp
    return kda.KdaFwdPlan(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                          cu_seqlens=dev(inp.cu_seqlens), initial_state=dev(inp.h0),
                          output_final_state=output_final_state, chunk=chunk,
                          use_qk_l2norm=pre.get("l2", False),
                          use_beta_sigmoid=pre.get("sig", False), gate=pre.get("gate"),
                          A_log=dev(raw.A_log), dt_bias=dev(raw.dt_bias),
                          gate_lower_bound=pre.get("lb", -5.0))


def raw_oracle(raw, pre, units=None):
    # the pre-stage in fp64 (oracle/prestage.py), then the recurrence: fp64 numpy for small
    # cases; the C recurrence (inputs rounded to fp32, ~1e-7) when units are sampled
    from oracle.prestage import prestage
    from oracle.recurrent import kda_recurrent
    inp = raw.inp
    f = W.as_f32_numpy
    q, k, g, beta = prestage(f(inp.q), f(inp.k), f(inp.g), f(inp.beta),
                             qk_l2norm=pre.get("l2", False), beta_sigmoid=pre.get("sig", False),
                             gate=pre.get("gate"), A_log=raw.A_log.numpy(),
                             dt_bias=raw.dt_bias.numpy(), lower_bound=pre.get("lb", -5.0))
    h0 = None if inp.h0 is None else inp.h0.numpy()
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()
    if units is None:
        return kda_recurrent(q, k, f(inp.v), g, beta, inp.scale, h0, cu)
    return kda_oracle_c(q, k, f(inp.v), g, beta, inp.scale, h0, cu, units=units,
                        n_threads=ORACLE_THREADS)


PRE_SHAPES = {
    "bf16_gva_b2_t100_h0": W.custom(B=2, T=100, H=2, HV=4, K=128, V=128, h0_std=0.1),
    "bf16_varlen_edges": W.custom(H=1, HV=2, K=128, V=128, h0_std=0.1,
                                  lengths=(0, 1, 17, 33, 64)),
    "bf16_k64v64_t50": W.custom(B=1, T=50, H=2, HV=2, K=64, V=64),
    "fp32_k128v64_t70": W.custom(B=1, T=70, H=1, HV=2, K=128, V=64, dtype="fp32"),
}
PRE_CASES = [(n, c, gate) for n in PRE_SHAPES for c in CHUNKS[PRE_SHAPES[n].dtype]
             for gate in ("softplus", "bounded")]


@pytest.mark.parametrize("name,chunk,gate", PRE_CASES)
def test_prestage_parity(name, chunk, gate):
    # raw q/k, raw gate input, beta logits: all three pre-stage steps inside the kernels
    w = PRE_SHAPES[name]
    raw = W.make_raw_inputs(w, seed=21)
    pre = {"l2": True, "sig": True, "gate": gate, "lb": -4.0}
    plan = raw_plan(raw, chunk, pre)
    o, fin = plan()
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    fin = fin.cpu().numpy().astype(np.float64)
    o_ref, f_ref = raw_oracle(raw, pre)
    check_all(raw.inp, o, fin, o_ref, f_ref, w.dtype)


@pytest.mark.parametrize("chunk", [1, 16, 32, 64])
@pytest.mark.parametrize("pre", [{"l2": True}, {"sig": True}, {"gate": "softplus"},
                                 {"gate": "bounded", "lb": -2.5}],
                         ids=["l2norm", "beta_sigmoid", "softplus_gate", "bounded_gate"])
def test_prestage_steps_one_at_a_time(pre, chunk):
    w = W.custom(B=1, T=77, H=2, HV=2, K=128, V=128, h0_std=0.1)
    raw = W.make_raw_inputs(w, seed=22)
    if not pre.get("sig"):           # logits are not a valid beta: use a plain one
        raw.inp.beta = torch.sigmoid(raw.inp.beta.float()).to(raw.inp.beta.dtype)
    if not pre.get("l2"):            # unnormalised q, k of std 2 would make the state blow up
        raw.inp.q = (raw.inp.q.float() / 23.0).to(raw.inp.q.dtype)
        raw.inp.k = (raw.inp.k.float() / 23.0).to(raw.inp.k.dtype)
    if not pre.get("gate"):          # the raw gate input is not a decay: use a plain one
        raw.inp.g = (-torch.rand(raw.inp.g.shape, generator=torch.Generator().manual_seed(3))
                     * 0.1).to(raw.inp.g.dtype)
    o, fin = raw_plan(raw, chunk, pre)()
    torch.cuda.synchronize()
    o_ref, f_ref = raw_oracle(raw, pre)
    check_all(raw.inp, o.float().cpu().numpy(), fin.cpu().numpy().astype(np.float64), o_ref,
              f_ref, "bf16")


def test_prestage_full_size_bounded_gate():
    # the throughput shape with raw inputs and FlashKDA's bounded gate (lower bound -5), every
    # unit against the oracle
    w = W.WORKLOADS["h16_t4096"]
    raw = W.make_raw_inputs(w, seed=0)
    pre = {"l2": True, "sig": True, "gate": "bounded", "lb": -5.0}
    o, fin = raw_plan(raw, 32, pre)()
    torch.cuda.synchronize()
    units = [(0, j) for j in range(w.HV)]
    o_ref, f_ref = raw_oracle(raw, pre, units=units)
    check_all(raw.inp, o.float().cpu().numpy(), fin.cpu().numpy().astype(np.float64), o_ref,
              f_ref, "bf16", units=units)


# --------------------------------------------------------------------------- strong gates
# Decays far beyond what factors centred on a reference token can hold (their exponents
# would span more than 2^100 within a 16- or 32-token chunk). The kernels then form the
# diagonal Gram blocks from exact per-token decay products; the result must meet the same bars.
# One case stays just inside the factored form's range.

STRONG_G = {
    # log decays of -3.8 .. -4.2 per token: the 32-token blocks' factors span 2^82 .. 2^92,
    # still on the factored path (hi + lo bf16 factors)
    "span90_g": W.custom(B=1, T=100, H=2, HV=2, K=128, V=128, h0_std=0.1, g_lo=0.015,
                         g_hi=0.022),
    # plain log decays of -6.9 .. -18.4 per token and key dim
    "strong_g": W.custom(B=1, T=100, H=2, HV=2, K=128, V=128, h0_std=0.1, g_lo=1e-8,
                         g_hi=1e-3),
    # per-dim decays from almost none to -13.8 per token: chunks and blocks of both kinds
    "mixed_g": W.custom(B=2, T=77, H=1, HV=2, K=128, V=128, g_lo=1e-6, g_hi=0.999),
    "strong_g_k64_varlen": W.custom(H=1, HV=2, K=64, V=64, h0_std=0.1, g_lo=1e-8, g_hi=1e-3,
                                    lengths=(0, 5, 16, 33, 70)),
}


@pytest.mark.parametrize("chunk", [1, 16, 32, 64])
@pytest.mark.parametrize("name", list(STRONG_G))
def test_strong_decay_parity(name, chunk):
    w = STRONG_G[name]
    inp = W.make_inputs(w, seed=31)
    o, fin = gpu_run(inp, chunk=chunk)
    o_ref, f_ref = oracle_run(inp)
    check_all(inp, o, fin, o_ref, f_ref, w.dtype, what=f"{name} chunk {chunk}")


# gate parameters for strong activated decays: the softplus gate with exp(A_log) = 8 and raw
# gate inputs ~ N(2, 1) (about -17 per token); the bounded gate at lower bound -5 with raw
# inputs ~ N(3, 1) (close to -5 per token, -80 over 16 tokens)
STRONG_PRE = {
    "softplus_A8": (dict(g_mean=2.0, A_lo=7.99, A_hi=8.01), {"gate": "softplus"}),
    "bounded_lb5": (dict(g_mean=3.0), {"gate": "bounded", "lb": -5.0}),
}


@pytest.mark.parametrize("chunk", [1, 16, 32, 64])
@pytest.mark.parametrize("case", list(STRONG_PRE))
def test_strong_gate_parity(case, chunk):
    kw, gate = STRONG_PRE[case]
    w = W.custom(B=2, T=90, H=2, HV=4, K=128, V=128, h0_std=0.1)
    raw = W.make_raw_inputs(w, seed=32, **kw)
    pre = {"l2": True, "sig": True, **gate}
    o, fin = raw_plan(raw, chunk, pre)()
    torch.cuda.synchronize()
    o_ref, f_ref = raw_oracle(raw, pre)
    check_all(raw.inp, o.float().cpu().numpy(), fin.cpu().numpy().astype(np.float64), o_ref,
              f_ref, "bf16", what=f"{case} chunk {chunk}")


@pytest.mark.parametrize("chunk", [64, 32, 16])
@pytest.mark.parametrize("case", list(STRONG_PRE))
def test_strong_gate_full_size_every_unit(case, chunk):
    # the throughput shape with raw inputs and a strong gate: every chunk takes the exact
    # diagonal path; every unit and row against the oracle
    kw, gate = STRONG_PRE[case]
    w = W.WORKLOADS["h16_t4096"]
    raw = W.make_raw_inputs(w, seed=0, **kw)
    pre = {"l2": True, "sig": True, **gate}
    o, fin = raw_plan(raw, chunk, pre)()
    torch.cuda.synchronize()
    units = [(0, j) for j in range(w.HV)]
    o_ref, f_ref = raw_oracle(raw, pre, units=units)
    check_all(raw.inp, o.float().cpu().numpy(), fin.cpu().numpy().astype(np.float64), o_ref,
              f_ref, "bf16", units=units, what=f"{case} chunk {chunk}")
