"""The parity bars of parity_check.py, exercised on the CPU with the oracle's own outputs: an
output rounded like the GPU's (o to bf16) passes, and planted mistakes that one global relative
L2 error over the whole tensor lets through are caught."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle.native import kda_oracle_c
from parity_check import TOL, check_outputs, rel_l2


@pytest.fixture(scope="module")
def h16():
    # the throughput workload: 16 heads x 4096 tokens, zero initial state
    inp = W.make_inputs(W.WORKLOADS["h16_t4096"], seed=0)
    f = W.as_f32_numpy
    o_ref, f_ref = kda_oracle_c(f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta), inp.scale)
    # what a correct bf16 kernel returns at best: o rounded to bf16, the state in fp32
    o = torch.from_numpy(o_ref).to(torch.bfloat16).float().numpy()
    fin = f_ref.astype(np.float32).astype(np.float64)
    return inp, o, fin, o_ref, f_ref


def test_rounded_output_passes(h16):
    inp, o, fin, o_ref, f_ref = h16
    worst = check_outputs(o, fin, o_ref, f_ref, inp.seq_bounds(), "bf16")
    assert worst["o_unit"] < 2.5e-3 and worst["o_row"] < 4e-3


def test_zeroed_row_is_caught_where_a_global_norm_is_not(h16):
    inp, o, fin, o_ref, f_ref = h16
    bad = o.copy()
    bad[0, 1234, 7, :] = 0.0                   # one token of one head never written
    # a single relative L2 over the whole tensor stays under the bar ...
    assert rel_l2(bad, o_ref) <= TOL["bf16"]
    # ... the per-unit and per-row bars do not
    with pytest.raises(AssertionError, match="o rel L2 above|o row error"):
        check_outputs(bad, fin, o_ref, f_ref, inp.seq_bounds(), "bf16")


def test_row_bar_catches_what_the_unit_bar_does_not(h16):
    inp, o, fin, o_ref, f_ref = h16
    for fix in ("scaled", "stale"):
        bad = o.copy()
        if fix == "scaled":
            bad[0, 2000, 3, :] *= 1.1          # one row 10% off
        else:
            bad[0, 3000, 9, :] = 0.95 * bad[0, 3000, 9, :] + 0.05 * bad[0, 2999, 9, :]
        from parity_check import o_errors
        ue, _, _ = o_errors(bad, o_ref, inp.seq_bounds())
        assert np.nanmax(ue) <= TOL["bf16"]    # invisible to the per-unit bar
        with pytest.raises(AssertionError, match="o row error"):
            check_outputs(bad, fin, o_ref, f_ref, inp.seq_bounds(), "bf16")


def test_wrong_unit_is_caught(h16):
    inp, o, fin, o_ref, f_ref = h16
    bad = o.copy()
    bad[0, :, 5, :] *= 1.01                    # one head 1% off everywhere
    assert rel_l2(bad, o_ref) <= TOL["bf16"]
    with pytest.raises(AssertionError, match="o rel L2 above"):
        check_outputs(bad, fin, o_ref, f_ref, inp.seq_bounds(), "bf16")


def test_final_state_row_is_caught(h16):
    inp, o, fin, o_ref, f_ref = h16
    bad = fin.copy()
    bad[0, 9, 77, :] *= 0.95                   # one key row of one head's final state
    assert rel_l2(bad, f_ref) <= TOL["bf16"]
    with pytest.raises(AssertionError, match="final-state row error"):
        check_outputs(o, bad, o_ref, f_ref, inp.seq_bounds(), "bf16")


def test_varlen_units_and_empty_sequences():
    # per-unit bookkeeping over packed sequences, with empty ones: a planted error in one
    # sequence is reported in that sequence only
    w = W.custom(H=1, HV=2, K=64, V=64, h0_std=0.1, lengths=(0, 40, 0, 17, 64))
    inp = W.make_inputs(w, seed=1)
    f = W.as_f32_numpy
    cu = inp.cu_seqlens.numpy()
    o_ref, f_ref = kda_oracle_c(f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta),
                                inp.scale, inp.h0.numpy(), cu)
    check_outputs(o_ref, f_ref, o_ref, f_ref, inp.seq_bounds(), "fp32")
    bad = o_ref.copy()
    bad[0, 40 + 5, 1, :] *= 1.001             # sequence 3 (tokens 40..56), head 1
    with pytest.raises(AssertionError, match=r"first \(s, j\) = \(3, 1\)"):
        check_outputs(bad, f_ref, o_ref, f_ref, inp.seq_bounds(), "fp32")


# --------------------------------------------------------------------------- gradient bars

@pytest.fixture(scope="module")
def grads_small():
    # packed sequences with grouped value heads; the C backward oracle's gradients
    from oracle.native import kda_oracle_bwd_c
    w = W.custom(H=2, HV=4, K=64, V=64, h0_std=0.2, lengths=(40, 0, 300, 17))
    inp = W.make_inputs(w, seed=4)
    gr = W.make_grads(inp, seed=4)
    f = W.as_f32_numpy
    ref = kda_oracle_bwd_c(f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta), inp.scale,
                           inp.h0.numpy(), inp.cu_seqlens.numpy(), f(gr.d_o), gr.dht.numpy(),
                           n_threads=2)
    return inp, ref


def test_fp32_rounded_gradients_pass(grads_small):
    from parity_check import check_grads
    inp, ref = grads_small
    got = tuple(x.astype(np.float32) for x in ref)
    worst = check_grads(got, ref, inp.seq_bounds())
    assert max(worst.values()) < 1e-6


@pytest.mark.parametrize("name,where", [("dk", (0, 320, 1)), ("dg", (0, 5, 2)),
                                        ("dbeta", (0, 100, 3)), ("dv", (0, 341, 0))])
def test_planted_gradient_row_is_caught(grads_small, name, where):
    from parity_check import GRAD_NAMES, check_grads
    inp, ref = grads_small
    got = [x.copy() for x in ref]
    i = GRAD_NAMES.index(name)
    got[i][where] = 0.0                        # one token row (one value for dbeta) unwritten
    with pytest.raises(AssertionError, match=f"{name} (rel L2 above|row error)"):
        check_grads(got, ref, inp.seq_bounds())


def test_planted_dh0_row_is_caught(grads_small):
    from parity_check import check_grads
    inp, ref = grads_small
    got = [x.copy() for x in ref]
    got[5][2, 1, 7, :] *= 1.001                # one key row of one unit's dh0, 0.1% off
    with pytest.raises(AssertionError, match="dh0 (rel L2 above|row error)"):
        check_grads(got, ref, inp.seq_bounds())
