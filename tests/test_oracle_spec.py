"""Pins for the speculative multi-token decode of the oracle
(vllm.cpp cpu_ops.cpp, CausalConv1dSpecUpdateKernel and GdnSpecDecodeKernel).

The pages state the property that makes speculative decoding work: the
recurrence is sequential and the slot of column t receives the state after
t+1 tokens, so starting the next step from column j-1 is the same as having
run only the first j tokens.  The same holds for the widened conv row: the
next step's window, read at offset num_accepted-1, is the history that plain
decode would hold after the accepted tokens.  These tests check both against
plain one-token decode (itself pinned in test_oracle_pins.py), token by
token, on inputs where a wrong offset, column or snapshot time changes the
result.
"""
import numpy as np
import pytest

import oracle
from gdn_inputs import Dims, spec_inputs

D = Dims(Hk=2, Hv=4, Dk=8, Dv=4, K=4)   # Dk != Dv, Hv != Hk
SCALE = 1.0 / np.sqrt(D.Dk)


def _plain(inp, tok_ids, hist, S):
    """Plain decode of tokens ``tok_ids`` one at a time, from conv history
    ``hist`` [Cc, K-1] and state ``S`` [Hv, Dv, Dk] (unrounded).  Returns the
    outputs, and the history and state after each token."""
    cp = hist[None].copy()
    sp = S[None].copy()
    outs, hists, states = [], [], []
    for t in tok_ids:
        o, cp, sp = oracle.decode(D, inp["x"][t:t + 1], inp["w"], inp["a"][t:t + 1], inp["b"][t:t + 1],
                                  inp["A_log"], inp["dt_bias"], cp, sp, [0], SCALE, state_dtype="f64",
                                  out_dtype="f64")
        outs.append(o[0])
        hists.append(cp[0].copy())
        states.append(sp[0].copy())
    return outs, hists, states


def _step(inp, **kw):
    return oracle.decode_spec(D, inp["cu"], inp["x"], inp["w"], inp["a"], inp["b"], inp["A_log"],
                              inp["dt_bias"], inp["conv_pool"], inp["ssm_pool"], inp["state_idx"],
                              inp["num_accepted"], SCALE, **{"state_dtype": "f64", "out_dtype": "f64", **kw})


@pytest.mark.parametrize("lens", [None, [4, 1, 3, 2, 4]])
def test_snapshots_are_prefix_decodes(lens):
    """First step after a prefill (num_accepted = 1, window at the row's
    start): output t and the snapshot in column t equal plain decode of the
    first t+1 tokens; taps past K-1 of the widened row are never read."""
    cols = 4
    inp = spec_inputs(D, 5, cols, 32, "f32", "f32", seed=11, lens=lens)
    inp["num_accepted"][:] = 1
    out, cp, sp = _step(inp)
    Km1 = D.K - 1
    for i in range(5):
        lo, hi = inp["cu"][i], inp["cu"][i + 1]
        row = inp["conv_pool"][inp["state_idx"][i, 0]]
        S0 = inp["ssm_pool"][inp["state_idx"][i, 0]]
        outs, hists, states = _plain(inp, range(lo, hi), row[:, :Km1], S0)
        for t in range(hi - lo):
            np.testing.assert_allclose(out[lo + t], outs[t], rtol=0, atol=1e-12)
            np.testing.assert_allclose(sp[inp["state_idx"][i, t]], states[t], rtol=0, atol=1e-12)
        for t in range(hi - lo, cols):   # columns past the request's tokens are not written
            np.testing.assert_array_equal(sp[inp["state_idx"][i, t]], inp["ssm_pool"][inp["state_idx"][i, t]])
        if hi - lo == cols:
            # the window that num_accepted = n selects next step is plain decode's history after n tokens
            new_row = cp[inp["state_idx"][i, 0]]
            for n in range(1, cols + 1):
                np.testing.assert_array_equal(new_row[:, n - 1:n - 1 + Km1], hists[n - 1])


def test_next_step_rolls_back_to_accepted_prefix():
    """Two steps: the second starts at column num_accepted-1.  Its outputs and
    snapshots equal plain decode of the accepted prefix of step one followed
    by step two's tokens."""
    cols, N = 4, 6
    one = spec_inputs(D, N, cols, 40, "f32", "f32", seed=21)
    one["num_accepted"][:] = 1
    _, cp1, sp1 = _step(one)
    two = spec_inputs(D, N, cols, 40, "f32", "f32", seed=22)
    two["state_idx"] = one["state_idx"]
    two["conv_pool"], two["ssm_pool"] = cp1, sp1
    two["num_accepted"] = np.array([1, 2, 3, 4, 2, 3], np.int32)
    out2, _, sp2 = _step(two)
    Km1 = D.K - 1
    for i in range(N):
        n = int(two["num_accepted"][i])
        row0 = one["conv_pool"][one["state_idx"][i, 0]]
        S0 = one["ssm_pool"][one["state_idx"][i, 0]]
        _, hists, states = _plain(one, range(one["cu"][i], one["cu"][i] + n), row0[:, :Km1], S0)
        lo, hi = two["cu"][i], two["cu"][i + 1]
        outs, _, states2 = _plain(two, range(lo, hi), hists[-1], states[-1])
        for t in range(hi - lo):
            np.testing.assert_allclose(out2[lo + t], outs[t], rtol=0, atol=1e-12)
            np.testing.assert_allclose(sp2[two["state_idx"][i, t]], states2[t], rtol=0, atol=1e-12)


def test_null_columns_and_inert_requests():
    """A -1 column skips only its own store; a request whose initial column is
    -1 gets zero outputs and leaves both pools as they were."""
    N, cols, S = 6, 4, 32
    inp = spec_inputs(D, N, cols, S, "f32", "f32", seed=31, null_reqs=2, null_cols=4)
    sidx, nat = inp["state_idx"], inp["num_accepted"]
    live = sidx[np.arange(N), nat - 1] >= 0
    assert live.sum() == N - 2 and (sidx[live] < 0).sum() > 0
    out, cp, sp = _step(inp)
    # the same step with every -1 column of a live request given a spare slot
    spare = iter(sorted(set(range(S)) - set(sidx[sidx >= 0].tolist())))
    full_sidx = sidx.copy()
    for i, c in zip(*np.nonzero(sidx < 0)):
        if live[i]:
            full_sidx[i, c] = next(spare)
    out_f, cp_f, sp_f = _step({**inp, "state_idx": full_sidx})
    ssm_written = set(sidx[live][sidx[live] >= 0].tolist())
    conv_written = set(sidx[live, 0].tolist())
    for s in range(S):
        if s in ssm_written:
            np.testing.assert_array_equal(sp[s], sp_f[s])
        else:
            np.testing.assert_array_equal(sp[s], inp["ssm_pool"][s])
        if s in conv_written:
            np.testing.assert_array_equal(cp[s], cp_f[s])
        else:
            np.testing.assert_array_equal(cp[s], inp["conv_pool"][s])
    for i in range(N):
        lo, hi = inp["cu"][i], inp["cu"][i + 1]
        if live[i]:
            np.testing.assert_array_equal(out[lo:hi], out_f[lo:hi])
            assert np.all(np.abs(out[lo:hi]).sum(axis=(1, 2)) > 0)
        else:
            assert np.all(out[lo:hi] == 0)


def test_single_column_is_plain_decode():
    """One column, one token, a row of exactly K-1 taps: the same as plain
    decode, pools and rounded outputs included."""
    inp = spec_inputs(D, 7, 1, 16, "bf16", "bf16", seed=41)
    out, cp, sp = _step(inp, state_dtype="bf16", out_dtype="bf16")
    slots = inp["state_idx"][:, 0]
    o2, cp2, sp2 = oracle.decode(D, inp["x"], inp["w"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
                                 inp["conv_pool"], inp["ssm_pool"], slots, SCALE, state_dtype="bf16",
                                 out_dtype="bf16")
    np.testing.assert_array_equal(out, o2)
    np.testing.assert_array_equal(cp, cp2)
    np.testing.assert_array_equal(sp, sp2)


def test_rounding_only_at_snapshots():
    """The running state is not rounded between tokens: with a bf16 pool each
    snapshot is the rounding of the unrounded (f64) snapshot."""
    inp = spec_inputs(D, 4, 4, 32, "f32", "bf16", seed=51)
    _, _, sp_exact = _step(inp, state_dtype="f64")
    _, _, sp_bf = _step(inp, state_dtype="bf16")
    live = inp["state_idx"][inp["state_idx"] >= 0]
    np.testing.assert_array_equal(sp_bf[live], oracle.round_to(sp_exact[live], "bf16"))


@pytest.mark.parametrize("W_extra", [0, 3])
def test_widened_pool_uses_leading_taps(W_extra):
    """Plain decode and prepare on a widened conv pool act on each row's
    leading K-1 taps and leave the rest untouched."""
    rng = np.random.default_rng(61)
    S, B = 10, 4
    Km1 = D.K - 1
    wide = rng.normal(size=(S, D.Cc, Km1 + W_extra))
    x = rng.normal(size=(B, D.Cc))
    w = rng.normal(size=(D.Cc, D.K)) * 0.5
    a, b = rng.normal(size=(B, D.Hv)), rng.normal(size=(B, D.Hv))
    A_log, dt = rng.uniform(0, 2.7, D.Hv), rng.uniform(-1, 1, D.Hv)
    ssm = rng.normal(size=(S, D.Hv, D.Dv, D.Dk)) * 0.05
    slots = np.array([3, 7, 1, 8])
    o_w, cp_w, sp_w = oracle.decode(D, x, w, a, b, A_log, dt, wide, ssm, slots, SCALE)
    o_n, cp_n, sp_n = oracle.decode(D, x, w, a, b, A_log, dt, wide[:, :, :Km1].copy(), ssm, slots, SCALE)
    np.testing.assert_array_equal(o_w, o_n)
    np.testing.assert_array_equal(sp_w, sp_n)
    np.testing.assert_array_equal(cp_w[:, :, :Km1], cp_n)
    np.testing.assert_array_equal(cp_w[:, :, Km1:], wide[:, :, Km1:])
    cu = np.array([0, 1, 3, 4], np.int32)
    pre_w = oracle.prepare(D, cu, x, w, a, b, A_log, dt, wide, slots[:3], np.ones(3, np.uint8))
    pre_n = oracle.prepare(D, cu, x, w, a, b, A_log, dt, wide[:, :, :Km1].copy(), slots[:3], np.ones(3, np.uint8))
    for key in ("q", "k", "v", "g", "beta"):
        np.testing.assert_array_equal(pre_w[key], pre_n[key])
    np.testing.assert_array_equal(pre_w["conv_pool"][:, :, :Km1], pre_n["conv_pool"])
    np.testing.assert_array_equal(pre_w["conv_pool"][:, :, Km1:], wide[:, :, Km1:])
