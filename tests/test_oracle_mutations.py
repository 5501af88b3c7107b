"""Planted mistakes in the oracle (on the CPU) must be caught by its pins.

Each case swaps one oracle function for a copy with a plausible bug -- start
offsets passed as end offsets, a lower bound instead of an upper bound, a
dropped routing weight, a transposed operand -- and checks that at least one
pin of tests/test_oracle_pins.py then fails.  This shows the pins constrain
the oracle rather than restate it.
"""
import numpy as np
import pytest

from oracle import moe_oracle as O
import tests.test_oracle_pins as P


def _fails(fn, *args):
    try:
        fn(*args)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def _mut_start_offsets(orig):
    def f(expert_ids, topk_weights, E):
        s = orig(expert_ids, topk_weights, E)
        s.offsets = s.starts.astype(np.int32)        # wrong convention
        return s
    return f


def _mut_unstable(orig):
    def f(expert_ids, topk_weights, E):
        s = orig(expert_ids, topk_weights, E)
        ids = np.asarray(expert_ids).reshape(-1)
        order = np.argsort(-np.arange(ids.size), kind="stable")
        perm = order[np.argsort(ids[order], kind="stable")]   # ties in descending s
        s.perm = perm
        s.row_to_token = perm // np.asarray(expert_ids).shape[1]
        if topk_weights is not None:
            s.row_weight = np.asarray(topk_weights).reshape(-1)[perm]
        return s
    return f


def _lower_bound(ts, tau):
    return np.searchsorted(ts.tile_start, np.asarray(tau), side="left") - 1


def _row_block_major(orig):
    def f(ts, counts, offsets, tau):
        g = int(O.tile_owner(ts, tau))
        local = int(tau) - int(ts.tile_start[g])
        mb, nb = divmod(local, ts.tiles_n)
        start = 0 if g == 0 else int(offsets[g - 1])
        return g, mb, nb, start + mb * ts.BM, min(ts.BM, int(counts[g]) - mb * ts.BM)
    return f


def _fwd_no_weight(x, W, expert_ids, topk_weights, E, *, acc=np.float64):
    return _ORIG["moe_forward"](x, W, expert_ids, None, E, acc=acc)


def _fwd_untransposed(x, W, expert_ids, topk_weights, E, *, acc=np.float64):
    Wt = np.swapaxes(np.asarray(W), 1, 2)      # multiplies by W[e] instead of W[e]^T
    return _ORIG["moe_forward"](x, Wt, expert_ids, topk_weights, E, acc=acc)


def _gg_untransposed(A, W, offsets, *, acc=np.float64, out=None):
    return _ORIG["grouped_gemm"](A, np.swapaxes(np.asarray(W), 1, 2), offsets, acc=acc, out=out)


def _bwd_weighted_dw(dY, x, W, expert_ids, topk_weights, E, *, acc=np.float64):
    dX, dW, d_w = _ORIG["moe_backward"](dY, x, W, expert_ids, topk_weights, E, acc=acc)
    return dX, dW, d_w * np.asarray(topk_weights)  # uses the weighted product


def _bwd_unweighted_dx(dY, x, W, expert_ids, topk_weights, E, *, acc=np.float64):
    _, dW, d_w = _ORIG["moe_backward"](dY, x, W, expert_ids, topk_weights, E, acc=acc)
    dX, _, _ = _ORIG["moe_backward"](dY, x, W, expert_ids, None, E, acc=acc)
    return dX, dW, d_w


def _bwd_dw_transposed_sum(dY, x, W, expert_ids, topk_weights, E, *, acc=np.float64):
    dX, dW, d_w = _ORIG["moe_backward"](dY, x, W, expert_ids, None, E, acc=acc)
    dX2, _, d_w2 = _ORIG["moe_backward"](dY, x, W, expert_ids, topk_weights, E, acc=acc)
    return dX2, dW, d_w2                       # dW without the routing weight


def _gated_swapped(gu, *, acc=np.float64, round_h=False):
    F = gu.shape[1] // 2
    return _ORIG["gated_activation"](np.concatenate([gu[:, F:], gu[:, :F]], axis=1), acc=acc,
                                     round_h=round_h)


def _gated_sigmoid(gu, *, acc=np.float64, round_h=False):
    F = gu.shape[1] // 2
    g = np.asarray(gu[:, :F], dtype=np.float64)
    return (1.0 / (1.0 + np.exp(-g)) * gu[:, F:]).astype(acc)   # sigmoid instead of silu


def _gated_down_untransposed(x, W_gu, W_down, expert_ids, topk_weights, E, *, acc=np.float64,
                             round_h=False):
    Wd = np.swapaxes(np.asarray(W_down), 1, 2)
    if Wd.shape[2] != W_gu.shape[1] // 2:
        raise ValueError("shape")
    return _ORIG["gated_ffn_forward"](x, W_gu, Wd, expert_ids, topk_weights, E, acc=acc)


def _gated_no_weight(x, W_gu, W_down, expert_ids, topk_weights, E, *, acc=np.float64,
                     round_h=False):
    return _ORIG["gated_ffn_forward"](x, W_gu, W_down, expert_ids, None, E, acc=acc)


def _e4m3_bias8(bits):
    return _ORIG["decode_e4m3"](bits) / 2.0            # exponent bias 8 instead of 7


def _e4m3_no_subnormals(bits):
    v = _ORIG["decode_e4m3"](bits)
    e = (np.asarray(bits, dtype=np.uint8) >> 3) & 0xF
    return np.where(e == 0, 0.0, v)                    # subnormals flushed


def _fp8_no_token_scale(xq, x_scale, Wq, w_scale, expert_ids, topk_weights, E, *, acc=np.float64):
    return _ORIG["moe_forward_fp8"](xq, np.ones(len(x_scale)), Wq, w_scale, expert_ids, topk_weights,
                                    E, acc=acc)


def _fp8_channel_scale_on_rows(xq, x_scale, Wq, w_scale, expert_ids, topk_weights, E, *,
                               acc=np.float64):
    sw = np.asarray(w_scale)
    return _ORIG["moe_forward_fp8"](xq, x_scale, Wq, np.broadcast_to(sw[:, :1], sw.shape), expert_ids,
                                    topk_weights, E, acc=acc)      # one scale per expert only


def _gated_bwd_sigmoid_derivative(dY, x, W_gu, W_down, expert_ids, topk_weights, E, *, acc=np.float64,
                                  round_h=False):
    """silu' taken as the logistic function alone (the g s (1 - s) term dropped)."""
    saved = np.exp
    dX, dWgu, dWd, d_w = _ORIG["gated_ffn_backward"](dY, x, W_gu, W_down, expert_ids, topk_weights, E,
                                                      acc=acc)
    F = W_gu.shape[1] // 2
    ids = np.asarray(expert_ids).reshape(-1)
    k = np.asarray(expert_ids).shape[1]
    wflat = np.asarray(topk_weights).reshape(-1)
    dX2 = np.zeros_like(dX)
    for e in range(E):
        s_e = np.nonzero(ids == e)[0]
        if s_e.size == 0:
            continue
        tok = s_e // k
        xe = np.asarray(x)[tok]
        gu = xe @ W_gu[e].T
        g, u = gu[:, :F], gu[:, F:]
        sg = 1.0 / (1.0 + saved(-g))
        dh = wflat[s_e][:, None] * (np.asarray(dY)[tok] @ W_down[e])
        dgu = np.concatenate([dh * u * sg, dh * g * sg], axis=1)
        np.add.at(dX2, tok, dgu @ W_gu[e])
    return dX2, dWgu, dWd, d_w


def _gated_bwd_weighted_dw(dY, x, W_gu, W_down, expert_ids, topk_weights, E, *, acc=np.float64,
                           round_h=False):
    dX, dWgu, dWd, d_w = _ORIG["gated_ffn_backward"](dY, x, W_gu, W_down, expert_ids, topk_weights, E,
                                                      acc=acc)
    return dX, dWgu, dWd, d_w * np.asarray(topk_weights)


def _mx_first_block_scale(q, scales):
    sc = np.asarray(scales)
    return _ORIG["mx_values"](q, np.repeat(sc[..., :1], sc.shape[-1], axis=-1))   # one scale per row


def _mx_masked_no_weight_scales(xq, x_bs, Wq, w_bs, ms, T, *, acc=np.float64):
    return O.masked_forward(O.mx_values(xq, x_bs), O.decode_e4m3(Wq), ms, T, acc=acc)


def _rank_counts_invalid_slots(expert_ids, topk_weights, E):
    # ranks counted over all earlier slots, valid or not
    ids = np.asarray(expert_ids)
    T, k = ids.shape
    shifted = np.where((ids >= 0) & (ids < E), ids, 0)   # every slot looks valid to the rank
    rs = _ORIG["rank_schedule"](shifted, topk_weights, E)
    return rs


_ORIG = {n: getattr(O, n) for n in ["rank_schedule", "masked_forward_mx", "mx_values", "routing_schedule", "tile_owner", "tile_coords", "moe_forward",
                                     "grouped_gemm", "moe_backward", "gated_activation",
                                     "gated_ffn_forward", "decode_e4m3", "moe_forward_fp8",
                                     "gated_ffn_backward"]}

CASES = [
    ("end offsets replaced by start offsets", "routing_schedule", lambda: _mut_start_offsets(_ORIG["routing_schedule"]),
     [P.test_offsets_page_examples]),
    ("unstable sort", "routing_schedule", lambda: _mut_unstable(_ORIG["routing_schedule"]),
     [P.test_sorted_rows_brute_force]),
    ("lower bound owner lookup", "tile_owner", lambda: _lower_bound,
     [lambda: P.test_tile_owner_brute_force.hypothesis.inner_test([2, 0, 0, 5], 7, 16, 16)]),
    ("row-block-major walk", "tile_coords", lambda: _row_block_major(_ORIG["tile_coords"]),
     [P.test_column_block_major_walk]),
    ("routing weight dropped", "moe_forward", lambda: _fwd_no_weight,
     [lambda: P.test_moe_forward_brute_force(0), P.test_rank_one_closed_form]),
    ("weights not transposed", "moe_forward", lambda: _fwd_untransposed,
     [P.test_rank_one_closed_form]),
    ("grouped GEMM weights not transposed", "grouped_gemm", lambda: _gg_untransposed,
     [P.test_single_expert_is_plain_matmul]),
    ("routing-weight gradient from the weighted product", "moe_backward", lambda: _bwd_weighted_dw,
     [P.test_backward_finite_differences, P.test_backward_euler_identities]),
    ("token gradient without the routing weight", "moe_backward", lambda: _bwd_unweighted_dx,
     [P.test_backward_finite_differences, P.test_backward_euler_identities]),
    ("weight gradient without the routing weight", "moe_backward", lambda: _bwd_dw_transposed_sum,
     [P.test_backward_finite_differences, P.test_backward_euler_identities]),
    ("gate and up halves swapped", "gated_activation", lambda: _gated_swapped,
     [P.test_gated_gate_and_up_halves, P.test_gated_ffn_reduces_to_dense_swiglu]),
    ("sigmoid in place of silu", "gated_activation", lambda: _gated_sigmoid,
     [P.test_gated_gate_and_up_halves, lambda: P.test_gated_ffn_brute_force(0)]),
    ("down projection not transposed", "gated_ffn_forward", lambda: _gated_down_untransposed,
     [P.test_gated_ffn_reduces_to_dense_swiglu, lambda: P.test_gated_ffn_brute_force(1)]),
    ("gated routing weight dropped", "gated_ffn_forward", lambda: _gated_no_weight,
     [P.test_gated_gate_and_up_halves, P.test_gated_ffn_homogeneity]),
    ("e4m3 exponent bias 8", "decode_e4m3", lambda: _e4m3_bias8,
     [P.test_e4m3_decode_against_torch]),
    ("e4m3 subnormals flushed", "decode_e4m3", lambda: _e4m3_no_subnormals,
     [P.test_e4m3_decode_against_torch]),
    ("fp8 token scale dropped", "moe_forward_fp8", lambda: _fp8_no_token_scale,
     [P.test_fp8_forward_brute_force, P.test_fp8_power_of_two_scales_are_exact]),
    ("silu derivative without its g term", "gated_ffn_backward", lambda: _gated_bwd_sigmoid_derivative,
     [P.test_gated_backward_finite_differences]),
    ("gated routing-weight gradient from the weighted product", "gated_ffn_backward",
     lambda: _gated_bwd_weighted_dw,
     [P.test_gated_backward_finite_differences, P.test_gated_backward_identities]),
    ("block scales collapsed to one per row", "mx_values", lambda: _mx_first_block_scale,
     [P.test_mx_forward_brute_force_and_block_structure]),
    ("masked block-scaled forward without the weight block scales", "masked_forward_mx",
     lambda: _mx_masked_no_weight_scales,
     [P.test_mx_masked_equals_contiguous, P.test_mx_masked_overflow_brute_force]),
    ("rank counted over invalid slots too", "rank_schedule", lambda: _rank_counts_invalid_slots,
     [lambda: P.test_rank_schedule_brute_force(2, 31, 3, 4, 0.2)]),
    ("fp8 channel scale collapsed to one per expert", "moe_forward_fp8",
     lambda: _fp8_channel_scale_on_rows,
     [P.test_fp8_forward_brute_force, P.test_fp8_power_of_two_scales_are_exact]),
]


@pytest.mark.parametrize("name,attr,make,checks", CASES, ids=[c[0] for c in CASES])
def test_planted_mistake_is_caught(monkeypatch, name, attr, make, checks):
    for chk in checks:
        assert not _fails(chk), f"pin fails on the unmodified oracle: {chk}"
    monkeypatch.setattr(O, attr, make())
    assert all(_fails(chk) for chk in checks), f"planted mistake not caught: {name}"
