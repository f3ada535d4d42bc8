"""The fp64 oracle against its pins (CPU only)."""
import math

import numpy as np
import pytest

import oracle
import pins
from workloads import WORKLOADS, make_inputs, to_f64, workload


@pytest.mark.parametrize("pin", pins.ATTENTION_PINS, ids=lambda f: f.__name__)
def test_attention_pin(pin):
    pin(oracle.attention)


@pytest.mark.parametrize("merge", [oracle.merge_fold, oracle.merge_closed_form],
                         ids=["fold", "closed_form"])
@pytest.mark.parametrize("pin", pins.MERGE_PINS, ids=lambda f: f.__name__)
def test_merge_pin(pin, merge):
    pin(merge)


@pytest.mark.parametrize("merge", [oracle.merge_fold, oracle.merge_closed_form],
                         ids=["fold", "closed_form"])
def test_chunked_equals_full(merge):
    pins.pin_chunked_equals_full(oracle.attention, merge, oracle.chunk_bounds)


def test_chunk_bounds():
    pins.pin_chunk_bounds(oracle.chunk_bounds)
    with pytest.raises(ValueError):
        oracle.chunk_bounds(10, 3, [3, 3, 3])
    with pytest.raises(ValueError):
        oracle.chunk_bounds(10, 0)


def test_layout():
    pins.pin_layout(oracle.seq2head, oracle.head2seq)


def test_ulysses_share():
    pins.pin_ulysses_share(oracle.attention, oracle.seq2head)


def test_head_groups():
    pins.pin_head_groups(oracle.head_groups, oracle.groups_to_seq, oracle.seq2head)


def test_ulysses_anything_share():
    pins.pin_ulysses_anything_share(oracle.attention, oracle.head_groups)
    # the named share function is the group of that split
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((1, 9, 5, 4)) for _ in range(3))
    o, l = oracle.ulysses_anything_share(q, k, v, 2, 1)
    o_ref, l_ref = oracle.attention(q[:, :, 3:], k[:, :, 3:], v[:, :, 3:])
    assert np.abs(o - o_ref).max() == 0 and np.abs(l - l_ref).max() == 0


def test_usp():
    pins.pin_usp(oracle.attention, oracle.usp_attention, oracle.usp_share)


def test_fold_equals_closed_form_at_workload_splits():
    """The in-order fold and the one-step merge agree on real chunk partials of
    the ring-anything workload's split (S = 4645, 8 uneven chunks), and both
    equal the unchunked result; a sample of query rows keeps it fast."""
    q, k, v = (to_f64(t) for t in make_inputs(4, heads=2))
    qs = q[:, ::97]
    o_ref, l_ref = oracle.attention(qs, k, v)
    for merge in ("fold", "closed"):
        o, l = oracle.chunked_attention(qs, k, v, 8, merge=merge)
        assert np.abs(o - o_ref).max() < 1e-12
        assert np.abs(l - l_ref).max() < 1e-12


@pytest.mark.parametrize("idx,rank", [(1, 0), (1, 3), (3, 0), (3, 7), (4, 0), (4, 7)])
def test_ring_share_equals_rows_of_full(idx, rank):
    w = workload(idx)
    q, k, v = (to_f64(t) for t in make_inputs(idx, heads=1))
    o_s, l_s = oracle.ring_share(q, k, v, w.ring_degree, rank)
    a, b = oracle.chunk_bounds(w.S, w.ring_degree)[rank]
    o_f, l_f = oracle.attention(q[:, a:b], k, v)
    assert np.abs(o_s - o_f).max() < 1e-12
    assert np.abs(l_s - l_f).max() < 1e-12


def test_workload_generator():
    # deterministic, right shapes and dtypes
    for w in WORKLOADS:
        assert w.flops() == 4.0 * w.B * w.H * w.S * w.S * w.D
    q1, k1, v1 = make_inputs(1)
    q2, k2, v2 = make_inputs(1)
    assert (q1 == q2).all() and (v1 == v2).all()
    assert tuple(q1.shape) == (1, 256, 2, 64) and str(q1.dtype) == "torch.float32"
    q, k, v = make_inputs(2, heads=4)
    assert tuple(q.shape) == (1, 1536, 4, 128) and str(q.dtype) == "torch.bfloat16"
    # the head slice is a slice of the full draw
    qf, _, _ = make_inputs(2)
    assert (qf[:, :, :4] == q).all()
    # logit standard deviation ~3 for the FLUX workloads
    qd, kd = to_f64(q), to_f64(k)
    s = np.einsum("bihd,bjhd->bhij", qd[:, :256], kd[:, :256]) / math.sqrt(128)
    assert 2.7 < s.std() < 3.3
    assert float(workload(3).S) == 4608 and workload(4).S == 4645 and workload(5).S == 4276


def test_video_outliers():
    w = workload(5)
    _, k, _ = make_inputs(5, heads=2)
    kd = to_f64(k)
    norms = np.sqrt((kd ** 2).sum(-1))            # [B, S, H]
    n_out = int(round(w.outlier_frac * w.S))
    assert n_out == 43
    for b in range(w.B):
        for h in range(2):
            big = (norms[b, :, h] > 4 * math.sqrt(w.D)).sum()
            assert big == n_out
