"""Stride and aliasing rules of the C-ABI (include/sigattn.h, sigattn_strides),
checked on the host through sigattn_validate: nothing is enqueued and the
(fake) pointers are never dereferenced."""
import pytest

import sigmoid_attention_amd as sa

OK, NULL, SHAPE, SEQLEN, ALIGN, ALIAS, BIAS, PREC, HIP, PASS, STRIDE = range(11)
BIG = 1 << 40
P = [0x100000000000 + i * BIG for i in range(8)]  # far-apart fake device addresses

B, H, L, D = 2, 4, 256, 64


def contiguous():
    return (H * L * D, L * D, D)


def blhd():
    return (L * H * D, D, H * D)


def fused(which):
    """Stride triple and element offset of slice `which` of a [B, L, 3, H, d] buffer."""
    return (L * 3 * H * D, D, 3 * H * D), which * H * D


def check(pass_, strides, ptrs, lens=(256, 100)):
    a, keep = sa.make_args(B, H, L, D, lens, strides=strides)
    return sa.validate(a, pass_, ptrs)


def test_default_layout_still_validates():
    a, keep = sa.make_args(B, H, L, D, (256, 100))
    assert sa.validate(a, "fwd", P[:4]) == OK
    assert sa.validate(a, "bwd_dkdv", P[:6]) == OK


def test_blhd_layout_accepted_for_every_pass():
    for pass_, n in (("fwd", 4), ("bwd_dq", 5), ("bwd_dkdv", 6)):
        assert check(pass_, [blhd()] * n, P[:n]) == OK


def test_fused_qkv_inputs_and_fused_gradient_outputs_accepted():
    st, _ = fused(0)
    q = P[0]
    ins = [q + 2 * fused(i)[1] for i in range(3)]
    g = P[1]
    outs = [g + 2 * fused(i)[1] for i in range(3)]
    # dK/dV written into the k and v slices of one fused gradient buffer
    assert check("bwd_dkdv", [st] * 3 + [blhd()] + [st, st], ins + [P[2], outs[1], outs[2]]) == OK
    # dQ into the q slice of the same buffer shape
    assert check("bwd_dq", [st] * 3 + [blhd(), st], ins + [P[2], outs[0]]) == OK


def test_interleaved_outputs_that_collide_are_rejected():
    st, _ = fused(0)
    g = P[1]
    # dV placed half a head-block after dK: the slices interleave and collide
    assert check("bwd_dkdv", [st] * 3 + [blhd(), st, st], [P[0]] * 3 + [P[2], g, g + 2 * (H * D // 2)]) == ALIAS
    # identical outputs
    assert check("bwd_dkdv", [blhd()] * 6, P[:4] + [P[5], P[5]]) == ALIAS


def test_output_overlapping_input_rejected_inputs_may_alias():
    assert check("fwd", [blhd()] * 4, [P[0], P[0], P[0], P[0] + 64]) == ALIAS
    assert check("fwd", [blhd()] * 4, [P[0], P[0], P[0], P[3]]) == OK


@pytest.mark.parametrize("bad", [(H * L * D, L * D, 4), (H * L * D, L * D, 60), (H * L * D, 12, D),
                                 (-8, L * D, D), (H * L * D, L * D, 1 << 24)])
def test_bad_strides_rejected(bad):
    for pass_, n in (("fwd", 4), ("bwd_dq", 5), ("bwd_dkdv", 6)):
        st = [contiguous()] * n
        st[1] = bad  # an input
        assert check(pass_, st, P[:n]) == STRIDE


def test_broadcast_input_allowed_broadcast_output_rejected():
    mqa = (L * D, 0, D)  # one K/V head shared by all query heads
    assert check("fwd", [contiguous(), mqa, mqa, contiguous()], P[:4]) == OK
    assert check("fwd", [contiguous()] * 3 + [mqa], P[:4]) == STRIDE


def test_output_rows_overlapping_within_one_view_rejected():
    # heads 8 elements apart: head h row l and head h+1 overlap
    assert check("fwd", [contiguous()] * 3 + [(H * L * D, 8, H * D)], P[:4]) == STRIDE


def test_validate_reports_argument_errors_in_order():
    a, keep = sa.make_args(B, H, L, D, (256, 100))
    assert sa.validate(a, "fwd", [P[0], 0, P[2], P[3]]) == NULL
    assert sa.validate(a, "fwd", [P[0], P[1] + 8, P[2], P[3]]) == ALIGN
    assert sa.validate(a, "fwd", P[:4]) == OK
    a, keep = sa.make_args(B, H, L, D, (257, 100))
    assert sa.validate(a, "fwd", P[:4]) == SEQLEN
    lib = sa.load()
    a, keep = sa.make_args(B, H, L, D, (256, 100))
    import ctypes
    arr = (ctypes.c_void_p * 4)(*P[:4])
    assert lib.sigattn_validate(ctypes.byref(a), 7, arr) == PASS
    assert lib.sigattn_validate(ctypes.byref(a), 0, None) == NULL


def test_layout_strides_of_torch_views():
    import torch

    from sigmoid_attention_amd._binding import layout_strides
    x = torch.empty(2, 5, 3, 4, 64)  # [B, L, 3, H, d] fused projection
    q = x[:, :, 0]
    assert layout_strides(q, "blhd") == ((2, 4, 5, 64), (5 * 3 * 4 * 64, 64, 3 * 4 * 64))
    c = torch.empty(2, 4, 5, 64)
    assert layout_strides(c, "bhld") == ((2, 4, 5, 64), (4 * 5 * 64, 5 * 64, 64))
    assert layout_strides(c.permute(0, 2, 1, 3), "blhd") == ((2, 4, 5, 64), (4 * 5 * 64, 5 * 64, 64))


def test_softmax_entry_points_validate_row_arrays():
    import ctypes
    lib = sa.load()
    a, keep = sa.make_args(B, H, L, D, (256, 100))
    r0, r1 = 0x500000000000, 0x600000000000
    q, k, v, o = P[:4]
    assert lib.sigattn_softmax_fwd(ctypes.byref(a), q, k, v, o, None) == NULL
    assert lib.sigattn_softmax_fwd(ctypes.byref(a), q, k, v, o, r0 + 4) == ALIGN
    assert lib.sigattn_softmax_fwd(ctypes.byref(a), q, k, v, o, o + 64) == ALIAS  # lse2 inside O
    assert lib.sigattn_softmax_bwd_prep(ctypes.byref(a), o, P[4], o + 1024) == ALIAS  # delta inside O
    assert lib.sigattn_softmax_bwd_prep(ctypes.byref(a), o, P[4], None) == NULL
    # an output overlapping an input row array
    assert lib.sigattn_softmax_bwd_dq(ctypes.byref(a), q, k, v, P[4], r0, r1, r1) == ALIAS
    assert lib.sigattn_softmax_bwd_dkdv(ctypes.byref(a), q, k, v, P[4], r0, r1, r0, P[6]) == ALIAS
    assert lib.sigattn_softmax_bwd_dkdv(ctypes.byref(a), q, k, v, P[4], None, r1, P[5], P[6]) == NULL
