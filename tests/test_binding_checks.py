"""The Python binding's argument checks (CPU only, nothing is launched).

The C calls take bare pointers, so a tensor of the wrong shape or element
size would become an out-of-bounds device access; the binding must refuse it
with ValueError before any call into the library.  Host tensors are used
here: every check except the last one (device residence) runs on them, so a
well-formed call ends in "must be a device tensor" and each malformed one in
a message that names the argument."""
import pytest
import torch

import bit_quantized_moe_diffrouter_amd as q

T, H, E, K, I = 4, 128, 8, 2, 64


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def u8(n):
    return torch.zeros(n, dtype=torch.uint8)


def router():
    return q.QuantWeight(i32(E, H // 8), bf(E, H // 64), bf(E, H // 64))


def tiled(experts, rows, inf, split=0):
    return q.TiledWeight(u8(64), experts, rows, inf, split)


def raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


ROUTE_OK = dict(x_router=bf(T, H), norm_scale=bf(H), eps=1e-6, proj=router(), per_expert_scale=bf(E), k=K)


@pytest.mark.parametrize("change,match", [
    (dict(), "device tensor"),
    (dict(x_router=bf(T, H + 64)), "in_features"),
    (dict(x_router=f32(T, H)), "x_router: element size"),
    (dict(norm_scale=bf(H - 1)), "norm_scale: shape"),
    (dict(norm_scale=f32(H)), "norm_scale: element size"),
    (dict(per_expert_scale=bf(E + 1)), "per_expert_scale: shape"),
    (dict(logit_bias=bf(E)), "logit_bias .*element size"),
    (dict(logit_bias=f32(E - 1)), "logit_bias .*shape"),
    (dict(logits_out=f32(T, E + 1)), "logits_out .*shape"),
    (dict(indices=i32(T, K + 1)), "indices: shape"),
    (dict(weights=bf(T, K)), "weights .*element size"),
])
def test_moe_route_checks(change, match):
    kw = dict(ROUTE_OK, **change)
    raises(match, q.moe_route, **kw)


@pytest.mark.parametrize("change,match", [
    (dict(), "device tensor"),
    (dict(expert_offsets=i32(E)), "expert_offsets: shape"),
    (dict(sorted_assign=i32(T * K - 1)), "sorted_assign: shape"),
    (dict(indices=bf(T, K)), "indices: element size"),
])
def test_moe_sort_checks(change, match):
    kw = dict(dict(indices=i32(T, K), E=E), **change)
    raises(match, q.moe_sort, **kw)


GU_OK = dict(x_expert=bf(T, H), gate_up=tiled(E, 2 * I, H, I), I=I, k=K, expert_offsets=i32(E + 1),
             sorted_assign=i32(T * K))


@pytest.mark.parametrize("change,match", [
    (dict(), "device tensor"),
    (dict(x_expert=bf(T, H + 64)), "in_features"),
    (dict(I=2 * I), "rows vs 2 \\* I"),
    (dict(expert_offsets=i32(E + 2)), "expert_offsets: shape"),
    (dict(sorted_assign=i32(T * K + 1)), "sorted_assign: shape"),
])
def test_gate_up_checks(change, match):
    raises(match, q.qswitch_gate_up_geglu, **dict(GU_OK, **change))


DN_OK = dict(mid=u8(1 << 20), T=T, k=K, down=tiled(E, H, I), weights=f32(T, K), expert_offsets=i32(E + 1),
             sorted_assign=i32(T * K))


@pytest.mark.parametrize("change,match", [
    (dict(), "device tensor"),
    (dict(weights=bf(T, K)), "weights .*element size"),
    (dict(weights=f32(T, K + 1)), "weights .*shape"),
    (dict(expert_offsets=i32(E)), "expert_offsets: shape"),
    (dict(sorted_assign=i32(T)), "sorted_assign: shape"),
    (dict(y=bf(T, H - 64)), "y: shape"),
    (dict(mid=u8(16)), "mid: 16 bytes"),
])
def test_down_combine_checks(change, match):
    raises(match, q.qswitch_down_combine, **dict(DN_OK, **change))


@pytest.mark.parametrize("fn,W,y,match", [
    (q.qlinear, tiled(1, 64, H), None, "device tensor"),
    (q.qlinear, tiled(1, 64, H + 64), None, "x: shape"),
    (q.qlinear, tiled(1, 64, H), bf(T, 128), "y: shape"),
    (q.qlinear_geglu, tiled(1, 128, H, 64), None, "device tensor"),
    (q.qlinear_geglu, tiled(1, 128, 2 * H, 64), None, "x: shape"),
    (q.qlinear_geglu, tiled(1, 128, H, 64), bf(T, 128), "y: shape"),
    (q.qlinear_softcap, tiled(1, 64, H), None, "device tensor"),
    (q.qlinear_softcap, tiled(1, 64, 64), None, "x: shape"),
    (q.qlinear_softcap, tiled(1, 64, H), f32(T, 65), "y: shape"),
])
def test_dense_checks(fn, W, y, match):
    raises(match, fn, bf(T, H), W, y=y)


def test_embed_checks():
    W = q.TiledTWeight(u8(64), 256, H)
    raises("device tensor", q.embed_matmul_t, bf(T, 256), W, 1.0)
    raises("probs: shape", q.embed_matmul_t, bf(T, 255), W, 1.0)
    raises("probs: element size", q.embed_matmul_t, f32(T, 256), W, 1.0)
    raises("out: shape", q.embed_matmul_t, bf(T, 256), W, 1.0, out=bf(T, H + 1))


def test_unsorted_checks():
    gu = tiled(E, 2 * I, H, I)
    dn = tiled(E, H, I)
    ws = u8(1024)
    raises("device tensor", q.qswitch_gate_up_geglu_unsorted, bf(T, H), gu, I, i32(T, K), ws)
    raises("in_features", q.qswitch_gate_up_geglu_unsorted, bf(T, 2 * H), gu, I, i32(T, K), ws)
    raises("indices: element size", q.qswitch_gate_up_geglu_unsorted, bf(T, H), gu, I, f32(T, K).half(), ws)
    raises("mid_rows: shape", q.qswitch_gate_up_geglu_unsorted, bf(T, H), gu, I, i32(T, K), ws, bf(T * K, I + 1))
    raises("device tensor", q.qswitch_down_combine_unsorted, bf(T * K, I), T, K, dn, i32(T, K), f32(T, K), ws)
    raises("mid_rows: shape", q.qswitch_down_combine_unsorted, bf(T * K, 2 * I), T, K, dn, i32(T, K), f32(T, K), ws)
    raises("weights .*element size", q.qswitch_down_combine_unsorted, bf(T * K, I), T, K, dn, i32(T, K),
           bf(T, K), ws)
    raises("y: shape", q.qswitch_down_combine_unsorted, bf(T * K, I), T, K, dn, i32(T, K), f32(T, K), ws,
           y=bf(T, H + 1))
