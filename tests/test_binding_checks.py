"""Host-side argument checks of the Python binding (CPU only: no tensor here
is on a GPU, and no check may need the library). Every shape, dtype or rank
mismatch between the tensors of a call must raise before any pointer reaches a
kernel; with consistent shapes the only complaint left is the device."""
import pytest
import torch

import exact_attention_amd as ea

bf, u8, i32, f32 = torch.bfloat16, torch.uint8, torch.int32, torch.float32


def z(shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def raises(match, fn, *a, **kw):
    with pytest.raises((ValueError, TypeError), match=match):
        fn(*a, **kw)


# ------------------------------------------------------------------ dense forward

def fwd_args(B=2, Nq=8, Nk=8, Hq=4, Hkv=2, d=64, dv=None):
    return z((B, Nq, Hq, d)), z((B, Nk, Hkv, d)), z((B, Nk, Hkv, dv or d))


def test_fwd_consistent_shapes_only_fail_on_device():
    raises("on a GPU", ea.attn_fwd, *fwd_args())


@pytest.mark.parametrize("bad", ["k_batch", "k_dim", "v_rows", "v_heads"])
def test_fwd_qkv_mismatch(bad):
    q, k, v = fwd_args()
    if bad == "k_batch":
        k = z((3, 8, 2, 64))
    elif bad == "k_dim":
        k = z((2, 8, 2, 128))
    elif bad == "v_rows":
        v = z((2, 9, 2, 64))
    else:
        v = z((2, 8, 4, 64))
    raises("k must be", ea.attn_fwd, q, k, v)


def test_fwd_out_and_lse_checked():
    q, k, v = fwd_args()
    raises("out must have shape", ea.attn_fwd, q, k, v, out=z((2, 8, 4, 32)))
    raises("out must be", ea.attn_fwd, q, k, v, out=z((2, 8, 4, 64), f32))
    raises("lse must have shape", ea.attn_fwd, q, k, v, lse=z((2, 8, 4), f32))
    raises("lse must be", ea.attn_fwd, q, k, v, lse=z((2, 4, 8), bf))
    raises("contiguous", ea.attn_fwd, q, k, v, out=z((2, 4, 8, 64)).transpose(1, 2))


def test_fwd_dtype_and_rank():
    q, k, v = fwd_args()
    raises("q must be", ea.attn_fwd, q.float(), k, v)
    raises("4 dims", ea.attn_fwd, q[0], k, v)


# ------------------------------------------------------------------ varlen forward

def vl_args(Tq=20, Tk=20, Hq=4, Hkv=2, d=64, S=3):
    cu = torch.tensor([0, 5, 12, 20][:S + 1], dtype=i32)
    return z((Tq, Hq, d)), z((Tk, Hkv, d)), z((Tk, Hkv, d)), cu, cu.clone()


def test_varlen_consistent_shapes_only_fail_on_device():
    q, k, v, cq, ck = vl_args()
    raises("on a GPU", ea.attn_fwd_varlen, q, k, v, cq, ck, 8)


def test_varlen_mismatches():
    q, k, v, cq, ck = vl_args()
    raises("head dim", ea.attn_fwd_varlen, q, z((20, 2, 128)), v, cq, ck, 8)
    raises("v must have shape", ea.attn_fwd_varlen, q, k, z((19, 2, 64)), cq, ck, 8)
    raises("same length", ea.attn_fwd_varlen, q, k, v, cq, ck[:3], 8)
    raises("seq_order", ea.attn_fwd_varlen, q, k, v, cq, ck, 8, seq_order=torch.zeros(2, dtype=i32))
    raises("at least two", ea.attn_fwd_varlen, q, k, v, cq[:1], ck[:1], 8)


# ------------------------------------------------------------------ MX fp8 forward

def mx_args(B=1, N=64, Hq=2, Hkv=1, d=128):
    return (z((B, N, Hq, d), u8), z((B, N, Hkv, d), u8), z((B, N, Hkv, d), u8),
            z((B, Hq, N, d // 32), u8), z((B, Hkv, N, d // 32), u8), z((B, N // 32, Hkv, d), u8))


def test_mx8_consistent_shapes_only_fail_on_device():
    raises("on a GPU", ea.attn_fwd_mx8, *mx_args())


@pytest.mark.parametrize("i,shape,name", [
    (1, (1, 32, 1, 128), "k8"), (2, (1, 32, 1, 128), "v8"), (3, (1, 1, 64, 8), "q_scale"),
    (4, (1, 64, 1, 4), "k_scale"), (5, (1, 64, 1, 128), "v_scale")])
def test_mx8_mismatch(i, shape, name):
    a = list(mx_args())
    a[i] = z(shape, u8)
    raises(f"{name} must have shape", ea.attn_fwd_mx8, *a)


def test_mx8_block_multiple():
    a = list(mx_args(N=48))
    raises("multiples of 32", ea.attn_fwd_mx8, *a)


# ------------------------------------------------------------------ backward

def test_bwd_mismatches():
    q, k, v = fwd_args(Hkv=2)
    o, do = z(q.shape), z(q.shape)
    lse = z((2, 4, 8), f32)
    raises("on a GPU", ea.attn_bwd, q, k, v, o, do, lse)
    raises("shapes", ea.attn_bwd, q, k, v, z((2, 8, 4, 32)), do, lse)
    raises("lse must be", ea.attn_bwd, q, k, v, o, do, z((2, 8, 4), f32))
    raises("k must be", ea.attn_bwd, q, z((3, 8, 2, 64)), z((3, 8, 2, 64)), o, do, lse)
    raises("workspace must be", ea.attn_bwd, q, k, v, o, do, lse, workspace=z((16,), f32))


# ------------------------------------------------------------------ paged decode

def dec_args(B=3, Hq=8, Hkv=2, d=128, P=10, ps=16, mp=4):
    return (z((B, Hq, d)), z((P, ps, Hkv, d)), z((P, ps, Hkv, d)), torch.zeros((B, mp), dtype=i32),
            torch.zeros((B,), dtype=i32))


def test_decode_consistent_shapes_only_fail_on_device():
    raises("on a GPU", ea.attn_decode_paged, *dec_args())


def test_decode_mismatches():
    q, kc, vc, bt, sl = dec_args()
    raises("v_cache must have shape", ea.attn_decode_paged, q, kc, z((10, 16, 2, 64)), bt, sl)
    raises("v_cache must have shape", ea.attn_decode_paged, q, kc, z((10, 16, 4, 128)), bt, sl)
    raises("head dim", ea.attn_decode_paged, q, z((10, 16, 2, 64)), z((10, 16, 2, 64)), bt, sl)
    raises("block_table must have 3 rows", ea.attn_decode_paged, q, kc, vc, torch.zeros((2, 4), dtype=i32), sl)
    raises("seq_lens must have shape", ea.attn_decode_paged, q, kc, vc, bt, torch.zeros((4,), dtype=i32))
    raises("page_size", ea.attn_decode_paged, q, kc, vc, bt, sl, 8)
    raises("block_table must be", ea.attn_decode_paged, q, kc, vc, bt.long(), sl)
    raises("workspace must be", ea.attn_decode_paged, q, kc, vc, bt, sl, workspace=z((16,), f32))
