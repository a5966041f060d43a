"""moga_permute_vt_noalloc (the entry point that allocates nothing: its sort
scratch is a fixed per-GPU device array in the library) against
moga_permute_vt with a caller workspace, through the C ABI: every output
bit for bit, on two calls in a row, the second with a smaller input, so that
the scratch left by the first call must not leak into the second."""

import ctypes

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def moga():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_long_router_amd as m
    return m


def _case(N, H, D, M, seed, with_q):
    g = torch.Generator(device="cpu").manual_seed(seed)
    # uneven groups, some empty: ids drawn from a skewed distribution over [0, M)
    w = torch.arange(1, M + 1, dtype=torch.float64) ** -1.3
    w[M // 2] = 0.0
    gid = torch.multinomial(w, N, replacement=True, generator=g).to(torch.int32)
    K, V = (torch.randn((N, H, D), generator=g).bfloat16() for _ in range(2))
    Q = torch.randn((N, H, D), generator=g).bfloat16() if with_q else None
    return gid.to(DEV), (None if Q is None else Q.to(DEV)), K.to(DEV), V.to(DEV)


def _noalloc_raw(moga, gid, M, Q, K, V, outs):
    """Direct ctypes call of the C entry point on preallocated outputs."""
    from sparse_attention_long_router_amd import _lib
    N, H, D = K.shape
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    return _lib.LIB.moga_permute_vt_noalloc(p(gid), p(Q), p(K), p(V), N, H, D, M, p(outs["Qp"]), p(outs["Kp"]),
                                            p(outs["Vt"]), p(outs["perm"]), p(outs["cu_seqlens"]),
                                            p(outs["max_seqlen"]), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("with_q", [False, True])
def test_noalloc_matches_workspace_path(moga, with_q):
    cases = [(120000, 4, 128, 48, 1), (5000, 2, 64, 7, 2)]   # second call: smaller N, fewer groups
    for N, H, D, M, seed in cases:
        print(f"[no-alloc] N={N} H={H} D={D} M={M} with_q={with_q}", flush=True)
        gid, Q, K, V = _case(N, H, D, M, seed, with_q)
        ref = moga.moga_permute_vt(gid, M, Q, K, V)
        outs = {k: (torch.full_like(v, -7) if v is not None and v.dtype == torch.int32 else
                    (torch.full_like(v, float("nan")) if v is not None else None)) for k, v in ref.items()}
        rc = _noalloc_raw(moga, gid, M, Q, K, V, outs)
        assert rc == 0, rc
        torch.cuda.synchronize()
        for k in ("perm", "cu_seqlens", "max_seqlen"):
            assert torch.equal(outs[k], ref[k]), k
        assert torch.equal(outs["Kp"].view(torch.int16), ref["Kp"].view(torch.int16))
        assert torch.equal(outs["Vt"].view(torch.int16), ref["Vt"].view(torch.int16))
        if with_q:
            assert torch.equal(outs["Qp"].view(torch.int16), ref["Qp"].view(torch.int16))
        # and through the binding
        b = moga.moga_permute_vt_noalloc(gid, M, Q, K, V)
        torch.cuda.synchronize()
        assert torch.equal(b["perm"], ref["perm"]) and torch.equal(b["cu_seqlens"], ref["cu_seqlens"])


def test_noalloc_rejects_sizes_beyond_its_scratch(moga):
    """8 * M * ceil(N / 1024) bytes above 1 MiB: refused before any launch."""
    from sparse_attention_long_router_amd import _lib
    fake = ctypes.c_void_p(4096)  # never dereferenced: the size check fails first
    N, M = (1 << 21) + 1024, 64
    rc = _lib.LIB.moga_permute_vt_noalloc(fake, None, fake, fake, N, 1, 64, M, None, fake, fake, fake, fake, fake,
                                          None)
    assert rc == -4  # MOGA_ERR_WORKSPACE
