"""gs_sparse_adam_noalloc (the allocation-free variant of gs_sparse_adam,
for callers that cannot allocate device memory) against gs_sparse_adam,
through the C ABI: two calls in a row on the same GPU (its scratch array
keeps the first call's contents), the second on a smaller input; results
bit-identical (the same kernels, the same arithmetic).  Also the host-side
rejection of a size beyond the scratch, which launches nothing."""
import ctypes as C

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(n, seed, density):
    """Seeded parameters, gradients, moments and union flags of n rows."""
    rng = np.random.default_rng(seed)
    ld = n + 7
    state = [rng.standard_normal((59, ld)).astype(np.float32) for _ in range(2)]
    m = (0.1 * rng.standard_normal((59, ld))).astype(np.float32)
    v = (0.01 * rng.random((59, ld))).astype(np.float32)
    flags = np.zeros(((n + 15) // 16) * 16, np.uint8)
    flags[:n] = rng.random(n) < density
    return ld, state[0], state[1], m, v, flags


def _run(fn_name, n, ld, p, g, m, v, flags, with_ws):
    import differentiable_gaussian_splatting_dgs_amd as gs
    L = gs.lib()
    dev = torch.device("cuda:0")
    tp, tg, tm, tv = (torch.from_numpy(a.copy()).to(dev) for a in (p, g, m, v))
    tf = torch.from_numpy(flags.copy()).to(dev)
    idx = torch.full((max(n, 1),), -1, dtype=torch.int32, device=dev)
    cnt = torch.full((1,), -1, dtype=torch.int64, device=dev)
    lr, b1, b2, eps = 2e-3, 0.9 ** 4, 0.999 ** 4, 1e-15
    bc1, bc2 = 1 - b1 ** 3, 1 - b2 ** 3
    s = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: C.c_void_p(t.data_ptr())
    args = [P(tp), P(tg), P(tm), P(tv), n, ld, P(tf), P(idx), P(cnt), C.c_float(lr), C.c_float(b1), C.c_float(b2),
            C.c_float(eps), C.c_float(bc1), C.c_float(bc2)]
    if with_ws:
        ws = torch.empty(gs.gs_workspace_size(gs.GS_OP_SPARSE_ADAM, n), dtype=torch.uint8, device=dev)
        args += [P(ws), C.c_size_t(ws.numel())]
    st = getattr(L, fn_name)(*args, s)
    assert st == gs.GS_OK, gs.gs_last_error()
    torch.cuda.synchronize()
    k = int(cnt.item())
    return dict(p=tp.cpu().numpy(), g=tg.cpu().numpy(), m=tm.cpu().numpy(), v=tv.cpu().numpy(),
                flags=tf.cpu().numpy(), idx=idx[:k].cpu().numpy(), count=k)


def test_noalloc_adam_matches_the_workspace_entry_point():
    """Two calls in a row (the second smaller: its compaction reads fewer
    scratch words than the first left), each against gs_sparse_adam on the
    same inputs; then the first size again after the smaller one."""
    for n, seed, dens in ((300_001, 1, 0.35), (5_003, 2, 0.8), (300_001, 3, 0.05)):
        ld, p, g, m, v, flags = _case(n, seed, dens)
        print(f"[noalloc] n={n} ld={ld} listed={int(flags.sum())}", flush=True)
        a = _run("gs_sparse_adam", n, ld, p, g, m, v, flags, True)
        b = _run("gs_sparse_adam_noalloc", n, ld, p, g, m, v, flags, False)
        assert a["count"] == b["count"] == int(flags.sum())
        assert np.array_equal(a["idx"], b["idx"])
        assert np.array_equal(b["idx"], np.flatnonzero(flags[:n]).astype(np.int32))
        for key in ("p", "g", "m", "v", "flags"):
            assert np.array_equal(a[key].view(np.uint32), b[key].view(np.uint32)), key
        # rows outside the union and the padding columns untouched
        out = np.ones(ld, bool)
        out[b["idx"]] = False
        assert np.array_equal(b["p"][:, out], p[:, out]) and np.array_equal(b["m"][:, out], m[:, out])
        assert not b["flags"].any()


def test_noalloc_adam_rejects_sizes_beyond_its_scratch():
    import differentiable_gaussian_splatting_dgs_amd as gs
    L = gs.lib()
    n = gs.GS_NOALLOC_MAX_N + 1
    one = torch.zeros(16, dtype=torch.float32, device="cuda:0")
    P = C.c_void_p(one.data_ptr())
    st = L.gs_sparse_adam_noalloc(P, P, P, P, n, n, P, P, P, C.c_float(1e-3), C.c_float(0.9), C.c_float(0.999),
                                  C.c_float(1e-15), C.c_float(0.1), C.c_float(0.001),
                                  C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == gs.GS_ERR_INVALID_ARG
    assert "scratch" in gs.gs_last_error()
    torch.cuda.synchronize()
