"""View coupling on the GPU (gs_view_overlap, gs_view_priority) against the
oracle (Odin summary page, "Relative locality graph"): every intersection
count exactly, every Jaccard weight and priority bit for bit (both sides
divide and add in IEEE fp64 in the same order).

Inputs: seeded synthetic index lists (runs and scattered indices, empty
and full sets, ragged word and tile edges) and the visible lists the
preprocess emits for orbit and flight cameras, those compared first with
the oracle's own visible lists so that every expected value comes from the
oracle."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def gpu_overlap(lists, n, ld=None, counts=None, fill_seed=0, weights=True):
    """Rows of a [B][ld] device buffer hold the lists; the tail of each row
    is filled with valid-looking indices that must not be read."""
    import differentiable_gaussian_splatting_dgs_amd as gs
    B = len(lists)
    ld = ld or max(n, 1)
    rng = np.random.default_rng(fill_seed)
    host = rng.integers(0, max(n, 1), (max(B, 1), ld)).astype(np.int32)
    for v, l in enumerate(lists):
        host[v, :l.size] = l
    cnt = np.array([l.size for l in lists] if counts is None else counts, np.int64)
    dev = torch.from_numpy(host).cuda()
    dcnt = torch.from_numpy(cnt).cuda() if B > 0 else torch.zeros(1, dtype=torch.int64, device="cuda")
    inter = torch.full((max(B, 1), max(B, 1)), -7, dtype=torch.int64, device="cuda")
    w = torch.full((max(B, 1), max(B, 1)), -7.0, dtype=torch.float64, device="cuda") if weights else None
    ws = torch.empty(max(gs.gs_workspace_size(gs.GS_OP_VIEW_OVERLAP, n, B), 256), dtype=torch.uint8,
                     device="cuda")
    gs.gs_view_overlap(dev, ld, dcnt, B, n, inter, w, ws)
    torch.cuda.synchronize()
    return inter.cpu().numpy()[:B, :B], (w.cpu().numpy()[:B, :B] if weights else None)


def gpu_priority(w, prev):
    import differentiable_gaussian_splatting_dgs_amd as gs
    B = w.shape[0]
    dw = torch.from_numpy(np.ascontiguousarray(w)).cuda()
    dp = torch.from_numpy(np.asarray(prev, np.int32)).cuda() if len(prev) else None
    s = torch.full((B,), -7.0, dtype=torch.float64, device="cuda")
    gs.gs_view_priority(dw, B, dp, len(prev), s)
    torch.cuda.synchronize()
    return s.cpu().numpy()


def check_exact(tag, inter, w, lists):
    oi = oracle.view_overlap(lists)
    ow = oracle.view_coupling(oi)
    bad = np.argwhere(inter != oi)
    assert bad.size == 0, f"{tag}: {len(bad)} counts differ, first {bad[0]}: {inter[tuple(bad[0])]} vs " \
                          f"{oi[tuple(bad[0])]}"
    if w is not None:
        assert np.array_equal(w.view(np.uint64), ow.view(np.uint64)), f"{tag}: weights not bit-identical"
    say(f"[coupling {tag}] B={len(lists)} exact; max w off-diagonal "
        f"{(ow - np.eye(len(lists))).max() if len(lists) else 0:.3f}")
    return oi, ow


@pytest.mark.parametrize("n,B", [(20_011, 130), (4096, 64), (33, 65), (31, 1), (1, 3), (100_003, 17)])
def test_overlap_matches_oracle_on_random_lists(n, B):
    rng = np.random.default_rng(n * 1000 + B)
    lists = synth.random_visible_lists(rng, n, B)
    inter, w = gpu_overlap(lists, n, fill_seed=B)
    check_exact(f"random n={n}", inter, w, lists)


def test_overlap_edge_cases():
    # no Gaussians: every set empty, every weight 0
    inter, w = gpu_overlap([np.zeros(0, np.int32)] * 3, 0)
    assert (inter == 0).all() and (w == 0).all()
    # disjoint sets: zero off the diagonal, ones on it
    n = 640
    lists = [np.arange(v, n, 5, dtype=np.int32) for v in range(5)]
    inter, w = gpu_overlap(lists, n)
    check_exact("disjoint", inter, w, lists)
    assert (w == np.eye(5)).all()
    # a narrower row stride than n, weights not asked for
    inter, w = gpu_overlap(lists, n, ld=200, weights=False)
    assert w is None
    check_exact("ld < n", inter, None, lists)
    # entries outside [0, n) are skipped and counts are read as
    # min(max(count, 0), ld): the oracle sees the lists without them
    raw = [np.array([-9, -1, 3, 7, 31, 32, 600], np.int32),
           np.array([0, 3, 32, 639, 640, 700], np.int32),
           np.arange(0, 640, dtype=np.int32)]
    inter, w = gpu_overlap(raw, n, ld=640, counts=[7, 6, 10_000])
    check_exact("out of range", inter, w, [l[(l >= 0) & (l < n)] for l in raw])
    inter, w = gpu_overlap(raw[:2], n, counts=[-5, 2])
    check_exact("negative count", inter, w, [raw[0][:0], raw[1][:2]])


def test_overlap_of_preprocess_visible_lists():
    """Visible lists from gs_preprocess for 70 orbit views of a cut-down
    small scene and 40 flight views over a cut-down aerial ground: the lists
    equal the oracle's, then the coupling equals the oracle's on them."""
    import differentiable_gaussian_splatting_dgs_amd as gs
    base = synth.workload(1)
    idx = np.linspace(0, base.n - 1, 5003).round().astype(np.int64)
    params = np.ascontiguousarray(base.params[:, idx])
    for tag, cams in (("orbit", synth.orbit_cameras(160, 120, 70, radius=2.5)),
                      ("flight", synth.flight_cameras(192, 108, 40, height_above=2.0))):
        vc = gs.ViewCoupling(params.shape[1], len(cams), "cuda")
        dp = torch.from_numpy(params).cuda()
        vc.visible_lists(dp, params.shape[1], cams)
        inter, w = vc.overlap()
        torch.cuda.synchronize()
        olists = [oracle.visible_list(params, c) for c in cams]
        counts = vc.counts.cpu().numpy()
        rows = vc.lists.cpu().numpy()
        for v, ol in enumerate(olists):
            assert counts[v] == ol.size and np.array_equal(rows[v, :ol.size], ol), f"{tag} view {v} list"
        oi, ow = check_exact(f"preprocess {tag}", inter.cpu().numpy(), w.cpu().numpy(), olists)
        assert 0 < (oi > 0).sum() < oi.size or tag == "orbit"


def test_priority_matches_oracle():
    rng = np.random.default_rng(5)
    n, B = 20_011, 130
    lists = synth.random_visible_lists(rng, n, B)
    oi = oracle.view_overlap(lists)
    ow = oracle.view_coupling(oi)
    for prev in ([], [3], [0, 5, 5, 129], list(rng.permutation(B)[:40]), list(range(B))):
        s = gpu_priority(ow, prev)
        so = oracle.view_priority(ow, prev)
        assert np.array_equal(s.view(np.uint64), so.view(np.uint64)), f"priority prev={prev[:6]}"
    # entries outside [0, B) are skipped
    s = gpu_priority(ow, [-1, 2, B, 7])
    assert np.array_equal(s, oracle.view_priority(ow, [2, 7]))
    say("[coupling priority] bit-exact")


def test_overlap_many_views_sampled():
    """4,096 views (64 tiles of 64 views a side, 2,080 tiles on or above the
    diagonal): 3,000 sampled pairs against the oracle on just those two
    lists, the diagonal against the list lengths, symmetry."""
    rng = np.random.default_rng(4096)
    n, B = 3001, 4096
    lists = synth.random_visible_lists(rng, n, B)
    inter, w = gpu_overlap(lists, n)
    assert np.array_equal(inter, inter.T)
    assert np.array_equal(np.diag(inter), [l.size for l in lists])
    pairs = rng.integers(0, B, (3000, 2))
    for i, j in pairs:
        oi = oracle.view_overlap([lists[i], lists[j]])
        ow = oracle.view_coupling(oi)
        assert inter[i, j] == oi[0, 1], (i, j)
        assert w[i, j].view(np.uint64) == ow[0, 1].view(np.uint64), (i, j)
    say(f"[coupling B={B}] 3000 sampled pairs exact")
