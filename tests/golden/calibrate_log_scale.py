"""Find the mean of the per-axis log-scale normal for which about 90% of the
Gaussians visible in view 0 have a screen radius below 2% of the image width
(the Grendel-GS notes, "Sparse All-to-All communication", report this share
for real scenes).  Calls only ``synth`` and ``oracle``; prints the constants
that ``synth`` carries as LOG_SCALE_MU_SCENE / LOG_SCALE_MU_AERIAL.

    python tests/golden/calibrate_log_scale.py
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "..", ".."))
import oracle  # noqa: E402
import synth   # noqa: E402


def share_below(w, mu, sigma):
    p = w.params.copy()
    rng = np.random.default_rng(777)
    p[3:6] = rng.normal(mu, sigma, (3, w.n)).astype(np.float32)
    cam = w.cameras[0]
    pre = oracle.preprocess(p, cam)
    r = pre["radius"][pre["visible"]]
    return float(np.mean(r < 0.02 * cam.width))


def bisect(w, sigma, lo=-7.0, hi=-2.0, target=0.90):
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        if share_below(w, mid, sigma) > target:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


if __name__ == "__main__":
    scene = synth.plane_scene(1, 200_000, 1920, 1080, [0.0], seed=1)
    mu_s = bisect(scene, 0.5)
    print(f"LOG_SCALE_MU_SCENE  = {mu_s:.2f}   (share {share_below(scene, round(mu_s, 2), 0.5):.4f})")
    aer = synth.aerial(n=300_000)
    mu_a = bisect(aer, 0.8)
    print(f"LOG_SCALE_MU_AERIAL = {mu_a:.2f}   (share {share_below(aer, round(mu_a, 2), 0.8):.4f})")
