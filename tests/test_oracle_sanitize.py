"""The oracle's C++ under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

`oracle/sanitize_main.cpp` includes the oracle's source unchanged and runs
every C entry point once (preprocess in fp32 and fp64, binning, tiled,
brute-force and sampled-pixel rendering, the loss, the backward with and
without a magnitude map, the projection backward, the frozen fp64 forward
and loss, Adam, the SH basis and the exponential).  Built single-threaded
with -fsanitize=address,undefined and no recovery, so any out-of-bounds
access, use after free, signed overflow or invalid shift ends the run with
an error.  Its image, loss, image gradient and parameter gradients must also
equal the OpenMP shared-library build's bit for bit: the oracle's results
do not depend on the thread count.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sanitize_main.cpp")


@pytest.fixture(scope="module")
def sanitized_exe(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("san") / "sanitize_main")
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fno-fast-math",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", exe, SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("case", ["tiny_l1", "tiny_ssim", "small_cut"])
def test_oracle_clean_under_sanitizers(sanitized_exe, tmp_path, case):
    if case.startswith("tiny"):
        w = synth.workload(0)
        weights = (1.0, 0.0) if case == "tiny_l1" else (0.8, 0.2)
    else:
        w = synth.cut_down(synth.workload(1), 200, 136, n=6000)
        weights = (0.8, 0.2)
    cam, tgt = w.cameras[0], w.targets[0]
    np.ascontiguousarray(w.params, np.float32).tofile(tmp_path / "params.f32")
    (tmp_path / "camera.bin").write_bytes(bytes(oracle.cam_struct(cam)))
    np.ascontiguousarray(tgt, np.float32).tofile(tmp_path / "target.f32")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sanitized_exe, str(tmp_path), str(w.n), str(weights[0]), str(weights[1])],
                       capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr
    # the same results as the OpenMP shared-library build
    H, W = cam.height, cam.width
    img, _, _, _ = oracle.render(w.params, cam)
    L, dL, _, _ = oracle.loss(img, tgt, *weights)
    _, _, grads, _ = oracle.backward(w.params, cam, dL, at_fp32=True)
    assert np.array_equal(np.fromfile(tmp_path / "out_image.f32", np.float32).reshape(3, H, W), img)
    assert np.fromfile(tmp_path / "out_loss.f64")[0] == L
    assert np.array_equal(np.fromfile(tmp_path / "out_dl.f64").reshape(3, H, W), dL)
    assert np.array_equal(np.fromfile(tmp_path / "out_grads.f64").reshape(59, w.n), grads)
    assert int(np.fromfile(tmp_path / "out_misc.f64")[0]) == len(oracle.bin_sort(w.params, cam)[0])
