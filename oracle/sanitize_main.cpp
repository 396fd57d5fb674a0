// TEST INFRASTRUCTURE ONLY: a command-line driver that runs every C entry
// point of the oracle once on inputs read from files, built by the tests
// with AddressSanitizer and UndefinedBehaviorSanitizer (g++, host code) so
// that an out-of-bounds access, a use after free or undefined arithmetic in
// the oracle stops the run.  It includes the oracle's source unchanged and
// writes the image, loss, image gradient and parameter gradients it got, so
// the test can also compare them with the shared-library build (the
// oracle's results must not depend on the thread count or the build).
//
//   sanitize_main <dir> <n> <w_l1> <w_ssim>
//     reads  <dir>/params.f32 [59][n], <dir>/camera.bin (or_camera),
//            <dir>/target.f32 [3][H][W]
//     writes <dir>/out_image.f32, out_dl.f64, out_grads.f64, out_loss.f64,
//            out_misc.f64 (checksums of the other entry points' outputs)
#include "gs_oracle.cpp"

#include <cstdio>
#include <cstdlib>
#include <string>

namespace {

template <class T>
std::vector<T> read_file(const std::string& path, size_t count) {
  std::vector<T> v(count);
  FILE* f = std::fopen(path.c_str(), "rb");
  if (f == nullptr || std::fread(v.data(), sizeof(T), count, f) != count) {
    std::fprintf(stderr, "cannot read %zu items from %s\n", count, path.c_str());
    std::exit(2);
  }
  std::fclose(f);
  return v;
}

template <class T>
void write_file(const std::string& path, const std::vector<T>& v) {
  FILE* f = std::fopen(path.c_str(), "wb");
  if (f == nullptr || std::fwrite(v.data(), sizeof(T), v.size(), f) != v.size()) {
    std::fprintf(stderr, "cannot write %s\n", path.c_str());
    std::exit(2);
  }
  std::fclose(f);
}

double sum(const std::vector<double>& v) {
  double s = 0.0;
  for (double x : v) s += x;
  return s;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 5) {
    std::fprintf(stderr, "usage: %s dir n w_l1 w_ssim\n", argv[0]);
    return 2;
  }
  const std::string dir = argv[1];
  const int64_t n = std::atoll(argv[2]);
  const double w_l1 = std::atof(argv[3]), w_ssim = std::atof(argv[4]);
  const std::vector<float> params = read_file<float>(dir + "/params.f32", size_t(59) * n);
  const or_camera cam = read_file<or_camera>(dir + "/camera.bin", 1)[0];
  const int W = cam.width, H = cam.height;
  const size_t P = size_t(W) * H;
  const int TX = (W + 15) / 16, TY = (H + 15) / 16;
  const std::vector<float> target = read_file<float>(dir + "/target.f32", 3 * P);

  // preprocess (fp32 and fp64) and the projection's internals
  std::vector<float> mean2d(2 * n), depth(n), cov2d(3 * n), conic(3 * n), opac(n), rgb(3 * n);
  std::vector<uint8_t> rgb_pos(3 * n), visible(n);
  std::vector<int32_t> radius(n), rect(4 * n);
  std::vector<uint32_t> tiles(n);
  or_preprocess(params.data(), n, n, &cam, mean2d.data(), depth.data(), cov2d.data(), conic.data(), opac.data(),
                rgb.data(), rgb_pos.data(), radius.data(), rect.data(), tiles.data(), visible.data());
  std::vector<double> p64(params.begin(), params.end());
  std::vector<double> m2(2 * n), d1(n), c3(3 * n), k3(3 * n), o1(n), r3(3 * n);
  or_preprocess_f64(p64.data(), n, n, &cam, m2.data(), d1.data(), c3.data(), k3.data(), o1.data(), r3.data());
  std::vector<double> Rq(9 * n), Sig(9 * n), craw(3 * n);
  or_projection_internals_f64(p64.data(), n, n, &cam, Rq.data(), Sig.data(), craw.data());

  // binning: count, then fill
  const int64_t M = or_bin(params.data(), n, n, &cam, nullptr, nullptr, 0, nullptr);
  std::vector<uint64_t> keys(M > 0 ? M : 1);
  std::vector<int32_t> vals(M > 0 ? M : 1);
  std::vector<uint32_t> ranges(2 * size_t(TX) * TY);
  or_bin(params.data(), n, n, &cam, keys.data(), vals.data(), M, ranges.data());

  // render, brute-force render, sampled pixels
  std::vector<float> image(3 * P), Tf(P), image_b(3 * P), Tf_b(P);
  std::vector<uint32_t> last(P), proc(size_t(TX) * TY), last_b(P);
  or_render(params.data(), n, n, &cam, image.data(), Tf.data(), last.data(), proc.data());
  or_render_brute(params.data(), n, n, &cam, image_b.data(), Tf_b.data(), last_b.data());
  if (image != image_b || last != last_b) {
    std::fprintf(stderr, "brute-force render differs from the tiled one\n");
    return 3;
  }
  const int K = 64;
  std::vector<int32_t> px(K), py(K);
  for (int k = 0; k < K; ++k) {
    px[k] = int32_t((uint64_t(k) * 2654435761u) % uint64_t(W));
    py[k] = int32_t((uint64_t(k) * 40503u + 7u) % uint64_t(H));
  }
  std::vector<float> srgb(3 * K), sT(K);
  std::vector<uint32_t> slast(K);
  or_composite_pixels(params.data(), n, n, &cam, vals.data(), ranges.data(), px.data(), py.data(), K, srgb.data(),
                      sT.data(), slast.data());

  // loss, backward (with and without a magnitude map), projection backward
  std::vector<double> dL(3 * P);
  double l1 = 0.0, ss = 0.0;
  const double L = or_loss(image.data(), target.data(), W, H, w_l1, w_ssim, dL.data(), &l1, &ss);
  std::vector<double> g2d(9 * n), m2d(9 * n), grads(59 * size_t(n), 0.0), mags(59 * size_t(n), 0.0);
  or_backward(params.data(), n, n, &cam, dL.data(), nullptr, g2d.data(), m2d.data(), grads.data(), mags.data(), 1);
  std::vector<double> gmag(3 * P, 1e-4), g2d_b(9 * n), m2d_b(9 * n), gr_b(59 * size_t(n), 0.0),
      mg_b(59 * size_t(n), 0.0);
  or_backward(params.data(), n, n, &cam, dL.data(), gmag.data(), g2d_b.data(), m2d_b.data(), gr_b.data(),
              mg_b.data(), 0);
  std::vector<double> pg(59 * size_t(n), 0.0);
  or_project_backward(params.data(), n, n, &cam, g2d.data(), pg.data());
  std::vector<double> out9(9 * n);
  or_project_outputs_f64(params.data(), p64.data(), n, n, &cam, out9.data());

  // frozen fp64 forward and loss
  std::vector<double> img64(3 * P);
  or_render_frozen_f64(params.data(), p64.data(), n, n, &cam, img64.data());
  const double Lf = or_loss_frozen_f64(img64.data(), image.data(), target.data(), W, H, w_l1, w_ssim);

  // Adam over the visible rows
  std::vector<int32_t> rows;
  for (int64_t i = 0; i < n; ++i)
    if (visible[i]) rows.push_back(int32_t(i));
  std::vector<double> pa(p64), ma(59 * size_t(n), 0.0), va(59 * size_t(n), 0.0);
  or_adam(pa.data(), grads.data(), ma.data(), va.data(), n, rows.data(), int64_t(rows.size()), 1e-3, 0.9, 0.999,
          1e-15, 0.1, 0.001);

  // SH basis and the exponential
  std::vector<double> dirs = {1.0, 0.0, 0.0, 0.0, 0.6, 0.8}, Y(32);
  or_sh_basis_f64(dirs.data(), 2, Y.data());
  std::vector<float> dirs32 = {0.0f, 1.0f, 0.0f}, Y32(16);
  or_sh_basis_f32(dirs32.data(), 1, Y32.data());

  write_file(dir + "/out_image.f32", image);
  write_file(dir + "/out_dl.f64", dL);
  write_file(dir + "/out_grads.f64", grads);
  write_file(dir + "/out_loss.f64", std::vector<double>{L, l1, ss, Lf});
  write_file(dir + "/out_misc.f64",
             std::vector<double>{double(M), sum(d1), sum(Sig), sum(craw), sum(std::vector<double>(srgb.begin(), srgb.end())),
                                 sum(gr_b), sum(mg_b), sum(pg), sum(out9), sum(img64), sum(pa), sum(Y),
                                 double(Y32[1]), double(or_pexp(-1.0f))});
  std::printf("ok n=%lld M=%lld loss=%.9g\n", (long long)n, (long long)M, L);
  return 0;
}
