// Driver for the sanitizer build of the host Lloyd-Max solver: runs it over a
// grid of (d, bits), checks that every centroid is finite, strictly
// increasing inside (0, 1) on the positive half, and that d = 3 gives the
// uniform grid's positive half, (2 k + 1) / L. Exit status 0 on success.
#include <cmath>
#include <cstdio>
#include <vector>

namespace tq {
bool lloyd_max_positive_half(int d, int bits, std::vector<double> &c);
}

int main() {
  const int dims[] = {3, 4, 5, 7, 16, 64, 128, 256};
  int bad = 0;
  for (int d : dims) {
    for (int bits = 1; bits <= 6; ++bits) {
      std::vector<double> c;
      if (!tq::lloyd_max_positive_half(d, bits, c)) {
        std::printf("d=%d bits=%d did not settle\n", d, bits);
        ++bad;
        continue;
      }
      const int H = 1 << (bits - 1);
      for (int k = 0; k < H; ++k) {
        const bool ok = std::isfinite(c[k]) && c[k] > 0.0 && c[k] < 1.0 && (k == 0 || c[k] > c[k - 1]);
        if (!ok) {
          std::printf("d=%d bits=%d c[%d]=%.17g\n", d, bits, k, c[k]);
          ++bad;
        }
        if (d == 3 && std::fabs(c[k] - (2.0 * k + 1.0) / (2.0 * H)) > 1e-12) {
          std::printf("d=3 bits=%d c[%d]=%.17g not uniform\n", bits, k, c[k]);
          ++bad;
        }
      }
    }
  }
  std::printf("%s\n", bad ? "FAILED" : "ok");
  return bad ? 1 : 0;
}
