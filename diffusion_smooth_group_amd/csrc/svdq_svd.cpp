// svdq_svd.cpp -- host truncated SVD used by the offline pack.
//
// The SVDQuant paper splits the smoothed weight W_hat into a rank-r branch
// L1 L2 and a residual; the truncated SVD gives the split with the smallest
// residual (Eckart-Young-Mirsky; SVDQuant §4.2, Fig. 5).  Only the top r
// singular triplets are needed, and r (16..64) is tiny next to K and N, so:
//   1. Gram matrix of the shorter side in float64 (blocked, multithreaded),
//   2. Lanczos on the Gram matrix with full reorthogonalisation (two
//      classical Gram-Schmidt passes) and restarts on invariant subspaces,
//   3. the tridiagonal eigenproblem by implicit symmetric QR steps with a
//      Wilkinson shift (Golub & Van Loan, "Matrix Computations", §8.3),
//   4. back-transformation to the other side's singular vectors.
// No LAPACK: the library depends on nothing beyond the HIP runtime.
#include <immintrin.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <thread>
#include <vector>

#include "svdq_host.h"

namespace svdq {

int host_threads() {
  static int n = [] {
    int t = int(std::thread::hardware_concurrency());
    const char* e = std::getenv("SVDQ_NUM_THREADS");
    if (!e) e = std::getenv("OMP_NUM_THREADS");
    if (e && std::atoi(e) > 0) t = std::min(t > 0 ? t : 1, std::atoi(e));
    return std::max(1, std::min(t, 64));
  }();
  return n;
}

void parallel_for(int64_t n, const std::function<void(int64_t, int64_t)>& f) {
  int nt = host_threads();
  if (n <= 0) return;
  if (nt <= 1 || n < 2) { f(0, n); return; }
  nt = int(std::min<int64_t>(nt, n));
  std::vector<std::thread> th;
  th.reserve(nt);
  for (int t = 0; t < nt; ++t) {
    int64_t b = n * t / nt, e = n * (t + 1) / nt;
    th.emplace_back([&f, b, e] { f(b, e); });
  }
  for (auto& x : th) x.join();
}

namespace {

// G = B B^T for B (s x L, row-major).  Full symmetric result.  32 x 32
// tiles of G (upper triangle) over 512-long slices of L; 2 x 4 register
// micro-tiles with AVX2 FMA accumulators.
void gram(const double* B, int64_t s, int64_t L, double* G) {
  const int64_t TB = 32, LC = 512;
  int64_t nt = (s + TB - 1) / TB;
  std::vector<std::pair<int64_t, int64_t>> tiles;
  for (int64_t i = 0; i < nt; ++i)
    for (int64_t j = i; j < nt; ++j) tiles.push_back({i, j});
  parallel_for(int64_t(tiles.size()), [&](int64_t tb, int64_t te) {
    std::vector<double> acc(TB * TB);
    for (int64_t t = tb; t < te; ++t) {
      int64_t i0 = tiles[t].first * TB, j0 = tiles[t].second * TB;
      int64_t ni = std::min(TB, s - i0), nj = std::min(TB, s - j0);
      std::fill(acc.begin(), acc.end(), 0.0);
      for (int64_t l0 = 0; l0 < L; l0 += LC) {
        int64_t nl = std::min(LC, L - l0);
        int64_t nl4 = nl & ~int64_t(3);
        for (int64_t ii = 0; ii < ni; ii += 2) {
          int64_t ri = std::min<int64_t>(2, ni - ii);
          for (int64_t jj = 0; jj < nj; jj += 4) {
            int64_t rj = std::min<int64_t>(4, nj - jj);
            const double* a0p = B + (i0 + ii) * L + l0;
            const double* a1p = B + (i0 + ii + std::min<int64_t>(1, ri - 1)) * L + l0;
            const double* b0p = B + (j0 + jj) * L + l0;
            const double* b1p = B + (j0 + jj + std::min<int64_t>(1, rj - 1)) * L + l0;
            const double* b2p = B + (j0 + jj + std::min<int64_t>(2, rj - 1)) * L + l0;
            const double* b3p = B + (j0 + jj + std::min<int64_t>(3, rj - 1)) * L + l0;
            __m256d c00 = _mm256_setzero_pd(), c01 = c00, c02 = c00, c03 = c00;
            __m256d c10 = c00, c11 = c00, c12 = c00, c13 = c00;
            for (int64_t l = 0; l < nl4; l += 4) {
              const __m256d a0 = _mm256_loadu_pd(a0p + l), a1 = _mm256_loadu_pd(a1p + l);
              __m256d b = _mm256_loadu_pd(b0p + l);
              c00 = _mm256_fmadd_pd(a0, b, c00); c10 = _mm256_fmadd_pd(a1, b, c10);
              b = _mm256_loadu_pd(b1p + l);
              c01 = _mm256_fmadd_pd(a0, b, c01); c11 = _mm256_fmadd_pd(a1, b, c11);
              b = _mm256_loadu_pd(b2p + l);
              c02 = _mm256_fmadd_pd(a0, b, c02); c12 = _mm256_fmadd_pd(a1, b, c12);
              b = _mm256_loadu_pd(b3p + l);
              c03 = _mm256_fmadd_pd(a0, b, c03); c13 = _mm256_fmadd_pd(a1, b, c13);
            }
            double r[2][4];
            const __m256d cs[2][4] = {{c00, c01, c02, c03}, {c10, c11, c12, c13}};
            for (int x = 0; x < 2; ++x)
              for (int y = 0; y < 4; ++y) {
                alignas(32) double v[4];
                _mm256_store_pd(v, cs[x][y]);
                r[x][y] = (v[0] + v[1]) + (v[2] + v[3]);
              }
            const double* ap[2] = {a0p, a1p};
            const double* bp[4] = {b0p, b1p, b2p, b3p};
            for (int64_t l = nl4; l < nl; ++l)
              for (int x = 0; x < 2; ++x)
                for (int y = 0; y < 4; ++y) r[x][y] += ap[x][l] * bp[y][l];
            for (int64_t x = 0; x < ri; ++x)
              for (int64_t y = 0; y < rj; ++y) acc[(ii + x) * TB + jj + y] += r[x][y];
          }
        }
      }
      for (int64_t x = 0; x < ni; ++x)
        for (int64_t y = 0; y < nj; ++y) {
          G[(i0 + x) * s + j0 + y] = acc[x * TB + y];
          G[(j0 + y) * s + i0 + x] = acc[x * TB + y];
        }
    }
  });
}

// Symmetric tridiagonal eigenproblem: d[n] diagonal, e[n-1] off-diagonal
// (e[i] couples i and i+1).  On return d holds the eigenvalues; Z (zr x n
// row-major) holds rows row0 .. row0+zr-1 of the eigenvector matrix, whose
// column i belongs to d[i] (zr = n, row0 = 0 gives all eigenvectors; zr = 1,
// row0 = n-1 only the last components, enough for the Ritz residuals).
// Implicit QR steps with a Wilkinson shift on the trailing unreduced block;
// each step chases the bulge down with Givens similarities.
bool tridiag_eig(int n, double* d, double* e, double* Z, int zr, int row0) {
  std::fill(Z, Z + size_t(zr) * n, 0.0);
  for (int i = 0; i < zr; ++i) Z[size_t(i) * n + row0 + i] = 1.0;
  if (n <= 1) return true;
  const double eps = 2.220446049250313e-16;
  int q = n - 1;
  long iters = 0, max_iters = 60L * n;
  while (q > 0) {
    for (int i = 0; i < q; ++i)
      if (std::fabs(e[i]) <= eps * (std::fabs(d[i]) + std::fabs(d[i + 1]))) e[i] = 0.0;
    if (e[q - 1] == 0.0) { --q; continue; }
    int p = q - 1;
    while (p > 0 && e[p - 1] != 0.0) --p;
    if (++iters > max_iters) return false;
    // Wilkinson shift from the trailing 2 x 2 block
    double dd = 0.5 * (d[q - 1] - d[q]);
    double ee = e[q - 1];
    double den = dd + std::copysign(std::hypot(dd, ee), dd == 0.0 ? 1.0 : dd);
    double mu = d[q] - (den != 0.0 ? ee * ee / den : 0.0);
    double x = d[p] - mu, z = e[p];
    for (int k = p; k < q; ++k) {
      double r = std::hypot(x, z);
      double c = 1.0, s = 0.0;
      if (r != 0.0) { c = x / r; s = z / r; }
      if (k > p) e[k - 1] = r;
      double a = d[k], b = e[k], cc = d[k + 1];
      d[k] = c * c * a + 2.0 * c * s * b + s * s * cc;
      d[k + 1] = s * s * a - 2.0 * c * s * b + c * c * cc;
      e[k] = c * s * (cc - a) + (c * c - s * s) * b;
      if (k < q - 1) {
        z = s * e[k + 1];
        e[k + 1] = c * e[k + 1];
        x = e[k];
      }
      for (int i = 0; i < zr; ++i) {
        double zk = Z[size_t(i) * n + k], zk1 = Z[size_t(i) * n + k + 1];
        Z[size_t(i) * n + k] = c * zk + s * zk1;
        Z[size_t(i) * n + k + 1] = -s * zk + c * zk1;
      }
    }
  }
  return true;
}

struct Rng {
  uint64_t s;
  explicit Rng(uint64_t seed) : s(seed ? seed : 0x9E3779B97F4A7C15ull) {}
  double next() {  // xorshift64*, uniform in (-1, 1)
    s ^= s >> 12; s ^= s << 25; s ^= s >> 27;
    uint64_t v = s * 0x2545F4914F6CDD1Dull;
    return (double(v >> 11) * (1.0 / 9007199254740992.0)) * 2.0 - 1.0;
  }
};

// w -= Q[0..nq) (Q^T w), twice; Q rows are orthonormal vectors of length s.
void reorth(const std::vector<double>& Q, int64_t nq, int64_t s, double* w) {
  if (nq == 0) return;
  int nt = host_threads();
  for (int pass = 0; pass < 2; ++pass) {
    std::vector<double> part(size_t(nt) * nq, 0.0);
    int64_t nchunk = std::min<int64_t>(nt, std::max<int64_t>(1, s / 256));
    parallel_for(nchunk, [&](int64_t cb, int64_t ce) {
      for (int64_t c = cb; c < ce; ++c) {
        int64_t b = s * c / nchunk, e = s * (c + 1) / nchunk;
        for (int64_t i = 0; i < nq; ++i) {
          const double* qi = &Q[size_t(i) * s];
          double h = 0.0;
          for (int64_t t = b; t < e; ++t) h += qi[t] * w[t];
          part[size_t(c) * nq + i] = h;
        }
      }
    });
    std::vector<double> h(nq, 0.0);
    for (int64_t c = 0; c < nchunk; ++c)
      for (int64_t i = 0; i < nq; ++i) h[i] += part[size_t(c) * nq + i];
    parallel_for(nchunk, [&](int64_t cb, int64_t ce) {
      for (int64_t c = cb; c < ce; ++c) {
        int64_t b = s * c / nchunk, e = s * (c + 1) / nchunk;
        for (int64_t i = 0; i < nq; ++i) {
          const double* qi = &Q[size_t(i) * s];
          double hi = h[i];
          for (int64_t t = b; t < e; ++t) w[t] -= hi * qi[t];
        }
      }
    });
  }
}

double norm2(const double* v, int64_t n) {
  double a = 0.0;
  for (int64_t i = 0; i < n; ++i) a += v[i] * v[i];
  return std::sqrt(a);
}

}  // namespace

// Top-r eigenpairs of the symmetric s x s matrix G: theta[r] in descending
// order, Y (s x r row-major) orthonormal eigenvectors.
bool lanczos_top(const double* G, int64_t s, int r, double* theta, double* Y, int* steps_out) {
  if (r <= 0) return true;
  const int64_t mmax = std::min<int64_t>(s, std::max<int64_t>(int64_t(r) + 64, int64_t(12) * r + 200));
  std::vector<double> Q;          // Lanczos vectors, row per vector
  Q.reserve(size_t(mmax + 1) * s);
  std::vector<double> alpha, beta;
  std::vector<double> w(s), qv(s);
  Rng rng(0x5EEDull + uint64_t(s) * 7919u);
  for (int64_t i = 0; i < s; ++i) qv[i] = rng.next();
  double nq = norm2(qv.data(), s);
  for (int64_t i = 0; i < s; ++i) qv[i] /= nq;
  Q.insert(Q.end(), qv.begin(), qv.end());
  double gnorm = 0.0;   // running estimate of ||G|| for the breakdown test
  std::vector<double> Z, dd, ee, th;
  int64_t m = 0, next_check = 0;
  bool done = false;
  while (!done) {
    const double* qj = &Q[size_t(m) * s];
    parallel_for(s, [&](int64_t b, int64_t e) {
      for (int64_t i = b; i < e; ++i) {
        const double* g = G + i * s;
        double a = 0.0;
        for (int64_t t = 0; t < s; ++t) a += g[t] * qj[t];
        w[i] = a;
      }
    });
    double a = 0.0;
    for (int64_t i = 0; i < s; ++i) a += qj[i] * w[i];
    alpha.push_back(a);
    for (int64_t i = 0; i < s; ++i) w[i] -= a * qj[i];
    if (m > 0) {
      const double* qp = &Q[size_t(m - 1) * s];
      double bprev = beta[m - 1];
      for (int64_t i = 0; i < s; ++i) w[i] -= bprev * qp[i];
    }
    reorth(Q, m + 1, s, w.data());
    double b = norm2(w.data(), s);
    gnorm = std::max(gnorm, std::fabs(a) + b + (m > 0 ? beta[m - 1] : 0.0));
    ++m;
    bool last = (m >= mmax);
    if (!last) {
      if (b <= 1e-13 * gnorm || b == 0.0) {
        // invariant subspace: continue from a fresh direction orthogonal to Q
        b = 0.0;
        for (int attempt = 0; attempt < 4; ++attempt) {
          for (int64_t i = 0; i < s; ++i) w[i] = rng.next();
          reorth(Q, m, s, w.data());
          double nw = norm2(w.data(), s);
          if (nw > 1e-6) { for (int64_t i = 0; i < s; ++i) w[i] /= nw; break; }
        }
        beta.push_back(0.0);
      } else {
        for (int64_t i = 0; i < s; ++i) w[i] /= b;
        beta.push_back(b);
      }
      Q.insert(Q.end(), w.begin(), w.end());
    } else {
      beta.push_back(b);
    }
    bool check = last || (m >= r + 8 && m >= next_check);
    if (!check) continue;
    next_check = m + std::max<int64_t>(10, m / 8);
    dd.assign(alpha.begin(), alpha.begin() + m);
    ee.assign(beta.begin(), beta.begin() + (m - 1));
    ee.push_back(0.0);
    Z.assign(size_t(m), 0.0);
    if (!tridiag_eig(int(m), dd.data(), ee.data(), Z.data(), 1, int(m - 1))) return false;
    // order Ritz values descending
    std::vector<int> idx(m);
    for (int i = 0; i < m; ++i) idx[i] = i;
    std::sort(idx.begin(), idx.end(), [&](int x, int y) { return dd[x] > dd[y]; });
    double bm = beta[m - 1];
    double top = std::max(std::fabs(dd[idx[0]]), 1e-300);
    bool conv = true;
    for (int i = 0; i < r && i < m; ++i) {
      double res = std::fabs(bm * Z[idx[i]]);
      if (res > 1e-10 * top) { conv = false; break; }
    }
    if (m < r) conv = false;
    if (conv || last) {
      // all eigenvectors of the final tridiagonal matrix
      dd.assign(alpha.begin(), alpha.begin() + m);
      ee.assign(beta.begin(), beta.begin() + (m - 1));
      ee.push_back(0.0);
      Z.assign(size_t(m) * m, 0.0);
      if (!tridiag_eig(int(m), dd.data(), ee.data(), Z.data(), int(m), 0)) return false;
      for (int i = 0; i < m; ++i) idx[i] = i;
      std::sort(idx.begin(), idx.end(), [&](int x, int y) { return dd[x] > dd[y]; });
      int rr = int(std::min<int64_t>(r, m));
      for (int i = 0; i < r; ++i) theta[i] = i < rr ? dd[idx[i]] : 0.0;
      std::fill(Y, Y + size_t(s) * r, 0.0);
      parallel_for(s, [&](int64_t b0, int64_t e0) {
        for (int64_t t = b0; t < e0; ++t)
          for (int i = 0; i < rr; ++i) {
            double acc = 0.0;
            for (int64_t k = 0; k < m; ++k) acc += Q[size_t(k) * s + t] * Z[size_t(k) * m + idx[i]];
            Y[size_t(t) * r + i] = acc;
          }
      });
      if (steps_out) *steps_out = int(m);
      if (std::getenv("SVDQ_DEBUG_SVD")) std::fprintf(stderr, "svdq: lanczos s=%lld r=%d steps=%lld\n", (long long)s, r, (long long)m);
      done = true;
    }
  }
  return true;
}

bool truncated_svd(const double* A, int64_t K, int64_t N, int r, double* L1, double* L2, double* sigma) {
  if (r <= 0) return true;
  const bool rows = (K <= N);      // Gram of the K rows, else of the N columns
  const int64_t s = rows ? K : N, L = rows ? N : K;
  std::vector<double> Bt;
  const double* B = A;
  if (!rows) {
    Bt.resize(size_t(N) * K);
    parallel_for(N, [&](int64_t b, int64_t e) {
      for (int64_t n = b; n < e; ++n)
        for (int64_t k = 0; k < K; ++k) Bt[size_t(n) * K + k] = A[size_t(k) * N + n];
    });
    B = Bt.data();
  }
  const bool dbg = std::getenv("SVDQ_DEBUG_SVD") != nullptr;
  auto t0 = std::chrono::steady_clock::now();
  auto lap = [&](const char* what) {
    if (!dbg) return;
    auto t1 = std::chrono::steady_clock::now();
    std::fprintf(stderr, "svdq: %s %.3f s\n", what, std::chrono::duration<double>(t1 - t0).count());
    t0 = t1;
  };
  std::vector<double> G(size_t(s) * s);
  gram(B, s, L, G.data());
  lap("gram");
  std::vector<double> theta(r), Y(size_t(s) * r);
  if (!lanczos_top(G.data(), s, r, theta.data(), Y.data(), nullptr)) return false;
  lap("lanczos");
  G.clear(); G.shrink_to_fit();
  // Directions with sigma_i <= 1e-6 sigma_1 are numerical noise of the Gram
  // matrix (its eigenvalues carry an absolute error of about eps * sigma_1^2);
  // they are dropped from the branch and stay in the residual.
  const double cut = std::max(theta[0], 0.0) * 1e-12;
  std::vector<double> sg(r), inv(r);
  for (int i = 0; i < r; ++i) {
    double t = theta[i];
    bool keep = (t > cut) && (t > 0.0);
    sg[i] = keep ? std::sqrt(t) : 0.0;
    inv[i] = keep ? 1.0 / sg[i] : 0.0;
    if (sigma) sigma[i] = sg[i];
  }
  if (rows) {
    // U = Y; L1 = U S; L2 = (Y^T A) / S
    for (int64_t k = 0; k < K; ++k)
      for (int i = 0; i < r; ++i) L1[size_t(k) * r + i] = Y[size_t(k) * r + i] * sg[i];
    parallel_for(N, [&](int64_t b, int64_t e) {
      std::vector<double> acc(size_t(r) * (e - b), 0.0);
      for (int64_t k = 0; k < K; ++k) {
        const double* a = A + size_t(k) * N;
        for (int i = 0; i < r; ++i) {
          double y = Y[size_t(k) * r + i];
          if (y == 0.0) continue;
          double* ac = &acc[size_t(i) * (e - b)];
          for (int64_t n = b; n < e; ++n) ac[n - b] += y * a[n];
        }
      }
      for (int i = 0; i < r; ++i)
        for (int64_t n = b; n < e; ++n) L2[size_t(i) * N + n] = acc[size_t(i) * (e - b) + n - b] * inv[i];
    });
  } else {
    // V = Y; L2 = V^T; L1 = A V (= U S)
    for (int i = 0; i < r; ++i)
      for (int64_t n = 0; n < N; ++n) L2[size_t(i) * N + n] = sg[i] > 0.0 ? Y[size_t(n) * r + i] : 0.0;
    parallel_for(K, [&](int64_t b, int64_t e) {
      for (int64_t k = b; k < e; ++k) {
        const double* a = A + size_t(k) * N;
        for (int i = 0; i < r; ++i) {
          double acc = 0.0;
          if (sg[i] > 0.0)
            for (int64_t n = 0; n < N; ++n) acc += a[n] * Y[size_t(n) * r + i];
          L1[size_t(k) * r + i] = acc;
        }
      }
    });
  }
  lap("factors");
  return true;
}

}  // namespace svdq
