// Symmetric eigensolver in fp64 for the per-layer latent rotation.
//
// The rotation is the eigenbasis of the latent covariance with eigenvectors
// ordered by ascending eigenvalue [OSCAR issue #10, maintainer reply, part
// "How the rotation adapts to the latent"].  The matrix is small (r x r,
// r = kv_lora_rank <= a few thousand) and computed once per layer offline, so
// a sequential host solver is the right tool: Householder reduction to
// tridiagonal form followed by implicit symmetric QR steps with a Wilkinson
// shift (Golub & Van Loan, Matrix Computations, 4th ed., sections 8.3.1 and
// 8.3.3), accumulating the orthogonal factors into the eigenvectors.
#include "eigh.hpp"

#include <algorithm>
#include <cmath>
#include <numeric>
#include <vector>

namespace mla {
namespace {

// A <- H A H with H = I - beta v v^T acting on indices k+1..n-1, for every k.
// On return d/e hold the tridiagonal matrix and Q the accumulated reflectors
// (A_in = Q T Q^T).
void tridiagonalize(int n, std::vector<double> &a, std::vector<double> &q,
                    std::vector<double> &d, std::vector<double> &e) {
  q.assign(static_cast<size_t>(n) * n, 0.0);
  for (int i = 0; i < n; ++i) q[static_cast<size_t>(i) * n + i] = 1.0;
  std::vector<double> v(n), p(n), w(n), qv(n);
  auto A = [&](int i, int j) -> double & {
    return a[static_cast<size_t>(i) * n + j];
  };
  for (int k = 0; k + 2 < n; ++k) {
    const int m0 = k + 1;
    double norm2 = 0.0;
    for (int i = m0; i < n; ++i) norm2 += A(i, k) * A(i, k);
    const double norm = std::sqrt(norm2);
    if (norm == 0.0) continue;
    const double x0 = A(m0, k);
    const double alpha = (x0 > 0.0) ? -norm : norm;  // avoid cancellation
    for (int i = m0; i < n; ++i) v[i] = A(i, k);
    v[m0] -= alpha;
    double vtv = 0.0;
    for (int i = m0; i < n; ++i) vtv += v[i] * v[i];
    if (vtv == 0.0) continue;
    const double beta = 2.0 / vtv;
    // p = beta * A_sub v
    for (int i = m0; i < n; ++i) {
      double s = 0.0;
      for (int j = m0; j < n; ++j) s += A(i, j) * v[j];
      p[i] = beta * s;
    }
    double ptv = 0.0;
    for (int i = m0; i < n; ++i) ptv += p[i] * v[i];
    const double kk = 0.5 * beta * ptv;
    for (int i = m0; i < n; ++i) w[i] = p[i] - kk * v[i];
    // A_sub -= v w^T + w v^T
    for (int i = m0; i < n; ++i)
      for (int j = m0; j < n; ++j) A(i, j) -= v[i] * w[j] + w[i] * v[j];
    // column/row k: H maps x to alpha e1
    A(m0, k) = alpha;
    A(k, m0) = alpha;
    for (int i = m0 + 1; i < n; ++i) {
      A(i, k) = 0.0;
      A(k, i) = 0.0;
    }
    // Q <- Q H
    for (int i = 0; i < n; ++i) {
      double s = 0.0;
      for (int j = m0; j < n; ++j) s += q[static_cast<size_t>(i) * n + j] * v[j];
      qv[i] = beta * s;
    }
    for (int i = 0; i < n; ++i)
      for (int j = m0; j < n; ++j) q[static_cast<size_t>(i) * n + j] -= qv[i] * v[j];
  }
  d.resize(n);
  e.assign(n > 1 ? n - 1 : 0, 0.0);
  for (int i = 0; i < n; ++i) d[i] = A(i, i);
  for (int i = 0; i + 1 < n; ++i) e[i] = A(i + 1, i);
}

// Implicit symmetric QR with Wilkinson shift on the tridiagonal (d, e);
// rotations are accumulated into the columns of V.  Returns false if an
// unreduced block fails to converge within the iteration budget.
bool tridiagonal_qr(int n, std::vector<double> &d, std::vector<double> &e,
                    std::vector<double> &V) {
  const double eps = std::numeric_limits<double>::epsilon();
  long budget = 60L * n + 100;
  int qe = n - 1;
  while (qe > 0) {
    if (std::fabs(e[qe - 1]) <= eps * (std::fabs(d[qe - 1]) + std::fabs(d[qe]))) {
      e[qe - 1] = 0.0;
      --qe;
      continue;
    }
    int p = qe - 1;
    while (p > 0 &&
           std::fabs(e[p - 1]) > eps * (std::fabs(d[p - 1]) + std::fabs(d[p])))
      --p;
    if (--budget < 0) return false;
    // Wilkinson shift from the trailing 2x2 block of [p, qe]
    const double a = d[qe - 1], b = e[qe - 1], c = d[qe];
    const double delta = 0.5 * (a - c);
    const double sgn = (delta >= 0.0) ? 1.0 : -1.0;
    const double mu = c - (b * b) / (delta + sgn * std::hypot(delta, b));
    double x = d[p] - mu;
    double z = e[p];
    for (int k = p; k < qe; ++k) {
      // rotation G in plane (k, k+1) with G^T [x; z] = [r; 0]
      const double r = std::hypot(x, z);
      double cs = 1.0, sn = 0.0;
      if (r != 0.0) {
        cs = x / r;
        sn = -z / r;
      }
      if (k > p) e[k - 1] = r;
      const double dk = d[k], ek = e[k], dk1 = d[k + 1];
      d[k] = cs * cs * dk - 2.0 * cs * sn * ek + sn * sn * dk1;
      d[k + 1] = sn * sn * dk + 2.0 * cs * sn * ek + cs * cs * dk1;
      e[k] = cs * sn * (dk - dk1) + (cs * cs - sn * sn) * ek;
      if (k + 1 < qe) {
        x = e[k];
        z = -sn * e[k + 1];
        e[k + 1] = cs * e[k + 1];
      }
      for (int i = 0; i < n; ++i) {
        double &vk = V[static_cast<size_t>(i) * n + k];
        double &vk1 = V[static_cast<size_t>(i) * n + k + 1];
        const double t0 = vk, t1 = vk1;
        vk = cs * t0 - sn * t1;
        vk1 = sn * t0 + cs * t1;
      }
    }
  }
  return true;
}

}  // namespace

bool eigh_ascending(int n, const double *sym, double *eigvals, double *eigvecs) {
  if (n <= 0) return false;
  std::vector<double> a(sym, sym + static_cast<size_t>(n) * n);
  for (double x : a)
    if (!std::isfinite(x)) return false;
  // symmetrise (the covariance is symmetric up to rounding)
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < i; ++j) {
      const double m = 0.5 * (a[static_cast<size_t>(i) * n + j] +
                              a[static_cast<size_t>(j) * n + i]);
      a[static_cast<size_t>(i) * n + j] = m;
      a[static_cast<size_t>(j) * n + i] = m;
    }
  std::vector<double> q, d, e;
  tridiagonalize(n, a, q, d, e);
  if (!tridiagonal_qr(n, d, e, q)) return false;
  std::vector<int> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int x, int y) { return d[x] < d[y]; });
  for (int j = 0; j < n; ++j) {
    const int src = order[j];
    eigvals[j] = d[src];
    // sign rule: the entry of largest magnitude is positive (ties: lowest row)
    int imax = 0;
    double vmax = -1.0;
    for (int i = 0; i < n; ++i) {
      const double m = std::fabs(q[static_cast<size_t>(i) * n + src]);
      if (m > vmax) {
        vmax = m;
        imax = i;
      }
    }
    const double sgn = (q[static_cast<size_t>(imax) * n + src] < 0.0) ? -1.0 : 1.0;
    for (int i = 0; i < n; ++i)
      eigvecs[static_cast<size_t>(i) * n + j] = sgn * q[static_cast<size_t>(i) * n + src];
  }
  return true;
}

}  // namespace mla
