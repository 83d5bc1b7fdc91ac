// Host fp64 symmetric eigensolver used by mla_calibrate_rotation.
#pragma once

namespace mla {
// sym: n x n row-major symmetric matrix.  On success eigvals[j] ascending and
// eigvecs[i*n + j] = component i of eigenvector j, each eigenvector signed so
// that its largest-magnitude entry is positive (ties: lowest row).  Returns
// false on non-finite input or if the QR iteration does not converge.
bool eigh_ascending(int n, const double *sym, double *eigvals, double *eigvecs);
}  // namespace mla
