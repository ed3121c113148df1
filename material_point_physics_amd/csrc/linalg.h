// linalg.h -- 3x3 linear algebra: determinant, Jacobi eigenvector, polar rotation
// Part of mpm.hip: included there, inside its anonymous namespace, after the
// parts before it; not a standalone header.

// ------------------------------------------------------- 3x3 linear algebra

__device__ __forceinline__ float det3(const float A[9]) {
  return A[0] * (A[4] * A[8] - A[5] * A[7]) - A[1] * (A[3] * A[8] - A[5] * A[6]) +
         A[2] * (A[3] * A[7] - A[4] * A[6]);
}

// For X = I + Y: the cofactor matrix of X minus I (K, row-major, so that
// X^{-T} = (I + K) / det X) and det X - 1 (returned), formed without adding
// and then subtracting I: both keep the relative precision of a small Y (the
// deformation of an element that has barely strained).
__device__ __forceinline__ float cofactor_minus_identity(const float Y[9], float K[9]) {
  const float o0 = 1.f + Y[0], o1 = 1.f + Y[4], o2 = 1.f + Y[8];
  K[0] = Y[4] + Y[8] + (Y[4] * Y[8] - Y[5] * Y[7]);
  K[1] = Y[5] * Y[6] - Y[3] * o2;
  K[2] = Y[3] * Y[7] - o1 * Y[6];
  K[3] = Y[2] * Y[7] - Y[1] * o2;
  K[4] = Y[0] + Y[8] + (Y[0] * Y[8] - Y[2] * Y[6]);
  K[5] = Y[1] * Y[6] - o0 * Y[7];
  K[6] = Y[1] * Y[5] - Y[2] * o1;
  K[7] = Y[2] * Y[3] - o0 * Y[5];
  K[8] = Y[0] + Y[4] + (Y[0] * Y[4] - Y[1] * Y[3]);
  // first-row expansion: (1 + Y00)(1 + K00) + Y01 K01 + Y02 K02 - 1
  return Y[0] + K[0] + Y[0] * K[0] + Y[1] * K[1] + Y[2] * K[2];
}

// Eigenvector of the smallest eigenvalue of a symmetric 3x3 matrix by cyclic
// Jacobi rotations (Rutishauser's formulation of the symmetric Jacobi method,
// as in Golub & Van Loan, "Matrix Computations"): accurate to about eps/gap
// even when two eigenvalues nearly coincide.  Only used for reflected F.
__device__ void smallest_eigvec_sym3(const float Hin[9], float v[3]) {
  float a[3][3], W[3][3];
#pragma unroll
  for (int r = 0; r < 3; ++r)
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      a[r][c] = Hin[r * 3 + c];
      W[r][c] = (r == c) ? 1.f : 0.f;
    }
  for (int sweep = 0; sweep < 10; ++sweep) {
    const float off = a[0][1] * a[0][1] + a[0][2] * a[0][2] + a[1][2] * a[1][2];
    const float dia = a[0][0] * a[0][0] + a[1][1] * a[1][1] + a[2][2] * a[2][2];
    if (off <= 1e-14f * dia) break;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int p = k == 2 ? 1 : 0, q = k == 0 ? 1 : 2;
      const float apq = a[p][q];
      if (apq == 0.f) continue;
      const float theta = (a[q][q] - a[p][p]) / (2.f * apq);
      const float t = copysignf(1.f, theta) / (fabsf(theta) + sqrtf(theta * theta + 1.f));
      const float c = rsqrtf(t * t + 1.f), sn = t * c;
#pragma unroll
      for (int r = 0; r < 3; ++r) {  // columns p, q
        const float xp = a[r][p], xq = a[r][q];
        a[r][p] = c * xp - sn * xq;
        a[r][q] = sn * xp + c * xq;
      }
#pragma unroll
      for (int r = 0; r < 3; ++r) {  // rows p, q
        const float xp = a[p][r], xq = a[q][r];
        a[p][r] = c * xp - sn * xq;
        a[q][r] = sn * xp + c * xq;
      }
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        const float xp = W[r][p], xq = W[r][q];
        W[r][p] = c * xp - sn * xq;
        W[r][q] = sn * xp + c * xq;
      }
    }
  }
  // column of the smallest diagonal entry (selects, no dynamic indexing)
  const bool c1 = a[1][1] < a[0][0];
  const float d01 = c1 ? a[1][1] : a[0][0];
  const bool c2 = a[2][2] < d01;
#pragma unroll
  for (int r = 0; r < 3; ++r) v[r] = c2 ? W[r][2] : (c1 ? W[r][1] : W[r][0]);
}

// Rotation R in SO(3) closest to F (the fixed-corotated model's rotation).
// Higham's scaled Newton iteration for the polar decomposition (Higham 1986,
// "Computing the polar decomposition -- with applications"):
//   X <- (zeta X + X^{-T} / zeta) / 2,  zeta = |det X|^{-1/3},
// which converges quadratically to the orthogonal polar factor Q.  When
// det F < 0, Q is a reflection; the SO(3) rotation with the sign on the
// smallest singular value is Q (I - 2 v v^T), v the right singular vector of
// the smallest singular value (smallest eigenvector of H = Q^T F).
// Returns status bits (inverted / no convergence).
__device__ uint32_t rotation_of(const float F[9], float R[9]) {
  float X[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) X[k] = F[k];
  uint32_t st = 0;
  float detF = det3(F);
  if (!(fabsf(detF) > 1e-20f) || !isfinite(detF)) {
#pragma unroll
    for (int k = 0; k < 9; ++k) R[k] = (k % 4 == 0) ? 1.f : 0.f;
    return MPM_STATUS_INVERTED;
  }
  bool done = false;
  for (int it = 0; it < 24 && !done; ++it) {
    const float c00 = X[4] * X[8] - X[5] * X[7], c01 = X[5] * X[6] - X[3] * X[8], c02 = X[3] * X[7] - X[4] * X[6];
    const float c10 = X[2] * X[7] - X[1] * X[8], c11 = X[0] * X[8] - X[2] * X[6], c12 = X[1] * X[6] - X[0] * X[7];
    const float c20 = X[1] * X[5] - X[2] * X[4], c21 = X[2] * X[3] - X[0] * X[5], c22 = X[0] * X[4] - X[1] * X[3];
    const float det = X[0] * c00 + X[1] * c01 + X[2] * c02;
    const float ad = fabsf(det);
    // Determinant scaling speeds up the first iterations of a strongly
    // stretched F; near a rotation it is ~1 and is skipped.
    float zeta = 1.f;
    if (fabsf(ad - 1.f) > 0.05f) zeta = exp2f(-0.333333333f * log2f(ad));
    // the iteration is self-correcting, so the hardware reciprocal suffices
    const float a = 0.5f * zeta, b = 0.5f * __builtin_amdgcn_rcpf(zeta * det);
    const float Y[9] = {a * X[0] + b * c00, a * X[1] + b * c01, a * X[2] + b * c02,
                        a * X[3] + b * c10, a * X[4] + b * c11, a * X[5] + b * c12,
                        a * X[6] + b * c20, a * X[7] + b * c21, a * X[8] + b * c22};
    float diff = 0.f;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      const float d = Y[k] - X[k];
      diff += d * d;
      X[k] = Y[k];
    }
    done = diff < 1e-11f;
  }
  if (!done) st |= MPM_STATUS_NO_CONVERGE;
  if (detF < 0.f) {
    st |= MPM_STATUS_INVERTED;
    float H[9];  // Q^T F
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
      for (int c = 0; c < 3; ++c) H[r * 3 + c] = X[0 * 3 + r] * F[0 * 3 + c] + X[1 * 3 + r] * F[1 * 3 + c] + X[2 * 3 + r] * F[2 * 3 + c];
    float Hs[9];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
      for (int c = 0; c < 3; ++c) Hs[r * 3 + c] = 0.5f * (H[r * 3 + c] + H[c * 3 + r]);
    float v[3];
    smallest_eigvec_sym3(Hs, v);
    const float qv[3] = {X[0] * v[0] + X[1] * v[1] + X[2] * v[2], X[3] * v[0] + X[4] * v[1] + X[5] * v[2],
                         X[6] * v[0] + X[7] * v[1] + X[8] * v[2]};
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
      for (int c = 0; c < 3; ++c) X[r * 3 + c] -= 2.0f * qv[r] * v[c];
  }
#pragma unroll
  for (int k = 0; k < 9; ++k) R[k] = X[k];
  return st;
}

// The same rotation for F = I + H, returned as Q = R - I with the scaled
// Newton iteration written for Y = X - I: with the cofactor form above,
// X' = a X + b (I + K) becomes Y' = a Y + b K + (a + b - 1) I, a = zeta / 2,
// b = 1 / (2 zeta det X); near a rotation (zeta = 1) a + b - 1 =
// -d / (2 (1 + d)) with d = det X - 1.  No term subtracts I from a value
// near I, so F - R = H - Q keeps the relative precision of a small H.  *dF
// receives det F - 1.  A reflected F (det F < 0) takes the full-matrix path.
__device__ uint32_t rotation_minus_identity(const float H[9], float Q[9], float *dF) {
  float K[9];
  const float d0 = cofactor_minus_identity(H, K);
  *dF = d0;
  const float detF = 1.f + d0;
  if (!(fabsf(detF) > 1e-20f) || !isfinite(detF)) {
#pragma unroll
    for (int k = 0; k < 9; ++k) Q[k] = 0.f;
    return MPM_STATUS_INVERTED;
  }
  if (detF < 0.f) {
    float F[9], R[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) F[k] = H[k] + ((k % 4 == 0) ? 1.f : 0.f);
    const uint32_t st = rotation_of(F, R);
#pragma unroll
    for (int k = 0; k < 9; ++k) Q[k] = R[k] - ((k % 4 == 0) ? 1.f : 0.f);
    return st;
  }
  float Y[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) Y[k] = H[k];
  bool done = false;
  float d = d0;
  for (int it = 0; it < 24 && !done; ++it) {
    if (it > 0) d = cofactor_minus_identity(Y, K);
    float a = 0.5f, b, c;
    if (fabsf(d) > 0.05f) {
      // determinant scaling for a strongly stretched F
      const float zeta = exp2f(-0.333333333f * log2f(1.f + d));
      a = 0.5f * zeta;
      b = 0.5f * __builtin_amdgcn_rcpf(zeta * (1.f + d));
      c = a + b - 1.f;
    } else {
      // (the iteration corrects the hardware reciprocal's error in b, and c
      // carries it only relative to d)
      const float r = __builtin_amdgcn_rcpf(1.f + d);
      b = 0.5f * r;
      c = -0.5f * d * r;
    }
    float diff = 0.f;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      const float yn = a * Y[k] + b * K[k] + ((k % 4 == 0) ? c : 0.f);
      const float e = yn - Y[k];
      diff += e * e;
      Y[k] = yn;
    }
    done = diff < 1e-11f;
  }
#pragma unroll
  for (int k = 0; k < 9; ++k) Q[k] = Y[k];
  return done ? 0u : (uint32_t)MPM_STATUS_NO_CONVERGE;
}
