// materials.h -- per-particle material updates: deformation gradient, stress, sand and snow plasticity
// Part of mpm.hip: included there, inside its anonymous namespace, after the
// parts before it; not a standalone header.

// The deformation state is stored as its difference from the identity: the
// displacement gradient H = F - I (nine values), or j = J - 1 for the fluid.
// Near the rest state F - I is many times smaller than F, and stored this way
// it keeps full single precision, where F itself would round it away (an
// element strained by 1e-7 would carry about 30% error in F - I and in the
// stress formed from it).  Every formula below is the textbook one rewritten
// in H (or j) so that no step subtracts I from a value near I.

// Deferred deformation-gradient update with the C of the G2P before it:
// F <- (I + dt C) F, i.e. H <- H + dt C (I + H); for the fluid
// J <- J det(I + dt C), i.e. j <- j + dd + j dd with dd = det(I + dt C) - 1.
template <int MAT>
__device__ __forceinline__ void update_F(float *Hp, const float Cp[9], float dt) {
  if (MAT == MPM_J_FLUID) {
    float G[9], K[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) G[k] = dt * Cp[k];
    const float dd = cofactor_minus_identity(G, K);
    Hp[0] = Hp[0] + dd + Hp[0] * dd;
  } else {
    float Hn[9];
#pragma unroll
    for (int r2 = 0; r2 < 3; ++r2)
#pragma unroll
      for (int c2 = 0; c2 < 3; ++c2)
        Hn[r2 * 3 + c2] = Hp[r2 * 3 + c2] + dt * (Cp[r2 * 3 + c2] + Cp[r2 * 3 + 0] * Hp[0 * 3 + c2] +
                                                  Cp[r2 * 3 + 1] * Hp[1 * 3 + c2] + Cp[r2 * 3 + 2] * Hp[2 * 3 + c2]);
#pragma unroll
    for (int k = 0; k < 9; ++k) Hp[k] = Hn[k];
  }
}

// Kirchhoff stress of the fixed-corotated model, tau = 2 mu (F - R) F^T +
// lam (J - 1) J I with R the rotation closest to F (fluid: tau = K J (J - 1) I,
// K = E), and the APIC affine momentum matrix A = m C - dt V0 (4/dx^2) tau.
// In the displacement form: F - R = H - (R - I) and F^T = I + H^T.
// Returns status bits (inverted or unconverged F; fluid: J <= 0).
template <int MAT>
__device__ __forceinline__ uint32_t affine_momentum(const SimDev &s, const float *Hp, float E, const float Cp[9],
                                                    float A[9]) {
  const float mass = s.mass;
  if (MAT == MPM_J_FLUID) {
    const float j = Hp[0];
    const float tau_diag = E * (1.f + j) * j;
#pragma unroll
    for (int k = 0; k < 9; ++k) A[k] = mass * Cp[k] - s.stress_k * ((k % 4 == 0) ? tau_diag : 0.f);
    return (1.f + j > 0.f) ? 0u : (uint32_t)MPM_STATUS_INVERTED;
  }
  const float mu = E * s.mu_per_E, lam = E * s.lam_per_E;
  float Q[9], dJ;
  const uint32_t st = rotation_minus_identity(Hp, Q, &dJ);
  float D[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) D[k] = 2.f * mu * (Hp[k] - Q[k]);
  const float vl = lam * dJ * (1.f + dJ);
#pragma unroll
  for (int r2 = 0; r2 < 3; ++r2)
#pragma unroll
    for (int c2 = 0; c2 < 3; ++c2) {
      // (D F^T)_{rc} = D_rc + sum_k D_rk H_ck
      const float tau = D[r2 * 3 + c2] + D[r2 * 3 + 0] * Hp[c2 * 3 + 0] + D[r2 * 3 + 1] * Hp[c2 * 3 + 1] +
                        D[r2 * 3 + 2] * Hp[c2 * 3 + 2] + (r2 == c2 ? vl : 0.f);
      A[r2 * 3 + c2] = mass * Cp[r2 * 3 + c2] - s.stress_k * tau;
    }
  return st;
}

// ------------------------------------------------------------------ sand
// Drucker-Prager elastoplasticity in Hencky strain (Klar et al. 2016,
// "Drucker-Prager elastoplasticity for sand animation"), with a constant
// friction angle.  [RT-MPM] merges the SVD, the plasticity projection and
// the stress into the particle phase of P2G; so does the sand instance of
// P2G here, after the deferred F update.  Principal stretches are unsigned:
// F^T F = V diag(l) V^T, s = sqrt(l), Hencky strain e = ln(l) / 2, with l
// floored at 1e-6 (an element crushed below 1/1000 of its length).

// log(1 + x) and exp(x) - 1 for the principal strains, kept accurate for
// small x with the hardware logarithm and exponential: with u = 1 + x
// rounded, log(1 + x) = log(u) x / (u - 1) (Goldberg 1991, "What every
// computer scientist should know about floating-point arithmetic",
// Theorem 4); with u = exp(x) rounded, exp(x) - 1 = (u - 1) x / log(u)
// (Kahan's method, in the same paper).
__device__ __forceinline__ float log1p_strain(float x) {
  const float u = 1.f + x, d = u - 1.f;
  return d == 0.f ? x : logf(u) * (x * __builtin_amdgcn_rcpf(d));
}
__device__ __forceinline__ float expm1_strain(float x) {
  const float u = expf(x), d = u - 1.f;
  if (d == 0.f) return x;
  if (d == -1.f) return -1.f;
  return d * (x * __builtin_amdgcn_rcpf(logf(u)));
}

// Eigen-decomposition of a symmetric 3x3 matrix by cyclic Jacobi rotations
// (Rutishauser's formulation, Golub & Van Loan, "Matrix Computations"):
// A becomes diagonal, W's columns the eigenvectors.  Used on F^T F - I.
__device__ __forceinline__ void eigen_sym3(float a[3][3], float W[3][3]) {
#pragma unroll
  for (int r = 0; r < 3; ++r)
#pragma unroll
    for (int c = 0; c < 3; ++c) W[r][c] = (r == c) ? 1.f : 0.f;
  for (int sweep = 0; sweep < 10; ++sweep) {
    // (off-diagonal entries below 1e-6 of the diagonal's: the matrix here is
    // F^T F - I, whose entries are as small as the strain, and single
    // precision rounding floors the ratio near 1e-7)
    const float off = a[0][1] * a[0][1] + a[0][2] * a[0][2] + a[1][2] * a[1][2];
    const float dia = a[0][0] * a[0][0] + a[1][1] * a[1][1] + a[2][2] * a[2][2];
    if (off <= 1e-12f * dia) break;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int p = k == 2 ? 1 : 0, q = k == 0 ? 1 : 2;
      const float apq = a[p][q];
      // (an entry this small is zero for the strains here, and skipping it
      // keeps the reciprocal below finite)
      if (fabsf(apq) < 1e-30f) continue;
      // The angle needs no correct rounding: c and s = t c form an exact
      // rotation up to rounding for any t, and the sweeps converge from
      // whatever angle they take, so the hardware reciprocal and square
      // root serve.
      const float theta = (a[q][q] - a[p][p]) * __builtin_amdgcn_rcpf(2.f * apq);
      const float t = copysignf(1.f, theta) * __builtin_amdgcn_rcpf(fabsf(theta) + __builtin_amdgcn_sqrtf(theta * theta + 1.f));
      const float c = __builtin_amdgcn_rsqf(t * t + 1.f), sn = t * c;
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
}

// F V diag(m) V^T (F with its principal stretches scaled by m).
__device__ __forceinline__ void stretch_scaled(const float F[9], const float W[3][3], const float m[3], float out[9]) {
  float M[9];
#pragma unroll
  for (int r = 0; r < 3; ++r)
#pragma unroll
    for (int c = 0; c < 3; ++c)
      M[r * 3 + c] = W[r][0] * m[0] * W[c][0] + W[r][1] * m[1] * W[c][1] + W[r][2] * m[2] * W[c][2];
#pragma unroll
  for (int r = 0; r < 3; ++r)
#pragma unroll
    for (int c = 0; c < 3; ++c)
      out[r * 3 + c] = F[r * 3 + 0] * M[0 * 3 + c] + F[r * 3 + 1] * M[1 * 3 + c] + F[r * 3 + 2] * M[2 * 3 + c];
}

// ------------------------------------------------------------------ snow
// Non-associative Cam-clay (Wolper et al. 2019, "CD-MPM: continuum damage
// material point methods for dynamic fracture animation"; [RT-MPM] names it,
// with its parameters, for its snow scene) on the Hencky elasticity of the
// sand model.  With t = sum e and d = e - t/3 the Kirchhoff stress has
// pressure p = -kappa t and shear measure q = sqrt(3/2) |dev tau| =
// sqrt(6) mu |d|, so the return mapping onto the yield ellipse
// (1 + 2 beta) q^2 + M^2 (p + beta p0)(p - p0) <= 0 is closed-form: past p0
// the compression tip (t = -p0 / kappa, d = 0), below -beta p0 the tension
// tip (t = beta p0 / kappa), between them with y > 0 the deviator scaled so
// that q lands on the ellipse (t kept).  p0 = kappa sinh(xi max(-a, 0))
// hardens with the log plastic volume a = ln J_P, which takes the log-volume
// the projection removes from the elastic part (a += t - t_new); the
// exponent is capped at 40 so that p0 stays finite.

// Sand and snow, per particle: the plasticity projection of F (in place,
// when project; snow also updates its log plastic volume a) and the APIC
// affine momentum A = m C - dt V0 (4/dx^2) tau with the Hencky Kirchhoff
// stress tau = U diag(2 mu h + lam sum h) U^T of the projected principal
// strains h (U = F V diag(1/s) is unchanged by the projection, so tau is
// formed from the trial F and its l).  Sand's return mapping, with the
// deviator d = e - t/3: t > 0 -> tip (h = 0); else g = |d| + (1 + nu)/(1 -
// 2 nu) t alpha, g <= 0 -> unchanged, g > 0 -> h = e - g d / |d|.  Returns
// status bits (det F <= 0).
template <int MAT>
__device__ __forceinline__ uint32_t plastic_affine(const SimDev &s, float Hp[9], float E, float &a,
                                                   const float Cp[9], float A[9], bool project) {
  // F^T F - I = H + H^T + H^T H, diagonalised: F^T F = V diag(1 + sg) V^T
  float am[3][3], W[3][3];
#pragma unroll
  for (int r = 0; r < 3; ++r)
#pragma unroll
    for (int c = 0; c < 3; ++c)
      am[r][c] = Hp[r * 3 + c] + Hp[c * 3 + r] +
                 (Hp[0 * 3 + r] * Hp[0 * 3 + c] + Hp[1 * 3 + r] * Hp[1 * 3 + c] + Hp[2 * 3 + r] * Hp[2 * 3 + c]);
  eigen_sym3(am, W);
  float l[3], e[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const float sg = fmaxf(am[i][i], 1e-6f - 1.f);
    l[i] = 1.f + sg;
    e[i] = 0.5f * log1p_strain(sg);
  }
  float K[9];
  const uint32_t st = cofactor_minus_identity(Hp, K) > -1.f ? 0u : (uint32_t)MPM_STATUS_INVERTED;
  const float mu = E * s.mu_per_E, lam = E * s.lam_per_E;
  float h[3] = {e[0], e[1], e[2]};
  bool moved = false;
  if (project) {
    const float t = e[0] + e[1] + e[2];
    const float d[3] = {e[0] - t / 3.f, e[1] - t / 3.f, e[2] - t / 3.f};
    const float nd2 = d[0] * d[0] + d[1] * d[1] + d[2] * d[2];
    if (MAT == MPM_SAND) {
      const float nd = sqrtf(nd2);
      if (t > 0.f) {
        h[0] = h[1] = h[2] = 0.f;
        moved = true;
      } else {
        const float g = nd + s.dp_c * t * s.alpha;
        if (g > 0.f) {
          const float k = g / nd;
#pragma unroll
          for (int i = 0; i < 3; ++i) h[i] = e[i] - k * d[i];
          moved = true;
        }
      }
    } else {
      const float kappa = E * s.kappa_per_E;
      const float p = -kappa * t;
      const float p0 = kappa * sinhf(fminf(s.snow_xi * fmaxf(-a, 0.f), 40.f));
      float tn = t, k = 0.f;
      if (p > p0) {
        tn = -p0 / kappa;
        moved = true;
      } else if (p < -s.snow_beta * p0) {
        tn = s.snow_beta * p0 / kappa;
        moved = true;
      } else {
        // y > 0  <=>  (1 + 2 beta) q^2 > X = M^2 (p + beta p0)(p0 - p) >= 0
        const float q2 = 6.f * mu * mu * nd2;
        const float X = s.snow_m2 * (p + s.snow_beta * p0) * (p0 - p);
        if (s.snow_1p2b * q2 > X) {
          k = sqrtf(X / (s.snow_1p2b * q2));
          moved = true;
        }
      }
      if (moved) {
#pragma unroll
        for (int i = 0; i < 3; ++i) h[i] = tn / 3.f + k * d[i];
        a += t - tn;
      }
    }
  }
  // tau = F V diag((2 mu h + lam sum h) / l) V^T F^T, F the trial F (F = I + H
  // only multiplies here, so its rounding costs no relative precision)
  float Fp[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) Fp[k] = Hp[k] + ((k % 4 == 0) ? 1.f : 0.f);
  const float ht = h[0] + h[1] + h[2];
  float q[3], G[9];
#pragma unroll
  for (int i = 0; i < 3; ++i) q[i] = (2.f * mu * h[i] + lam * ht) / l[i];
  stretch_scaled(Fp, W, q, G);
#pragma unroll
  for (int r2 = 0; r2 < 3; ++r2)
#pragma unroll
    for (int c2 = 0; c2 < 3; ++c2) {
      const float tau = G[r2 * 3 + 0] * Fp[c2 * 3 + 0] + G[r2 * 3 + 1] * Fp[c2 * 3 + 1] + G[r2 * 3 + 2] * Fp[c2 * 3 + 2];
      A[r2 * 3 + c2] = s.mass * Cp[r2 * 3 + c2] - s.stress_k * tau;
    }
  if (moved) {
    // F becomes the projected one, its stretches scaled by m = exp(h - e):
    // F V diag(m) V^T = F (I + M1) with M1 = V diag(m - 1) V^T, so
    // H <- M1 + H + H M1 (m - 1 formed without cancellation near m = 1)
    float mm1[3], M1[9];
#pragma unroll
    for (int i = 0; i < 3; ++i) mm1[i] = expm1_strain(h[i] - e[i]);
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
      for (int c = 0; c < 3; ++c)
        M1[r * 3 + c] = W[r][0] * mm1[0] * W[c][0] + W[r][1] * mm1[1] * W[c][1] + W[r][2] * mm1[2] * W[c][2];
    float Hn[9];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
      for (int c = 0; c < 3; ++c)
        Hn[r * 3 + c] = M1[r * 3 + c] + Hp[r * 3 + c] +
                        (Hp[r * 3 + 0] * M1[0 * 3 + c] + Hp[r * 3 + 1] * M1[1 * 3 + c] + Hp[r * 3 + 2] * M1[2 * 3 + c]);
#pragma unroll
    for (int k = 0; k < 9; ++k) Hp[k] = Hn[k];
  }
  return st;
}
