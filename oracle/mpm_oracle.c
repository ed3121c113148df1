/*
 * mpm_oracle.c -- plain, serial CPU reference of one explicit MLS-MPM step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file exists to check the GPU library.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it.  It shares no code, header, table or helper with the HIP path.
 *
 * Source of the method.  The page "Principles towards Real-Time Simulation of
 * Material Point Method on Modern GPUs" (below: [RT-MPM]) describes the step's
 * phases but prints none of the equations.  The step here is the textbook
 * MLS-MPM with quadratic B-splines and APIC transfer (Hu et al. 2018, "A
 * moving least squares material point method with displacement discontinuity
 * and two-way rigid body coupling"; Jiang et al. 2015, "The affine
 * particle-in-cell method"), with the fixed-corotated elastic model
 * (Stomakhin et al. 2012), and for sand the Drucker-Prager plasticity of
 * Klar et al. 2016 ("Drucker-Prager elastoplasticity for sand animation":
 * Hencky-strain elasticity and its return mapping, here with a constant
 * friction angle), and for snow the non-associative Cam-clay (NACC) model
 * of Wolper et al. 2019 ("CD-MPM: continuum damage material point methods
 * for dynamic fracture animation"), which [RT-MPM] names for its snow scene
 * together with its parameters (bulk modulus, Poisson ratio, friction M,
 * cohesion beta, hardening xi), here on the same Hencky elasticity as sand.
 * Each step below names the passage of [RT-MPM] it matches:
 *   - P2G adds weighted mass and momenta to grid nodes            [RT-MPM §4.3]
 *   - three quadratic B-spline weights per axis ("nine floats")   [RT-MPM, on-chip
 *                                                                  memory principle, §6.2.5]
 *   - the particle stress is a temporary evaluated with P2G        [RT-MPM, kernel
 *                                                                  merging discussion]
 *   - grid update: nodal velocities, then collisions                [RT-MPM §6.3.2 paragraph]
 *   - G2P gathers velocities and updates the deformation gradient  [RT-MPM, kernel
 *                                                                  merging discussion]
 * Readings where the page is silent (grid convention, walls, clamp, fluid
 * equation of state) are listed in the design notes of the repository.
 *
 * Precision: compiled with ORC_REAL=double (the reference) and, separately,
 * ORC_REAL=float (to measure the envelope fp32 arithmetic can reach).  Never
 * compiled with -ffast-math.
 *
 * Layout: particle arrays are AoS, row-major: x[p*3+a], C[p*9+r*3+c].
 * Grid: n nodes per axis at x_i = i*dx, dx = 1/n, domain [0,1]^3.  Node
 * (i,j,k) has linear index i + n*(j + n*k); momentum and velocity are
 * interleaved, three values per node.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifndef ORC_REAL
#define ORC_REAL double
#endif
typedef ORC_REAL real;

typedef struct {
  int32_t n;          /* grid nodes per axis */
  int32_t wall;       /* sticky-wall thickness, in nodes */
  int32_t material;   /* 0 fixed-corotated elastic, 1 weakly compressible fluid, 2 sand, 3 snow */
  int32_t pad;
  double dt;
  double gravity[3];
  double E;           /* Young's modulus (bulk modulus K for the fluid) when E_p is NULL */
  double nu;          /* Poisson ratio */
  double rho;         /* density */
  double p_vol;       /* initial particle volume V0 */
  double friction_deg; /* sand: friction angle, degrees */
  double snow_M;      /* snow: slope M of the critical-state line (the page's friction coefficient) */
  double snow_beta;   /* snow: cohesion beta (tension tip at -beta p0) */
  double snow_xi;     /* snow: hardening xi */
} orc_params;

int orc_real_bytes(void) { return (int)sizeof(real); }

/* ---------------------------------------------------------------- splines */

/* Quadratic B-spline kernel N(d) on the unit grid (textbook definition). */
static real bspline2(real d) {
  d = d < 0 ? -d : d;
  if (d < (real)0.5) return (real)0.75 - d * d;
  if (d < (real)1.5) return (real)0.5 * ((real)1.5 - d) * ((real)1.5 - d);
  return (real)0;
}

/* Base node of a coordinate given in grid units: floor(xn - 1/2). */
int64_t orc_base(real xn) { return (int64_t)floor(xn - (real)0.5); }

/* Weights of the three nodes base+o (o = 0,1,2) for a particle at
 * fractional offset f = xn - base in [0.5, 1.5): w[o] = N(f - o). */
void orc_weights(real f, real w[3]) {
  for (int o = 0; o < 3; ++o) w[o] = bspline2(f - (real)o);
}

/* ----------------------------------------------------------- 3x3 algebra */

static void mat_mul(const real A[9], const real B[9], real out[9]) {
  real t[9];
  for (int r = 0; r < 3; ++r)
    for (int c = 0; c < 3; ++c) {
      real s = 0;
      for (int k = 0; k < 3; ++k) s += A[r * 3 + k] * B[k * 3 + c];
      t[r * 3 + c] = s;
    }
  memcpy(out, t, sizeof t);
}

static void mat_mul_bt(const real A[9], const real B[9], real out[9]) { /* A B^T */
  real t[9];
  for (int r = 0; r < 3; ++r)
    for (int c = 0; c < 3; ++c) {
      real s = 0;
      for (int k = 0; k < 3; ++k) s += A[r * 3 + k] * B[c * 3 + k];
      t[r * 3 + c] = s;
    }
  memcpy(out, t, sizeof t);
}

static real mat_det(const real A[9]) {
  return A[0] * (A[4] * A[8] - A[5] * A[7]) - A[1] * (A[3] * A[8] - A[5] * A[6]) +
         A[2] * (A[3] * A[7] - A[4] * A[6]);
}

static real dot3(const real a[3], const real b[3]) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2]; }

static void cross3(const real a[3], const real b[3], real out[3]) {
  out[0] = a[1] * b[2] - a[2] * b[1];
  out[1] = a[2] * b[0] - a[0] * b[2];
  out[2] = a[0] * b[1] - a[1] * b[0];
}

static int normalize3(real a[3]) {
  real l = sqrt(dot3(a, a));
  if (!(l > 0)) return 0;
  a[0] /= l; a[1] /= l; a[2] /= l;
  return 1;
}

/* ------------------------------------------------------------------- SVD */

/* Cyclic Jacobi eigen-decomposition of a symmetric 3x3 matrix (Golub & Van
 * Loan, "Matrix Computations", symmetric Schur decomposition and the cyclic
 * Jacobi method).  On return S is (numerically) diagonal and V holds the
 * eigenvectors as columns. */
static void jacobi_eigen_sym3(real S[9], real V[9]) {
  static const int P[3] = {0, 0, 1}, Q[3] = {1, 2, 2};
  for (int i = 0; i < 9; ++i) V[i] = (i % 4 == 0) ? (real)1 : (real)0;
  const real eps = sizeof(real) == 8 ? (real)1e-30 : (real)1e-14;
  for (int sweep = 0; sweep < 60; ++sweep) {
    real off = S[1] * S[1] + S[2] * S[2] + S[5] * S[5];
    real dia = S[0] * S[0] + S[4] * S[4] + S[8] * S[8];
    if (off <= eps * dia || off == 0) break;
    for (int k = 0; k < 3; ++k) {
      int p = P[k], q = Q[k];
      real apq = S[p * 3 + q];
      if (apq == 0) continue;
      real app = S[p * 3 + p], aqq = S[q * 3 + q];
      real theta = (aqq - app) / (2 * apq);
      real t = (theta >= 0 ? (real)1 : (real)-1) / (fabs(theta) + sqrt(theta * theta + 1));
      real c = 1 / sqrt(t * t + 1), s = t * c;
      /* S <- S J (columns p, q), then S <- J^T S (rows p, q); V <- V J. */
      for (int r = 0; r < 3; ++r) {
        real sp = S[r * 3 + p], sq = S[r * 3 + q];
        S[r * 3 + p] = c * sp - s * sq;
        S[r * 3 + q] = s * sp + c * sq;
      }
      for (int col = 0; col < 3; ++col) {
        real sp = S[p * 3 + col], sq = S[q * 3 + col];
        S[p * 3 + col] = c * sp - s * sq;
        S[q * 3 + col] = s * sp + c * sq;
      }
      for (int r = 0; r < 3; ++r) {
        real vp = V[r * 3 + p], vq = V[r * 3 + q];
        V[r * 3 + p] = c * vp - s * vq;
        V[r * 3 + q] = s * vp + c * vq;
      }
    }
  }
}

/* Signed SVD F = U diag(s) V^T with U, V proper rotations (det = +1).
 * V and s^2 come from the Jacobi eigen-decomposition of F^T F, sorted so that
 * s[0] >= s[1] >= |s[2]|; U's first two columns are F v_k normalised (the
 * second orthogonalised against the first), the third is their cross product,
 * and s_k = u_k . F v_k, so that when det F < 0 the sign lands on the
 * smallest singular value. */
void orc_svd3(const real F[9], real U[9], real s[3], real V[9]) {
  real S[9];
  for (int r = 0; r < 3; ++r)
    for (int c = 0; c < 3; ++c) {
      real a = 0;
      for (int k = 0; k < 3; ++k) a += F[k * 3 + r] * F[k * 3 + c];
      S[r * 3 + c] = a;
    }
  real W[9];
  jacobi_eigen_sym3(S, W);
  real ev[3] = {S[0], S[4], S[8]};
  int ord[3] = {0, 1, 2};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (ev[ord[j]] > ev[ord[i]]) { int t = ord[i]; ord[i] = ord[j]; ord[j] = t; }
  real v[3][3]; /* v[k] = k-th right singular vector */
  for (int k = 0; k < 3; ++k)
    for (int r = 0; r < 3; ++r) v[k][r] = W[r * 3 + ord[k]];
  real v3x[3];
  cross3(v[0], v[1], v3x);
  if (dot3(v3x, v[2]) < 0) { v[2][0] = -v[2][0]; v[2][1] = -v[2][1]; v[2][2] = -v[2][2]; }

  real Fv[3][3];
  for (int k = 0; k < 3; ++k)
    for (int r = 0; r < 3; ++r) Fv[k][r] = F[r * 3 + 0] * v[k][0] + F[r * 3 + 1] * v[k][1] + F[r * 3 + 2] * v[k][2];

  real u[3][3];
  for (int r = 0; r < 3; ++r) u[0][r] = Fv[0][r];
  if (!normalize3(u[0])) { u[0][0] = 1; u[0][1] = 0; u[0][2] = 0; }
  real proj = dot3(u[0], Fv[1]);
  for (int r = 0; r < 3; ++r) u[1][r] = Fv[1][r] - proj * u[0][r];
  real s0 = sqrt(ev[ord[0]] > 0 ? ev[ord[0]] : 0);
  real tol = (sizeof(real) == 8 ? (real)1e-12 : (real)1e-6) * (s0 > 0 ? s0 : 1);
  if (!(sqrt(dot3(u[1], u[1])) > tol) || !normalize3(u[1])) {
    /* any unit vector orthogonal to u0 */
    real e[3] = {0, 0, 0};
    int m = fabs(u[0][0]) < fabs(u[0][1]) ? (fabs(u[0][0]) < fabs(u[0][2]) ? 0 : 2)
                                          : (fabs(u[0][1]) < fabs(u[0][2]) ? 1 : 2);
    e[m] = 1;
    real d = dot3(e, u[0]);
    for (int r = 0; r < 3; ++r) u[1][r] = e[r] - d * u[0][r];
    normalize3(u[1]);
  }
  cross3(u[0], u[1], u[2]);
  for (int k = 0; k < 3; ++k) s[k] = dot3(u[k], Fv[k]);
  for (int r = 0; r < 3; ++r)
    for (int k = 0; k < 3; ++k) {
      U[r * 3 + k] = u[k][r];
      V[r * 3 + k] = v[k][r];
    }
}

/* Rotation closest to F: R = U V^T from the signed SVD. */
void orc_rotation(const real F[9], real R[9]) {
  real U[9], s[3], V[9];
  orc_svd3(F, U, s, V);
  mat_mul_bt(U, V, R);
}

/* Lame parameters from Young's modulus and Poisson ratio. */
void orc_lame(real E, real nu, real *mu, real *lam) {
  *mu = E / (2 * (1 + nu));
  *lam = E * nu / ((1 + nu) * (1 - 2 * nu));
}

/* Fixed-corotated Kirchhoff stress tau = P F^T with
 * P = 2 mu (F - R) + lam (J - 1) J F^{-T}, i.e.
 * tau = 2 mu (F - R) F^T + lam (J - 1) J I. */
void orc_kirchhoff_fc(const real F[9], real mu, real lam, real tau[9]) {
  real R[9], D[9];
  orc_rotation(F, R);
  for (int i = 0; i < 9; ++i) D[i] = F[i] - R[i];
  mat_mul_bt(D, F, tau);
  real J = mat_det(F);
  for (int i = 0; i < 9; ++i) tau[i] *= 2 * mu;
  for (int a = 0; a < 3; ++a) tau[a * 4] += lam * (J - 1) * J;
}

/* Weakly compressible fluid, linear equation of state p = K (1 - J):
 * tau = -p J I = K J (J - 1) I.  Returns the diagonal value. */
real orc_kirchhoff_fluid(real J, real K) { return K * J * (J - 1); }

/* ------------------------------------------------------------------ sand
 * Drucker-Prager elastoplasticity in Hencky strain (Klar et al. 2016), with
 * unsigned singular values: F^T F = V diag(l) V^T, s_i = sqrt(l_i), and the
 * principal Hencky strain e_i = ln s_i = ln(l_i) / 2.  A value l_i below
 * ORC_SAND_LFLOOR is taken as that floor (an element crushed to less than
 * 1/1000 of its length along a principal axis). */
#define ORC_SAND_LFLOOR 1e-6

/* Principal strains of F: V (eigenvectors of F^T F as columns), l (its
 * eigenvalues, floored) and e = ln(l) / 2. */
static void sand_principal(const real F[9], real V[9], real l[3], real e[3]) {
  real S[9];
  for (int r = 0; r < 3; ++r)
    for (int c = 0; c < 3; ++c) {
      real a = 0;
      for (int k = 0; k < 3; ++k) a += F[k * 3 + r] * F[k * 3 + c];
      S[r * 3 + c] = a;
    }
  jacobi_eigen_sym3(S, V);
  for (int i = 0; i < 3; ++i) {
    l[i] = S[i * 4] > (real)ORC_SAND_LFLOOR ? S[i * 4] : (real)ORC_SAND_LFLOOR;
    e[i] = (real)0.5 * log(l[i]);
  }
}

/* F V diag(m) V^T: F with its principal stretches s_i scaled by m_i. */
static void sand_scale(const real F[9], const real V[9], const real m[3], real out[9]) {
  real M[9];
  for (int r = 0; r < 3; ++r)
    for (int c = 0; c < 3; ++c) M[r * 3 + c] = V[r * 3 + 0] * m[0] * V[c * 3 + 0] + V[r * 3 + 1] * m[1] * V[c * 3 + 1] +
                                           V[r * 3 + 2] * m[2] * V[c * 3 + 2];
  real t[9];
  mat_mul(F, M, t);
  for (int i = 0; i < 9; ++i) out[i] = t[i];
}

/* Cone slope alpha = sqrt(2/3) 2 sin(phi) / (3 - sin(phi)) of the friction
 * angle phi (degrees). */
real orc_sand_alpha(real friction_deg) {
  const real sp = sin(friction_deg * (real)3.14159265358979323846 / 180);
  return sqrt((real)2 / 3) * 2 * sp / (3 - sp);
}

/* Return mapping of F (in place) onto the Drucker-Prager cone in principal
 * Hencky strain e:  with the trace t = sum e and the deviator d = e - t/3,
 *   t > 0   : expansion, projected to the cone's tip, e = 0 (F -> U V^T);
 *   else, with g = |d| + (3 lam + 2 mu) / (2 mu) t alpha
 *   g <= 0  : inside the cone, unchanged (this includes a purely volumetric
 *             compression, d = 0, which the published mapping sends to the
 *             tip with the expansions);
 *   g > 0   : e <- e - g d / |d| (onto the cone's surface; |d| > 0 here).
 * (3 lam + 2 mu) / (2 mu) = (1 + nu) / (1 - 2 nu) depends on nu only.
 * Returns 0 (unchanged), 1 (tip) or 2 (surface). */
int orc_sand_project(real F[9], real nu, real alpha) {
  real V[9], l[3], e[3];
  sand_principal(F, V, l, e);
  const real t = e[0] + e[1] + e[2];
  real d[3], nd2 = 0;
  for (int i = 0; i < 3; ++i) {
    d[i] = e[i] - t / 3;
    nd2 += d[i] * d[i];
  }
  const real nd = sqrt(nd2);
  real h[3];
  int kind;
  if (t > 0) {
    kind = 1;
    for (int i = 0; i < 3; ++i) h[i] = 0;
  } else {
    const real g = nd + (1 + nu) / (1 - 2 * nu) * t * alpha;
    if (g <= 0) return 0;
    kind = 2;
    for (int i = 0; i < 3; ++i) h[i] = e[i] - g * d[i] / nd;
  }
  real m[3];
  for (int i = 0; i < 3; ++i) m[i] = exp(h[i] - e[i]); /* new stretch / old stretch */
  sand_scale(F, V, m, F);
  return kind;
}

/* Kirchhoff stress of the Hencky (St. Venant-Kirchhoff in log strain)
 * energy psi = mu sum e_i^2 + lam/2 (sum e_i)^2:
 *   tau = U diag(2 mu e_i + lam sum e) U^T,  U = F V diag(1/s),
 * i.e. tau = F V diag((2 mu e_i + lam sum e) / l_i) V^T F^T. */
void orc_kirchhoff_sand(const real F[9], real mu, real lam, real tau[9]) {
  real V[9], l[3], e[3];
  sand_principal(F, V, l, e);
  const real t = e[0] + e[1] + e[2];
  real m[3];
  for (int i = 0; i < 3; ++i) m[i] = (2 * mu * e[i] + lam * t) / l[i];
  real G[9];
  sand_scale(F, V, m, G);
  mat_mul_bt(G, F, tau);
}

/* ------------------------------------------------------------------ snow
 * Non-associative Cam-clay (Wolper et al. 2019; [RT-MPM]'s snow scene) on
 * the Hencky elasticity above.  In principal Hencky strain e, with trace
 * t = sum e and deviator d = e - t/3, the Kirchhoff stress has
 *   pressure      p = -tr(tau)/3 = -kappa t          (kappa = lam + 2 mu / 3)
 *   shear measure q = sqrt(3/2) |dev tau| = sqrt(6) mu |d|.
 * Yield surface (an ellipse in the p-q plane between p = -beta p0 and p0):
 *   y(p, q) = (1 + 2 beta) q^2 + M^2 (p + beta p0) (p - p0) <= 0,
 * with the hardening p0 = kappa sinh(xi max(-a, 0)), where a = ln J_P is the
 * log of the plastic volume ratio carried by each particle.  The exponent is
 * capped at ORC_SNOW_XCAP so that p0 stays finite in single precision (a
 * state 10^17 times the bulk modulus, never reached in practice).
 * Return mapping of the trial strain (non-associative: q moves, p stays,
 * except at the tips):
 *   p > p0        : compression tip, e = (-p0 / kappa) / 3 per axis (d = 0);
 *   p < -beta p0  : tension tip, e = (beta p0 / kappa) / 3 per axis;
 *   y <= 0        : elastic, unchanged;
 *   y > 0         : d scaled so that q lands on the surface, t kept.
 * The total volume ratio J = J_E J_P is not changed by a projection, so the
 * log plastic volume takes what leaves the elastic one: a += t - t_new
 * (compaction lowers a and raises p0; expansion past the tension tip
 * softens). */
#define ORC_SNOW_XCAP 40

/* Hardening p0 = kappa sinh(xi max(-a, 0)), exponent capped. */
real orc_snow_p0(real a, real kappa, real xi) {
  real x = xi * (a < 0 ? -a : 0);
  if (x > (real)ORC_SNOW_XCAP) x = (real)ORC_SNOW_XCAP;
  return kappa * sinh(x);
}

/* The NACC return mapping of F (in place) and of the log plastic volume *a.
 * Returns 0 (elastic), 1 (compression tip), 2 (tension tip) or 3 (onto the
 * ellipse). */
int orc_snow_project(real F[9], real *a, real mu, real lam, real M, real beta, real xi) {
  real V[9], l[3], e[3];
  sand_principal(F, V, l, e);
  const real kappa = lam + 2 * mu / 3;
  const real t = e[0] + e[1] + e[2];
  real d[3], nd2 = 0;
  for (int i = 0; i < 3; ++i) {
    d[i] = e[i] - t / 3;
    nd2 += d[i] * d[i];
  }
  const real p = -kappa * t;
  const real p0 = orc_snow_p0(*a, kappa, xi);
  real t_new = t, k = 1;
  int kind;
  if (p > p0) {
    kind = 1;
    t_new = -p0 / kappa;
    k = 0;
  } else if (p < -beta * p0) {
    kind = 2;
    t_new = beta * p0 / kappa;
    k = 0;
  } else {
    const real q2 = 6 * mu * mu * nd2;
    const real y = (1 + 2 * beta) * q2 + M * M * (p + beta * p0) * (p - p0);
    if (y <= 0) return 0;
    kind = 3;
    /* q_new^2 = M^2 (p + beta p0) (p0 - p) / (1 + 2 beta); q2 > 0 here */
    k = sqrt(M * M * (p + beta * p0) * (p0 - p) / ((1 + 2 * beta) * q2));
  }
  real m[3];
  for (int i = 0; i < 3; ++i) m[i] = exp(t_new / 3 + k * d[i] - e[i]); /* new stretch / old stretch */
  sand_scale(F, V, m, F);
  *a += t - t_new;
  return kind;
}

/* ------------------------------------------------------------ MPM phases */

static int64_t node_index(int64_t n, int64_t i, int64_t j, int64_t k) { return i + n * (j + n * k); }

/* Locate a particle: base node b and the per-axis weights.  Returns 0 when
 * the 3x3x3 stencil leaves the grid. */
static int locate(const orc_params *P, const real x[3], int64_t b[3], real w[3][3]) {
  const int64_t n = P->n;
  for (int a = 0; a < 3; ++a) {
    real xn = x[a] * (real)n;
    if (!(xn == xn)) return 0;
    b[a] = orc_base(xn);
    if (b[a] < 0 || b[a] + 2 > n - 1) return 0;
    orc_weights(xn - (real)b[a], w[a]);
  }
  return 1;
}

void orc_grid_clear(const orc_params *P, real *gm, real *gp) {
  int64_t nn = (int64_t)P->n * P->n * P->n;
  memset(gm, 0, sizeof(real) * nn);
  memset(gp, 0, sizeof(real) * 3 * nn);
}

/* Particle-to-grid transfer, particles in index order.  Adds into gm (mass)
 * and gp (momentum).  For the elastic materials (fixed-corotated, sand, snow)
 * F holds the deformation gradients (snow, sand: their elastic parts); for the
 * fluid J holds the volume ratios, for snow the log plastic volumes a.
 * E_p may be NULL (and is NULL for snow, whose modulus is P->E).
 * Returns the number of particles skipped because their stencil left the
 * grid (0 for valid input). */
int64_t orc_p2g(const orc_params *P, int64_t N, const real *x, const real *v, const real *C,
                const real *F, const real *J, const real *E_p, real *gm, real *gp) {
  const real dx = (real)1 / (real)P->n;
  const real inv_dx2x4 = 4 * (real)P->n * (real)P->n; /* D^{-1} = 4/dx^2 for quadratic splines */
  const real dt = (real)P->dt, vol = (real)P->p_vol, mass = (real)P->rho * (real)P->p_vol;
  const int64_t n = P->n;
  int64_t skipped = 0;
  for (int64_t p = 0; p < N; ++p) {
    int64_t b[3];
    real w[3][3];
    if (!locate(P, x + 3 * p, b, w)) { ++skipped; continue; }
    real tau[9];
    real E = E_p ? E_p[p] : (real)P->E;
    if (P->material == 1) {
      real t = orc_kirchhoff_fluid(J[p], E);
      for (int i = 0; i < 9; ++i) tau[i] = (i % 4 == 0) ? t : 0;
    } else if (P->material == 2 || P->material == 3) { /* Hencky elasticity (sand, snow) */
      real mu, lam;
      orc_lame(E, (real)P->nu, &mu, &lam);
      orc_kirchhoff_sand(F + 9 * p, mu, lam, tau);
    } else {
      real mu, lam;
      orc_lame(E, (real)P->nu, &mu, &lam);
      orc_kirchhoff_fc(F + 9 * p, mu, lam, tau);
    }
    real A[9];
    for (int i = 0; i < 9; ++i) A[i] = mass * C[9 * p + i] - dt * vol * inv_dx2x4 * tau[i];
    for (int oz = 0; oz < 3; ++oz)
      for (int oy = 0; oy < 3; ++oy)
        for (int ox = 0; ox < 3; ++ox) {
          int64_t i = b[0] + ox, j = b[1] + oy, k = b[2] + oz;
          real wt = w[0][ox] * w[1][oy] * w[2][oz];
          real d[3] = {(real)i * dx - x[3 * p], (real)j * dx - x[3 * p + 1], (real)k * dx - x[3 * p + 2]};
          int64_t id = node_index(n, i, j, k);
          gm[id] += wt * mass;
          for (int a = 0; a < 3; ++a) {
            real ad = A[a * 3] * d[0] + A[a * 3 + 1] * d[1] + A[a * 3 + 2] * d[2];
            gp[3 * id + a] += wt * (mass * v[3 * p + a] + ad);
          }
        }
  }
  return skipped;
}

/* Grid update: v_i = p_i / m_i + dt g where m_i > 0, else 0; sticky walls set
 * all components to zero on nodes with any index < wall or >= n - wall. */
void orc_grid_update(const orc_params *P, const real *gm, const real *gp, real *gv) {
  const int64_t n = P->n, wall = P->wall;
  const real dt = (real)P->dt;
  for (int64_t k = 0; k < n; ++k)
    for (int64_t j = 0; j < n; ++j)
      for (int64_t i = 0; i < n; ++i) {
        int64_t id = node_index(n, i, j, k);
        int in_wall = i < wall || j < wall || k < wall || i >= n - wall || j >= n - wall || k >= n - wall;
        for (int a = 0; a < 3; ++a) {
          real va = 0;
          if (gm[id] > 0 && !in_wall) va = gp[3 * id + a] / gm[id] + dt * (real)P->gravity[a];
          gv[3 * id + a] = va;
        }
      }
}

/* Grid-to-particle transfer with the APIC affine matrix, deformation-gradient
 * (or volume-ratio) update (for sand and snow followed by the plasticity
 * projection; snow's also updates its log plastic volume in J),
 * advection and the position clamp to [2dx, (n-2)dx].  Returns the number of
 * clamped components. */
int64_t orc_g2p(const orc_params *P, int64_t N, real *x, real *v, real *C, real *F, real *J,
                const real *gv) {
  const real dx = (real)1 / (real)P->n;
  const real inv_dx2x4 = 4 * (real)P->n * (real)P->n;
  const real dt = (real)P->dt;
  const int64_t n = P->n;
  const real lo = 2 * dx, hi = (real)(n - 2) * dx;
  int64_t clamped = 0;
  for (int64_t p = 0; p < N; ++p) {
    int64_t b[3];
    real w[3][3];
    if (!locate(P, x + 3 * p, b, w)) continue;
    real vn[3] = {0, 0, 0}, B[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0};
    for (int oz = 0; oz < 3; ++oz)
      for (int oy = 0; oy < 3; ++oy)
        for (int ox = 0; ox < 3; ++ox) {
          int64_t i = b[0] + ox, j = b[1] + oy, k = b[2] + oz;
          real wt = w[0][ox] * w[1][oy] * w[2][oz];
          real d[3] = {(real)i * dx - x[3 * p], (real)j * dx - x[3 * p + 1], (real)k * dx - x[3 * p + 2]};
          const real *vi = gv + 3 * node_index(n, i, j, k);
          for (int a = 0; a < 3; ++a) {
            vn[a] += wt * vi[a];
            for (int c = 0; c < 3; ++c) B[a * 3 + c] += wt * vi[a] * d[c];
          }
        }
    real Cn[9], G[9];
    for (int i = 0; i < 9; ++i) Cn[i] = inv_dx2x4 * B[i];
    for (int i = 0; i < 9; ++i) G[i] = ((i % 4 == 0) ? (real)1 : (real)0) + dt * Cn[i];
    if (P->material == 1) {
      J[p] = J[p] * mat_det(G);
    } else {
      mat_mul(G, F + 9 * p, F + 9 * p);
      /* sand: the plasticity projection of the updated F ([RT-MPM] merges the
       * SVD, the plasticity projection and the stress into one particle phase) */
      if (P->material == 2) orc_sand_project(F + 9 * p, (real)P->nu, orc_sand_alpha((real)P->friction_deg));
      if (P->material == 3) {
        real mu, lam;
        orc_lame((real)P->E, (real)P->nu, &mu, &lam);
        orc_snow_project(F + 9 * p, J + p, mu, lam, (real)P->snow_M, (real)P->snow_beta, (real)P->snow_xi);
      }
    }
    for (int i = 0; i < 9; ++i) C[9 * p + i] = Cn[i];
    for (int a = 0; a < 3; ++a) {
      v[3 * p + a] = vn[a];
      real xa = x[3 * p + a] + dt * vn[a];
      if (xa < lo) { xa = lo; ++clamped; }
      if (xa > hi) { xa = hi; ++clamped; }
      x[3 * p + a] = xa;
    }
  }
  return clamped;
}

/* One full step: clear the grid, P2G, grid update, G2P.  The grid arrays
 * (gm: n^3, gp and gv: 3 n^3) are caller-owned and hold the step's grid
 * state on return.  Returns the clamp count, or -1 when a particle's
 * stencil left the grid. */
int64_t orc_step(const orc_params *P, int64_t N, real *x, real *v, real *C, real *F, real *J,
                 const real *E_p, real *gm, real *gp, real *gv) {
  orc_grid_clear(P, gm, gp);
  if (orc_p2g(P, N, x, v, C, F, J, E_p, gm, gp) != 0) return -1;
  orc_grid_update(P, gm, gp, gv);
  return orc_g2p(P, N, x, v, C, F, J, gv);
}
