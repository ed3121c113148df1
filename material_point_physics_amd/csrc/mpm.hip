// mpm.hip -- MI355X (gfx950) implementation of one explicit MLS-MPM step
// behind the C ABI declared in include/mpm.h.
//
// Method: "Principles towards Real-Time Simulation of Material Point Method on
// Modern GPUs" (below [RT-MPM]) splits a step into particle sorting, P2G,
// grid update and G2P; the equations are the textbook MLS-MPM with quadratic
// B-splines, APIC transfer and the fixed-corotated model (Hu et al. 2018;
// Jiang et al. 2015; Stomakhin et al. 2012).
//
// Step = 5 kernels, captured once into a HIP graph per buffer parity:
//   k_scan_*      two-phase exclusive scan of per-bin counts -> bin starts,
//                 chunk list (<= KMAX particles of one bin per chunk)
//   k_scatter     bucket scatter by 4^3-cell bin (first radix digit), one
//                 wavefront per chunk of the previous layout: particles that
//                 stay in their bin keep their order (ballot prefix counts),
//                 the few that change bin take wave-aggregated atomic cursors
//                 -> perm[slot] = source index, and the particle's cell
//                 within its bin at the same position
//   k_p2g         one wavefront per chunk: in-LDS counting sort by cell (second
//                 radix digit, 64 cells = 64 lanes), deferred F update, polar
//                 decomposition, Kirchhoff stress, APIC momentum, conflict-free
//                 accumulation into two private 6^3-node LDS windows, one
//                 native global atomic flush per window node and channel
//   k_g2p         one wavefront per chunk: the grid update (v = p/m + dt g,
//                 sticky walls) of the bin's 6^3-node window, staged in LDS;
//                 gather, APIC C, advection + clamp in the storage order P2G
//                 chose; the next step's bin keys/counts
//
// Deferred deformation gradient: [RT-MPM] (kernel-merging discussion) notes
// that the F update at the end of G2P can be postponed to the start of P2G
// to avoid writing F twice, and merges SVD and stress into P2G.  Here G2P
// produces C; the next P2G forms F = (I + dt C) F_prev, evaluates the stress
// and stores F.  mpm_read_particles applies the same pending update, so the
// state read back is F at the end of the step.
//
// Memory: every buffer is carved from the caller's workspace at creation;
// nothing is allocated afterwards ([RT-MPM], memory-reallocation principle).
// No kernel in a step reads a value back to the host ([RT-MPM], CPU-GPU
// synchronisation principle): launch shapes are fixed at creation, and the
// variable-length work lists (chunks, active blocks) are consumed by
// persistent workgroups that read their lengths on the device.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>

#include "../../include/mpm.h"

namespace {

constexpr int WG = 256;          // threads per workgroup (4 wave64)
constexpr int NB = 8;            // node-block edge of the grid layout (512 nodes per block)
constexpr int CB = 4;            // bin edge in cells: particles are bucketed by 4^3-cell bins
constexpr int CB3 = CB * CB * CB;  // 64 cells per bin = one wavefront
constexpr int PW = CB + 2;       // P2G window edge: base nodes of a bin + stencil reach
constexpr int PW3 = PW * PW * PW;  // 216 window nodes
constexpr int KMAX_SHIFT = 8;
constexpr int KMAX = 1 << KMAX_SHIFT;  // particles per P2G chunk at most (4 rounds of one wavefront)
constexpr int KMIN_SHIFT = 6;    // smallest chunk size: 64 particles (see mpm_create)
constexpr int NQ = 8;            // P2G work queues, one per XCD
// Each bin's slot range starts at a multiple of SLOT_ALIGN particles, so a
// particle field's 128-byte lines (32 fp32 values) never straddle two bins:
// chunks and their 64-particle rounds read and write whole lines.  The
// padding slots (holes) are never read: every kernel walks the chunk list.
constexpr int SLOT_ALIGN = 32;
constexpr int NUM_KERNELS = 5;
constexpr int STEP_BATCH = 8;    // steps per batched graph (a multiple of NACC: a batch ends on its starting phase)
// P2G accumulators.  Step n accumulates into gridA[n mod NACC] and its G2P
// reads it.  With the fused G2P2G kernel, the P2G of step n + 1 runs while
// other wavefronts still read step n's accumulator, so the buffer a P2G
// clears for later use is the one of step n - 2 (both its P2G and its G2P
// ended at least one kernel earlier): four buffers, step n clears n + 2.
constexpr int NACC = 4;
static_assert(STEP_BATCH % NACC == 0, "a batch must end on its starting phase");

enum Ctr : int {
  CTR_NCHUNKS = 0,       // + layout parity: chunks of each layout
  CTR_PENDING = 2,
  CTR_MOVERS = 3,        // particles outside their chunk's bin after the last G2P
  CTR_SINCE = 4,         // steps since the last sort
  CTR_SORT = 5,          // + buffer parity: whether the step that reads that buffer sorts
  CTR_MAX_INTERVAL = 7,  // sort policy: at least every this many steps (0 or 1: every step) ...
  CTR_MOVER_BUDGET = 8,  // ... and whenever more particles than this are outside their bins
  // Control words for the fused G2P2G kernel, per buffer parity (the step
  // that reads that buffer).  The step before writes them and the step
  // itself reads them, so no kernel writes a word that its own workgroups
  // read.
  CTR_LOOK = 9,          // + parity: that step's P2G was done by the fused kernel before it
  CTR_PRESET = 11,       // + parity: that step's sort decision (CTR_SORT) was taken before it
  CTR_MOVSNAP = 13,      // movers counted by the previous step's G2P, kept for the fused kernel
  CTR_WORDS = 16,
};
constexpr uint8_t MOVER_TAG = 0xFF;  // P2G order tag of a particle outside its chunk's bin

struct PBuf {
  float *x;      // [3][Np]
  float *v;      // [3][Np]
  float *C;      // [9][Np], row-major components
  float *F;      // [9][Np] (elastic) or [1][Np] (fluid J), one step behind: see header note
  float *E;      // [Np] per-particle Young's modulus, or nullptr
  uint32_t *id;  // [Np] creation index
};

struct SimDev {
  int32_t N, Np;
  int32_t n, nb, nblk;         // grid nodes per axis, node-blocks per axis, node-blocks
  int32_t nbin, nbins;         // bins per axis, bins (Morton-ordered: nbins = (2^ceil(log2 nbin))^3)
  int32_t wall, material, has_E;
  float dx, fn, dt;
  float g[3];
  float mass, vol, E;
  float mu_per_E, lam_per_E;  // Lame parameters per unit Young's modulus
  float alpha, dp_c;          // sand: cone slope of the friction angle, (1 + nu) / (1 - 2 nu)
  float stress_k;             // dt * V0 * 4 / dx^2
  float c_scale;              // 4 / dx (G2P: C = 4/dx^2 * sum w v (x_i - x_p), offsets in cells)
  float lo, hi;               // position clamp
  uint32_t max_chunks;
  int32_t chunk_shift;        // chunks hold up to 2^chunk_shift (64..KMAX) particles of one bin
  PBuf buf[2];
  uint32_t *perm, *key;         // key = bin | cell << KEY_CELL_SHIFT (cell of the base node in its bin)
  uint8_t *cellp;              // cell of the base node in its bin, in perm (sorted) order
  uint32_t *bin_count;         // particles per bin in the next layout (G2P counts)
  uint32_t *stay_count;        // of those, particles already in that bin (G2P counts)
  uint32_t *bin_start, *bin_cursor;  // first slot of each bin; next slot for particles entering it
  uint32_t *bin_stay;          // particles that stay in each bin at this sort (set by the scan)
  uint32_t *tile_sum;          // [ntiles][2] scan tile totals (particles, chunks)
  int32_t ntiles;
  // Chunk lists, one per layout (particle buffer) q: chunks[q][c] = (first
  // slot, count, bin, particles that stay in the bin at the next sort);
  // ctr[CTR_NCHUNKS + q] chunks.  The step that reads buffer q builds
  // layout q ^ 1; its scatter walks layout q.
  uint4 *chunks[2];
  // Grid accumulators, rotating by step number: step n accumulates into
  // gridA[n mod NACC] and marks the node-blocks it touched in the same
  // active_flag; its G2P reads them; the P2G of step n + 2 clears them (and
  // their flags) while it accumulates into its own.
  uint32_t *active_flag[NACC];  // per node-block: 1 = touched by that step's P2G
  float4 *gridA[NACC];          // P2G accumulator per node: (m, p_x, p_y, p_z)
  uint32_t *ctr;
  uint32_t *status;
};

// ------------------------------------------------------------ device utils

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Element of a particle field at a 32-bit byte offset from a uniform base
// (a component's first element).  All fields of one particle share the
// offset register, and each access takes the scalar-base global form: no
// per-access 64-bit address arithmetic.  Offsets are below 2^30 (N < 2^28).
template <typename T>
__device__ __forceinline__ T &at_byte(T *base, uint32_t off) {
  return *reinterpret_cast<T *>(reinterpret_cast<char *>(base) + off);
}

// Streaming accesses for particle fields that a step writes once and reads
// only in the next step (F, E, id, v, C, G2P's advected x) or reads once
// (P2G's C and F): the non-temporal hint keeps these lines from displacing
// the ones reused within the step -- the positions P2G stores for G2P, the
// keys G2P stores for the scatter, the grid lines of the windows.  Measured
// on the 12M slab: scatter + P2G + G2P 1.154 -> 1.063 ms.
template <typename T>
__device__ __forceinline__ void stream_store(T v, T &dst) {
  __builtin_nontemporal_store(v, &dst);
}
template <typename T>
__device__ __forceinline__ T stream_load(const T &src) {
  return __builtin_nontemporal_load(&src);
}

// Node-blocked grid index: blocks of 8^3 nodes (x fastest across blocks);
// inside a block, 4^3 cubes of 2x2x2 nodes (x fastest), and inside a cube
// the 8 nodes with x fastest.  A cube's 8 float4 records fill one 128-byte
// line, and every P2G/G2P window (6^3 nodes at an even origin) covers
// exactly 27 whole cubes, so its flush and its load touch 27 lines.
__device__ __forceinline__ uint32_t node_index(const SimDev &s, int gx, int gy, int gz) {
  const uint32_t blk = ((uint32_t)(gz >> 3) * s.nb + (uint32_t)(gy >> 3)) * s.nb + (uint32_t)(gx >> 3);
  const uint32_t cube = ((uint32_t)((gz >> 1) & 3) << 4) | ((uint32_t)((gy >> 1) & 3) << 2) | (uint32_t)((gx >> 1) & 3);
  const uint32_t in_cube = ((uint32_t)(gz & 1) << 2) | ((uint32_t)(gy & 1) << 1) | (uint32_t)(gx & 1);
  return (blk << 9) | (cube << 3) | in_cube;
}
// Inverse of the in-block part of node_index: local index -> node offsets.
__device__ __forceinline__ void block_local_coords(int local, int &lx, int &ly, int &lz) {
  const int cube = local >> 3, in_cube = local & 7;
  lx = ((cube & 3) << 1) | (in_cube & 1);
  ly = (((cube >> 2) & 3) << 1) | ((in_cube >> 1) & 1);
  lz = ((cube >> 4) << 1) | (in_cube >> 2);
}

// Base node floor(x/dx - 1/2) of a position already inside the clamp box.
__device__ __forceinline__ int base_node(float xn) { return (int)floorf(xn - 0.5f); }

// Spread the low 10 bits of v to every third bit (Morton interleave).
__device__ __forceinline__ uint32_t spread3(uint32_t v) {
  v &= 0x3FFu;
  v = (v | (v << 16)) & 0x030000FFu;
  v = (v | (v << 8)) & 0x0300F00Fu;
  v = (v | (v << 4)) & 0x030C30C3u;
  v = (v | (v << 2)) & 0x09249249u;
  return v;
}
__device__ __forceinline__ uint32_t compact3(uint32_t v) {
  v &= 0x09249249u;
  v = (v | (v >> 2)) & 0x030C30C3u;
  v = (v | (v >> 4)) & 0x0300F00Fu;
  v = (v | (v >> 8)) & 0x030000FFu;
  v = (v | (v >> 16)) & 0x3FFu;
  return v;
}

// Bin of a base node: 4^3-cell bins in Morton (Z-curve) order, so that bins
// adjacent in space are close in processing order (L2 reuse of shared grid
// nodes, compact per-XCD work ranges).
__device__ __forceinline__ uint32_t bin_key(const SimDev &, int bx, int by, int bz) {
  return spread3((uint32_t)bx >> 2) | (spread3((uint32_t)by >> 2) << 1) | (spread3((uint32_t)bz >> 2) << 2);
}

// Cell of a base node within its 4^3-cell bin (x fastest), and the key word
// that carries it above the bin index.  grid_n <= 1024 keeps bins below 2^24.
constexpr int KEY_CELL_SHIFT = 24;
__device__ __forceinline__ uint32_t cell_in_bin(int bx, int by, int bz) {
  return ((uint32_t)(bz & 3) << 4) | ((uint32_t)(by & 3) << 2) | (uint32_t)(bx & 3);
}

// Quadratic B-spline weights of nodes base+0,1,2 at fractional offset f in [0.5,1.5).
__device__ __forceinline__ void bspline_weights(float f, float w[3]) {
  const float a = 1.5f - f, b = f - 1.0f, c = f - 0.5f;
  w[0] = 0.5f * a * a;
  w[1] = 0.75f - b * b;
  w[2] = 0.5f * c * c;
}

// Wave-aggregated atomic add of 1 per valid lane into counters[key]: one
// atomic per distinct key in the wavefront.  Returns each lane's slot
// (old value + rank among the lanes with the same key).
__device__ __forceinline__ uint32_t wave_aggregated_increment(uint32_t *counters, uint32_t key, bool valid) {
  const int lane = lane_id();
  uint64_t todo = __ballot(valid);
  uint32_t slot = 0;
  while (todo) {
    const int leader = __ffsll((unsigned long long)todo) - 1;
    const uint32_t lkey = __shfl(key, leader);
    const uint64_t peers = __ballot(valid && key == lkey) & todo;
    uint32_t old = 0;
    if (lane == leader) old = atomicAdd(counters + lkey, (uint32_t)__popcll(peers));
    old = __shfl(old, leader);
    if ((peers >> lane) & 1ull) slot = old + (uint32_t)__popcll(peers & ((1ull << lane) - 1ull));
    todo &= ~peers;
  }
  return slot;
}

__device__ __forceinline__ void flag_status(const SimDev &s, uint32_t bit, int counter_word) {
  atomicOr(&s.status[0], bit);
  if (counter_word > 0) atomicAdd(&s.status[counter_word], 1u);
}

// ------------------------------------------------------- 3x3 linear algebra

__device__ __forceinline__ float det3(const float A[9]) {
  return A[0] * (A[4] * A[8] - A[5] * A[7]) - A[1] * (A[3] * A[8] - A[5] * A[6]) +
         A[2] * (A[3] * A[7] - A[4] * A[6]);
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

// --------------------------------------------------------------- kernels

// Creation: AoS inputs -> SoA buffer 0 (creation order), ids, first keys.
__global__ __launch_bounds__(WG) void k_init(SimDev s, const float *__restrict__ x0, const float *__restrict__ v0,
                                             const float *__restrict__ C0, const float *__restrict__ F0,
                                             const float *__restrict__ E_p) {
  const uint32_t i = blockIdx.x * WG + threadIdx.x;
  const bool valid = i < (uint32_t)s.N;
  const PBuf b = s.buf[0];
  const size_t Np = (size_t)s.Np;
  uint32_t key = 0;
  if (valid) {
    bool bad = false;
    int base[3];
    for (int a = 0; a < 3; ++a) {
      float xa = x0[3 * (size_t)i + a];
      if (!(xa >= s.lo && xa <= s.hi)) bad = true;  // also catches NaN
      xa = fminf(fmaxf(xa, s.lo), s.hi);
      b.x[a * Np + i] = xa;
      b.v[a * Np + i] = v0 ? v0[3 * (size_t)i + a] : 0.f;
      base[a] = base_node(xa * s.fn);
    }
    if (bad) flag_status(s, MPM_STATUS_BAD_INPUT, 0);
    for (int k = 0; k < 9; ++k) b.C[k * Np + i] = C0 ? C0[9 * (size_t)i + k] : 0.f;
    if (s.material == MPM_J_FLUID) {
      b.F[i] = F0 ? F0[i] : 1.f;
    } else {
      for (int k = 0; k < 9; ++k) b.F[k * Np + i] = F0 ? F0[9 * (size_t)i + k] : ((k % 4 == 0) ? 1.f : 0.f);
    }
    if (s.has_E) b.E[i] = E_p[i];
    b.id[i] = i;
    key = bin_key(s, base[0], base[1], base[2]);
  }
  wave_aggregated_increment(s.bin_count, key, valid);
}

// Sort policy words (see mpm_set_sort_policy).
__global__ void k_set_sort_policy(SimDev s, uint32_t max_interval, uint32_t mover_budget) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    s.ctr[CTR_MAX_INTERVAL] = max_interval;
    s.ctr[CTR_MOVER_BUDGET] = mover_budget;
  }
}

// Zero a uint32 range (fill kernel; graphs avoid memset nodes).
__global__ __launch_bounds__(WG) void k_zero_u32(uint32_t *p, size_t n) {
  for (size_t k = (size_t)blockIdx.x * WG + threadIdx.x; k < n; k += (size_t)gridDim.x * WG) p[k] = 0u;
}

__global__ __launch_bounds__(WG) void k_zero_f32(float *p, size_t n) {
  for (size_t k = (size_t)blockIdx.x * WG + threadIdx.x; k < n; k += (size_t)gridDim.x * WG) p[k] = 0.f;
}

// Block-wide inclusive scan of one value per thread (NT threads); returns the
// inclusive prefix and writes the workgroup total to *total.
template <int NT>
__device__ __forceinline__ uint32_t block_scan_incl(uint32_t v, uint32_t *wsum, uint32_t *total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  uint32_t inc = v;
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t t = __shfl_up(inc, d);
    if (lane >= d) inc += t;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t x = wsum[w];
    if (w < wave) before += x;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + inc;
}

constexpr int SCAN_PER = 8;                  // bins per thread
constexpr int SCAN_TILE = WG * SCAN_PER;     // bins per scan tile
constexpr int SCAN_SMALL_NT = 1024;          // grids of at most this many x SCAN_PER bins
                                             // scan in one workgroup, without k_scan_tiles

// A bin's slot range: its count rounded up to whole SLOT_ALIGN groups.
__device__ __forceinline__ uint32_t padded(uint32_t count) {
  return (count + (uint32_t)SLOT_ALIGN - 1u) & ~(uint32_t)(SLOT_ALIGN - 1);
}

// Whether the current step sorts (the free-zone policy of [RT-MPM],
// non-essential-phase discussion: particles stay in their bins' chunks
// between sorts, and the few that left their bin are handled one by one).
// Every step sorts unless a policy was set with mpm_set_sort_policy.
__device__ __forceinline__ bool sort_this_step(const SimDev &s) {
  const uint32_t maxint = s.ctr[CTR_MAX_INTERVAL];
  return maxint <= 1u || s.ctr[CTR_SINCE] + 1u >= maxint || s.ctr[CTR_MOVERS] > s.ctr[CTR_MOVER_BUDGET];
}

// The decision for the next step, taken by the fused kernel before that step
// begins (it must know whether to run the next step's P2G): the same rule,
// on the movers the previous step counted, since the current step's G2P is
// still running.
__device__ __forceinline__ bool sort_next_step(const SimDev &s) {
  const uint32_t maxint = s.ctr[CTR_MAX_INTERVAL];
  return maxint <= 1u || s.ctr[CTR_SINCE] + 1u >= maxint || s.ctr[CTR_MOVSNAP] > s.ctr[CTR_MOVER_BUDGET];
}

// The current step's decision: taken before it by the fused kernel, or now.
__device__ __forceinline__ bool decide_sort(const SimDev &s, int src) {
  return s.ctr[CTR_PRESET + src] != 0u ? s.ctr[CTR_SORT + src] != 0u : sort_this_step(s);
}

// Scan, phase 1: per-tile totals of (padded) slot counts and chunk counts.
// Also takes the step's sort decision (uniform: every thread reads the same
// counters) and publishes it for the step's other kernels.
__global__ __launch_bounds__(WG) void k_scan_tiles(SimDev s, int src) {
  __shared__ uint32_t wsum[WG / 64];
  const bool sort = decide_sort(s, src);
  // (a preset decision is already in the word, which other workgroups read)
  if (blockIdx.x == 0 && threadIdx.x == 0 && s.ctr[CTR_PRESET + src] == 0u) s.ctr[CTR_SORT + src] = sort ? 1u : 0u;
  if (!sort) return;
  const uint32_t nbins = (uint32_t)s.nbins;
  const uint32_t b0 = blockIdx.x * SCAN_TILE + threadIdx.x * SCAN_PER;
  uint32_t c = 0, ch = 0;
#pragma unroll
  for (int k = 0; k < SCAN_PER; ++k) {
    const uint32_t cnt = (b0 + k < nbins) ? s.bin_count[b0 + k] : 0u;
    c += padded(cnt);
    ch += (cnt + (1u << s.chunk_shift) - 1u) >> s.chunk_shift;
  }
  uint32_t tc, tch;
  block_scan_incl<WG>(c, wsum, &tc);
  block_scan_incl<WG>(ch, wsum, &tch);
  if (threadIdx.x == 0) {
    s.tile_sum[2 * blockIdx.x] = tc;
    s.tile_sum[2 * blockIdx.x + 1] = tch;
  }
}

// Scan, phase 2: each tile adds the totals of the tiles before it, scans its
// bins and writes the bin starts and cursors for k_scatter, the chunk list of
// layout lay for k_p2g, and zeroes the counts for k_g2p; the last tile
// publishes the chunk total.  A bin's particles that stay in it are placed
// first (in their previous order), so the cursor for the others starts after
// them.  NT threads per workgroup, one tile of NT * SCAN_PER bins per
// workgroup.
template <int NT>
__global__ __launch_bounds__(NT) void k_scan_bins(SimDev s, int lay) {
  constexpr int TILE = NT * SCAN_PER;
  __shared__ uint32_t wsum[NT / 64];
  constexpr int LTAB = (NT == SCAN_SMALL_NT) ? TILE + 1 : 1;
  __shared__ uint32_t cfirst[LTAB];  // tile-relative first chunk of each bin (+ the tile's total)
  __shared__ uint32_t pfirst[LTAB];  // tile-relative first slot of each bin (+ the tile's total)
  const uint32_t nbins = (uint32_t)s.nbins;
  const uint32_t t = blockIdx.x;
  const uint32_t shift = (uint32_t)s.chunk_shift;
  const int src = lay ^ 1;
  // The sort decision: taken here by the one-workgroup scan (no k_scan_tiles
  // before it), else read from k_scan_tiles.  The mover count is kept for
  // the fused kernel's decision and reset for this step's G2P to fill again
  // (every thread has read it before the barrier).
  bool sort;
  if (NT == SCAN_SMALL_NT) {
    sort = decide_sort(s, src);
    __syncthreads();
    if (threadIdx.x == 0) s.ctr[CTR_SORT + src] = sort ? 1u : 0u;
  } else {
    sort = s.ctr[CTR_SORT + src] != 0u;
  }
  if (t == 0 && threadIdx.x == 0) {
    s.ctr[CTR_MOVSNAP] = s.ctr[CTR_MOVERS];
    s.ctr[CTR_MOVERS] = 0u;
  }
  if (!sort) {
    // No sort: layout lay repeats layout src (its chunk list is copied),
    // and the bin counts are cleared for this step's G2P.
    const uint32_t nch_old = s.ctr[CTR_NCHUNKS + src];
    for (uint32_t c = t * NT + threadIdx.x; c < nch_old; c += gridDim.x * NT) s.chunks[lay][c] = s.chunks[src][c];
    const uint32_t b0 = t * TILE + threadIdx.x * SCAN_PER;
#pragma unroll
    for (int k = 0; k < SCAN_PER; ++k)
      if (b0 + k < nbins) {
        s.bin_count[b0 + k] = 0u;
        s.stay_count[b0 + k] = 0u;
      }
    if (t == 0 && threadIdx.x == 0) {
      s.ctr[CTR_NCHUNKS + lay] = nch_old;
      s.ctr[CTR_SINCE] = s.ctr[CTR_SINCE] + 1u;
    }
    return;
  }
  uint32_t pc = 0, pch = 0;
  for (uint32_t k = threadIdx.x; k < t; k += NT) {
    pc += s.tile_sum[2 * k];
    pch += s.tile_sum[2 * k + 1];
  }
  uint32_t tile_base_c, tile_base_ch;
  block_scan_incl<NT>(pc, wsum, &tile_base_c);
  block_scan_incl<NT>(pch, wsum, &tile_base_ch);
  const uint32_t lb0 = threadIdx.x * SCAN_PER, b0 = t * TILE + lb0;
  uint32_t c[SCAN_PER], st[SCAN_PER], ch[SCAN_PER], csum = 0, chsum = 0;
#pragma unroll
  for (int k = 0; k < SCAN_PER; ++k) {
    c[k] = (b0 + k < nbins) ? s.bin_count[b0 + k] : 0u;
    st[k] = (b0 + k < nbins) ? s.stay_count[b0 + k] : 0u;  // (loaded with the counts: no second round trip)
    ch[k] = (c[k] + (1u << shift) - 1u) >> shift;
    csum += padded(c[k]);
    chsum += ch[k];
  }
  uint32_t tc, tch;
  const uint32_t ic = block_scan_incl<NT>(csum, wsum, &tc);
  const uint32_t ich = block_scan_incl<NT>(chsum, wsum, &tch);
  uint32_t run = ic - csum, chrun = ich - chsum;  // tile-relative, in slots (multiples of SLOT_ALIGN)
  // Many-tile grids are sparse per bin (a chunk or two): each thread writes
  // its bins' chunk records.  The one-workgroup path (small, often dense
  // scenes, many chunks per bin) spreads the records over all threads.
  constexpr bool spread = NT == SCAN_SMALL_NT;
#pragma unroll
  for (int k = 0; k < SCAN_PER; ++k) {
    const uint32_t b = b0 + k;
    if (spread) {
      cfirst[lb0 + k] = chrun;
      pfirst[lb0 + k] = run | (c[k] & (uint32_t)(SLOT_ALIGN - 1));  // (run is aligned: the low bits carry the count)
    }
    if (b < nbins) {
      s.bin_count[b] = 0u;
      if (c[k] > 0u) {  // (stay_count <= bin_count: both are zero otherwise)
        const uint32_t stay = min(st[k], c[k]);
        s.stay_count[b] = 0u;
        s.bin_start[b] = tile_base_c + run;
        s.bin_stay[b] = stay;
        s.bin_cursor[b] = tile_base_c + run + stay;
      }
      if (!spread)
        for (uint32_t j = 0; j < ch[k]; ++j) {
          const uint32_t off = j << shift, cnt = min(1u << shift, c[k] - off);
          s.chunks[lay][tile_base_ch + chrun + j] = make_uint4(tile_base_c + run + off, cnt, b, cnt);
        }
    }
    run += padded(c[k]);
    chrun += ch[k];
  }
  if (spread && threadIdx.x == 0) {
    cfirst[TILE] = tch;
    pfirst[TILE] = tc;
  }
  __syncthreads();
  // (spread) chunk c belongs to the last bin whose first chunk is <= c
  // (binary search in LDS)
  for (uint32_t cc = threadIdx.x; spread && cc < tch; cc += NT) {
    uint32_t lo = 0, hi = TILE - 1;
    while (lo < hi) {
      const uint32_t mid = (lo + hi + 1u) >> 1;
      if (cfirst[mid] <= cc) lo = mid;
      else hi = mid - 1u;
    }
    const uint32_t off = (cc - cfirst[lo]) << shift, amask = (uint32_t)(SLOT_ALIGN - 1);
    const uint32_t pstart = pfirst[lo] & ~amask, span = (pfirst[lo + 1] & ~amask) - pstart, rem = pfirst[lo] & amask;
    const uint32_t pcount = rem ? span - (uint32_t)SLOT_ALIGN + rem : span;  // the bin's particle count
    const uint32_t cnt = min(1u << shift, pcount - off);
    s.chunks[lay][tile_base_ch + cc] = make_uint4(tile_base_c + pstart + off, cnt, t * TILE + lo, cnt);
  }
  if (t == gridDim.x - 1 && threadIdx.x == 0) s.ctr[CTR_NCHUNKS + lay] = tile_base_ch + tch;
  if (t == 0 && threadIdx.x == 0) s.ctr[CTR_SINCE] = 0u;
}

// Creation: move the initial state (buffer 0, creation order) into bin order
// in buffer 1 (layout 1, whose chunk list the scan wrote): particle i goes to
// the next free slot of its bin (one atomic per distinct bin per wavefront;
// the order within a bin is the order the atomics happen to run in).  Writes
// the keys of the new order and counts every particle as a stayer of its bin
// (the chunk records already say so), for the first step's scan.
__global__ __launch_bounds__(WG) void k_scatter_init(SimDev s) {
  const uint32_t i = blockIdx.x * WG + threadIdx.x;
  const bool valid = i < (uint32_t)s.N;
  const PBuf a = s.buf[0], b = s.buf[1];
  const size_t Np = (size_t)s.Np;
  int base[3] = {0, 0, 0};
  float xi[3] = {0.f, 0.f, 0.f};
  uint32_t key = 0;
  if (valid) {
    for (int c = 0; c < 3; ++c) {
      xi[c] = a.x[c * Np + i];
      base[c] = base_node(xi[c] * s.fn);
    }
    key = bin_key(s, base[0], base[1], base[2]);
  }
  const uint32_t slot = wave_aggregated_increment(s.bin_cursor, key, valid);
  if (valid && slot < (uint32_t)s.Np) {
    for (int c = 0; c < 3; ++c) {
      b.x[c * Np + slot] = xi[c];
      b.v[c * Np + slot] = a.v[c * Np + i];
    }
    for (int k = 0; k < 9; ++k) b.C[k * Np + slot] = a.C[k * Np + i];
    const int fw = s.material == MPM_J_FLUID ? 1 : 9;
    for (int k = 0; k < fw; ++k) b.F[k * Np + slot] = a.F[k * Np + i];
    if (s.has_E) b.E[slot] = a.E[i];
    b.id[slot] = a.id[i];
    s.key[slot] = key | (cell_in_bin(base[0], base[1], base[2]) << KEY_CELL_SHIFT);
  }
  wave_aggregated_increment(s.bin_count, key, valid);
  wave_aggregated_increment(s.stay_count, key, valid);
}

// Bucket scatter of a step that reads buffer (layout) src.  Persistent
// single-wavefront workgroups walk the chunks of layout src.  A particle that
// stays in its chunk's bin goes to bin_start + (stayers of the bin's earlier
// chunks, recorded by G2P) + (stayers before it in the chunk): the bin's
// stayers keep their previous order, so P2G's processing order, and with it
// the storage order, repeats from step to step and its gathers read
// consecutive addresses.  A particle that changes bin takes the bin's atomic
// cursor, which starts after the bin's stayers.
// Position of the bin's stayer number j (in their previous order) in the
// bin's new slot range.  A dense bin's stayers fill several chunks of K =
// 2^kshift; each chunk was stored in P2G's (super-rank, window, cell) order,
// so its rounds of 64 hold about one particle per cell, while its cells as a
// whole may be far from balanced (particles created cell by cell stay
// together).  For Cp = 2 or 4 full chunks (the most with blocks of at least
// one round), the blocks are transposed -- new chunk q takes block q of every
// old chunk -- so each new chunk draws evenly from all of them and needs
// fewer read-modify-write passes.  Other stayers keep their order.
__device__ __forceinline__ uint32_t stayer_slot(uint32_t j, uint32_t stay, uint32_t kshift) {
  const uint32_t full = stay >> kshift, cap = 1u << (kshift - KMIN_SHIFT);  // blocks >= 64 particles
  const uint32_t cp = min(full, cap) >= 4u ? 4u : (min(full, cap) >= 2u ? 2u : 1u);
  if (cp == 1u || j >= (cp << kshift)) return j;
  const uint32_t K = 1u << kshift, B = K / cp;
  const uint32_t m = j >> kshift, r = j & (K - 1u), q = r / B, i = r % B;
  return (q << kshift) + m * B + i;
}

__global__ __launch_bounds__(64) void k_scatter(SimDev s, int src) {
  if (s.ctr[CTR_SORT + src] == 0u) return;  // a step without a sort
  const int lane = threadIdx.x;
  const uint32_t kshift = (uint32_t)s.chunk_shift;
  const uint64_t below = (1ull << lane) - 1ull;
  const uint32_t nch = s.ctr[CTR_NCHUNKS + src];
  const uint4 *chunks = s.chunks[src];
  // The record of the next chunk, and the bin of the chunk before it, are
  // loaded one chunk ahead.
  uint4 ch_next = make_uint4(0u, 0u, 0u, 0u);
  uint32_t prev_next = 0xFFFFFFFFu;
  if (blockIdx.x < nch) {
    ch_next = chunks[blockIdx.x];
    if (blockIdx.x > 0) prev_next = chunks[blockIdx.x - 1].z;
  }
  for (uint32_t c = blockIdx.x; c < nch; c += gridDim.x) {
    const uint4 ch = ch_next;
    const uint32_t prev_bin = prev_next;
    const uint32_t start = ch.x, count = min(ch.y, (uint32_t)KMAX), bin = ch.z;
    if (c + gridDim.x < nch) {
      ch_next = chunks[c + gridDim.x];
      prev_next = chunks[c + gridDim.x - 1].z;
    }
    // all of the chunk's keys at once (lanes past the count read none)
    uint32_t kc[KMAX / 64];
#pragma unroll
    for (int j = 0; j < KMAX / 64; ++j) {
      const uint32_t r = (uint32_t)(64 * j + lane);
      kc[j] = r < count ? s.key[start + r] : 0u;
    }
    const uint32_t bstart = s.bin_start[bin], bstay = s.bin_stay[bin];
    uint32_t base = 0;  // stayers before this chunk's, in the bin
    // stayers of the bin's earlier chunks (a bin's chunks are consecutive;
    // nearly always none, or a few records)
    for (uint32_t c0 = c; prev_bin == bin && c0 > 0;) {
      const uint32_t lo = c0 > 64u ? c0 - 64u : 0u;
      const uint32_t cj = lo + (uint32_t)lane;
      uint4 r = make_uint4(0u, 0u, 0xFFFFFFFFu, 0u);
      if (cj < c0) r = chunks[cj];
      const bool same = cj < c0 && r.z == bin;
      uint32_t add = same ? r.w : 0u;
      for (int d = 32; d >= 1; d >>= 1) add += (uint32_t)__shfl_xor((int)add, d);
      base += add;
      // all 64 earlier records belong to the bin: keep walking back
      if (__ballot(same) != ~0ull || lo == 0u) break;
      c0 = lo;
    }
#pragma unroll
    for (int j = 0; j < KMAX / 64; ++j) {
      const uint32_t r = (uint32_t)(64 * j + lane);
      if ((uint32_t)(64 * j) >= count) break;
      const bool valid = r < count;
      const uint32_t key = kc[j] & ((1u << KEY_CELL_SHIFT) - 1u);
      const bool stay = valid && key == bin;
      const uint64_t sm = __ballot(stay);
      uint32_t slot = bstart + stayer_slot(base + (uint32_t)__popcll(sm & below), bstay, kshift);
      base += (uint32_t)__popcll(sm);
      if (__ballot(valid && !stay) != 0ull) {
        const uint32_t mslot = wave_aggregated_increment(s.bin_cursor, key, valid && !stay);
        if (!stay) slot = mslot;
      }
      if (valid && slot < (uint32_t)s.Np) {
        s.perm[slot] = start + r;
        s.cellp[slot] = (uint8_t)(kc[j] >> KEY_CELL_SHIFT);
      }
    }
  }
}

// P2G.  Persistent single-wavefront workgroups take chunks (<= KMAX particles
// of one 4^3-cell bin) from their XCD's queue.
//
// Accumulation without atomics: on gfx950, LDS float atomics serialise per
// lane, so the windows are private to the wavefront and updated with plain
// read-modify-writes.  There are NWIN windows; the particle of rank r in its
// cell (r-th of that cell in the chunk) accumulates into window r % NWIN and
// has super-rank r / NWIN.  The chunk's particles are ordered by (super-rank,
// window, cell): lanes that share a super-rank differ in (window, cell), so
// for a fixed stencil offset their target addresses are distinct, and one
// masked ds_read/ds_write pair per offset adds all of them.  A round of 64
// lanes that spans several super-ranks runs one pass per super-rank.  The LDS
// executes a wavefront's accesses in issue order; compiler fences keep that
// order.  The flush adds the windows and issues one native global atomic per
// node and channel.
constexpr int NWIN = 2;                  // accumulation windows per wavefront
constexpr int KSR = KMAX / NWIN;         // super-ranks per chunk, at most

struct P2GRankTables {                   // lives in the window space while a chunk is ordered
  uint32_t hist[CB3];                    // particles per cell
  uint32_t subcnt[KMAX / 64][CB3];       // particles per cell in each sub-round of 64
  uint32_t rstart[KSR + 2];              // first position of each super-rank
  uint64_t rmask[NWIN * KSR];            // per (super-rank, window): cells present (bit = cell)
};
static_assert(sizeof(P2GRankTables) <= sizeof(float4) * NWIN * PW3, "rank tables must fit the windows");

union P2GShared {
  float4 win[NWIN * PW3];
  P2GRankTables rk;
};

// Deferred deformation-gradient update with the C of the G2P before it:
// F <- (I + dt C) F, or for the fluid J <- J det(I + dt C).
template <int MAT>
__device__ __forceinline__ void update_F(float *Fp, const float Cp[9], float dt) {
  if (MAT == MPM_J_FLUID) {
    const float G[9] = {1.f + dt * Cp[0], dt * Cp[1], dt * Cp[2], dt * Cp[3], 1.f + dt * Cp[4],
                        dt * Cp[5], dt * Cp[6], dt * Cp[7], 1.f + dt * Cp[8]};
    Fp[0] = Fp[0] * det3(G);
  } else {
    float Fn[9];
#pragma unroll
    for (int r2 = 0; r2 < 3; ++r2)
#pragma unroll
      for (int c2 = 0; c2 < 3; ++c2)
        Fn[r2 * 3 + c2] = Fp[r2 * 3 + c2] + dt * (Cp[r2 * 3 + 0] * Fp[0 * 3 + c2] + Cp[r2 * 3 + 1] * Fp[1 * 3 + c2] +
                                                  Cp[r2 * 3 + 2] * Fp[2 * 3 + c2]);
#pragma unroll
    for (int k = 0; k < 9; ++k) Fp[k] = Fn[k];
  }
}

// Kirchhoff stress of the fixed-corotated model, tau = 2 mu (F - R) F^T +
// lam (J - 1) J I with R the rotation closest to F (fluid: tau = K J (J - 1) I,
// K = E), and the APIC affine momentum matrix A = m C - dt V0 (4/dx^2) tau.
// Returns status bits (inverted or unconverged F; fluid: J <= 0).
template <int MAT>
__device__ __forceinline__ uint32_t affine_momentum(const SimDev &s, const float *Fp, float E, const float Cp[9],
                                                    float A[9]) {
  const float mass = s.mass;
  if (MAT == MPM_J_FLUID) {
    const float J = Fp[0];
    const float tau_diag = E * J * (J - 1.f);
#pragma unroll
    for (int k = 0; k < 9; ++k) A[k] = mass * Cp[k] - s.stress_k * ((k % 4 == 0) ? tau_diag : 0.f);
    return (J > 0.f) ? 0u : (uint32_t)MPM_STATUS_INVERTED;
  }
  const float mu = E * s.mu_per_E, lam = E * s.lam_per_E;
  float R[9];
  const uint32_t st = rotation_of(Fp, R);
  const float J = det3(Fp);
  float D[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) D[k] = 2.f * mu * (Fp[k] - R[k]);
  const float vl = lam * (J - 1.f) * J;
#pragma unroll
  for (int r2 = 0; r2 < 3; ++r2)
#pragma unroll
    for (int c2 = 0; c2 < 3; ++c2) {
      const float tau = D[r2 * 3 + 0] * Fp[c2 * 3 + 0] + D[r2 * 3 + 1] * Fp[c2 * 3 + 1] + D[r2 * 3 + 2] * Fp[c2 * 3 + 2] +
                        (r2 == c2 ? vl : 0.f);
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

// Eigen-decomposition of a symmetric 3x3 matrix by cyclic Jacobi rotations
// (Rutishauser's formulation, Golub & Van Loan, "Matrix Computations"):
// A becomes diagonal, W's columns the eigenvectors.
__device__ __forceinline__ void eigen_sym3(float a[3][3], float W[3][3]) {
#pragma unroll
  for (int r = 0; r < 3; ++r)
#pragma unroll
    for (int c = 0; c < 3; ++c) W[r][c] = (r == c) ? 1.f : 0.f;
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

// Sand, per particle: the plasticity projection of F (in place, when
// project) and the APIC affine momentum A = m C - dt V0 (4/dx^2) tau with the
// Hencky Kirchhoff stress tau = U diag(2 mu h + lam sum h) U^T of the
// projected principal strains h (U = F V diag(1/s) is unchanged by the
// projection, so tau is formed from the trial F and its l).  Return
// mapping, with t = sum e and the deviator d = e - t/3: t > 0 -> tip
// (h = 0); else g = |d| + (1 + nu)/(1 - 2 nu) t alpha, g <= 0 -> unchanged,
// g > 0 -> h = e - g d / |d|.  Returns status bits (det F <= 0).
__device__ __forceinline__ uint32_t sand_affine(const SimDev &s, float Fp[9], float E, const float Cp[9], float A[9],
                                                bool project) {
  float a[3][3], W[3][3];
#pragma unroll
  for (int r = 0; r < 3; ++r)
#pragma unroll
    for (int c = 0; c < 3; ++c) a[r][c] = Fp[0 * 3 + r] * Fp[0 * 3 + c] + Fp[1 * 3 + r] * Fp[1 * 3 + c] + Fp[2 * 3 + r] * Fp[2 * 3 + c];
  eigen_sym3(a, W);
  float l[3], e[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    l[i] = fmaxf(a[i][i], 1e-6f);
    e[i] = 0.5f * logf(l[i]);
  }
  const uint32_t st = det3(Fp) > 0.f ? 0u : (uint32_t)MPM_STATUS_INVERTED;
  float h[3] = {e[0], e[1], e[2]};
  bool moved = false;
  if (project) {
    const float t = e[0] + e[1] + e[2];
    const float d[3] = {e[0] - t / 3.f, e[1] - t / 3.f, e[2] - t / 3.f};
    const float nd = sqrtf(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
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
  }
  // tau = F V diag((2 mu h + lam sum h) / l) V^T F^T, F the trial F
  const float mu = E * s.mu_per_E, lam = E * s.lam_per_E, ht = h[0] + h[1] + h[2];
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
  if (moved) {  // F becomes the projected one: its stretches scaled by exp(h - e)
    float m[3], Fn[9];
#pragma unroll
    for (int i = 0; i < 3; ++i) m[i] = expf(h[i] - e[i]);
    stretch_scaled(Fp, W, m, Fn);
#pragma unroll
    for (int k = 0; k < 9; ++k) Fp[k] = Fn[k];
  }
  return st;
}

// Base node b = floor(x/dx - 1/2), fractional offset f and quadratic
// B-spline weights w[axis][o] of a position.
__device__ __forceinline__ void particle_weights(const float xp[3], float fn, int b[3], float f[3], float w[3][3]) {
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    const float xn = xp[a] * fn;
    b[a] = base_node(xn);
    f[a] = xn - (float)b[a];
    bspline_weights(f[a], w[a]);
  }
}

// APIC momentum at stencil node o: m v + A (o - f) dx = q0 + Ad o.
__device__ __forceinline__ void momentum_terms(float mass, float dx, const float vp[3], const float A[9],
                                               const float f[3], float q0[3], float Ad[9]) {
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    q0[a] = mass * vp[a] - dx * (A[a * 3 + 0] * f[0] + A[a * 3 + 1] * f[1] + A[a * 3 + 2] * f[2]);
#pragma unroll
    for (int c2 = 0; c2 < 3; ++c2) Ad[a * 3 + c2] = dx * A[a * 3 + c2];
  }
}

// One particle's 27 node contributions (w m, w (q0 + Ad o)) added to an LDS
// window, li0 = the window index of stencil offset 0: plain read-modify-
// writes, which the caller makes conflict-free across the wavefront's lanes.
__device__ __forceinline__ void deposit_window(float4 *win, int li0, float w[3][3], float q0[3], float Ad[9],
                                               float mass) {
  // Form the 27 node contributions here rather than keeping all 108 of them
  // live across the caller's pass loop (register pressure limits occupancy).
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    __asm__ __volatile__("" : "+v"(q0[k]), "+v"(w[0][k]), "+v"(w[1][k]), "+v"(w[2][k]));
  }
#pragma unroll
  for (int k = 0; k < 9; ++k) __asm__ __volatile__("" : "+v"(Ad[k]));
  // Momentum at node o is q0 + Ad (ox, oy, oz): running sums along z, y and
  // x (one add per component per step; no multiplications by the constant
  // offsets, which IEEE rules keep the compiler from folding).
  float qz[3] = {q0[0], q0[1], q0[2]};
#pragma unroll
  for (int oz = 0; oz < 3; ++oz) {
    if (oz > 0) {
      qz[0] += Ad[2];
      qz[1] += Ad[5];
      qz[2] += Ad[8];
    }
    float qy[3] = {qz[0], qz[1], qz[2]};
#pragma unroll
    for (int oy = 0; oy < 3; ++oy) {
      if (oy > 0) {
        qy[0] += Ad[1];
        qy[1] += Ad[4];
        qy[2] += Ad[7];
      }
      const float wyz = w[1][oy] * w[2][oz];
      float qx[3] = {qy[0], qy[1], qy[2]};
#pragma unroll
      for (int ox = 0; ox < 3; ++ox) {
        if (ox > 0) {
          qx[0] += Ad[0];
          qx[1] += Ad[3];
          qx[2] += Ad[6];
        }
        const float wt = w[0][ox] * wyz;
        const int li = li0 + (oz * PW + oy) * PW + ox;
        float4 g = win[li];
        g.x = fmaf(wt, mass, g.x);
        g.y = fmaf(wt, qx[0], g.y);
        g.z = fmaf(wt, qx[1], g.z);
        g.w = fmaf(wt, qx[2], g.w);
        win[li] = g;
        // keep this read-modify-write ahead of the next one in issue order
        __asm__ __volatile__("" ::: "memory");
      }
    }
  }
}

// Clear accumulator a (that of the step two before the one accumulating
// now: its P2G and its G2P have ended): the node-blocks it marked, and their
// marks.  Workgroup b takes blocks G-1-b, 2G-1-b, ... (G workgroups; counted
// from the last one because in a small scene the first ones have chunks and
// the flag loads would delay them); the stores drain while it works on its
// chunks.  One wavefront per workgroup.
__device__ __forceinline__ void clear_accumulator(const SimDev &s, int a) {
  const int lane = threadIdx.x;
  for (uint32_t blk = gridDim.x - 1u - blockIdx.x; blk < (uint32_t)s.nblk; blk += gridDim.x) {
    if (s.active_flag[a][blk] == 0u) continue;
    float4 *g = s.gridA[a] + ((size_t)blk << 9);
#pragma unroll
    for (int k = 0; k < 8; ++k) g[k * 64 + lane] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane == 0) s.active_flag[a][blk] = 0u;
  }
}

// Flush: the sum of the NWIN windows (window origin = first base node of
// the bin, ox0, oy0, oz0), one native global float atomic per nonzero value
// (adding zero changes nothing) into accumulator a, in whole cubes: lane =
// (cube of the pair, node in cube, channel), so each atomic instruction
// covers two cubes = two full 128-byte lines (the memory-side atomic units
// work per line).  A window cube's node index is separable per axis; with
// the window origin a multiple of 4, the axis terms of cube coordinate 0..2
// are uniform (relative to the origin's node-block: at most one block step
// per axis), so a lane's address is a uniform block pointer plus the cube
// offset of its half of the wavefront plus its node and channel.  Then the
// (at most 2x2x2) node-blocks the window overlaps are marked: the P2G two
// steps later clears exactly these (and mpm_read_grid reads them).  A marked
// block whose nodes got no mass is cleared for nothing, which is harmless.
// Plain stores: every writer stores the same value.
__device__ __forceinline__ void flush_windows(const SimDev &s, const float4 *win, int ox0, int oy0, int oz0, int a) {
  const int lane = threadIdx.x;
  {
    const int h = lane >> 5, j = (lane >> 2) & 7, chn = lane & 3;
    const int jx = j & 1, jy = (j >> 1) & 1, jz = j >> 2;
    const uint32_t nbs = (uint32_t)s.nb;
    uint32_t XC[3], YC[3], ZC[3];  // node offsets of cube coordinate 0..2 per axis
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const uint32_t ux = (uint32_t)(ox0 >> 1) + (uint32_t)k, uy = (uint32_t)(oy0 >> 1) + (uint32_t)k,
                     uz = (uint32_t)(oz0 >> 1) + (uint32_t)k;
      XC[k] = (((ux >> 2) - (uint32_t)(ox0 >> 3)) << 9) + ((ux & 3u) << 3);
      YC[k] = (((uy >> 2) - (uint32_t)(oy0 >> 3)) * nbs << 9) + ((uy & 3u) << 5);
      ZC[k] = (((uz >> 2) - (uint32_t)(oz0 >> 3)) * nbs * nbs << 9) + ((uz & 3u) << 7);
    }
    float4 *gblk = s.gridA[a] +
                   (((size_t)(oz0 >> 3) * nbs + (size_t)(oy0 >> 3)) * nbs + (size_t)(ox0 >> 3)) * 512u;
    const uint32_t lane_b = (uint32_t)(16 * j + 4 * chn);
    const float *winl = reinterpret_cast<const float *>(win) + 4 * ((jz * PW + jy) * PW + jx) + chn;
    // the window reaches past the grid only at the grid's upper faces
    const bool interior = ox0 + PW <= s.n && oy0 + PW <= s.n && oz0 + PW <= s.n;
#pragma unroll
    for (int t = 0; t < 14; ++t) {
      const int c0 = 2 * t, c1 = 2 * t + 1;  // the two cubes of this step
      const int x0 = c0 % 3, y0 = (c0 / 3) % 3, z0 = c0 / 9;
      const int x1 = c1 % 3, y1 = (c1 / 3) % 3, z1 = (c1 < 27) ? c1 / 9 : 0;
      const uint32_t o0 = XC[x0] + YC[y0] + ZC[z0], o1 = XC[x1] + YC[y1] + ZC[z1];
      const int kw0 = ((2 * z0) * PW + 2 * y0) * PW + 2 * x0, kw1 = ((2 * z1) * PW + 2 * y1) * PW + 2 * x1;
      if (c1 >= 27 && h) continue;
      const int kw = h ? kw1 : kw0;
      float val = 0.f;
#pragma unroll
      for (int w = 0; w < NWIN; ++w) val += winl[4 * (kw + w * PW3)];
      bool inb = val != 0.f;
      if (!interior) {
        const int cx = h ? x1 : x0, cy = h ? y1 : y0, cz = h ? z1 : z0;
        inb = inb && ox0 + 2 * cx + jx < s.n && oy0 + 2 * cy + jy < s.n && oz0 + 2 * cz + jz < s.n;
      }
      if (inb) unsafeAtomicAdd(&at_byte(reinterpret_cast<float *>(gblk), 16u * (h ? o1 : o0) + lane_b), val);
    }
  }
  if (lane < 8) {
    const int bx = (ox0 >> 3) + (lane & 1), by = (oy0 >> 3) + ((lane >> 1) & 1), bz = (oz0 >> 3) + (lane >> 2);
    const int ex = min(ox0 + PW - 1, s.n - 1) >> 3, ey = min(oy0 + PW - 1, s.n - 1) >> 3,
              ez = min(oz0 + PW - 1, s.n - 1) >> 3;
    if (bx <= ex && by <= ey && bz <= ez)
      s.active_flag[a][((uint32_t)bz * (uint32_t)s.nb + (uint32_t)by) * (uint32_t)s.nb + (uint32_t)bx] = 1u;
  }
}

// A particle whose stencil is outside its chunk's window (only in steps
// without a sort; rare) deposits its 27 nodes into accumulator a with direct
// global atomics and marks the node-blocks its stencil touches, for the
// clear two steps later and the grid readback.  Momentum at node o is
// q0 + Ad o.
__device__ __forceinline__ void deposit_global(const SimDev &s, int a, const int b[3], const float w[3][3],
                                               const float q0[3], const float Ad[9]) {
  const float mass = s.mass;
#pragma unroll 1
  for (int oz = 0; oz < 3; ++oz)
#pragma unroll 1
    for (int oy = 0; oy < 3; ++oy)
#pragma unroll 1
      for (int ox = 0; ox < 3; ++ox) {
        const int gx = b[0] + ox, gy = b[1] + oy, gz = b[2] + oz;
        if (gx < 0 || gy < 0 || gz < 0 || gx >= s.n || gy >= s.n || gz >= s.n) continue;
        const float wt = w[0][ox] * w[1][oy] * w[2][oz];
        float *g = reinterpret_cast<float *>(s.gridA[a] + node_index(s, gx, gy, gz));
        unsafeAtomicAdd(g + 0, wt * mass);
        unsafeAtomicAdd(g + 1, wt * (q0[0] + Ad[0] * ox + Ad[1] * oy + Ad[2] * oz));
        unsafeAtomicAdd(g + 2, wt * (q0[1] + Ad[3] * ox + Ad[4] * oy + Ad[5] * oz));
        unsafeAtomicAdd(g + 3, wt * (q0[2] + Ad[6] * ox + Ad[7] * oy + Ad[8] * oz));
      }
#pragma unroll 1
  for (int k = 0; k < 8; ++k) {
    const int gx = min(b[0] + 2 * (k & 1), s.n - 1), gy = min(b[1] + ((k >> 1) & 1) * 2, s.n - 1),
              gz = min(b[2] + (k >> 2) * 2, s.n - 1);
    if (gx < 0 || gy < 0 || gz < 0) continue;
    s.active_flag[a][((uint32_t)(gz >> 3) * (uint32_t)s.nb + (uint32_t)(gy >> 3)) * (uint32_t)s.nb +
                     (uint32_t)(gx >> 3)] = 1u;
  }
}

// The P2G of one step.  FREE: a step without a sort (free-zone policy), with
// the paths for particles outside their chunk's bin; the per-step-sort
// instance has none of that code.
template <int MAT, bool HAS_E, bool FREE>
__device__ __forceinline__ void p2g_step(const SimDev &s, int src, int acc, P2GShared &sm, uint32_t *order,
                                         uint8_t *ordtag) {
  const PBuf in = s.buf[src], out = s.buf[src ^ 1];
  const int lane = threadIdx.x;
  const uint32_t Np = (uint32_t)s.Np;  // Np < 2^29: component offsets k Np (k < 9) are exact in 32 bits
  // Workgroup b runs on XCD b % 8 and takes every (grid/8)-th chunk of that
  // XCD's contiguous (Morton-ordered, so spatially compact) share of the
  // chunk list.  Static assignment: no contended atomics on a work queue.
  const uint32_t q = blockIdx.x & (NQ - 1), wq = blockIdx.x / NQ, nwq = gridDim.x / NQ;
  const uint32_t nch = s.ctr[CTR_NCHUNKS + (src ^ 1)];
  const uint4 *chunks = s.chunks[src ^ 1];  // the layout this step builds
  const uint32_t qbeg = (uint32_t)(((uint64_t)nch * q) / NQ), qend = (uint32_t)(((uint64_t)nch * (q + 1)) / NQ);
  const bool pending = s.ctr[CTR_PENDING] != 0u;
  // Without a sort this step (free-zone policy), the layout is the previous
  // one: each slot is its own source, its cell comes from the key G2P wrote,
  // and a particle whose key names another bin is outside the chunk's window
  // (a mover: deposited with direct global atomics).
  constexpr bool sorted = !FREE;
  const float dt = s.dt, mass = s.mass, fn = s.fn, dx = s.dx;

  // A chunk's sorted source indices and cells are loaded one chunk ahead,
  // during the previous chunk's pass B, so pass A starts with them in
  // registers (lanes past the count get an invalid source and cell 0).  The
  // raw values are kept: clamping them here would wait for the loads.
  uint32_t pf_src[KMAX / 64], pf_cell[KMAX / 64];
  auto prefetch = [&](const uint4 &chrec) {
    const uint32_t pstart = chrec.x, pcount = min(chrec.y, (uint32_t)KMAX);
#pragma unroll
    for (int j = 0; j < KMAX / 64; ++j) {
      const uint32_t qi = (uint32_t)(64 * j + lane);
      pf_src[j] = 0xFFFFFFFFu;
      pf_cell[j] = 0u;
      if (qi < pcount) {
        if (sorted) {
          pf_src[j] = s.perm[pstart + qi];
          pf_cell[j] = s.cellp[pstart + qi];
        } else {
          pf_src[j] = pstart + qi;
          pf_cell[j] = s.key[pstart + qi];  // the whole key: bin and cell
        }
      }
    }
  };
  clear_accumulator(s, (acc + 2) & (NACC - 1));
  uint4 ch_next = make_uint4(0u, 0u, 0u, 0u);
  if (qbeg + wq < qend) {
    ch_next = chunks[qbeg + wq];
    prefetch(ch_next);
  }
  for (uint32_t c = qbeg + wq; c < qend; c += nwq) {
    const uint4 ch = ch_next;
    const uint32_t start = ch.x, count = min(ch.y, (uint32_t)KMAX), bin = ch.z;
    const int ox0 = (int)compact3(bin) * CB, oy0 = (int)compact3(bin >> 1) * CB, oz0 = (int)compact3(bin >> 2) * CB;  // first base node of the bin = window origin
    const bool has_next = c + nwq < qend;
    if (has_next) ch_next = chunks[c + nwq];

    // Pass A: cell of each particle and its rank within the cell.  Ranks
    // follow the particles' previous storage order (their source index), so
    // the processing order -- which is also the order the new state is
    // stored in -- is stable from step to step and the gathers below run over
    // nearly consecutive addresses.  The chunk is read as KMAX/64 sub-rounds
    // of consecutive slots, each a run of consecutive sources; sub-rounds
    // are ranked in the order of their smallest source.  Lanes with the same
    // cell are matched bit by bit with ballots; the lowest lane of each group
    // records the group's size (leaders have distinct cells: no atomics).
    P2GRankTables &rk = sm.rk;
    const uint64_t below = (1ull << lane) - 1ull;
    // (source index and cell come in sorted order: the scatter carried the
    // cell that G2P computed with the key, so no position gather is needed)
    // (sub-rounds past the chunk's count are skipped with uniform branches)
    const uint32_t nsub = (count + 63u) / 64u;
    // cells[j]: the cell (bits 0-5) and, bit 6, a mover (never in a sorted step)
    uint32_t cells[KMAX / 64], srcs[KMAX / 64], srcmin[KMAX / 64];
    uint32_t nmov = 0;
#pragma unroll
    for (int j = 0; j < KMAX / 64; ++j) {
      const uint32_t kc = pf_cell[j];
      const bool mv = !sorted && (uint32_t)(64 * j + lane) < count && (kc & ((1u << KEY_CELL_SHIFT) - 1u)) != bin;
      cells[j] = ((sorted ? kc : (kc >> KEY_CELL_SHIFT)) & (uint32_t)(CB3 - 1)) | (mv ? (uint32_t)CB3 : 0u);
      if (FREE) nmov += (uint32_t)__popcll(__ballot(mv));
      uint32_t src = (uint32_t)(64 * j + lane) < count ? min(pf_src[j], Np - 1u) : 0xFFFFFFFFu;
      srcs[j] = src;
      srcmin[j] = 0xFFFFFFFFu;
      if ((uint32_t)j >= nsub) continue;
      for (int d = 32; d >= 1; d >>= 1) src = min(src, (uint32_t)__shfl_xor((int)src, d));
      srcmin[j] = src;
      rk.subcnt[j][lane] = 0u;
    }
    __syncthreads();
    uint32_t rin[KMAX / 64];
#pragma unroll
    for (int j = 0; j < KMAX / 64; ++j) {
      rin[j] = 0u;
      if ((uint32_t)j >= nsub) continue;
      const bool v = (uint32_t)(64 * j + lane) < count && (!FREE || cells[j] < (uint32_t)CB3);
      const uint32_t cell = cells[j] & (uint32_t)(CB3 - 1);
      uint64_t peers = __ballot(v);
#pragma unroll
      for (int k = 0; k < 6; ++k) {
        const uint64_t bk = __ballot((cell >> k) & 1u);
        peers &= ((cell >> k) & 1u) ? bk : ~bk;
      }
      rin[j] = (uint32_t)__popcll(peers & below);
      if (v && (peers & below) == 0ull) rk.subcnt[j][cell] = (uint32_t)__popcll(peers);
    }
    __syncthreads();
    uint32_t rank[KMAX / 64];
#pragma unroll
    for (int j = 0; j < KMAX / 64; ++j) {
      rank[j] = 0u;
      if ((uint32_t)j >= nsub) continue;
      uint32_t before = 0u;
#pragma unroll
      for (int k = 0; k < KMAX / 64; ++k) {
        if ((uint32_t)k >= nsub) continue;
        const bool earlier = srcmin[k] < srcmin[j] || (srcmin[k] == srcmin[j] && k < j);
        if (k != j && earlier) before += rk.subcnt[k][cells[j] & (uint32_t)(CB3 - 1)];
      }
      rank[j] = before + rin[j];
    }
    {
      uint32_t total = 0u;
#pragma unroll
      for (int k = 0; k < KMAX / 64; ++k)
        if ((uint32_t)k < nsub) total += rk.subcnt[k][lane];
      rk.hist[lane] = total;
    }
    __syncthreads();
    // Rank tables: rmask[NWIN sr + w] = cells holding a particle of rank
    // NWIN sr + w (lane = cell), rstart[sr] = position of the first particle
    // of super-rank sr.
    {
      const uint32_t cnt = rk.hist[lane];
      uint32_t mx = cnt;
      for (int d = 32; d >= 1; d >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, d));
      uint32_t run = 0;
      for (uint32_t sr = 0; NWIN * sr < mx; ++sr) {
        uint32_t here = 0;
#pragma unroll
        for (int w = 0; w < NWIN; ++w) {
          const uint64_t m = __ballot(cnt > NWIN * sr + w);
          if (lane == 0) rk.rmask[NWIN * sr + w] = m;
          here += (uint32_t)__popcll(m);
        }
        if (lane == 0) rk.rstart[sr] = run;
        run += here;
      }
    }
    __syncthreads();
    uint32_t mbefore = count - nmov;  // movers go after the ranked particles
#pragma unroll
    for (int j = 0; j < KMAX / 64; ++j) {
      const uint32_t qi = (uint32_t)(64 * j + lane);
      const uint64_t mmask = FREE ? __ballot(cells[j] >= (uint32_t)CB3) : 0ull;
      if ((uint32_t)j < nsub && qi < count) {
        if (FREE && cells[j] >= (uint32_t)CB3) {
          const uint32_t pos = min(mbefore + (uint32_t)__popcll(mmask & below), (uint32_t)KMAX - 1u);
          order[pos] = srcs[j];
          ordtag[pos] = MOVER_TAG;
        } else {
          const uint32_t cell = cells[j], sr = rank[j] / NWIN, w = rank[j] % NWIN;
          uint32_t pos = rk.rstart[sr] + (uint32_t)__popcll(rk.rmask[NWIN * sr + w] & ((1ull << cell) - 1ull));
          for (uint32_t w2 = 0; w2 < w; ++w2) pos += (uint32_t)__popcll(rk.rmask[NWIN * sr + w2]);
          pos = min(pos, (uint32_t)KMAX - 1u);
          order[pos] = srcs[j];
          ordtag[pos] = (uint8_t)(sr * NWIN + w);
        }
      }
      mbefore += (uint32_t)__popcll(mmask);
    }
    __syncthreads();
    // the tables are dead: clear the windows
    for (int k = lane; k < NWIN * PW3; k += 64) sm.win[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();

    if (has_next) prefetch(ch_next);

    // Pass B: rounds of 64 particles in (super-rank, window, cell) order.
    for (uint32_t r0 = 0; r0 < count; r0 += 64) {
      const uint32_t pos = r0 + (uint32_t)lane;
      const bool valid = pos < count;
      const uint32_t at = min(pos, count - 1u);
      const uint32_t i = order[at];
      const uint32_t tag = ordtag[at];
      // The new state is stored in this processing order, (bin, super-rank,
      // window, cell): the next step's gathers then run over nearly
      // consecutive addresses.  P2G writes x and id there; G2P reads x from
      // the same slot, without an index indirection, and overwrites it with
      // the advected position.
      const uint32_t dst = start + at;
      const uint32_t io = 4u * i, od = 4u * dst;  // byte offsets of the source and destination slots
      float xp[3], vp[3], Cp[9];
#pragma unroll
      for (int a = 0; a < 3; ++a) {
        xp[a] = at_byte(in.x + a * Np, io);
        vp[a] = at_byte(in.v + a * Np, io);
      }
#pragma unroll
      for (int k = 0; k < 9; ++k) Cp[k] = stream_load(at_byte(in.C + k * Np, io));
      if (valid) {
#pragma unroll
        for (int a = 0; a < 3; ++a) at_byte(out.x + a * Np, od) = xp[a];
        stream_store(at_byte(in.id, io), at_byte(out.id, od));
      }

      // Deferred deformation-gradient update, stress, APIC momentum.
      float Fp[MAT == MPM_J_FLUID ? 1 : 9];
#pragma unroll
      for (int k = 0; k < (MAT == MPM_J_FLUID ? 1 : 9); ++k) Fp[k] = stream_load(at_byte(in.F + k * Np, io));
      if (pending) update_F<MAT>(Fp, Cp, dt);
      const float E = HAS_E ? at_byte(in.E, io) : s.E;
      float A[9];
      uint32_t st = 0;
      // sand: the plasticity projection of the updated F, with the stress
      if (MAT == MPM_SAND) st = sand_affine(s, Fp, E, Cp, A, pending);
      if (valid) {
#pragma unroll
        for (int k = 0; k < (MAT == MPM_J_FLUID ? 1 : 9); ++k) stream_store(Fp[k], at_byte(out.F + k * Np, od));
        if (HAS_E) stream_store(E, at_byte(out.E, od));
      }
      if (MAT != MPM_SAND) st = affine_momentum<MAT>(s, Fp, E, Cp, A);
      if (st && valid) flag_status(s, st, (st & MPM_STATUS_INVERTED) ? 2 : 0);
      int b[3];
      float f[3], w[3][3], q0[3], Ad[9];
      particle_weights(xp, fn, b, f, w);
      momentum_terms(mass, dx, vp, A, f, q0, Ad);
      const int lx = min(max(b[0] - ox0, 0), CB - 1), ly = min(max(b[1] - oy0, 0), CB - 1),
                lz = min(max(b[2] - oz0, 0), CB - 1);
      const int li0 = (int)(tag % NWIN) * PW3 + (lz * PW + ly) * PW + lx;

      // Passes: lanes conflict only when they share (window, cell).  The
      // lane's pass is its occurrence index among the earlier lanes of the
      // round with the same (window, cell) (ballot-matched, 7 bits), which
      // gives the fewest conflict-free passes; lanes of one super-rank never
      // share (window, cell), so this is at most one pass per super-rank.
      // (a mover's stencil is outside the window: it takes no pass)
      const bool mov = FREE && tag == MOVER_TAG;
      const bool inwin = valid && !mov;
      uint32_t pass_id;
      {
        const uint32_t wc = (tag % NWIN) * (uint32_t)CB3 + (uint32_t)((lz * CB + ly) * CB + lx);
        uint64_t peers = __ballot(inwin);
#pragma unroll
        for (int k = 0; k < 7; ++k) {
          const uint64_t bk = __ballot((wc >> k) & 1u);
          peers &= ((wc >> k) & 1u) ? bk : ~bk;
        }
        pass_id = (uint32_t)__popcll(peers & ((1ull << lane) - 1ull));
      }
      // A mover (only in a step without a sort; rare) deposits directly.
      if (FREE && valid && mov) deposit_global(s, acc, b, w, q0, Ad);
      bool todo = inwin;
      for (uint32_t pnow = 0;; ++pnow) {
        // (occurrence indices of a key are 0, 1, ..., so no lane waits for a
        // pass after an empty one)
        if (__ballot(todo && pass_id == pnow) == 0ull) break;
        if (todo && pass_id == pnow) {
          deposit_window(sm.win, li0, w, q0, Ad, mass);
          todo = false;
        }
      }
    }
    __syncthreads();
    flush_windows(s, sm.win, ox0, oy0, oz0, acc);
    __syncthreads();
  }
}

template <int MAT, bool HAS_E>
__global__ __launch_bounds__(64) void k_p2g(SimDev s, int src, int acc) {
  __shared__ P2GShared sm;
  __shared__ uint32_t order[KMAX];  // source index of each processing position
  __shared__ uint8_t ordtag[KMAX];  // super-rank * NWIN + window of each position (or MOVER_TAG)
  if (s.ctr[CTR_LOOK + src] != 0u) return;  // done by the fused kernel of the step before
  if (s.ctr[CTR_SORT + src] != 0u) p2g_step<MAT, HAS_E, false>(s, src, acc, sm, order, ordtag);
  else p2g_step<MAT, HAS_E, true>(s, src, acc, sm, order, ordtag);
}

// The grid update -- v = p/m + dt g where m > 0, sticky walls -- is
// evaluated by G2P on its window nodes as it loads them (grid_velocity), and
// the accumulator is cleared by the next step's P2G, so the step needs no
// separate pass over the grid.
__device__ __forceinline__ float4 grid_velocity(const SimDev &s, float4 acc, int gx, int gy, int gz) {
  const int n = s.n, wall = s.wall;
  float4 o = make_float4(0.f, 0.f, 0.f, acc.x);
  const bool in_wall = gx < wall || gy < wall || gz < wall || gx >= n - wall || gy >= n - wall || gz >= n - wall;
  if (acc.x > 0.f && !in_wall) {
    // one division per node (G2P evaluates each node once per window that
    // covers it): p (1/m) is within an ulp of p/m
    const float inv = 1.f / acc.x;
    o.x = acc.y * inv + s.dt * s.g[0];
    o.y = acc.z * inv + s.dt * s.g[1];
    o.z = acc.w * inv + s.dt * s.g[2];
  }
  return o;
}

// G2P: gather, APIC C, advection and clamp.  Persistent single-wavefront
// workgroups walk the same per-XCD chunk list as P2G.  A chunk's particles
// occupy the consecutive slots [start, start + count) (P2G stored them
// there), and all of their stencils lie in the bin's 6^3-node window, which
// is loaded once into LDS; each particle then gathers its 27 nodes from LDS.

// Window load in whole cubes (one 128-byte line each): lane = (cube, node in
// cube), 8 cubes per load instruction, 4 instructions.  This lane's window
// node of instruction t, packed wx | wy << 8 | wz << 16 (all ones when cube
// 8t + lane / 8 is past the 27th).
__device__ __forceinline__ void window_lanes(uint32_t wpack[4]) {
  const int lane = threadIdx.x;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int cb = 8 * t + (lane >> 3), j = lane & 7;
    const int wx = 2 * (cb % 3) + (j & 1), wy = 2 * ((cb / 3) % 3) + ((j >> 1) & 1), wz = 2 * (cb / 9) + (j >> 2);
    wpack[t] = cb < 27 ? (uint32_t)(wx | (wy << 8) | (wz << 16)) : 0xFFFFFFFFu;
  }
}

// Requests the accumulator values (m, p) of the window at (ox0, oy0, oz0)
// from accumulator a; nodes outside the grid read as zero.
__device__ __forceinline__ void fetch_window(const SimDev &s, int a, int ox0, int oy0, int oz0, const uint32_t wpack[4],
                                             float4 acc[4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    acc[t] = make_float4(0.f, 0.f, 0.f, 0.f);
    const int gx = ox0 + (int)(wpack[t] & 0xFFu), gy = oy0 + (int)((wpack[t] >> 8) & 0xFFu),
              gz = oz0 + (int)((wpack[t] >> 16) & 0xFFu);
    if (wpack[t] != 0xFFFFFFFFu && gx < s.n && gy < s.n && gz < s.n) acc[t] = s.gridA[a][node_index(s, gx, gy, gz)];
  }
}

// Converts fetched window values to grid velocities (the grid update) in LDS.
__device__ __forceinline__ void store_window(const SimDev &s, const float4 acc[4], const uint32_t wpack[4], int ox0,
                                             int oy0, int oz0, float4 *win) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (wpack[t] == 0xFFFFFFFFu) continue;
    const int wx = (int)(wpack[t] & 0xFFu), wy = (int)((wpack[t] >> 8) & 0xFFu), wz = (int)((wpack[t] >> 16) & 0xFFu);
    const int gx = ox0 + wx, gy = oy0 + wy, gz = oz0 + wz;
    win[(wz * PW + wy) * PW + wx] =
        (gx < s.n && gy < s.n && gz < s.n) ? grid_velocity(s, acc[t], gx, gy, gz) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// Gather of one particle at xp: v = sum w v_i and B = sum w v_i (o - f)^T
// (C = 4/dx^2 B dx, applied by the caller), from the velocity window of the
// bin at (ox0, oy0, oz0), or from accumulator a with the grid update for a
// particle whose stencil is outside the window (it left the chunk's bin
// since the last sort: only in steps without a sort; rare).
__device__ __forceinline__ void gather_particle(const SimDev &s, const float4 *win, int a, const float xp[3], int ox0,
                                                int oy0, int oz0, float v[3], float B[9]) {
  int b[3];
  float w[3][3], d[3][3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const float xn = xp[k] * s.fn;
    b[k] = base_node(xn);
    const float f = xn - (float)b[k];
    bspline_weights(f, w[k]);
    d[k][0] = -f;
    d[k][1] = 1.f - f;
    d[k][2] = 2.f - f;
  }
  const bool outside = b[0] - ox0 < 0 || b[0] - ox0 >= CB || b[1] - oy0 < 0 || b[1] - oy0 >= CB || b[2] - oz0 < 0 ||
                       b[2] - oz0 >= CB;
  const int lx = min(max(b[0] - ox0, 0), CB - 1), ly = min(max(b[1] - oy0, 0), CB - 1),
            lz = min(max(b[2] - oz0, 0), CB - 1);
  const int li0 = (lz * PW + ly) * PW + lx;
  // The quadratic B-spline's first moment sum_o w_o (o - f) = 0 gives the
  // columns of B as B_a = sum w o_a v_i - f_a v.  Reduced along x first for
  // each (y, z) row: S = sum_x w_x v_i and U = sum_x w_x ox v_i; offsets
  // equal to zero add nothing, so rows with oy = 0 (oz = 0) skip the y (z)
  // column.
  const float w2x = 2.f * w[0][2];
#pragma unroll
  for (int k = 0; k < 3; ++k) v[k] = 0.f;
#pragma unroll
  for (int k = 0; k < 9; ++k) B[k] = 0.f;
  if (outside) {
    // node rows of three, their loads issued together
#pragma unroll 1
    for (int r = 0; r < 9; ++r) {
      const int oy = r % 3, oz = r / 3;
      const int gy = b[1] + oy, gz = b[2] + oz;
      float4 acc[3];
#pragma unroll
      for (int ox = 0; ox < 3; ++ox) {
        const int gx = b[0] + ox;
        acc[ox] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (gx >= 0 && gy >= 0 && gz >= 0 && gx < s.n && gy < s.n && gz < s.n)
          acc[ox] = s.gridA[a][node_index(s, gx, gy, gz)];
      }
#pragma unroll
      for (int ox = 0; ox < 3; ++ox) {
        const float4 g = grid_velocity(s, acc[ox], b[0] + ox, gy, gz);
        const float wt = w[0][ox] * w[1][oy] * w[2][oz];
        const float vel[3] = {g.x, g.y, g.z};
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          v[k] = fmaf(wt, vel[k], v[k]);
          B[k * 3 + 0] = fmaf(wt * (float)ox, vel[k], B[k * 3 + 0]);
          B[k * 3 + 1] = fmaf(wt * (float)oy, vel[k], B[k * 3 + 1]);
          B[k * 3 + 2] = fmaf(wt * (float)oz, vel[k], B[k * 3 + 2]);
        }
      }
    }
  } else {
#pragma unroll
    for (int oz = 0; oz < 3; ++oz)
#pragma unroll
      for (int oy = 0; oy < 3; ++oy) {
        float S[3], U[3];
        const float4 g0 = win[li0 + (oz * PW + oy) * PW + 0];
        const float4 g1 = win[li0 + (oz * PW + oy) * PW + 1];
        const float4 g2 = win[li0 + (oz * PW + oy) * PW + 2];
        S[0] = w[0][0] * g0.x;
        S[1] = w[0][0] * g0.y;
        S[2] = w[0][0] * g0.z;
        U[0] = w[0][1] * g1.x;
        U[1] = w[0][1] * g1.y;
        U[2] = w[0][1] * g1.z;
        S[0] = fmaf(w[0][1], g1.x, S[0]);
        S[1] = fmaf(w[0][1], g1.y, S[1]);
        S[2] = fmaf(w[0][1], g1.z, S[2]);
        S[0] = fmaf(w[0][2], g2.x, S[0]);
        S[1] = fmaf(w[0][2], g2.y, S[1]);
        S[2] = fmaf(w[0][2], g2.z, S[2]);
        U[0] = fmaf(w2x, g2.x, U[0]);
        U[1] = fmaf(w2x, g2.y, U[1]);
        U[2] = fmaf(w2x, g2.z, U[2]);
        const float wyz = w[1][oy] * w[2][oz];
        const float wyz2 = wyz + wyz;
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          v[k] = fmaf(wyz, S[k], v[k]);
          B[k * 3 + 0] = fmaf(wyz, U[k], B[k * 3 + 0]);
          if (oy > 0) B[k * 3 + 1] = fmaf(oy == 1 ? wyz : wyz2, S[k], B[k * 3 + 1]);
          if (oz > 0) B[k * 3 + 2] = fmaf(oz == 1 ? wyz : wyz2, S[k], B[k * 3 + 2]);
        }
      }
  }
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int c2 = 0; c2 < 3; ++c2) B[k * 3 + c2] = fmaf(d[c2][0], v[k], B[k * 3 + c2]);  // d[c2][0] = -f_c2
}

// Advection x + dt v, clamped to the box; status bits for a clamp or a
// non-finite value (of x, v or C = c_scale B, which the caller stores).
__device__ __forceinline__ void advect(const SimDev &s, const float xp[3], const float v[3], const float B[9],
                                       float xn[3], float C[9], bool &clamped, bool &nonfinite) {
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    float xa = xp[k] + s.dt * v[k];
    if (!isfinite(xa) || !isfinite(v[k])) nonfinite = true;
    if (xa < s.lo || xa > s.hi) clamped = true;
    xn[k] = fminf(fmaxf(xa, s.lo), s.hi);
  }
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    C[k] = s.c_scale * B[k];
    if (!isfinite(C[k])) nonfinite = true;
  }
}

// The G2P of the step that accumulated into a: particles of layout lay (the
// one P2G built), x, v, C written in place, and the next step's bin keys and
// counts.
template <int MAT>
__device__ __forceinline__ void g2p_step(const SimDev &s, int lay, int a, float4 *win) {
  const PBuf out = s.buf[lay];
  const int lane = threadIdx.x;
  const uint32_t Np = (uint32_t)s.Np;  // Np < 2^29: component offsets k Np (k < 9) are exact in 32 bits
  const float fn = s.fn;
  const uint32_t q = blockIdx.x & (NQ - 1), wq = blockIdx.x / NQ, nwq = gridDim.x / NQ;
  const uint32_t nch = s.ctr[CTR_NCHUNKS + lay];
  uint4 *chunks = s.chunks[lay];
  const uint32_t qbeg = (uint32_t)(((uint64_t)nch * q) / NQ), qend = (uint32_t)(((uint64_t)nch * (q + 1)) / NQ);
  uint32_t wpack[4];
  window_lanes(wpack);
  for (uint32_t c = qbeg + wq; c < qend; c += nwq) {
    const uint4 ch = chunks[c];
    const uint32_t start = ch.x, count = min(ch.y, (uint32_t)KMAX), bin = ch.z;
    const int ox0 = (int)compact3(bin) * CB, oy0 = (int)compact3(bin >> 1) * CB, oz0 = (int)compact3(bin >> 2) * CB;
    // The window's accumulator values and the first round's positions are
    // requested together, then the window is converted to velocities (the
    // grid update) in LDS.
    float4 acc[4];
    fetch_window(s, a, ox0, oy0, oz0, wpack, acc);
    float xnext[3] = {0.f, 0.f, 0.f};  // positions of the next round, written by this step's P2G in this order
    if ((uint32_t)lane < count) {
#pragma unroll
      for (int k = 0; k < 3; ++k) xnext[k] = at_byte(out.x + k * Np, 4u * (start + (uint32_t)lane));
    }
    store_window(s, acc, wpack, ox0, oy0, oz0, win);
    __syncthreads();
    uint32_t nstay = 0;
    for (uint32_t r0 = 0; r0 < count; r0 += 64) {
      const uint32_t slot = start + r0 + (uint32_t)lane, so = 4u * slot;
      const bool valid = r0 + (uint32_t)lane < count;
      float xp[3] = {xnext[0], xnext[1], xnext[2]};
      if (r0 + 64u < count && r0 + 64u + (uint32_t)lane < count) {
#pragma unroll
        for (int k = 0; k < 3; ++k) xnext[k] = at_byte(out.x + k * Np, so + 256u);
      }
      uint32_t key = 0;
      if (valid) {
        float v[3], B[9], xn[3], Cn[9];
        gather_particle(s, win, a, xp, ox0, oy0, oz0, v, B);
        bool clamped = false, nonfinite = false;
        advect(s, xp, v, B, xn, Cn, clamped, nonfinite);
        int b[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          stream_store(xn[k], at_byte(out.x + k * Np, so));
          stream_store(v[k], at_byte(out.v + k * Np, so));
          b[k] = base_node(xn[k] * fn);
        }
#pragma unroll
        for (int k = 0; k < 9; ++k) stream_store(Cn[k], at_byte(out.C + k * Np, so));
        // the next bin: nearly always the chunk's own (Morton encoding only
        // when some lane of the wavefront left it)
        const bool same_bin = (b[0] >> 2) == (ox0 >> 2) && (b[1] >> 2) == (oy0 >> 2) && (b[2] >> 2) == (oz0 >> 2);
        key = (__ballot(!same_bin) == 0ull) ? bin : bin_key(s, b[0], b[1], b[2]);
        at_byte(s.key, so) = key | (cell_in_bin(b[0], b[1], b[2]) << KEY_CELL_SHIFT);
        if (clamped) flag_status(s, MPM_STATUS_CLAMPED, 1);
        if (nonfinite) flag_status(s, MPM_STATUS_NONFINITE, 3);
      }
      wave_aggregated_increment(s.bin_count, key, valid);
      nstay += (uint32_t)__popcll(__ballot(valid && key == bin));
    }
    // The chunk's particles that stay in its bin: the next scatter keeps them
    // in this order, after the stayers of the bin's earlier chunks.
    if (lane == 0) {
      chunks[c].w = nstay;
      if (nstay) atomicAdd(s.stay_count + bin, nstay);
      if (nstay < count) atomicAdd(s.ctr + CTR_MOVERS, count - nstay);  // for the next sort decision
    }
    __syncthreads();  // the window is reloaded for the next chunk
  }
}

// The control words a G2P leaves for the next step (that reads buffer lay):
// F is one update behind, and that step's P2G and sort decision are its own.
__device__ __forceinline__ void g2p_handoff(const SimDev &s, int lay) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    s.ctr[CTR_PENDING] = 1u;
    s.ctr[CTR_LOOK + lay] = 0u;
    s.ctr[CTR_PRESET + lay] = 0u;
  }
}

// G2P of a step that reads buffer src (accumulator a): writes x, v, C in
// place in layout src ^ 1 and the next step's bin keys and counts.
template <int MAT>
__global__ __launch_bounds__(64) void k_g2p(SimDev s, int src, int a) {
  __shared__ float4 win[PW3];
  g2p_step<MAT>(s, src ^ 1, a, win);
  g2p_handoff(s, src ^ 1);
}

// Fused G2P2G ([RT-MPM], the fused-kernel variant of the step: the G2P of
// one step and the P2G of the next in one pass over the particles).  In a
// step without a sort the next P2G needs no new order, so each chunk's
// particles go from the G2P straight into the next step's deposit, and the
// state carried from step to step is only x, F (or J), E and the ids:
// velocity and C stay in registers (they are stored for readback only when
// the launch asks for it).  Runs only when the next step does not sort (the
// decision is taken here, on the movers the previous step counted); before
// a sort it runs the plain G2P, which writes the keys the sort needs.
struct FusedShared {
  float4 vel[PW3];          // the step's grid velocities around the bin
  float4 win[NWIN * PW3];   // the next step's accumulation windows
};

// Step n reads buffer src, accumulated into a, and its G2P works on layout
// lay = src ^ 1.  The P2G of step n + 1 reads the particles there and writes
// them to the same slots of buffer src (the layout of step n + 1 repeats
// layout lay), accumulating into a + 1.  Particles are processed in their
// storage order, which the last sort's P2G chose ((super-rank, window,
// cell) within each chunk) and which changes little between sorts: a lane's
// window and pass follow from its occurrence index among the lanes of its
// round in the same cell.
template <int MAT, bool HAS_E>
__device__ __forceinline__ void fused_step(const SimDev &s, int src, int a, bool write_vc, FusedShared &sm) {
  const int lay = src ^ 1;
  const PBuf in = s.buf[lay], out = s.buf[src];
  const int a1 = (a + 1) & (NACC - 1);
  const int lane = threadIdx.x;
  const uint64_t below = (1ull << lane) - 1ull;
  const uint32_t Np = (uint32_t)s.Np;  // Np < 2^29: component offsets k Np (k < 9) are exact in 32 bits
  const float dt = s.dt, mass = s.mass, fn = s.fn, dx = s.dx;
  const uint32_t q = blockIdx.x & (NQ - 1), wq = blockIdx.x / NQ, nwq = gridDim.x / NQ;
  const uint32_t nch = s.ctr[CTR_NCHUNKS + lay];
  const uint4 *chunks = s.chunks[lay];
  const uint32_t qbeg = (uint32_t)(((uint64_t)nch * q) / NQ), qend = (uint32_t)(((uint64_t)nch * (q + 1)) / NQ);
  constexpr int FW = MAT == MPM_J_FLUID ? 1 : 9;
  clear_accumulator(s, (a1 + 2) & (NACC - 1));
  uint32_t wpack[4];
  window_lanes(wpack);
  // The next step's layout repeats this one: its chunk list is this list
  // (copied here, for a next step that runs no scan).
  if (blockIdx.x == 0 && lane == 0) s.ctr[CTR_NCHUNKS + src] = nch;
  uint4 ch_next = make_uint4(0u, 0u, 0u, 0u);  // chunk records are loaded one chunk ahead
  if (qbeg + wq < qend) ch_next = chunks[qbeg + wq];
  for (uint32_t c = qbeg + wq; c < qend; c += nwq) {
    const uint4 ch = ch_next;
    if (c + nwq < qend) ch_next = chunks[c + nwq];
    if (lane == 0) s.chunks[src][c] = ch;
    const uint32_t start = ch.x, count = min(ch.y, (uint32_t)KMAX), bin = ch.z;
    const int ox0 = (int)compact3(bin) * CB, oy0 = (int)compact3(bin >> 1) * CB, oz0 = (int)compact3(bin >> 2) * CB;
    // the window and the first round's x, F, E and ids are requested
    // together; later rounds are loaded one round ahead
    float4 acc[4];
    fetch_window(s, a, ox0, oy0, oz0, wpack, acc);
    float xq[3], Fq[FW], Eq = s.E;
    uint32_t idq;
    {
      const uint32_t sn = 4u * (start + ((uint32_t)lane < count ? (uint32_t)lane : 0u));
#pragma unroll
      for (int k = 0; k < 3; ++k) xq[k] = at_byte(in.x + k * Np, sn);
#pragma unroll
      for (int k = 0; k < FW; ++k) Fq[k] = stream_load(at_byte(in.F + k * Np, sn));
      if (HAS_E) Eq = stream_load(at_byte(in.E, sn));
      idq = stream_load(at_byte(in.id, sn));
    }
    for (int k = lane; k < NWIN * PW3; k += 64) sm.win[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    store_window(s, acc, wpack, ox0, oy0, oz0, sm.vel);
    __syncthreads();
    uint32_t nmov = 0;
    for (uint32_t r0 = 0; r0 < count; r0 += 64) {
      const bool valid = r0 + (uint32_t)lane < count;
      // lanes past the count read the chunk's first particle and store nothing
      const uint32_t so = 4u * (start + (valid ? r0 + (uint32_t)lane : 0u));
      float xp[3] = {xq[0], xq[1], xq[2]}, Fp[FW];
#pragma unroll
      for (int k = 0; k < FW; ++k) Fp[k] = Fq[k];
      const float E = Eq;
      if (valid) stream_store(idq, at_byte(out.id, so));
      if (r0 + 64u < count) {
        const bool vn = r0 + 64u + (uint32_t)lane < count;
        const uint32_t sn = 4u * (start + (vn ? r0 + 64u + (uint32_t)lane : 0u));
#pragma unroll
        for (int k = 0; k < 3; ++k) xq[k] = at_byte(in.x + k * Np, sn);
#pragma unroll
        for (int k = 0; k < FW; ++k) Fq[k] = stream_load(at_byte(in.F + k * Np, sn));
        if (HAS_E) Eq = stream_load(at_byte(in.E, sn));
        idq = stream_load(at_byte(in.id, sn));
      }
      float v[3], B[9], xn[3], Cn[9];
      gather_particle(s, sm.vel, a, xp, ox0, oy0, oz0, v, B);
      bool clamped = false, nonfinite = false;
      advect(s, xp, v, B, xn, Cn, clamped, nonfinite);
      // P2G of step n + 1: F update with the new C, stress, deposit at xn
      update_F<MAT>(Fp, Cn, dt);
      float A[9];
      uint32_t st = 0;
      if (MAT == MPM_SAND) st = sand_affine(s, Fp, E, Cn, A, true);  // projection and stress
      if (valid) {
#pragma unroll
        for (int k = 0; k < 3; ++k) at_byte(out.x + k * Np, so) = xn[k];
#pragma unroll
        for (int k = 0; k < FW; ++k) stream_store(Fp[k], at_byte(out.F + k * Np, so));
        if (HAS_E) stream_store(E, at_byte(out.E, so));
        if (write_vc) {
#pragma unroll
          for (int k = 0; k < 3; ++k) stream_store(v[k], at_byte(out.v + k * Np, so));
#pragma unroll
          for (int k = 0; k < 9; ++k) stream_store(Cn[k], at_byte(out.C + k * Np, so));
        }
        if (clamped) flag_status(s, MPM_STATUS_CLAMPED, 1);
        if (nonfinite) flag_status(s, MPM_STATUS_NONFINITE, 3);
      }
      if (MAT != MPM_SAND) st = affine_momentum<MAT>(s, Fp, E, Cn, A);
      if (st && valid) flag_status(s, st, (st & MPM_STATUS_INVERTED) ? 2 : 0);
      int b[3];
      float f[3], w[3][3], q0[3], Ad[9];
      particle_weights(xn, fn, b, f, w);
      momentum_terms(mass, dx, v, A, f, q0, Ad);
      // A particle whose new base node left the chunk's bin deposits directly
      // (and counts toward the sort decision).
      const bool mov = valid && (b[0] - ox0 < 0 || b[0] - ox0 >= CB || b[1] - oy0 < 0 || b[1] - oy0 >= CB ||
                                 b[2] - oz0 < 0 || b[2] - oz0 >= CB);
      nmov += (uint32_t)__popcll(__ballot(mov));
      if (mov) deposit_global(s, a1, b, w, q0, Ad);
      const bool inwin = valid && !mov;
      const int lx = min(max(b[0] - ox0, 0), CB - 1), ly = min(max(b[1] - oy0, 0), CB - 1),
                lz = min(max(b[2] - oz0, 0), CB - 1);
      // occurrence index among the earlier lanes of the round in the same
      // cell (ballot-matched, 6 bits): window = occ % NWIN, pass = occ / NWIN,
      // so lanes of one pass never share (window, cell)
      uint32_t occ;
      {
        const uint32_t cell = (uint32_t)((lz * CB + ly) * CB + lx);
        uint64_t peers = __ballot(inwin);
#pragma unroll
        for (int k = 0; k < 6; ++k) {
          const uint64_t bk = __ballot((cell >> k) & 1u);
          peers &= ((cell >> k) & 1u) ? bk : ~bk;
        }
        occ = (uint32_t)__popcll(peers & below);
      }
      const uint32_t pass_id = occ / NWIN;
      const int li0 = (int)(occ % NWIN) * PW3 + (lz * PW + ly) * PW + lx;
      bool todo = inwin;
      for (uint32_t pnow = 0;; ++pnow) {
        if (__ballot(todo && pass_id == pnow) == 0ull) break;
        if (todo && pass_id == pnow) {
          deposit_window(sm.win, li0, w, q0, Ad, mass);
          todo = false;
        }
      }
    }
    __syncthreads();
    flush_windows(s, sm.win, ox0, oy0, oz0, a1);
    if (lane == 0 && nmov) atomicAdd(s.ctr + CTR_MOVERS, nmov);  // for the sort decision two steps on
    __syncthreads();  // the windows are cleared for the next chunk
  }
}

// Step n reads buffer src and accumulated into a; write_vc: store v and C
// (the last step of a launch, so that the state can be read back); sched:
// whether the next step sorts, 0 or 1 when the host schedules the sorts
// (a fixed interval), -1 to decide here by the policy.  Leaves the next
// step's sort decision and whether its P2G is done.
template <int MAT, bool HAS_E>
__global__ __launch_bounds__(64) void k_g2p2g(SimDev s, int src, int a, int write_vc, int sched) {
  __shared__ FusedShared sm;
  // uniform: the words sort_next_step reads do not change in this kernel
  const bool next_sort = sched < 0 ? sort_next_step(s) : sched != 0;
  if (next_sort) g2p_step<MAT>(s, src ^ 1, a, sm.vel);
  else fused_step<MAT, HAS_E>(s, src, a, write_vc != 0, sm);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    // F in layout src ^ 1 is one update behind after the plain G2P; after the
    // fused pass the state of the next step's P2G is in buffer src, current.
    s.ctr[CTR_PENDING] = 1u;
    s.ctr[CTR_LOOK + (src ^ 1)] = next_sort ? 0u : 1u;
    s.ctr[CTR_PRESET + (src ^ 1)] = 1u;
    s.ctr[CTR_SORT + (src ^ 1)] = next_sort ? 1u : 0u;
  }
}

// Readback: unpermute to creation order, apply the pending F (or J) update.
// Single-wavefront workgroups walk the chunk list of layout cur (the slots
// between bins are padding).  After a fused G2P2G pass the state is in the
// same slots of the other buffer, with F current.
template <int MAT>
__global__ __launch_bounds__(64) void k_read_particles(SimDev s, int cur, float *__restrict__ x, float *__restrict__ v,
                                                       float *__restrict__ C, float *__restrict__ F) {
  const bool fused = s.ctr[CTR_LOOK + cur] != 0u;
  const PBuf b = s.buf[fused ? cur ^ 1 : cur];
  const size_t Np = (size_t)s.Np;
  const bool pending = !fused && s.ctr[CTR_PENDING] != 0u;
  const float dt = s.dt;
  const uint32_t nch = s.ctr[CTR_NCHUNKS + cur];
  for (uint32_t c = blockIdx.x; c < nch; c += gridDim.x) {
    const uint4 ch = s.chunks[cur][c];
    for (uint32_t r = threadIdx.x; r < ch.y; r += 64) {
      const size_t slot = (size_t)ch.x + r;
      if (slot >= Np) break;
      const size_t id = b.id[slot];
      if (id >= (size_t)s.N) continue;
      float Cp[9];
#pragma unroll
      for (int k = 0; k < 9; ++k) Cp[k] = b.C[k * Np + slot];
      for (int a = 0; a < 3; ++a) {
        if (x) x[3 * id + a] = b.x[a * Np + slot];
        if (v) v[3 * id + a] = b.v[a * Np + slot];
      }
      if (C)
        for (int k = 0; k < 9; ++k) C[9 * id + k] = Cp[k];
      if (!F) continue;
      if (MAT == MPM_J_FLUID) {
        float J = b.F[slot];
        if (pending) {
          const float G[9] = {1.f + dt * Cp[0], dt * Cp[1], dt * Cp[2], dt * Cp[3], 1.f + dt * Cp[4],
                              dt * Cp[5], dt * Cp[6], dt * Cp[7], 1.f + dt * Cp[8]};
          J = J * det3(G);
        }
        F[id] = J;
      } else {
        float Fp[9];
        for (int k = 0; k < 9; ++k) Fp[k] = b.F[k * Np + slot];
        if (pending) {
          update_F<MPM_FIXED_COROTATED>(Fp, Cp, dt);
          if (MAT == MPM_SAND) {  // and the plasticity projection that follows the update
            float A[9];
            (void)sand_affine(s, Fp, s.E, Cp, A, true);
          }
        }
        for (int k = 0; k < 9; ++k) F[9 * id + k] = Fp[k];
      }
    }
  }
}

// Readback of the grid after the last step (parity q): the node-blocks it
// marked, updated as G2P saw them (v = p/m + dt g, walls) -> dense
// (i + n (j + n k)) arrays of m and m v.
__global__ __launch_bounds__(WG) void k_read_grid(SimDev s, int q, float *__restrict__ mass, float *__restrict__ mom) {
  const int n = s.n;
  for (uint32_t blk = blockIdx.x; blk < (uint32_t)s.nblk; blk += gridDim.x) {
    if (s.active_flag[q][blk] == 0u) continue;
    const int bx = (int)(blk % (uint32_t)s.nb), by = (int)((blk / (uint32_t)s.nb) % (uint32_t)s.nb),
              bz = (int)(blk / ((uint32_t)s.nb * (uint32_t)s.nb));
    for (int local = threadIdx.x; local < 512; local += WG) {
      int lx, ly, lz;
      block_local_coords(local, lx, ly, lz);
      const int gx = bx * NB + lx, gy = by * NB + ly, gz = bz * NB + lz;
      if (gx >= n || gy >= n || gz >= n) continue;
      const float4 g = grid_velocity(s, s.gridA[q][((size_t)blk << 9) + local], gx, gy, gz);
      const size_t lin = (size_t)gx + (size_t)n * ((size_t)gy + (size_t)n * gz);
      if (mass) mass[lin] = g.w;
      if (mom) {
        mom[3 * lin + 0] = g.w * g.x;
        mom[3 * lin + 1] = g.w * g.y;
        mom[3 * lin + 2] = g.w * g.z;
      }
    }
  }
}

// ------------------------------------------------------------- host side

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

// Slots per particle buffer: N plus the padding of every bin that can hold a
// particle (at most SLOT_ALIGN - 1 each), in whole wavefronts.
int64_t slot_capacity(int64_t N, int nbin) {
  const int64_t bins = (int64_t)nbin * nbin * nbin;
  return ((N + (int64_t)(SLOT_ALIGN - 1) * std::min(N, bins)) + 63) / 64 * 64;
}
constexpr int64_t MAX_SLOTS = int64_t(1) << 29;  // 8 Np < 2^32 (32-bit component offsets)

bool valid_params(const mpm_params *p) {
  if (!p || p->struct_size < sizeof(mpm_params)) return false;
  // grid_n <= 1024: at most 256^3 bins, so a bin index fits below the cell
  // bits of the key word (KEY_CELL_SHIFT)
  if (p->grid_n < 8 || p->grid_n > 1024) return false;
  if (!(p->dt > 0.f) || !std::isfinite(p->dt)) return false;
  for (int a = 0; a < 3; ++a)
    if (!std::isfinite(p->gravity[a])) return false;
  if (p->wall_nodes < 0 || p->wall_nodes > p->grid_n / 2) return false;
  if (p->material != MPM_FIXED_COROTATED && p->material != MPM_J_FLUID && p->material != MPM_SAND) return false;
  if (p->material == MPM_SAND && !(p->friction_deg > 0.f && p->friction_deg < 90.f)) return false;
  if (!(p->E >= 0.f) || !std::isfinite(p->E)) return false;
  if (p->material != MPM_J_FLUID && !(p->nu >= 0.f && p->nu < 0.5f)) return false;
  if (!(p->rho > 0.f) || !std::isfinite(p->rho)) return false;
  if (!(p->p_vol > 0.f) || !std::isfinite(p->p_vol)) return false;
  return true;
}

// Workspace layout; with base == nullptr only the size is computed.
size_t layout(const mpm_params *p, int64_t N, bool has_E, char *base, SimDev *d) {
  const int n = p->grid_n, nb = (n + NB - 1) / NB;
  const int64_t nblk = (int64_t)nb * nb * nb;
  const int nbin = (n + CB - 1) / CB;
  const int64_t Np = slot_capacity(N, nbin);
  int nbin2 = 1;
  while (nbin2 < nbin) nbin2 <<= 1;
  const int64_t nbins = (int64_t)nbin2 * nbin2 * nbin2;
  const int64_t max_chunks = (N + (1 << KMIN_SHIFT) - 1) / (1 << KMIN_SHIFT) + nbins;
  const int fw = p->material == MPM_J_FLUID ? 1 : 9;
  size_t off = 0;
  auto take = [&](size_t bytes) -> char * {
    char *ptr = base ? base + off : nullptr;
    off += align_up(bytes);
    return ptr;
  };
  // The grid first: its placement then does not depend on N or on the other
  // arrays (shifting it by tens of MB measurably changed the grid update).
  float4 *gA[NACC];
  for (int k = 0; k < NACC; ++k) gA[k] = (float4 *)take(sizeof(float4) * (size_t)nblk * 512);
  PBuf bufs[2];
  for (int k = 0; k < 2; ++k) {
    bufs[k].x = (float *)take(sizeof(float) * 3 * Np);
    bufs[k].v = (float *)take(sizeof(float) * 3 * Np);
    bufs[k].C = (float *)take(sizeof(float) * 9 * Np);
    bufs[k].F = (float *)take(sizeof(float) * fw * Np);
    bufs[k].E = has_E ? (float *)take(sizeof(float) * Np) : nullptr;
    bufs[k].id = (uint32_t *)take(sizeof(uint32_t) * Np);
  }
  uint32_t *perm = (uint32_t *)take(sizeof(uint32_t) * Np);
  uint32_t *key = (uint32_t *)take(sizeof(uint32_t) * Np);
  uint32_t *cnt = (uint32_t *)take(sizeof(uint32_t) * nbins);
  uint32_t *stay = (uint32_t *)take(sizeof(uint32_t) * nbins);
  uint32_t *bstart = (uint32_t *)take(sizeof(uint32_t) * nbins);
  uint32_t *bstay = (uint32_t *)take(sizeof(uint32_t) * nbins);
  uint32_t *cur = (uint32_t *)take(sizeof(uint32_t) * nbins);
  const int64_t ntiles = (nbins + SCAN_TILE - 1) / SCAN_TILE;
  uint32_t *tiles = (uint32_t *)take(sizeof(uint32_t) * 2 * ntiles);
  uint32_t *aflag[NACC];
  for (int k = 0; k < NACC; ++k) aflag[k] = (uint32_t *)take(sizeof(uint32_t) * nblk);
  uint4 *chunks0 = (uint4 *)take(sizeof(uint4) * max_chunks);
  uint4 *chunks1 = (uint4 *)take(sizeof(uint4) * max_chunks);
  uint32_t *ctr = (uint32_t *)take(sizeof(uint32_t) * CTR_WORDS);
  uint32_t *status = (uint32_t *)take(sizeof(uint32_t) * MPM_STATUS_WORDS);
  uint8_t *cellp = (uint8_t *)take(Np);
  if (d) {
    d->N = (int32_t)N;
    d->Np = (int32_t)Np;
    d->n = n;
    d->nb = nb;
    d->nblk = (int32_t)nblk;
    d->nbin = nbin;
    d->nbins = (int32_t)nbins;
    d->wall = p->wall_nodes;
    d->material = p->material;
    d->has_E = has_E ? 1 : 0;
    d->dx = 1.0f / (float)n;
    d->fn = (float)n;
    d->dt = p->dt;
    for (int a = 0; a < 3; ++a) d->g[a] = p->gravity[a];
    d->mass = p->rho * p->p_vol;
    d->vol = p->p_vol;
    d->E = p->E;
    const double nu = p->material == MPM_J_FLUID ? 0.0 : (double)p->nu;
    // Fluid: tau = K J (J-1) I uses E as K directly; mu/lam unused.
    d->mu_per_E = (float)(1.0 / (2.0 * (1.0 + nu)));
    d->lam_per_E = (float)(nu / ((1.0 + nu) * (1.0 - 2.0 * nu)));
    // sand (Klar et al. 2016): alpha = sqrt(2/3) 2 sin(phi) / (3 - sin(phi)), and
    // (3 lam + 2 mu) / (2 mu) = (1 + nu) / (1 - 2 nu)
    const double sp = std::sin((double)p->friction_deg * 3.14159265358979323846 / 180.0);
    d->alpha = p->material == MPM_SAND ? (float)(std::sqrt(2.0 / 3.0) * 2.0 * sp / (3.0 - sp)) : 0.f;
    d->dp_c = (float)((1.0 + nu) / (1.0 - 2.0 * nu));
    d->stress_k = (float)((double)p->dt * (double)p->p_vol * 4.0 * (double)n * (double)n);
    d->c_scale = (float)(4.0 * n);
    d->lo = 2.0f * d->dx;
    d->hi = (float)(n - 2) * d->dx;
    d->max_chunks = (uint32_t)max_chunks;
    d->chunk_shift = KMAX_SHIFT;
    d->buf[0] = bufs[0];
    d->buf[1] = bufs[1];
    d->perm = perm;
    d->key = key;
    d->cellp = cellp;
    d->bin_count = cnt;
    d->stay_count = stay;
    d->bin_start = bstart;
    d->bin_stay = bstay;
    d->bin_cursor = cur;
    d->tile_sum = tiles;
    d->ntiles = (int32_t)ntiles;
    for (int k = 0; k < NACC; ++k) d->active_flag[k] = aflag[k];
    d->chunks[0] = chunks0;
    d->chunks[1] = chunks1;
    d->ctr = ctr;
    d->status = status;
    for (int k = 0; k < NACC; ++k) d->gridA[k] = gA[k];
  }
  return off;
}

const char *const KERNEL_NAMES[NUM_KERNELS] = {"k_scan_tiles", "k_scan_bins", "k_scatter", "k_p2g",
                                               "k_g2p"};

}  // namespace

// Graph sets, one per mode: 0 = separate kernels; 1 = fused G2P2G steps,
// sorts decided on the device; 2 = fused steps with sorts at a fixed
// interval K (no mover budget), scheduled by the host, where a step without
// a sort launches the fused kernel alone.  A set holds, for each phase p of
// its period (the step number modulo NACC, or modulo max(K, 8) in mode 2),
// one step (graph p) and STEP_BATCH steps (graph period + p).
constexpr int MAX_PERIOD = 32;  // mode 2: K a power of two, at most this

struct mpm_sim {
  SimDev d;
  int device = 0;
  int cur = 0;  // buffer holding the current state (step n reads buffer (n + 1) mod 2)
  int64_t steps = 0;
  bool fused = false;             // mpm_set_fused_steps
  int32_t sort_interval = 0;      // the policy as last set (host copy)
  int64_t mover_budget = 0;
  int sched_K = 0;                // K of the built mode-2 graphs
  bool sched_ready = false;       // the last step left the state the mode-2 schedule expects
  hipStream_t cap = nullptr;
  hipGraph_t graph[3][2 * MAX_PERIOD] = {};
  hipGraphExec_t exec[3][2 * MAX_PERIOD] = {};
  int grid_particles = 0;  // ceil(N / WG), rounded up to a multiple of 8
  int grid_scatter = 0;
  int grid_p2g = 0;
  int grid_g2p = 0;
  int grid_g2p2g = 0;
  int grid_blocks = 0;   // node-block loops (grid readback)
};

namespace {

#define HIP_TRY(expr)                        \
  do {                                       \
    if ((expr) != hipSuccess) return MPM_ERR_HIP; \
  } while (0)

int step_mode(const mpm_sim *sim) {
  if (!sim->fused) return 0;
  const int K = sim->sort_interval;
  // a budget of at least N never triggers a sort
  const bool no_budget = sim->mover_budget >= (int64_t)sim->d.N;
  if (no_budget && K >= 2 && K <= MAX_PERIOD && (K & (K - 1)) == 0) return 2;
  return 1;
}

int mode_period(const mpm_sim *sim, int mode) {
  return mode == 2 ? std::max(sim->sort_interval, STEP_BATCH) : NACC;
}

// Kernel k of the step of phase p (reads buffer src = (p + 1) mod 2,
// accumulates into p); fused: the plain G2P is replaced by the G2P2G kernel,
// which stores v and C when write_vc is set and takes the next step's sort
// decision from sched (-1: by the policy, on the device).
int launch_kernel(mpm_sim *sim, int k, hipStream_t st, int p, bool fused, bool write_vc, int sched) {
  const int src = (p + 1) & 1;
  const SimDev &d = sim->d;
  switch (k) {
    case 0:
      // (a small grid's bins are scanned by one workgroup, without tile totals)
      if (d.nbins > SCAN_SMALL_NT * SCAN_PER) k_scan_tiles<<<d.ntiles, WG, 0, st>>>(d, src);
      break;
    case 1:
      if (d.nbins > SCAN_SMALL_NT * SCAN_PER) k_scan_bins<WG><<<d.ntiles, WG, 0, st>>>(d, src ^ 1);
      else k_scan_bins<SCAN_SMALL_NT><<<1, SCAN_SMALL_NT, 0, st>>>(d, src ^ 1);
      break;
    case 2:
      k_scatter<<<sim->grid_scatter, 64, 0, st>>>(d, src);
      break;
    case 3:
      if (d.material == MPM_J_FLUID) {
        if (d.has_E) k_p2g<MPM_J_FLUID, true><<<sim->grid_p2g, 64, 0, st>>>(d, src, p);
        else k_p2g<MPM_J_FLUID, false><<<sim->grid_p2g, 64, 0, st>>>(d, src, p);
      } else if (d.material == MPM_SAND) {
        if (d.has_E) k_p2g<MPM_SAND, true><<<sim->grid_p2g, 64, 0, st>>>(d, src, p);
        else k_p2g<MPM_SAND, false><<<sim->grid_p2g, 64, 0, st>>>(d, src, p);
      } else {
        if (d.has_E) k_p2g<MPM_FIXED_COROTATED, true><<<sim->grid_p2g, 64, 0, st>>>(d, src, p);
        else k_p2g<MPM_FIXED_COROTATED, false><<<sim->grid_p2g, 64, 0, st>>>(d, src, p);
      }
      break;
    case 4:
      if (fused) {
        const int wv = write_vc ? 1 : 0;
        const int g = sim->grid_g2p2g;
        if (d.material == MPM_J_FLUID) {
          if (d.has_E) k_g2p2g<MPM_J_FLUID, true><<<g, 64, 0, st>>>(d, src, p, wv, sched);
          else k_g2p2g<MPM_J_FLUID, false><<<g, 64, 0, st>>>(d, src, p, wv, sched);
        } else if (d.material == MPM_SAND) {
          if (d.has_E) k_g2p2g<MPM_SAND, true><<<g, 64, 0, st>>>(d, src, p, wv, sched);
          else k_g2p2g<MPM_SAND, false><<<g, 64, 0, st>>>(d, src, p, wv, sched);
        } else {
          if (d.has_E) k_g2p2g<MPM_FIXED_COROTATED, true><<<g, 64, 0, st>>>(d, src, p, wv, sched);
          else k_g2p2g<MPM_FIXED_COROTATED, false><<<g, 64, 0, st>>>(d, src, p, wv, sched);
        }
      } else {
        // (the gather does not depend on the material: sand uses the elastic instance)
        if (d.material == MPM_J_FLUID) k_g2p<MPM_J_FLUID><<<sim->grid_g2p, 64, 0, st>>>(d, src, p);
        else k_g2p<MPM_FIXED_COROTATED><<<sim->grid_g2p, 64, 0, st>>>(d, src, p);
      }
      break;
  }
  return hipGetLastError() == hipSuccess ? MPM_OK : MPM_ERR_HIP;
}

// Which kernels step n runs in a mode: all five, or (mode 2, a step after a
// fused pass) the fused kernel alone; and the fused kernel's sched argument.
// lean_ok = false forces all five (the first step under a new schedule,
// whose P2G may not have run).
void step_plan(const mpm_sim *sim, int64_t n, int mode, bool lean_ok, bool run[NUM_KERNELS], int &sched) {
  for (int k = 0; k < NUM_KERNELS; ++k) run[k] = true;
  sched = -1;
  if (mode == 2) {
    const int K = sim->sort_interval, c = (int)(n % K);
    sched = (c == K - 1) ? 1 : 0;
    if (c != 0 && lean_ok)
      for (int k = 0; k < NUM_KERNELS - 1; ++k) run[k] = false;
  }
}

int enqueue_step(mpm_sim *sim, hipStream_t st, int64_t n, int mode, bool lean_ok, bool write_vc) {
  bool run[NUM_KERNELS];
  int sched;
  step_plan(sim, n, mode, lean_ok, run, sched);
  for (int k = 0; k < NUM_KERNELS; ++k) {
    if (!run[k]) continue;
    const int rc = launch_kernel(sim, k, st, (int)(n % NACC), mode != 0, write_vc, sched);
    if (rc) return rc;
  }
  return MPM_OK;
}

void destroy_graphs(mpm_sim *sim, int mode) {
  for (int k = 0; k < 2 * MAX_PERIOD; ++k) {
    if (sim->exec[mode][k]) (void)hipGraphExecDestroy(sim->exec[mode][k]);
    if (sim->graph[mode][k]) (void)hipGraphDestroy(sim->graph[mode][k]);
    sim->exec[mode][k] = nullptr;
    sim->graph[mode][k] = nullptr;
  }
}

// The graphs of one mode, captured on the private stream.
int build_graphs(mpm_sim *sim, int mode) {
  const int P = mode_period(sim, mode);
  for (int g = 0; g < 2 * P; ++g) {
    const int p0 = g % P, nsteps = g < P ? 1 : STEP_BATCH;
    HIP_TRY(hipStreamBeginCapture(sim->cap, hipStreamCaptureModeThreadLocal));
    int rc = MPM_OK;
    for (int k = 0; k < nsteps && rc == MPM_OK; ++k)
      rc = enqueue_step(sim, sim->cap, p0 + k, mode, true, k == nsteps - 1);
    hipGraph_t gr = nullptr;
    const hipError_t e = hipStreamEndCapture(sim->cap, &gr);
    if (rc || e != hipSuccess) {
      if (gr) (void)hipGraphDestroy(gr);
      return MPM_ERR_HIP;
    }
    sim->graph[mode][g] = gr;
    HIP_TRY(hipGraphInstantiate(&sim->exec[mode][g], gr, nullptr, nullptr, 0));
  }
  return MPM_OK;
}

void release(mpm_sim *sim) {
  if (!sim) return;
  for (int m = 0; m < 3; ++m) destroy_graphs(sim, m);
  if (sim->cap) {
    (void)hipStreamSynchronize(sim->cap);
    (void)hipStreamDestroy(sim->cap);
  }
  delete sim;
}

}  // namespace

extern "C" {

size_t mpm_workspace_bytes(const mpm_params *params, int64_t n_particles) {
  if (!valid_params(params) || n_particles < 0 || n_particles >= (int64_t(1) << 28)) return 0;
  if (slot_capacity(n_particles, (params->grid_n + CB - 1) / CB) >= MAX_SLOTS) return 0;
  // The per-particle modulus array is always reserved so that one size fits
  // both the uniform and the per-particle case.
  return layout(params, n_particles, true, nullptr, nullptr);
}

int mpm_create(const mpm_params *params, int64_t n_particles, const float *x0, const float *v0, const float *C0,
               const float *F0, const float *E_p, void *workspace, size_t workspace_bytes, void *stream,
               mpm_sim **out) {
  if (!out) return MPM_ERR_INVALID_ARG;
  *out = nullptr;
  if (!valid_params(params) || n_particles < 0 || n_particles >= (int64_t(1) << 28)) return MPM_ERR_INVALID_ARG;
  if (slot_capacity(n_particles, (params->grid_n + CB - 1) / CB) >= MAX_SLOTS) return MPM_ERR_INVALID_ARG;
  if (n_particles > 0 && !x0) return MPM_ERR_INVALID_ARG;
  const size_t need = mpm_workspace_bytes(params, n_particles);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || workspace_bytes < need)
    return MPM_ERR_WORKSPACE;

  mpm_sim *sim = new (std::nothrow) mpm_sim();
  if (!sim) return MPM_ERR_STATE;
  const bool has_E = E_p != nullptr;
  layout(params, n_particles, has_E, static_cast<char *>(workspace), &sim->d);
  const SimDev &d = sim->d;
  hipStream_t st = static_cast<hipStream_t>(stream);

  int rc = MPM_OK;
  do {
    if (hipGetDevice(&sim->device) != hipSuccess) { rc = MPM_ERR_HIP; break; }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, sim->device) != hipSuccess || cus <= 0)
      cus = 256;
    sim->grid_particles = (int)(((d.N + WG - 1) / WG + 7) / 8 * 8);
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_p2g<MPM_FIXED_COROTATED, false>, 64, 0) != hipSuccess ||
        occ <= 0)
      occ = 16;
    // Measured: 4 waves per SIMD (16 single-wave workgroups per CU) is
    // P2G's best launch; fewer expose latency and more slowed the kernel.
    occ = occ < 16 ? occ : 16;
    sim->grid_p2g = ((cus * occ + NQ - 1) / NQ) * NQ;
    // Chunk size: KMAX particles when there is enough work for every P2G
    // wavefront, else smaller (down to 64), so that a small scene's few bins
    // still spread over many wavefronts: the step time of small scenes is
    // the latency of one wavefront's chunks.
    {
      int shift = KMAX_SHIFT;
      while (shift > KMIN_SHIFT && ((int64_t)d.N >> shift) < (int64_t)sim->grid_p2g) --shift;
      sim->d.chunk_shift = shift;
    }
    int occ_g = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ_g, k_g2p<MPM_FIXED_COROTATED>, 64, 0) != hipSuccess || occ_g <= 0)
      occ_g = 16;
    // Measured: 5 waves per SIMD (20 workgroups per CU) is G2P's best launch;
    // 24 per CU, which 74 VGPRs would allow, was slower.
    occ_g = occ_g < 20 ? occ_g : 20;
    sim->grid_g2p = ((cus * occ_g + NQ - 1) / NQ) * NQ;
    // The fused kernel holds the G2P velocity window and the P2G windows
    // (10 KB of LDS, at most 15 workgroups per CU) and, with its loads one
    // round ahead, 130-150 VGPRs (3 waves per SIMD); P2G's cap of 16 applies.
    int occ_f = 0;
    const void *fk = d.material == MPM_J_FLUID
                         ? (d.has_E ? (const void *)k_g2p2g<MPM_J_FLUID, true> : (const void *)k_g2p2g<MPM_J_FLUID, false>)
                     : d.material == MPM_SAND
                         ? (d.has_E ? (const void *)k_g2p2g<MPM_SAND, true> : (const void *)k_g2p2g<MPM_SAND, false>)
                         : (d.has_E ? (const void *)k_g2p2g<MPM_FIXED_COROTATED, true>
                                    : (const void *)k_g2p2g<MPM_FIXED_COROTATED, false>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ_f, fk, 64, 0) != hipSuccess || occ_f <= 0) occ_f = 8;
    occ_f = occ_f < 16 ? occ_f : 16;
    sim->grid_g2p2g = ((cus * occ_f + NQ - 1) / NQ) * NQ;
    sim->grid_blocks = cus * 8;
    // single-wavefront workgroups, 8 per SIMD: the scatter is a chain of
    // short dependent loads per chunk, so it wants many chunks in flight
    sim->grid_scatter = cus * 32;
    if (hipStreamCreateWithFlags(&sim->cap, hipStreamNonBlocking) != hipSuccess) { rc = MPM_ERR_HIP; break; }

    // Clear counters, flags, status and the P2G accumulator, then upload.
    k_zero_u32<<<1, WG, 0, st>>>(d.ctr, CTR_WORDS);
    k_zero_u32<<<1, WG, 0, st>>>(d.status, MPM_STATUS_WORDS);
    const int zb = (int)std::min<int64_t>(((int64_t)d.nbins + WG - 1) / WG, 4096);
    k_zero_u32<<<zb, WG, 0, st>>>(d.bin_count, (size_t)d.nbins);
    k_zero_u32<<<zb, WG, 0, st>>>(d.stay_count, (size_t)d.nbins);
    const int gb = (int)std::min<int64_t>(((int64_t)d.nblk * 512 * 4 + WG - 1) / WG, 16384);
    for (int k = 0; k < NACC; ++k) {
      k_zero_u32<<<zb, WG, 0, st>>>(d.active_flag[k], (size_t)d.nblk);
      // G2P may read a stencil node whose weight is exactly zero and that no
      // particle marked active; it must hold a finite value, so start at zero.
      k_zero_f32<<<gb, WG, 0, st>>>(reinterpret_cast<float *>(d.gridA[k]), (size_t)d.nblk * 512 * 4);
    }
    if (d.N > 0) {
      k_init<<<(d.N + WG - 1) / WG, WG, 0, st>>>(d, x0, v0, C0, F0, E_p);
      // one bucket pass to bring the initial state into bin order (buffer 1,
      // whose chunk list the scan writes): the scans of a step that reads
      // buffer 0 (phase 1)
      launch_kernel(sim, 0, st, 1, false, false, -1);
      launch_kernel(sim, 1, st, 1, false, false, -1);
      k_scatter_init<<<sim->grid_particles, WG, 0, st>>>(d);
      sim->cur = 1;
    }
    if (hipGetLastError() != hipSuccess) { rc = MPM_ERR_HIP; break; }
    if (d.N > 0) rc = build_graphs(sim, 0);
  } while (0);
  if (rc != MPM_OK) {
    release(sim);
    return rc;
  }
  *out = sim;
  return MPM_OK;
}

int mpm_step(mpm_sim *sim, int32_t n_steps, void *stream) {
  if (!sim || n_steps < 0) return MPM_ERR_INVALID_ARG;
  if (sim->d.N == 0) {
    sim->steps += n_steps;
    return MPM_OK;
  }
  const int mode = step_mode(sim);
  if (mode == 2 && sim->sched_K != sim->sort_interval) {
    destroy_graphs(sim, 2);
    sim->sched_K = 0;
  }
  if (mode != 0 && !sim->exec[mode][0]) {
    const int rc = build_graphs(sim, mode);
    if (rc) return rc;
    if (mode == 2) sim->sched_K = sim->sort_interval;
  }
  const int P = mode_period(sim, mode);
  for (int g = 0; g < 2 * P; ++g)
    if (!sim->exec[mode][g]) return MPM_ERR_STATE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t left = n_steps;
  if (mode == 2 && !sim->sched_ready && left > 0) {
    // the first step under the schedule runs all its kernels (its P2G may
    // not have run yet)
    const int rc = enqueue_step(sim, st, sim->steps, 2, false, left == 1);
    if (rc) return rc;
    sim->cur ^= 1;
    sim->steps += 1;
    left -= 1;
    sim->sched_ready = true;
  }
  while (left >= STEP_BATCH) {
    if (hipGraphLaunch(sim->exec[mode][P + (int)(sim->steps % P)], st) != hipSuccess) return MPM_ERR_HIP;
    sim->steps += STEP_BATCH;  // even: the buffer parity is unchanged
    left -= STEP_BATCH;
  }
  for (; left > 0; --left) {
    if (hipGraphLaunch(sim->exec[mode][sim->steps % P], st) != hipSuccess) return MPM_ERR_HIP;
    sim->cur ^= 1;
    sim->steps += 1;
  }
  return MPM_OK;
}

int mpm_set_fused_steps(mpm_sim *sim, int32_t enable) {
  if (!sim || enable < 0 || enable > 1) return MPM_ERR_INVALID_ARG;
  sim->fused = enable == 1;
  sim->sched_ready = false;
  return MPM_OK;
}

int mpm_set_sort_policy(mpm_sim *sim, int32_t max_interval, int64_t mover_budget, void *stream) {
  if (!sim || max_interval < 0 || mover_budget < 0) return MPM_ERR_INVALID_ARG;
  const uint32_t budget = mover_budget > 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)mover_budget;
  k_set_sort_policy<<<1, 64, 0, static_cast<hipStream_t>(stream)>>>(sim->d, (uint32_t)max_interval, budget);
  if (hipGetLastError() != hipSuccess) return MPM_ERR_HIP;
  sim->sort_interval = max_interval;
  sim->mover_budget = mover_budget;
  sim->sched_ready = false;
  return MPM_OK;
}

int mpm_step_profiled(mpm_sim *sim, int32_t n_steps, void *stream, float *kernel_ms) {
  if (!sim || n_steps < 0 || !kernel_ms) return MPM_ERR_INVALID_ARG;
  if (sim->d.N == 0) {
    sim->steps += n_steps;
    return MPM_OK;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int mode = step_mode(sim);
  hipEvent_t ev[NUM_KERNELS + 1];
  for (int k = 0; k <= NUM_KERNELS; ++k)
    if (hipEventCreate(&ev[k]) != hipSuccess) return MPM_ERR_HIP;
  int rc = MPM_OK;
  for (int32_t s = 0; s < n_steps && rc == MPM_OK; ++s) {
    // the same kernels as the graphs (a kernel a step does not run takes no time)
    bool run[NUM_KERNELS];
    int sched;
    step_plan(sim, sim->steps, mode, mode == 2 && sim->sched_ready, run, sched);
    if (hipEventRecord(ev[0], st) != hipSuccess) { rc = MPM_ERR_HIP; break; }
    for (int k = 0; k < NUM_KERNELS && rc == MPM_OK; ++k) {
      if (run[k]) rc = launch_kernel(sim, k, st, (int)(sim->steps % NACC), mode != 0, true, sched);
      if (rc == MPM_OK && hipEventRecord(ev[k + 1], st) != hipSuccess) rc = MPM_ERR_HIP;
    }
    if (rc != MPM_OK) break;
    if (hipEventSynchronize(ev[NUM_KERNELS]) != hipSuccess) { rc = MPM_ERR_HIP; break; }
    for (int k = 0; k < NUM_KERNELS; ++k) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, ev[k], ev[k + 1]) != hipSuccess) { rc = MPM_ERR_HIP; break; }
      kernel_ms[k] += ms;
    }
    sim->cur ^= 1;
    sim->steps += 1;
    sim->sched_ready = mode == 2;
  }
  for (int k = 0; k <= NUM_KERNELS; ++k) (void)hipEventDestroy(ev[k]);
  return rc;
}

int mpm_read_particles(mpm_sim *sim, float *x, float *v, float *C, float *F_or_J, void *stream) {
  if (!sim) return MPM_ERR_INVALID_ARG;
  if (sim->d.N == 0) return MPM_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int g = sim->grid_g2p;
  if (sim->d.material == MPM_J_FLUID) k_read_particles<MPM_J_FLUID><<<g, 64, 0, st>>>(sim->d, sim->cur, x, v, C, F_or_J);
  else if (sim->d.material == MPM_SAND) k_read_particles<MPM_SAND><<<g, 64, 0, st>>>(sim->d, sim->cur, x, v, C, F_or_J);
  else k_read_particles<MPM_FIXED_COROTATED><<<g, 64, 0, st>>>(sim->d, sim->cur, x, v, C, F_or_J);
  return hipGetLastError() == hipSuccess ? MPM_OK : MPM_ERR_HIP;
}

int mpm_read_grid(mpm_sim *sim, float *mass, float *momentum, void *stream) {
  if (!sim) return MPM_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t nn = (size_t)sim->d.n * sim->d.n * sim->d.n;
  const int zb = (int)std::min<size_t>((nn * 3 + WG - 1) / WG, 16384);
  if (mass) k_zero_f32<<<zb, WG, 0, st>>>(mass, nn);
  if (momentum) k_zero_f32<<<zb, WG, 0, st>>>(momentum, 3 * nn);
  // the last step accumulated into its phase's accumulator
  if (sim->d.N > 0 && sim->steps > 0)
    k_read_grid<<<sim->grid_blocks, WG, 0, st>>>(sim->d, (int)((sim->steps - 1) % NACC), mass, momentum);
  return hipGetLastError() == hipSuccess ? MPM_OK : MPM_ERR_HIP;
}

int mpm_status(mpm_sim *sim, uint32_t *status_device, void *stream) {
  if (!sim || !status_device) return MPM_ERR_INVALID_ARG;
  if (hipMemcpyAsync(status_device, sim->d.status, sizeof(uint32_t) * MPM_STATUS_WORDS, hipMemcpyDeviceToDevice,
                     static_cast<hipStream_t>(stream)) != hipSuccess)
    return MPM_ERR_HIP;
  return MPM_OK;
}

int64_t mpm_steps_taken(const mpm_sim *sim) { return sim ? sim->steps : -1; }

int32_t mpm_num_kernels(void) { return NUM_KERNELS; }

const char *mpm_kernel_name(int32_t k) { return (k >= 0 && k < NUM_KERNELS) ? KERNEL_NAMES[k] : nullptr; }

void mpm_destroy(mpm_sim *sim) { release(sim); }

const char *mpm_error_string(int code) {
  switch (code) {
    case MPM_OK: return "ok";
    case MPM_ERR_INVALID_ARG: return "invalid argument";
    case MPM_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MPM_ERR_HIP: return "HIP runtime error";
    case MPM_ERR_STATE: return "simulation handle not usable";
    default: return "unknown error";
  }
}

}  // extern "C"
