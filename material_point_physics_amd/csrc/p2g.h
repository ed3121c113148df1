// p2g.h -- P2G: ranking in LDS, conflict-free window accumulation, flush
// Part of mpm.hip: included there, inside its anonymous namespace, after the
// parts before it; not a standalone header.

// P2G.  Persistent single-wavefront workgroups take chunks (<= KMAX particles
// of one 4^3-cell bin) from their XCD's queue.
//
// Accumulation without atomics: on gfx950, LDS float atomics serialise per
// lane, so the windows are private to the wavefront and updated with plain
// read-modify-writes.  There are NW windows; the particle of rank r in its
// cell (r-th of that cell in the chunk) accumulates into window r % NW and
// has super-rank r / NW.  The chunk's particles are ordered by (super-rank,
// window, cell): lanes that share a super-rank differ in (window, cell), so
// for a fixed stencil offset their target addresses are distinct, and one
// masked ds_read/ds_write pair per offset adds all of them.  A round of 64
// lanes that spans several super-ranks runs one pass per super-rank.  The LDS
// executes a wavefront's accesses in issue order; compiler fences keep that
// order.  The flush adds the windows and issues one native global atomic per
// node and channel.
// NW windows per wavefront: two where many wavefronts share a compute unit
// (large scenes: 16 per CU, 8 KB of LDS each), eight for small scenes, whose
// few chunks leave most of the LDS free.  A small scene's P2G lasts as long as
// its slowest chunk, and a chunk drawn from a dense or partly filled bin may
// hold 16-32 particles of one cell: with eight windows it needs a quarter of
// the passes.  The fused G2P2G pass uses two.
constexpr int NWIN = 2;                  // windows of the large-scene P2G and of the fused pass
constexpr int NWIN_WIDE = 8;             // windows of the small-scene P2G

template <int NW>
struct P2GRankTables {                   // lives in the window space while a chunk is ordered
  uint32_t hist[CB3];                    // particles per cell
  uint32_t subcnt[KMAX / 64][CB3];       // particles per cell in each sub-round of 64
  uint32_t rstart[KMAX / NW + 2];        // first position of each super-rank
  uint64_t rmask[KMAX];                  // per (super-rank, window): cells present (bit = cell)
};

template <int NW>
union P2GShared {
  float4 win[NW * PW3];
  P2GRankTables<NW> rk;
};
static_assert(sizeof(P2GRankTables<NWIN>) <= sizeof(float4) * NWIN * PW3, "rank tables must fit the windows");

// LDS of the small-chunk P2G: the windows and a per-cell count.  Its
// windows are PW3_PAD nodes apart, a multiple of 256 bytes, so that the
// flush reads one node's value in two windows with one instruction.
constexpr int PW3_PAD = 224;
static_assert(PW3_PAD >= PW3 && (PW3_PAD * 16) % 256 == 0, "padded window stride");
struct P2GSmallShared {
  float4 win[NWIN_WIDE * PW3_PAD];
  uint32_t cnt[CB3];  // particles per cell of the chunk being ranked
};

// Zero NW windows: whole rows of 64 lanes, unrolled (a loop whose trip count
// depends on the lane runs as a divergent loop, several times slower for a
// single wavefront), then the partial row.  (The many-wavefront paths keep
// the loop: unrolled, it raised their register count past an occupancy
// step.)
template <int NW, int WS = PW3>
__device__ __forceinline__ void clear_windows(float4 *win) {
  constexpr int N = NW * WS;
  const int lane = threadIdx.x;
#pragma unroll
  for (int k = 0; k < N / 64; ++k) win[64 * k + lane] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (N % 64 != 0 && lane < N % 64) win[64 * (N / 64) + lane] = make_float4(0.f, 0.f, 0.f, 0.f);
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

// Flush: the sum of the NW windows (window origin = first base node of
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
template <int NW, int WS = PW3>
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
      for (int w = 0; w < NW; ++w) val += winl[4 * (kw + w * WS)];
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

// One round of up to 64 particles, one per lane: load the particle at
// source slot i, store x, id, F (and the per-particle scalar) at slot dst,
// apply the deferred deformation update, evaluate the stress, form the APIC
// momentum and deposit it into the windows (tag: window and pass, or
// MOVER_TAG).  Lanes with valid = false load a valid particle and store
// nothing.  P2G writes x and id at dst; G2P reads x from the same slot,
// without an index indirection, and leaves it: the position it advects to
// is formed again here from x and its v.
// The state P2G reads of one particle: x, v, C, F (or J), the per-particle
// scalar and the id, loaded at source byte offset io.
template <int MAT>
struct P2GIn {
  float x[3], v[3], C[9], F[MAT == MPM_J_FLUID ? 1 : 9], E;
  uint32_t id;
};
template <int MAT, bool HAS_E>
__device__ __forceinline__ void load_p2g(const SimDev &s, const PBuf &in, uint32_t io, P2GIn<MAT> &p) {
  const uint32_t Np = (uint32_t)s.Np;  // Np < 2^29: component offsets k Np (k < 9) are exact in 32 bits
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    p.x[a] = at_byte(in.x + a * Np, io);
    p.v[a] = at_byte(in.v + a * Np, io);
  }
#pragma unroll
  for (int k = 0; k < 9; ++k) p.C[k] = stream_load(at_byte(in.C + k * Np, io));
#pragma unroll
  for (int k = 0; k < (MAT == MPM_J_FLUID ? 1 : 9); ++k) p.F[k] = stream_load(at_byte(in.F + k * Np, io));
  p.E = HAS_E ? at_byte(in.E, io) : s.E;
  p.id = stream_load(at_byte(in.id, io));
}

// (mid, called once the particle's loaded state is used up and before the
// deposit: the caller requests its next round there, so that the loads
// overlap the deposit's LDS passes)
template <int MAT, bool HAS_E, bool FREE, int NW, bool RANK_PASS, int WS, typename Mid>
__device__ __forceinline__ void p2g_particle(const SimDev &s, const PBuf &out, bool pending, int acc, int ox0,
                                             int oy0, int oz0, bool valid, const P2GIn<MAT> &pin, uint32_t tag,
                                             uint32_t dst, float4 *win, Mid mid) {
  const int lane = threadIdx.x;
  const uint32_t Np = (uint32_t)s.Np;  // Np < 2^29: component offsets k Np (k < 9) are exact in 32 bits
  const float dt = s.dt, mass = s.mass, fn = s.fn, dx = s.dx;
  const uint32_t od = 4u * dst;  // byte offset of the destination slot
  float xp[3], vp[3], Cp[9];
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    xp[a] = pin.x[a];
    vp[a] = pin.v[a];
  }
#pragma unroll
  for (int k = 0; k < 9; ++k) Cp[k] = pin.C[k];
  // the pending advection of the G2P before (the same bits as its keys)
  if (pending)
#pragma unroll
    for (int a = 0; a < 3; ++a) xp[a] = advanced(s, xp[a], vp[a]);
  if (valid) {
#pragma unroll
    for (int a = 0; a < 3; ++a) at_byte(out.x + a * Np, od) = xp[a];
    stream_store(pin.id, at_byte(out.id, od));
  }

  // Deferred deformation-gradient update, stress, APIC momentum.
  float Fp[MAT == MPM_J_FLUID ? 1 : 9];
#pragma unroll
  for (int k = 0; k < (MAT == MPM_J_FLUID ? 1 : 9); ++k) Fp[k] = pin.F[k];
  if (pending) update_F<MAT>(Fp, Cp, dt);
  // the per-particle scalar: Young's modulus, or snow's log plastic volume
  const float Es = pin.E;
  const float E = MAT == MPM_SNOW ? s.E : Es;
  float ap = Es;
  float A[9];
  uint32_t st = 0;
  // sand, snow: the plasticity projection of the updated F, with the stress
  if (MAT == MPM_SAND || MAT == MPM_SNOW) st = plastic_affine<MAT>(s, Fp, E, ap, Cp, A, pending);
  if (valid) {
#pragma unroll
    for (int k = 0; k < (MAT == MPM_J_FLUID ? 1 : 9); ++k) stream_store(Fp[k], at_byte(out.F + k * Np, od));
    if (HAS_E) stream_store(MAT == MPM_SNOW ? ap : E, at_byte(out.E, od));
  }
  if (MAT != MPM_SAND && MAT != MPM_SNOW) st = affine_momentum<MAT>(s, Fp, E, Cp, A);
  if (st && valid) flag_status(s, st, (st & MPM_STATUS_INVERTED) ? 2 : 0);
  int b[3];
  float f[3], w[3][3], q0[3], Ad[9];
  particle_weights(xp, fn, b, f, w);
  momentum_terms(mass, dx, vp, A, f, q0, Ad);
  const int lx = min(max(b[0] - ox0, 0), CB - 1), ly = min(max(b[1] - oy0, 0), CB - 1),
            lz = min(max(b[2] - oz0, 0), CB - 1);
  const int li0 = (int)(tag % NW) * WS + (lz * PW + ly) * PW + lx;

  // Passes: lanes conflict only when they share (window, cell).  With
  // RANK_PASS the tag is the particle's rank r in its cell, which is its
  // occurrence index in window r % NW: its pass is r / NW.  Otherwise the
  // lane's pass is its occurrence index among the earlier lanes of the
  // round with the same (window, cell) (ballot-matched), which gives the
  // fewest conflict-free passes; lanes of one super-rank never share
  // (window, cell), so this is at most one pass per super-rank.
  // (a mover's stencil is outside the window: it takes no pass)
  const bool mov = FREE && tag == MOVER_TAG;
  const bool inwin = valid && !mov;
  uint32_t pass_id;
  if (RANK_PASS) {
    pass_id = tag / NW;
  } else {
    const uint32_t wc = (tag % NW) * (uint32_t)CB3 + (uint32_t)((lz * CB + ly) * CB + lx);
    uint64_t peers = __ballot(inwin);
    constexpr int WC_BITS = NW == 2 ? 7 : (NW == 4 ? 8 : 9);  // 6 cell bits + log2(NW)
    static_assert(NW == 2 || NW == 4 || NW == 8, "window counts with a bit width here");
#pragma unroll
    for (int k = 0; k < WC_BITS; ++k) {
      const uint64_t bk = __ballot((wc >> k) & 1u);
      peers &= ((wc >> k) & 1u) ? bk : ~bk;
    }
    pass_id = (uint32_t)__popcll(peers & ((1ull << lane) - 1ull));
  }
  mid();
  // A mover (only in a step without a sort; rare) deposits directly.
  if (FREE && valid && mov) deposit_global(s, acc, b, w, q0, Ad);
  bool todo = inwin;
  for (uint32_t pnow = 0;; ++pnow) {
    // (occurrence indices of a key are 0, 1, ..., so no lane waits for a
    // pass after an empty one)
    if (__ballot(todo && pass_id == pnow) == 0ull) break;
    if (todo && pass_id == pnow) {
      deposit_window(win, li0, w, q0, Ad, mass);
      todo = false;
    }
  }
}

// The P2G of one step.  FREE: a step without a sort (free-zone policy), with
// the paths for particles outside their chunk's bin; the per-step-sort
// instance has none of that code.
template <int MAT, bool HAS_E, bool FREE, int NW>
__device__ __forceinline__ void p2g_step(const SimDev &s, int src, int acc, P2GShared<NW> &sm, uint32_t *order,
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
    ch_next = load_record(chunks + qbeg + wq);
    prefetch(ch_next);
  }
  // (waited for here, as at the end of every chunk below, so that the first
  // use in the chunk loop needs no wait: see the note before the flush)
#pragma unroll
  for (int j = 0; j < KMAX / 64; ++j) __asm__ __volatile__("" ::"v"(pf_src[j]), "v"(pf_cell[j]));
  for (uint32_t c = qbeg + wq; c < qend; c += nwq) {
    const uint4 ch = ch_next;
    const uint32_t start = ch.x, count = min(ch.y, (uint32_t)KMAX), bin = ch.z;
    const int ox0 = (int)compact3(bin) * CB, oy0 = (int)compact3(bin >> 1) * CB, oz0 = (int)compact3(bin >> 2) * CB;  // first base node of the bin = window origin
    const bool has_next = c + nwq < qend;
    if (has_next) ch_next = load_record(chunks + c + nwq);

    // Pass A: cell of each particle and its rank within the cell.  Ranks
    // follow the particles' previous storage order (their source index), so
    // the processing order -- which is also the order the new state is
    // stored in -- is stable from step to step and the gathers below run over
    // nearly consecutive addresses.  The chunk is read as KMAX/64 sub-rounds
    // of consecutive slots, each a run of consecutive sources; sub-rounds
    // are ranked in the order of their smallest source.  Lanes with the same
    // cell are matched bit by bit with ballots; the lowest lane of each group
    // records the group's size (leaders have distinct cells: no atomics).
    P2GRankTables<NW> &rk = sm.rk;
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
    // Rank tables: rmask[NW sr + w] = cells holding a particle of rank
    // NW sr + w (lane = cell), rstart[sr] = position of the first particle
    // of super-rank sr.
    {
      const uint32_t cnt = rk.hist[lane];
      uint32_t mx = cnt;
      for (int d = 32; d >= 1; d >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, d));
      uint32_t run = 0;
      for (uint32_t sr = 0; NW * sr < mx; ++sr) {
        uint32_t here = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const uint64_t m = __ballot(cnt > NW * sr + w);
          if (lane == 0) rk.rmask[NW * sr + w] = m;
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
          const uint32_t cell = cells[j], sr = rank[j] / NW, w = rank[j] % NW;
          uint32_t pos = rk.rstart[sr] + (uint32_t)__popcll(rk.rmask[NW * sr + w] & ((1ull << cell) - 1ull));
          for (uint32_t w2 = 0; w2 < w; ++w2) pos += (uint32_t)__popcll(rk.rmask[NW * sr + w2]);
          pos = min(pos, (uint32_t)KMAX - 1u);
          order[pos] = srcs[j];
          ordtag[pos] = (uint8_t)(sr * NW + w);
        }
      }
      mbefore += (uint32_t)__popcll(mmask);
    }
    __syncthreads();
    // the tables are dead: clear the windows
    for (int k = lane; k < NW * PW3; k += 64) sm.win[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();

    if (has_next) prefetch(ch_next);

    // Pass B: rounds of 64 particles in (super-rank, window, cell) order.
    // (lanes past the count load the chunk's last particle and store nothing;
    // a round's loads are issued before the deposit of the round before)
    P2GIn<MAT> pin;
    load_p2g<MAT, HAS_E>(s, in, 4u * order[min((uint32_t)lane, count - 1u)], pin);
    for (uint32_t r0 = 0; r0 < count; r0 += 64) {
      const uint32_t pos = r0 + (uint32_t)lane;
      const bool valid = pos < count;
      const uint32_t at = min(pos, count - 1u);
      const uint32_t tag = ordtag[at];
      // The new state is stored in this processing order, (bin, super-rank,
      // window, cell): the next step's gathers then run over nearly
      // consecutive addresses.
      p2g_particle<MAT, HAS_E, FREE, NW, false, PW3>(s, out, pending, acc, ox0, oy0, oz0, valid, pin, tag, start + at,
                                                sm.win, [&]() {
                                                  if (r0 + 64u < count)
                                                    load_p2g<MAT, HAS_E>(
                                                        s, in, 4u * order[min(pos + 64u, count - 1u)], pin);
                                                });
    }
    // The next chunk's prefetched sources and cells are waited for here,
    // before the flush: a vector load is complete only once every vector
    // operation issued before it is, so a wait for them after the flush
    // would also wait for the flush's atomics.
#pragma unroll
    for (int j = 0; j < KMAX / 64; ++j) __asm__ __volatile__("" ::"v"(pf_src[j]), "v"(pf_cell[j]));
    __syncthreads();
    flush_windows<NW>(s, sm.win, ox0, oy0, oz0, acc);
    __syncthreads();
  }
}

// The P2G of one step for chunks of at most 64 particles (small scenes,
// NWIN_WIDE windows): one round per chunk, so the ordering needs no tables
// in LDS.  Each lane keeps its particle; its rank r in its cell gives its
// window (r % NW), its pass (r / NW) and its storage slot, the position of
// (r, cell) in (rank, cell) order -- the (super-rank, window, cell) order of
// the general path.  A single wavefront's step time is its chain of
// dependent operations: the windows are cleared while the first chunk's
// loads are in flight, and again after a flush only if another chunk
// follows.  Requires chunks of at most 64 particles (the scan makes them so
// when the scene takes this path).
template <int MAT, bool HAS_E, bool FREE>
__device__ __forceinline__ void p2g_step_small(const SimDev &s, int src, int acc, P2GSmallShared &sm) {
  constexpr int NW = NWIN_WIDE;
  const PBuf in = s.buf[src], out = s.buf[src ^ 1];
  const int lane = threadIdx.x;
  const uint64_t below = (1ull << lane) - 1ull;
  const uint32_t Np = (uint32_t)s.Np;
  const uint32_t q = blockIdx.x & (NQ - 1), wq = blockIdx.x / NQ, nwq = gridDim.x / NQ;
  const uint32_t nch = s.ctr[CTR_NCHUNKS + (src ^ 1)];
  const uint4 *chunks = s.chunks[src ^ 1];
  const uint32_t qbeg = (uint32_t)(((uint64_t)nch * q) / NQ), qend = (uint32_t)(((uint64_t)nch * (q + 1)) / NQ);
  const bool pending = s.ctr[CTR_PENDING] != 0u;
  constexpr bool sorted = !FREE;
  // a chunk's source index and cell (or, without a sort, whole key) per
  // lane, loaded one chunk ahead
  uint32_t pf_src = 0xFFFFFFFFu, pf_cell = 0u;
  auto prefetch = [&](const uint4 &chrec) {
    const uint32_t pstart = chrec.x, pcount = min(chrec.y, 64u);
    pf_src = 0xFFFFFFFFu;
    pf_cell = 0u;
    if ((uint32_t)lane < pcount) {
      pf_src = sorted ? s.perm[pstart + lane] : pstart + (uint32_t)lane;
      pf_cell = sorted ? (uint32_t)s.cellp[pstart + lane] : s.key[pstart + lane];
    }
  };
  clear_accumulator(s, (acc + 2) & (NACC - 1));
  // (k_sort_small) the bins' counts, stayer counts and mover counters, which
  // every workgroup of this step's sort read, cleared for this step's G2P
  if (!FREE && s.sort_small)
    for (uint32_t b = blockIdx.x * 64u + (uint32_t)lane; b < (uint32_t)s.nbins; b += gridDim.x * 64u) {
      s.bin_count[b] = 0u;
      s.stay_count[b] = 0u;
      s.bin_cursor[b] = 0u;
    }
  uint4 ch_next = make_uint4(0u, 0u, 0u, 0u);
  if (qbeg + wq < qend) {
    ch_next = load_record(chunks + qbeg + wq);
    prefetch(ch_next);
  }
  clear_windows<NW, PW3_PAD>(sm.win);
  for (uint32_t c = qbeg + wq; c < qend; c += nwq) {
    const uint4 ch = ch_next;
    const uint32_t start = ch.x, count = min(ch.y, 64u), bin = ch.z;
    const int ox0 = (int)compact3(bin) * CB, oy0 = (int)compact3(bin >> 1) * CB, oz0 = (int)compact3(bin >> 2) * CB;
    const bool has_next = c + nwq < qend;
    if (has_next) ch_next = load_record(chunks + c + nwq);
    const bool in_chunk = (uint32_t)lane < count;
    const uint32_t kc = pf_cell;
    const bool mov = FREE && in_chunk && (kc & ((1u << KEY_CELL_SHIFT) - 1u)) != bin;
    const uint32_t cell = (sorted ? kc : (kc >> KEY_CELL_SHIFT)) & (uint32_t)(CB3 - 1);
    const bool ranked = in_chunk && !mov;
    // (lanes past the count load the chunk's first particle and store nothing)
    const uint32_t i = in_chunk ? min(pf_src, Np - 1u) : __builtin_amdgcn_readfirstlane(min(pf_src, Np - 1u));
    // Rank within the cell: lanes with the same cell matched bit by bit.
    uint64_t peers = __ballot(ranked);
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      const uint64_t bk = __ballot((cell >> k) & 1u);
      peers &= ((cell >> k) & 1u) ? bk : ~bk;
    }
    const uint32_t r = (uint32_t)__popcll(peers & below);
    // Particles per cell, lane = cell: each group's lowest lane writes its
    // size (the wavefront's LDS accesses execute in issue order).
    sm.cnt[lane] = 0u;
    __asm__ __volatile__("" ::: "memory");
    if (ranked && r == 0u) sm.cnt[cell] = (uint32_t)__popcll(peers);
    __asm__ __volatile__("" ::: "memory");
    const uint32_t cnt = sm.cnt[lane];
    // Lane k of (mlo, mhi) = the cells holding a particle of rank k; lane k
    // of pre = the position of the first of them.
    uint32_t mlo = 0u, mhi = 0u, pre = 0u, run = 0u;
    for (uint32_t k = 0; k < 64u; ++k) {
      const uint64_t m = __ballot(cnt > k);
      if (m == 0ull) break;
      if ((uint32_t)lane == k) {
        mlo = (uint32_t)m;
        mhi = (uint32_t)(m >> 32);
        pre = run;
      }
      run += (uint32_t)__popcll(m);
    }
    const int rq = ranked ? (int)r : 0;
    const uint64_t gm = ((uint64_t)(uint32_t)__shfl((int)mhi, rq) << 32) | (uint32_t)__shfl((int)mlo, rq);
    uint32_t pos = (uint32_t)__shfl((int)pre, rq) + (uint32_t)__popcll(gm & ((1ull << cell) - 1ull));
    if (FREE) {
      // movers go after the ranked particles
      const uint64_t mm = __ballot(mov);
      if (mov) pos = run + (uint32_t)__popcll(mm & below);
    }
    if (has_next) prefetch(ch_next);
    P2GIn<MAT> pin;
    load_p2g<MAT, HAS_E>(s, in, 4u * i, pin);
    p2g_particle<MAT, HAS_E, FREE, NW, true, PW3_PAD>(s, out, pending, acc, ox0, oy0, oz0, in_chunk, pin,
                                             mov ? (uint32_t)MOVER_TAG : r, start + pos, sm.win, []() {});
    // (the next chunk's loads are waited for before the flush: a vector load
    // is complete only once every vector operation issued before it is)
    __asm__ __volatile__("" ::"v"(pf_src), "v"(pf_cell));
    flush_windows<NW, PW3_PAD>(s, sm.win, ox0, oy0, oz0, acc);
    if (has_next) {
      __asm__ __volatile__("" ::: "memory");
      clear_windows<NW, PW3_PAD>(sm.win);
    }
  }
}

template <int MAT, bool HAS_E, int NW>
// (snow: at least 4 waves per SIMD, which holds it at 128 VGPRs with no spill;
// measured 13% faster than its unconstrained 130 VGPRs at 3 waves)
__global__ __launch_bounds__(64, NW == NWIN ? 4 : 1) void k_p2g(SimDev s, int src, int acc) {
  if constexpr (NW == NWIN_WIDE) {
    // (k_sort_small, which only small scenes use, leaves these to the P2G:
    // all its workgroups read them)
    if (s.sort_small && blockIdx.x == 0 && threadIdx.x == 0) {
      s.ctr[CTR_MOVSNAP] = s.ctr[CTR_MOVERS];
      s.ctr[CTR_MOVERS] = 0u;
      s.ctr[CTR_SINCE] = s.ctr[CTR_SORT + src] != 0u ? 0u : s.ctr[CTR_SINCE] + 1u;
    }
  }
  if (s.ctr[CTR_LOOK + src] != 0u) return;  // done by the fused kernel of the step before
  if constexpr (NW == NWIN_WIDE) {
    __shared__ P2GSmallShared sm;
    if (s.ctr[CTR_SORT + src] != 0u) p2g_step_small<MAT, HAS_E, false>(s, src, acc, sm);
    else p2g_step_small<MAT, HAS_E, true>(s, src, acc, sm);
  } else {
    __shared__ P2GShared<NW> sm;
    __shared__ uint32_t order[KMAX];  // source index of each processing position
    __shared__ uint8_t ordtag[KMAX];  // super-rank * NW + window of each position (or MOVER_TAG)
    if (s.ctr[CTR_SORT + src] != 0u) p2g_step<MAT, HAS_E, false, NW>(s, src, acc, sm, order, ordtag);
    else p2g_step<MAT, HAS_E, true, NW>(s, src, acc, sm, order, ordtag);
  }
}
