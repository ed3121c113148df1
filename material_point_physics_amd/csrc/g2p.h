// g2p.h -- G2P: velocity window with the grid update, gather, advection, next keys
// Part of mpm.hip: included there, inside its anonymous namespace, after the
// parts before it; not a standalone header.

// 1/m as the hardware reciprocal (within 1 ulp) refined by one Newton step,
// r + r (1 - m r): one division per node (G2P evaluates each node once per
// window that covers it), and p (1/m) is within an ulp of p/m.
__device__ __forceinline__ float inv_mass(float m) {
  const float r0 = __builtin_amdgcn_rcpf(m);
  return fmaf(r0, fmaf(-m, r0, 1.f), r0);
}

// The grid update -- v = p/m + dt g where m > 0, sticky walls -- is
// evaluated by G2P on its window nodes as it loads them (grid_velocity), and
// the accumulator is cleared by the P2G two steps later, so the step needs
// no separate pass over the grid.
__device__ __forceinline__ float4 grid_velocity(const SimDev &s, float4 acc, int gx, int gy, int gz) {
  const int n = s.n, wall = s.wall;
  float4 o = make_float4(0.f, 0.f, 0.f, acc.x);
  const bool in_wall = gx < wall || gy < wall || gz < wall || gx >= n - wall || gy >= n - wall || gz >= n - wall;
  if (acc.x > 0.f && !in_wall) {
    const float inv = inv_mass(acc.x);
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
// cube), 8 cubes per load instruction, 4 instructions.  This lane's word for
// instruction t (all ones when cube 8t + lane / 8 is past the 27th) packs
//   bits 0-9   8 cx + 32 cy + 128 cz + j: the node's offset, in node-index
//              units, from the first node of the window origin's node-block
//              when each axis' origin is a multiple of 8 (cube (cx, cy, cz)
//              of the window, node j = jx + 2 jy + 4 jz in the cube);
//   bits 10-17 its window index (wz PW + wy) PW + wx;
//   bits 18-20 cx == 2, cy == 2, cz == 2.
// A window origin is a multiple of 4 per axis.  When it is 4 mod 8 on an
// axis, that axis' cube coordinates 0 and 1 fall on the origin block's
// cubes 2 and 3 (offset +16, +64, +128 x 2 node-index units for x, y, z) and
// coordinate 2 on the next block's cube 0: the offsets below add these as
// uniform terms.
constexpr uint32_t WIN_NONE = 0xFFFFFFFFu;
__device__ __forceinline__ void window_lanes(uint32_t wpack[4]) {
  const int lane = threadIdx.x;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int cb = 8 * t + (lane >> 3), j = lane & 7;
    const int cx = cb % 3, cy = (cb / 3) % 3, cz = cb / 9;
    const int wx = 2 * cx + (j & 1), wy = 2 * cy + ((j >> 1) & 1), wz = 2 * cz + (j >> 2);
    const uint32_t base = (uint32_t)(8 * cx + 32 * cy + 128 * cz + j);
    const uint32_t li = (uint32_t)((wz * PW + wy) * PW + wx);
    const uint32_t c2 = (cx == 2 ? 1u : 0u) | (cy == 2 ? 2u : 0u) | (cz == 2 ? 4u : 0u);
    wpack[t] = cb < 27 ? (base | li << 10 | c2 << 18) : WIN_NONE;
  }
}
__device__ __forceinline__ int wp_li(uint32_t w) { return (int)((w >> 10) & 0xFFu); }
__device__ __forceinline__ void wp_coords(uint32_t w, int &wx, int &wy, int &wz) {
  const int li = wp_li(w);
  wx = li % PW;
  wy = (li / PW) % PW;
  wz = li / (PW * PW);
}

// Whether the window at (ox0, oy0, oz0) lies inside the grid, and whether it
// also holds no sticky-wall node: uniform per chunk, so most windows take the
// fast paths below without per-node bounds and wall tests.
__device__ __forceinline__ bool window_inside(const SimDev &s, int ox0, int oy0, int oz0) {
  return ox0 + PW <= s.n && oy0 + PW <= s.n && oz0 + PW <= s.n;
}
__device__ __forceinline__ bool window_off_walls(const SimDev &s, int ox0, int oy0, int oz0) {
  const int lo = s.wall, hi = s.n - s.wall;
  return ox0 >= lo && oy0 >= lo && oz0 >= lo && ox0 + PW <= hi && oy0 + PW <= hi && oz0 + PW <= hi;
}

// Requests the accumulator values (m, p) of the window at (ox0, oy0, oz0)
// from accumulator a; nodes outside the grid read as zero.
__device__ __forceinline__ void fetch_window(const SimDev &s, int a, int ox0, int oy0, int oz0, const uint32_t wpack[4],
                                             float4 acc[4]) {
  if (window_inside(s, ox0, oy0, oz0)) {
    const uint32_t nbs = (uint32_t)s.nb;
    const uint32_t px = (uint32_t)(ox0 >> 2) & 1u, py = (uint32_t)(oy0 >> 2) & 1u, pz = (uint32_t)(oz0 >> 2) & 1u;
    const uint32_t s0 = 16u * px + 64u * py + 256u * pz;
    const uint32_t dx2 = px * 480u, dy2 = py * (nbs * 512u - 128u), dz2 = pz * (nbs * nbs * 512u - 512u);
    float4 *gblk = s.gridA[a] + (((size_t)(oz0 >> 3) * nbs + (size_t)(oy0 >> 3)) * nbs + (size_t)(ox0 >> 3)) * 512u;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc[t] = make_float4(0.f, 0.f, 0.f, 0.f);
      const uint32_t w = wpack[t];
      const uint32_t off = (w & 0x3FFu) + s0 + ((w >> 18) & 1u) * dx2 + ((w >> 19) & 1u) * dy2 + ((w >> 20) & 1u) * dz2;
      if (t < 3 || w != WIN_NONE) acc[t] = at_byte(gblk, 16u * off);
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    acc[t] = make_float4(0.f, 0.f, 0.f, 0.f);
    int wx, wy, wz;
    wp_coords(wpack[t], wx, wy, wz);
    const int gx = ox0 + wx, gy = oy0 + wy, gz = oz0 + wz;
    if (wpack[t] != WIN_NONE && gx < s.n && gy < s.n && gz < s.n) acc[t] = s.gridA[a][node_index(s, gx, gy, gz)];
  }
}

// Converts fetched window values to grid velocities (the grid update) in LDS,
// three floats per node: packed, the gather's reads of a round hit fewer
// banks together than at a 16-byte stride (measured: G2P 0.070 -> 0.063 ms
// on the 4M dam break, 0.059 -> 0.054 on the 3.1M sand column).
__device__ __forceinline__ void store_window(const SimDev &s, const float4 acc[4], const uint32_t wpack[4], int ox0,
                                             int oy0, int oz0, float3 *win) {
  if (window_inside(s, ox0, oy0, oz0) && window_off_walls(s, ox0, oy0, oz0)) {
    const float gx = s.dt * s.g[0], gy = s.dt * s.g[1], gz = s.dt * s.g[2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t == 3 && wpack[t] == WIN_NONE) continue;
      const float4 m = acc[t];
      float4 o = make_float4(0.f, 0.f, 0.f, m.x);
      if (m.x > 0.f) {
        const float inv = inv_mass(m.x);
        o.x = m.y * inv + gx;
        o.y = m.z * inv + gy;
        o.z = m.w * inv + gz;
      }
      win[wp_li(wpack[t])] = make_float3(o.x, o.y, o.z);
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (wpack[t] == WIN_NONE) continue;
    int wx, wy, wz;
    wp_coords(wpack[t], wx, wy, wz);
    const int gx = ox0 + wx, gy = oy0 + wy, gz = oz0 + wz;
    const float4 o =
        (gx < s.n && gy < s.n && gz < s.n) ? grid_velocity(s, acc[t], gx, gy, gz) : make_float4(0.f, 0.f, 0.f, 0.f);
    win[(wz * PW + wy) * PW + wx] = make_float3(o.x, o.y, o.z);
  }
}

// Gather of one particle at xp: v = sum w v_i and B = sum w v_i (o - f)^T
// (C = 4/dx^2 B dx, applied by the caller), from the velocity window of the
// bin at (ox0, oy0, oz0), or from accumulator a with the grid update for a
// particle whose stencil is outside the window (it left the chunk's bin
// since the last sort: only in steps without a sort; rare).
__device__ __forceinline__ void gather_particle(const SimDev &s, const float3 *win, int a, const float xp[3], int ox0,
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
  // columns of B as B_a = sum w o_a v_i - f_a v.
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
    // Reduced one axis at a time: along x for each (y, z) row, then along y
    // in each z plane, then along z.  With t = w_1 a_1 formed once, a sum
    // w_0 a_0 + w_1 a_1 + w_2 a_2 and its first moment w_1 a_1 + 2 w_2 a_2
    // share that product.  Per plane: P = sum_y w_y S, PU = sum_y w_y U,
    // PY = sum_y w_y oy S; then v = sum_z w_z P, B_x = sum_z w_z PU,
    // B_y = sum_z w_z PY, B_z = sum_z w_z oz P.
    const float w2y = 2.f * w[1][2], w2z = 2.f * w[2][2];
    float P[3][3], PU[3][3], PY[3][3];
#pragma unroll
    for (int oz = 0; oz < 3; ++oz) {
      float S[3][3], U[3][3];
#pragma unroll
      for (int oy = 0; oy < 3; ++oy) {
        const float3 g0 = win[li0 + (oz * PW + oy) * PW + 0];
        const float3 g1 = win[li0 + (oz * PW + oy) * PW + 1];
        const float3 g2 = win[li0 + (oz * PW + oy) * PW + 2];
        const float a0[3] = {g0.x, g0.y, g0.z}, a1[3] = {g1.x, g1.y, g1.z}, a2[3] = {g2.x, g2.y, g2.z};
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          const float t = w[0][1] * a1[k];
          S[oy][k] = fmaf(w[0][2], a2[k], fmaf(w[0][0], a0[k], t));
          U[oy][k] = fmaf(w2x, a2[k], t);
        }
      }
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const float t = w[1][1] * S[1][k];
        P[oz][k] = fmaf(w[1][2], S[2][k], fmaf(w[1][0], S[0][k], t));
        PY[oz][k] = fmaf(w2y, S[2][k], t);
        PU[oz][k] = fmaf(w[1][2], U[2][k], fmaf(w[1][1], U[1][k], w[1][0] * U[0][k]));
      }
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const float t = w[2][1] * P[1][k];
      v[k] = fmaf(w[2][2], P[2][k], fmaf(w[2][0], P[0][k], t));
      B[k * 3 + 2] = fmaf(w2z, P[2][k], t);
      B[k * 3 + 0] = fmaf(w[2][2], PU[2][k], fmaf(w[2][1], PU[1][k], w[2][0] * PU[0][k]));
      B[k * 3 + 1] = fmaf(w[2][2], PY[2][k], fmaf(w[2][1], PY[1][k], w[2][0] * PY[0][k]));
    }
  }
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int c2 = 0; c2 < 3; ++c2) B[k * 3 + c2] = fmaf(d[c2][0], v[k], B[k * 3 + c2]);  // d[c2][0] = -f_c2
}

// Advection x + dt v, clamped to the box; the number of clamped components
// and whether a value (of x, v or C = c_scale B, which the caller stores) is
// not finite.
__device__ __forceinline__ void advect(const SimDev &s, const float xp[3], const float v[3], const float B[9],
                                       float xn[3], float C[9], uint32_t &clamped, bool &nonfinite) {
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const float xa = fmaf(s.dt, v[k], xp[k]);
    if (!isfinite(xa) || !isfinite(v[k])) nonfinite = true;
    if (xa < s.lo || xa > s.hi) ++clamped;
    xn[k] = advanced(s, xp[k], v[k]);
  }
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    C[k] = s.c_scale * B[k];
    if (!isfinite(C[k])) nonfinite = true;
  }
}

// The G2P of the step that accumulated into a: particles of layout lay (the
// one P2G built), v and C written in place (x stays: the next P2G advances
// it with that v), and the next step's bin keys and
// counts.
template <int MAT>
__device__ __forceinline__ void g2p_step(const SimDev &s, int lay, int a, float3 *win) {
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
  uint4 ch_next = make_uint4(0u, 0u, 0u, 0u);  // chunk records are loaded one chunk ahead
  if (qbeg + wq < qend) ch_next = load_record(chunks + qbeg + wq);
  for (uint32_t c = qbeg + wq; c < qend; c += nwq) {
    const uint4 ch = ch_next;
    if (c + nwq < qend) ch_next = load_record(chunks + c + nwq);
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
        uint32_t clamped = 0;
        bool nonfinite = false;
        advect(s, xp, v, B, xn, Cn, clamped, nonfinite);
        int b[3];
        // (the new position is not stored: the next P2G, or the readback,
        // forms it again from x and the v stored here, bit for bit)
#pragma unroll
        for (int k = 0; k < 3; ++k) {
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
        if (clamped) flag_status(s, MPM_STATUS_CLAMPED, 1, clamped);
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

// G2P of a step that reads buffer src (accumulator a): writes v and C in
// place in layout src ^ 1 (x stays; the next P2G advances it) and the next
// step's bin keys and counts.
template <int MAT>
__global__ __launch_bounds__(64, 5) void k_g2p(SimDev s, int src, int a) {
  __shared__ float3 win[PW3];
  g2p_step<MAT>(s, src ^ 1, a, win);
  g2p_handoff(s, src ^ 1);
}
