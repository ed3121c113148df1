// readback.h -- readback of particles (creation order) and of the grid
// Part of mpm.hip: included there, inside its anonymous namespace, after the
// parts before it; not a standalone header.

// Readback: unpermute to creation order, apply the pending advection and F (or J) update
// (and for sand and snow the projection that follows it; alpha: snow's log
// plastic volume after that projection, or NULL).
// Single-wavefront workgroups walk the chunk list of layout cur (the slots
// between bins are padding).  After a fused G2P2G pass the state is in the
// same slots of the other buffer, with F current.
template <int MAT>
__global__ __launch_bounds__(64) void k_read_particles(SimDev s, int cur, float *__restrict__ x, float *__restrict__ v,
                                                       float *__restrict__ C, float *__restrict__ F,
                                                       float *__restrict__ alpha) {
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
        const float xa = b.x[a * Np + slot], va = b.v[a * Np + slot];
        if (x) x[3 * id + a] = pending ? advanced(s, xa, va) : xa;
        if (v) v[3 * id + a] = va;
      }
      if (C)
        for (int k = 0; k < 9; ++k) C[9 * id + k] = Cp[k];
      if (!F && !alpha) continue;
      // (stored as J - 1 and F - I: see update_F)
      if (MAT == MPM_J_FLUID) {
        float j = b.F[slot];
        if (pending) update_F<MPM_J_FLUID>(&j, Cp, dt);
        F[id] = 1.f + j;
      } else {
        float Hp[9];
        for (int k = 0; k < 9; ++k) Hp[k] = b.F[k * Np + slot];
        float ap = MAT == MPM_SNOW ? b.E[slot] : 0.f;
        if (pending) {
          update_F<MPM_FIXED_COROTATED>(Hp, Cp, dt);
          if (MAT == MPM_SAND || MAT == MPM_SNOW) {  // and the plasticity projection that follows the update
            float A[9];
            (void)plastic_affine<MAT>(s, Hp, s.E, ap, Cp, A, true);
          }
        }
        if (F)
          for (int k = 0; k < 9; ++k) F[9 * id + k] = Hp[k] + ((k % 4 == 0) ? 1.f : 0.f);
        if (MAT == MPM_SNOW && alpha) alpha[id] = ap;
      }
    }
  }
}

// Readback of the grid after the last step (its accumulator q): the node-blocks it
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
