// fused.h -- fused G2P2G pass for steps without a sort
// Part of mpm.hip: included there, inside its anonymous namespace, after the
// parts before it; not a standalone header.

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
  float3 vel[PW3];          // the step's grid velocities around the bin
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
__device__ __forceinline__ void fused_step(const SimDev &s, int src, int a, bool write_vc, bool copy_ids,
                                           FusedShared &sm) {
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
  if (qbeg + wq < qend) ch_next = load_record(chunks + qbeg + wq);
  for (uint32_t c = qbeg + wq; c < qend; c += nwq) {
    const uint4 ch = ch_next;
    if (c + nwq < qend) ch_next = load_record(chunks + c + nwq);
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
      idq = copy_ids ? stream_load(at_byte(in.id, sn)) : 0u;
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
      const float E = MAT == MPM_SNOW ? s.E : Eq;  // snow: the slot holds the log plastic volume
      float ap = Eq;
      if (valid && copy_ids) stream_store(idq, at_byte(out.id, so));
      if (r0 + 64u < count) {
        const bool vn = r0 + 64u + (uint32_t)lane < count;
        const uint32_t sn = 4u * (start + (vn ? r0 + 64u + (uint32_t)lane : 0u));
#pragma unroll
        for (int k = 0; k < 3; ++k) xq[k] = at_byte(in.x + k * Np, sn);
#pragma unroll
        for (int k = 0; k < FW; ++k) Fq[k] = stream_load(at_byte(in.F + k * Np, sn));
        if (HAS_E) Eq = stream_load(at_byte(in.E, sn));
        if (copy_ids) idq = stream_load(at_byte(in.id, sn));
      }
      float v[3], B[9], xn[3], Cn[9];
      gather_particle(s, sm.vel, a, xp, ox0, oy0, oz0, v, B);
      uint32_t clamped = 0;
      bool nonfinite = false;
      advect(s, xp, v, B, xn, Cn, clamped, nonfinite);
      // P2G of step n + 1: F update with the new C, stress, deposit at xn
      update_F<MAT>(Fp, Cn, dt);
      float A[9];
      uint32_t st = 0;
      if (MAT == MPM_SAND || MAT == MPM_SNOW) st = plastic_affine<MAT>(s, Fp, E, ap, Cn, A, true);  // projection and stress
      if (valid) {
#pragma unroll
        for (int k = 0; k < 3; ++k) at_byte(out.x + k * Np, so) = xn[k];
#pragma unroll
        for (int k = 0; k < FW; ++k) stream_store(Fp[k], at_byte(out.F + k * Np, so));
        if (HAS_E && (copy_ids || MAT == MPM_SNOW)) stream_store(MAT == MPM_SNOW ? ap : E, at_byte(out.E, so));
        if (write_vc) {
#pragma unroll
          for (int k = 0; k < 3; ++k) stream_store(v[k], at_byte(out.v + k * Np, so));
#pragma unroll
          for (int k = 0; k < 9; ++k) stream_store(Cn[k], at_byte(out.C + k * Np, so));
        }
        if (clamped) flag_status(s, MPM_STATUS_CLAMPED, 1, clamped);
        if (nonfinite) flag_status(s, MPM_STATUS_NONFINITE, 3);
      }
      if (MAT != MPM_SAND && MAT != MPM_SNOW) st = affine_momentum<MAT>(s, Fp, E, Cn, A);
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
    flush_windows<NWIN>(s, sm.win, ox0, oy0, oz0, a1);
    if (lane == 0 && nmov) atomicAdd(s.ctr + CTR_MOVERS, nmov);  // for the sort decision two steps on
    __syncthreads();  // the windows are cleared for the next chunk
  }
}

// Step n reads buffer src and accumulated into a; write_vc: store v and C
// (the last step of a launch, so that the state can be read back); sched:
// whether the next step sorts, 0 or 1 when the host schedules the sorts
// (a fixed interval), -1 to decide here by the policy; copy_ids: copy the
// ids and the per-particle modulus to the output buffer (0 only when the
// host knows that both buffers already hold them at these slots: a fused
// pass after the first one since a sort, which copied them; snow's log
// plastic volume changes and is always written).  Leaves the next step's
// sort decision and whether its P2G is done.
template <int MAT, bool HAS_E>
__global__ __launch_bounds__(64) void k_g2p2g(SimDev s, int src, int a, int write_vc, int sched, int copy_ids) {
  __shared__ FusedShared sm;
  // uniform: the words sort_next_step reads do not change in this kernel
  const bool next_sort = sched < 0 ? sort_next_step(s) : sched != 0;
  if (next_sort) g2p_step<MAT>(s, src ^ 1, a, sm.vel);
  else fused_step<MAT, HAS_E>(s, src, a, write_vc != 0, copy_ids != 0, sm);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    // F in layout src ^ 1 is one update behind after the plain G2P; after the
    // fused pass the state of the next step's P2G is in buffer src, current.
    s.ctr[CTR_PENDING] = 1u;
    s.ctr[CTR_LOOK + (src ^ 1)] = next_sort ? 0u : 1u;
    s.ctr[CTR_PRESET + (src ^ 1)] = 1u;
    s.ctr[CTR_SORT + (src ^ 1)] = next_sort ? 1u : 0u;
  }
}
