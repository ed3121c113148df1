// sort.h -- creation, sort policy, the bin scans and the bucket scatter
// Part of mpm.hip: included there, inside its anonymous namespace, after the
// parts before it; not a standalone header.

// --------------------------------------------------------------- kernels

// Creation: AoS inputs -> SoA buffer 0 (creation order), ids, first keys.
// F (J) is stored as F - I (J - 1).
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
    // the deformation is stored as F - I (J - 1): see update_F
    if (s.material == MPM_J_FLUID) {
      b.F[i] = F0 ? F0[i] - 1.f : 0.f;
    } else {
      for (int k = 0; k < 9; ++k) b.F[k * Np + i] = F0 ? F0[9 * (size_t)i + k] - ((k % 4 == 0) ? 1.f : 0.f) : 0.f;
    }
    if (s.has_E) b.E[i] = E_p ? E_p[i] : s.snow_a0;  // snow: the slot holds the log plastic volume
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

__global__ __launch_bounds__(WG) void k_copy_u32(uint32_t *dst, const uint32_t *src, int n) {
  for (int k = threadIdx.x; k < n; k += blockDim.x) dst[k] = src[k];
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
// so a run of consecutive slots holds about one particle per cell, while a
// chunk's cells as a whole may be far from balanced (particles created cell
// by cell stay together).  For Cp = 2, 4 or 8 full chunks, the blocks are
// transposed -- new chunk q takes block q of every old chunk -- so each new
// chunk draws evenly from all of them and needs fewer read-modify-write
// passes.  Blocks hold at least one round of 64 particles when a chunk has
// several rounds, and at least 8 particles in one-round chunks.  Other
// stayers keep their order.
__device__ __forceinline__ uint32_t stayer_slot(uint32_t j, uint32_t stay, uint32_t kshift) {
  const uint32_t full = stay >> kshift, cap = kshift == (uint32_t)KMIN_SHIFT ? 8u : 1u << (kshift - KMIN_SHIFT);
  const uint32_t f = min(full, cap);
  const uint32_t cp = f >= 8u ? 8u : (f >= 4u ? 4u : (f >= 2u ? 2u : 1u));
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
    ch_next = load_record(chunks + blockIdx.x);
    if (blockIdx.x > 0) prev_next = load_record(chunks + blockIdx.x - 1).z;
  }
  for (uint32_t c = blockIdx.x; c < nch; c += gridDim.x) {
    const uint4 ch = ch_next;
    const uint32_t prev_bin = prev_next;
    const uint32_t start = ch.x, count = min(ch.y, (uint32_t)KMAX), bin = ch.z;
    if (c + gridDim.x < nch) {
      ch_next = load_record(chunks + c + gridDim.x);
      prev_next = load_record(chunks + c + gridDim.x - 1).z;
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

// ----------------------------------------------------- small-scene sort
// For a grid of at most SMALL_SORT_BINS bins (and chunks of 64), the scan
// and the scatter are one kernel.  Every workgroup forms the whole slot and
// chunk prefix of the bins itself -- a few KB of counts, and a few
// wavefront scans -- into LDS tables, so that no kernel boundary separates
// the counts from the placement: a small scene's step time is a chain of
// latencies, and a boundary costs about a microsecond.  Workgroup g writes
// the new chunk records of every G-th row of 64 bins and places the
// particles of every G-th old chunk, as k_scatter does (stayers in their
// previous order, transposed by stayer_slot; movers after the stayers of
// their bin, through a per-bin counter that starts at zero).  The counts,
// stayer counts and mover counters are read by every workgroup, so the
// step's P2G clears them (and updates the control words the one-workgroup
// scan updates); without a sort this kernel clears the counts itself.
constexpr int SMALL_SORT_BINS = 4096;

// ROUNDS = ceil(nbins / 256): the rounds of the prefix, unrolled (the bin
// counts stay in registers).
template <int ROUNDS>
__global__ __launch_bounds__(64) void k_sort_small(SimDev s, int src) {
  __shared__ uint4 tstart4[SMALL_SORT_BINS / 4];  // first slot of each bin in the new layout
  __shared__ uint2 tchunk4[SMALL_SORT_BINS / 4];  // first chunk of each bin (16 bits each)
  const int lay = src ^ 1;
  const int lane = threadIdx.x;
  const uint64_t below = (1ull << lane) - 1ull;
  const uint32_t nbins = (uint32_t)s.nbins, kshift = (uint32_t)s.chunk_shift, K = 1u << kshift;
  const uint32_t G = gridDim.x, g = blockIdx.x;
  const uint32_t nch_old = s.ctr[CTR_NCHUNKS + src];
  const uint4 *old = s.chunks[src];
  const bool sort = decide_sort(s, src);
  // (a preset decision is already in the word, which other workgroups read)
  if (g == 0 && lane == 0 && s.ctr[CTR_PRESET + src] == 0u) s.ctr[CTR_SORT + src] = sort ? 1u : 0u;
  if (!sort) {
    // Layout lay repeats layout src: its chunk list is copied, and the
    // counts are cleared for this step's G2P.
    for (uint32_t c = g * 64u + (uint32_t)lane; c < nch_old; c += G * 64u) s.chunks[lay][c] = old[c];
    for (uint32_t b = g * 64u + (uint32_t)lane; b < nbins; b += G * 64u) {
      s.bin_count[b] = 0u;
      s.stay_count[b] = 0u;
    }
    if (g == 0 && lane == 0) s.ctr[CTR_NCHUNKS + lay] = nch_old;
    return;
  }
  // (a workgroup with no old chunk and no row of bins has nothing to do)
  if (g >= nch_old && 64u * g >= nbins) return;
  // This workgroup's first old chunk and its keys, and the count of the
  // bin whose records it writes first, are requested before the tables.
  uint4 rec = make_uint4(0u, 0u, 0u, 0u);
  uint32_t key = 0u, prev_bin = 0xFFFFFFFFu;
  if (g < nch_old) {
    rec = load_record(old + g);
    if (g > 0u) prev_bin = load_record(old + g - 1u).z;
    if ((uint32_t)lane < min(rec.y, 64u)) key = s.key[rec.x + (uint32_t)lane];
  }
  const uint32_t brow = 64u * g + (uint32_t)lane;
  const uint32_t crow = brow < nbins ? s.bin_count[brow] : 0u;
  // Slot and chunk prefix: rounds of 256 bins, four consecutive bins per lane.
  static_assert(ROUNDS * 256 <= SMALL_SORT_BINS, "tables hold SMALL_SORT_BINS bins");
  // (nbins = 8^k >= 8 is a multiple of 4; the loads are unconditional, from
  // bin 0 past the end, so that they are all in flight together)
  uint4 c4[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const uint32_t b = 256u * (uint32_t)r + 4u * (uint32_t)lane;
    c4[r] = *reinterpret_cast<const uint4 *>(s.bin_count + (b < nbins ? b : 0u));
  }
  uint32_t sbase = 0u, cbase = 0u;  // slots and chunks of the bins of the earlier rounds
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const bool in = 256u * (uint32_t)r + 4u * (uint32_t)lane < nbins;
    const uint4 c = make_uint4(in ? c4[r].x : 0u, in ? c4[r].y : 0u, in ? c4[r].z : 0u, in ? c4[r].w : 0u);
    const uint32_t p0 = padded(c.x), p1 = padded(c.y), p2 = padded(c.z), p3 = padded(c.w);
    const uint32_t k0 = (c.x + K - 1u) >> kshift, k1 = (c.y + K - 1u) >> kshift, k2 = (c.z + K - 1u) >> kshift,
                   k3 = (c.w + K - 1u) >> kshift;
    const uint32_t ps = p0 + p1 + p2 + p3, ks = k0 + k1 + k2 + k3;
    const uint32_t pi = wave_incl_scan(ps), ki = wave_incl_scan(ks);
    const uint32_t pe = sbase + pi - ps, ke = cbase + ki - ks;
    tstart4[64 * r + lane] = make_uint4(pe, pe + p0, pe + p0 + p1, pe + p0 + p1 + p2);
    tchunk4[64 * r + lane] = make_uint2(ke | ((ke + k0) << 16), (ke + k0 + k1) | ((ke + k0 + k1 + k2) << 16));
    sbase += (uint32_t)__builtin_amdgcn_readlane((int)pi, 63);
    cbase += (uint32_t)__builtin_amdgcn_readlane((int)ki, 63);
  }
  __syncthreads();
  const uint32_t *tstart = reinterpret_cast<const uint32_t *>(tstart4);
  const uint16_t *tchunk = reinterpret_cast<const uint16_t *>(tchunk4);
  // New chunk records of rows g, g + G, ... of 64 bins.
  for (uint32_t b = brow; b - (uint32_t)lane < nbins; b += 64u * G) {
    const uint32_t cnt = b == brow ? crow : (b < nbins ? s.bin_count[b] : 0u);
    if (b < nbins && cnt > 0u) {
      const uint32_t p0 = tstart[b], k0 = tchunk[b];
      for (uint32_t j = 0, off = 0; off < cnt; ++j, off += K)
        s.chunks[lay][k0 + j] = make_uint4(p0 + off, min(K, cnt - off), b, min(K, cnt - off));
    }
  }
  if (g == 0 && lane == 0) s.ctr[CTR_NCHUNKS + lay] = cbase;
  // Placement of the particles of old chunks g, g + G, ...
  for (uint32_t c = g; c < nch_old; c += G) {
    if (c != g) {
      rec = load_record(old + c);
      prev_bin = load_record(old + c - 1u).z;
      key = (uint32_t)lane < min(rec.y, 64u) ? s.key[rec.x + (uint32_t)lane] : 0u;
    }
    const uint32_t start = rec.x, count = min(rec.y, 64u), bin = rec.z;
    const uint32_t bstay = min(s.stay_count[bin], s.bin_count[bin]);
    // stayers of the bin's earlier chunks (a bin's chunks are consecutive;
    // nearly always none, or a few records)
    uint32_t base = 0u;
    for (uint32_t c0 = c; prev_bin == bin && c0 > 0u;) {
      const uint32_t lo = c0 > 64u ? c0 - 64u : 0u;
      const uint32_t cj = lo + (uint32_t)lane;
      uint4 r = make_uint4(0u, 0u, 0xFFFFFFFFu, 0u);
      if (cj < c0) r = old[cj];
      const bool same = cj < c0 && r.z == bin;
      uint32_t add = same ? r.w : 0u;
      for (int d = 32; d >= 1; d >>= 1) add += (uint32_t)__shfl_xor((int)add, d);
      base += add;
      if (__ballot(same) != ~0ull || lo == 0u) break;
      c0 = lo;
    }
    const bool valid = (uint32_t)lane < count;
    const uint32_t kb = min(key & ((1u << KEY_CELL_SHIFT) - 1u), nbins - 1u);
    const bool stay = valid && kb == bin;
    const uint64_t sm = __ballot(stay);
    uint32_t slot = tstart[bin] + stayer_slot(base + (uint32_t)__popcll(sm & below), bstay, kshift);
    if (__ballot(valid && !stay) != 0ull) {
      const uint32_t off = wave_aggregated_increment(s.bin_cursor, kb, valid && !stay);
      if (valid && !stay) slot = tstart[kb] + min(s.stay_count[kb], s.bin_count[kb]) + off;
    }
    if (valid && slot < (uint32_t)s.Np) {
      s.perm[slot] = start + (uint32_t)lane;
      s.cellp[slot] = (uint8_t)(key >> KEY_CELL_SHIFT);
    }
  }
}
