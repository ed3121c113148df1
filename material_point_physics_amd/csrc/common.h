// common.h -- constants, control words, device state and device utilities
// Part of mpm.hip: included there, inside its anonymous namespace, after the
// parts before it; not a standalone header.

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
  float *F;      // [9][Np] F - I (elastic, sand, snow) or [1][Np] J - 1 (fluid), one step behind: see update_F
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
  float kappa_per_E;          // snow: bulk modulus per unit Young's modulus, 1 / (3 (1 - 2 nu))
  float snow_m2, snow_beta, snow_xi, snow_1p2b;  // snow: M^2, beta, xi, 1 + 2 beta
  float snow_a0;              // snow: initial log plastic volume
  float stress_k;             // dt * V0 * 4 / dx^2
  float c_scale;              // 4 / dx (G2P: C = 4/dx^2 * sum w v (x_i - x_p), offsets in cells)
  float lo, hi;               // position clamp
  uint32_t max_chunks;
  int32_t chunk_shift;        // chunks hold up to 2^chunk_shift (64..KMAX) particles of one bin
  int32_t sort_small;         // 1: k_sort_small sorts (the step's P2G then keeps the control words)
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

// x + dt v, clamped into [lo, hi]: G2P's new position.  G2P does not store
// it; the next P2G and the readback form it again from the stored x and v,
// with this one expression (an explicit fused multiply-add), so every side
// gets the same bits.
__device__ __forceinline__ float advanced(const SimDev &s, float x, float v) {
  return fminf(fmaxf(fmaf(s.dt, v, x), s.lo), s.hi);
}

// ------------------------------------------------------------ device utils

// A uniform record (a chunk record) read through the scalar data cache: the
// address is made wave-uniform and read in the constant address space, so the
// load is a scalar one.  Chunk records are written by an earlier kernel and
// only read by the kernels that use this (a wave may write the stayer count
// of a record it has read; no wave reads a record another one writes).
// Scalar loads are counted apart from vector memory operations, so waiting
// for a record does not also wait for the wave's outstanding vector stores
// and float atomics (which a vector load issued after them would).
__device__ __forceinline__ uint4 load_record(const uint4 *p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 r = *reinterpret_cast<const __attribute__((address_space(4))) u32x4 *>(((uint64_t)hi << 32) | lo);
  return make_uint4(r.x, r.y, r.z, r.w);
}

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

// Cell of a base node within its 4^3-cell bin, and the key word that
// carries it above the bin index.  grid_n <= 1024 keeps bins below 2^24.
// The number only orders a chunk's particles (the deposit passes take lanes
// in cell order): x fastest, then z, then y, so that 16 consecutive cells
// form an (x, z) plane, whose window nodes (strides 1 and 36, which is 4 mod
// 16) fall in 16 distinct 16-byte LDS bank groups for every stencil offset.
constexpr int KEY_CELL_SHIFT = 24;
__device__ __forceinline__ uint32_t cell_in_bin(int bx, int by, int bz) {
  return ((uint32_t)(by & 3) << 4) | ((uint32_t)(bz & 3) << 2) | (uint32_t)(bx & 3);
}

// Quadratic B-spline weights of nodes base+0,1,2 at fractional offset f in [0.5,1.5).
__device__ __forceinline__ void bspline_weights(float f, float w[3]) {
  const float a = 1.5f - f, b = f - 1.0f, c = f - 0.5f;
  w[0] = 0.5f * a * a;
  w[1] = 0.75f - b * b;
  w[2] = 0.5f * c * c;
}

// Inclusive prefix sum over the wavefront's 64 lanes (Hillis-Steele with DPP
// row shifts by 1, 2, 4 and 8 lanes within each row of 16, then the
// broadcasts of lane 15 into rows 1 and 3 and of lane 31 into rows 2 and 3).
// Lanes a shift reaches past the row's start, and rows a broadcast skips,
// add the 0 they receive.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
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

__device__ __forceinline__ void flag_status(const SimDev &s, uint32_t bit, int counter_word, uint32_t amount = 1u) {
  atomicOr(&s.status[0], bit);
  if (counter_word > 0) atomicAdd(&s.status[counter_word], amount);
}
