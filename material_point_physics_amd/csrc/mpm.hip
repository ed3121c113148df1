// mpm.hip -- MI355X (gfx950) implementation of one explicit MLS-MPM step
// behind the C ABI declared in include/mpm.h.
//
// Method: "Principles towards Real-Time Simulation of Material Point Method on
// Modern GPUs" (below [RT-MPM]) splits a step into particle sorting, P2G,
// grid update and G2P; the equations are the textbook MLS-MPM with quadratic
// B-splines, APIC transfer and the fixed-corotated model (Hu et al. 2018;
// Jiang et al. 2015; Stomakhin et al. 2012), plus a weakly compressible
// fluid, Drucker-Prager sand (Klar et al. 2016) and non-associative Cam-clay
// snow (Wolper et al. 2019), the last two on Hencky elasticity.
//
// Step = 5 kernels, captured into HIP graphs per phase (step number mod 4:
// the particle buffer and the grid accumulator the step uses):
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
//                 chose; the next step's bin keys/counts (v and C are stored;
//                 the advected x is not: the next P2G forms it again from x
//                 and v, bit for bit)
//
// Between sorts (mpm_set_sort_policy), k_g2p2g can replace k_g2p: the G2P of
// the step and the P2G of the next in one pass (mpm_set_fused_steps).
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

#include <mutex>

// Static scratch of mpm_run_noalloc: the workspace of a run that allocates
// nothing.  Every device the library runs on holds its own copy until the
// process ends.  In host code the name `scratch` is only a stand-in for the
// array, never a device address: host code uses the address that
// hipGetSymbolAddress returns for the current device (noalloc_scratch).
static __device__ __align__(256) unsigned char scratch[MPM_NOALLOC_SCRATCH_BYTES];

namespace {

#include "common.h"
#include "linalg.h"
#include "sort.h"
#include "materials.h"
#include "p2g.h"
#include "g2p.h"
#include "fused.h"
#include "readback.h"

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
  if (p->material != MPM_FIXED_COROTATED && p->material != MPM_J_FLUID && p->material != MPM_SAND &&
      p->material != MPM_SNOW)
    return false;
  if (p->material == MPM_SAND && !(p->friction_deg > 0.f && p->friction_deg < 90.f)) return false;
  if (p->material == MPM_SNOW) {
    // (the tips divide by the bulk modulus: E > 0)
    if (!(p->E > 0.f) || !(p->snow_M > 0.f) || !std::isfinite(p->snow_M)) return false;
    if (!(p->snow_beta >= 0.f) || !std::isfinite(p->snow_beta)) return false;
    if (!(p->snow_xi >= 0.f) || !std::isfinite(p->snow_xi) || !std::isfinite(p->snow_alpha0)) return false;
  }
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
    // snow (non-associative Cam-clay): kappa = lam + 2 mu / 3 = E / (3 (1 - 2 nu))
    d->kappa_per_E = (float)(1.0 / (3.0 * (1.0 - 2.0 * nu)));
    d->snow_m2 = (float)((double)p->snow_M * (double)p->snow_M);
    d->snow_beta = p->snow_beta;
    d->snow_xi = p->snow_xi;
    d->snow_1p2b = (float)(1.0 + 2.0 * (double)p->snow_beta);
    d->snow_a0 = p->snow_alpha0;
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
  // Recorded after every operation the handle enqueues, on the caller's
  // stream: destroying graphs (or the handle) first waits for it, so no
  // graph is destroyed while a launch of it is pending, and the caller may
  // free the workspace once mpm_destroy returns.
  hipEvent_t done = nullptr;
  hipGraph_t graph[3][2 * MAX_PERIOD] = {};
  hipGraphExec_t exec[3][2 * MAX_PERIOD] = {};
  int grid_particles = 0;  // ceil(N / WG), rounded up to a multiple of 8
  int grid_scatter = 0;
  int grid_p2g = 0;
  bool p2g_wide = false;  // small scene: P2G with NWIN_WIDE windows per wavefront
  int grid_sort_small = 0;  // k_sort_small's launch (d.sort_small)
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

// P2G of the step of phase p with NW accumulation windows per wavefront.
template <int NW>
void launch_p2g(const mpm_sim *sim, hipStream_t st, int src, int p) {
  const SimDev &d = sim->d;
  const int g = sim->grid_p2g;
  if (d.material == MPM_J_FLUID) {
    if (d.has_E) k_p2g<MPM_J_FLUID, true, NW><<<g, 64, 0, st>>>(d, src, p);
    else k_p2g<MPM_J_FLUID, false, NW><<<g, 64, 0, st>>>(d, src, p);
  } else if (d.material == MPM_SAND) {
    if (d.has_E) k_p2g<MPM_SAND, true, NW><<<g, 64, 0, st>>>(d, src, p);
    else k_p2g<MPM_SAND, false, NW><<<g, 64, 0, st>>>(d, src, p);
  } else if (d.material == MPM_SNOW) {  // (its scalar slot always carries the log plastic volume)
    k_p2g<MPM_SNOW, true, NW><<<g, 64, 0, st>>>(d, src, p);
  } else {
    if (d.has_E) k_p2g<MPM_FIXED_COROTATED, true, NW><<<g, 64, 0, st>>>(d, src, p);
    else k_p2g<MPM_FIXED_COROTATED, false, NW><<<g, 64, 0, st>>>(d, src, p);
  }
}

// Phase 0 (tile totals) or 1 (bins) of the scan of a step that reads
// buffer src.  (A small grid's bins are scanned by one workgroup, without
// tile totals.)
void launch_scan(const mpm_sim *sim, hipStream_t st, int src, int phase) {
  const SimDev &d = sim->d;
  const bool tiles = d.nbins > SCAN_SMALL_NT * SCAN_PER;
  if (phase == 0) {
    if (tiles) k_scan_tiles<<<d.ntiles, WG, 0, st>>>(d, src);
  } else if (tiles) {
    k_scan_bins<WG><<<d.ntiles, WG, 0, st>>>(d, src ^ 1);
  } else {
    k_scan_bins<SCAN_SMALL_NT><<<1, SCAN_SMALL_NT, 0, st>>>(d, src ^ 1);
  }
}

// Kernel k of the step of phase p (reads buffer src = (p + 1) mod 2,
// accumulates into p); fused: the plain G2P is replaced by the G2P2G kernel,
// which stores v and C when write_vc is set and takes the next step's sort
// decision from sched (-1: by the policy, on the device).
int launch_kernel(mpm_sim *sim, int k, hipStream_t st, int p, bool fused, bool write_vc, int sched,
                  int copy_ids = 1) {
  const int src = (p + 1) & 1;
  const SimDev &d = sim->d;
  switch (k) {
    case 0:
      if (!d.sort_small) launch_scan(sim, st, src, 0);
      break;
    case 1:
      if (d.sort_small) {
        // (nbins = 8^k: 8, 64, 512 or 4096 bins, in 1, 1, 2 or 16 rounds of 256)
        if (d.nbins <= 256) k_sort_small<1><<<sim->grid_sort_small, 64, 0, st>>>(d, src);
        else if (d.nbins <= 512) k_sort_small<2><<<sim->grid_sort_small, 64, 0, st>>>(d, src);
        else k_sort_small<SMALL_SORT_BINS / 256><<<sim->grid_sort_small, 64, 0, st>>>(d, src);
      }
      else launch_scan(sim, st, src, 1);
      break;
    case 2:
      if (!d.sort_small) k_scatter<<<sim->grid_scatter, 64, 0, st>>>(d, src);
      break;
    case 3:
      if (sim->p2g_wide) launch_p2g<NWIN_WIDE>(sim, st, src, p);
      else launch_p2g<NWIN>(sim, st, src, p);
      break;
    case 4:
      if (fused) {
        const int wv = write_vc ? 1 : 0;
        const int g = sim->grid_g2p2g;
        if (d.material == MPM_J_FLUID) {
          if (d.has_E) k_g2p2g<MPM_J_FLUID, true><<<g, 64, 0, st>>>(d, src, p, wv, sched, copy_ids);
          else k_g2p2g<MPM_J_FLUID, false><<<g, 64, 0, st>>>(d, src, p, wv, sched, copy_ids);
        } else if (d.material == MPM_SAND) {
          if (d.has_E) k_g2p2g<MPM_SAND, true><<<g, 64, 0, st>>>(d, src, p, wv, sched, copy_ids);
          else k_g2p2g<MPM_SAND, false><<<g, 64, 0, st>>>(d, src, p, wv, sched, copy_ids);
        } else if (d.material == MPM_SNOW) {
          k_g2p2g<MPM_SNOW, true><<<g, 64, 0, st>>>(d, src, p, wv, sched, copy_ids);
        } else {
          if (d.has_E) k_g2p2g<MPM_FIXED_COROTATED, true><<<g, 64, 0, st>>>(d, src, p, wv, sched, copy_ids);
          else k_g2p2g<MPM_FIXED_COROTATED, false><<<g, 64, 0, st>>>(d, src, p, wv, sched, copy_ids);
        }
      } else {
        // (the gather does not depend on the material: sand and snow use the elastic instance)
        if (d.material == MPM_J_FLUID) k_g2p<MPM_J_FLUID><<<sim->grid_g2p, 64, 0, st>>>(d, src, p);
        else k_g2p<MPM_FIXED_COROTATED><<<sim->grid_g2p, 64, 0, st>>>(d, src, p);
      }
      break;
  }
  return hipGetLastError() == hipSuccess ? MPM_OK : MPM_ERR_HIP;
}

// Which kernels step n runs in a mode: all five, or (mode 2, a step after a
// fused pass) the fused kernel alone; and the fused kernel's sched and
// copy_ids arguments.  lean_ok = false forces all five (the first step
// under a new schedule, whose P2G may not have run).  A lean step's fused
// pass follows a fused pass (of the full step that sorted, or of the first
// step under the schedule) that copied the ids and moduli into the other
// buffer at the same slots, and no sort has moved them since: it leaves
// them in place.
void step_plan(const mpm_sim *sim, int64_t n, int mode, bool lean_ok, bool run[NUM_KERNELS], int &sched,
               int &copy_ids) {
  for (int k = 0; k < NUM_KERNELS; ++k) run[k] = true;
  sched = -1;
  copy_ids = 1;
  if (mode == 2) {
    const int K = sim->sort_interval, c = (int)(n % K);
    sched = (c == K - 1) ? 1 : 0;
    if (c != 0 && lean_ok) {
      for (int k = 0; k < NUM_KERNELS - 1; ++k) run[k] = false;
      copy_ids = 0;
    }
  }
}

int enqueue_step(mpm_sim *sim, hipStream_t st, int64_t n, int mode, bool lean_ok, bool write_vc) {
  bool run[NUM_KERNELS];
  int sched, copy_ids;
  step_plan(sim, n, mode, lean_ok, run, sched, copy_ids);
  for (int k = 0; k < NUM_KERNELS; ++k) {
    if (!run[k]) continue;
    const int rc = launch_kernel(sim, k, st, (int)(n % NACC), mode != 0, write_vc, sched, copy_ids);
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

// Record the handle's completion event after the work just enqueued on st.
int mark(mpm_sim *sim, hipStream_t st) {
  if (!sim->done) return MPM_OK;  // (a handle-free run: no event)
  return hipEventRecord(sim->done, st) == hipSuccess ? MPM_OK : MPM_ERR_HIP;
}

void release(mpm_sim *sim) {
  if (!sim) return;
  if (sim->done) {
    (void)hipEventSynchronize(sim->done);  // the last operation enqueued, on whatever stream
    (void)hipEventDestroy(sim->done);
  }
  for (int m = 0; m < 3; ++m) destroy_graphs(sim, m);
  if (sim->cap) {
    (void)hipStreamSynchronize(sim->cap);
    (void)hipStreamDestroy(sim->cap);
  }
  delete sim;
}

// Launch shapes of the simulation's kernels on the current device, and its
// chunk size (host queries only: nothing is allocated).
int launch_shapes(mpm_sim *sim) {
  const SimDev &d = sim->d;
  if (hipGetDevice(&sim->device) != hipSuccess) return MPM_ERR_HIP;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, sim->device) != hipSuccess || cus <= 0)
    cus = 256;
  sim->grid_particles = (int)(((d.N + WG - 1) / WG + 7) / 8 * 8);
  // (occupancy of the instance this material launches)
  int occ = 0;
  const void *pk = d.material == MPM_SNOW ? (const void *)k_p2g<MPM_SNOW, true, NWIN>
                                          : (const void *)k_p2g<MPM_FIXED_COROTATED, false, NWIN>;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, pk, 64, 0) != hipSuccess || occ <= 0) occ = 16;
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
  // A scene whose 64-particle chunks fit in about three quarters of the
  // launch the eight-window P2G allows (its LDS admits fewer wavefronts per
  // CU) takes that P2G: every chunk still has a wavefront to itself, and the
  // dense chunks that set the step time need a quarter of the passes.
  {
    int occ_w = 0;
    const void *pw = d.material == MPM_SNOW ? (const void *)k_p2g<MPM_SNOW, true, NWIN_WIDE>
                                            : (const void *)k_p2g<MPM_FIXED_COROTATED, false, NWIN_WIDE>;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ_w, pw, 64, 0) != hipSuccess || occ_w <= 0) occ_w = 1;
    const int grid_w = ((cus * occ_w) / NQ) * NQ;
    sim->p2g_wide = sim->d.chunk_shift == KMIN_SHIFT && grid_w >= NQ &&
                    4 * ((int64_t)d.N >> KMIN_SHIFT) <= 3 * (int64_t)grid_w;
    if (sim->p2g_wide) sim->grid_p2g = grid_w;
  }
  // A small scene whose bins fit k_sort_small's tables (and whose chunk
  // indexes fit their 16 bits) sorts with it: scan and scatter in one kernel.
  {
    int occ_s = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ_s, k_sort_small<SMALL_SORT_BINS / 256>, 64, 0) != hipSuccess ||
        occ_s <= 0)
      occ_s = 1;
    sim->d.sort_small = sim->p2g_wide && d.nbins <= SMALL_SORT_BINS && d.max_chunks < 65536u ? 1 : 0;
    sim->grid_sort_small = cus * occ_s;
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
                   : d.material == MPM_SNOW ? (const void *)k_g2p2g<MPM_SNOW, true>
                       : (d.has_E ? (const void *)k_g2p2g<MPM_FIXED_COROTATED, true>
                                  : (const void *)k_g2p2g<MPM_FIXED_COROTATED, false>);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ_f, fk, 64, 0) != hipSuccess || occ_f <= 0) occ_f = 8;
  occ_f = occ_f < 16 ? occ_f : 16;
  sim->grid_g2p2g = ((cus * occ_f + NQ - 1) / NQ) * NQ;
  sim->grid_blocks = cus * 8;
  // single-wavefront workgroups, 8 per SIMD: the scatter is a chain of
  // short dependent loads per chunk, so it wants many chunks in flight
  sim->grid_scatter = cus * 32;
  return MPM_OK;
}

// The initial state: clear the control words, counters, block flags and
// accumulators, upload the inputs (creation order) and bucket them into
// bin order in buffer 1.  Fill kernels only: no memset and no allocation.
int init_state(mpm_sim *sim, const float *x0, const float *v0, const float *C0, const float *F0,
               const float *E_p, hipStream_t st) {
  const SimDev &d = sim->d;
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
    // whose chunk list the scan writes): the scan of a step that reads
    // buffer 0, and the bin cursors it sets
    launch_scan(sim, st, 0, 0);
    launch_scan(sim, st, 0, 1);
    k_scatter_init<<<sim->grid_particles, WG, 0, st>>>(d);
    // (k_sort_small counts the movers into a bin from zero)
    if (d.sort_small) k_zero_u32<<<zb, WG, 0, st>>>(d.bin_cursor, (size_t)d.nbins);
    sim->cur = 1;
  }
  return hipGetLastError() == hipSuccess ? MPM_OK : MPM_ERR_HIP;
}

// Device address of `scratch` on device dev, looked up once per device with
// that device current (each device holds its own copy, at its own address).
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex noalloc_mu;
void *noalloc_ptr[NOALLOC_MAX_DEVICES] = {};

int noalloc_scratch(int dev, void **out) {
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return MPM_ERR_HIP;
  std::lock_guard<std::mutex> lock(noalloc_mu);
  if (!noalloc_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MPM_ERR_HIP;
    if ((reinterpret_cast<uintptr_t>(p) & 255u) != 0) return MPM_ERR_WORKSPACE;
    noalloc_ptr[dev] = p;
  }
  *out = noalloc_ptr[dev];
  return MPM_OK;
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
  // snow's per-particle slot holds its log plastic volume: no per-particle modulus
  if (params->material == MPM_SNOW && E_p) return MPM_ERR_INVALID_ARG;
  const size_t need = mpm_workspace_bytes(params, n_particles);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || workspace_bytes < need)
    return MPM_ERR_WORKSPACE;

  mpm_sim *sim = new (std::nothrow) mpm_sim();
  if (!sim) return MPM_ERR_STATE;
  const bool has_E = E_p != nullptr || params->material == MPM_SNOW;
  layout(params, n_particles, has_E, static_cast<char *>(workspace), &sim->d);
  const SimDev &d = sim->d;
  hipStream_t st = static_cast<hipStream_t>(stream);

  int rc = MPM_OK;
  do {
    if ((rc = launch_shapes(sim)) != MPM_OK) break;
    if (hipStreamCreateWithFlags(&sim->cap, hipStreamNonBlocking) != hipSuccess) { rc = MPM_ERR_HIP; break; }
    if (hipEventCreateWithFlags(&sim->done, hipEventDisableTiming) != hipSuccess) { rc = MPM_ERR_HIP; break; }
    if ((rc = init_state(sim, x0, v0, C0, F0, E_p, st)) != MPM_OK) break;
    if ((rc = mark(sim, st)) != MPM_OK) break;
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
    // (a rare host wait: launches of the old graphs may still be pending)
    if (hipEventSynchronize(sim->done) != hipSuccess) return MPM_ERR_HIP;
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
  return mark(sim, st);
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
  return mark(sim, static_cast<hipStream_t>(stream));
}

int mpm_launch_config(const mpm_sim *sim, int32_t *out) {
  if (!sim || !out) return MPM_ERR_INVALID_ARG;
  out[0] = 1 << sim->d.chunk_shift;
  out[1] = sim->p2g_wide ? NWIN_WIDE : NWIN;
  out[2] = sim->d.sort_small ? 1 : (sim->d.nbins > SCAN_SMALL_NT * SCAN_PER ? 3 : 2);
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
    int sched, copy_ids;
    step_plan(sim, sim->steps, mode, mode == 2 && sim->sched_ready, run, sched, copy_ids);
    if (hipEventRecord(ev[0], st) != hipSuccess) { rc = MPM_ERR_HIP; break; }
    for (int k = 0; k < NUM_KERNELS && rc == MPM_OK; ++k) {
      if (run[k]) rc = launch_kernel(sim, k, st, (int)(sim->steps % NACC), mode != 0, true, sched, copy_ids);
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
  if (rc == MPM_OK) rc = mark(sim, st);
  return rc;
}

int mpm_read_particles(mpm_sim *sim, float *x, float *v, float *C, float *F_or_J, void *stream) {
  if (!sim) return MPM_ERR_INVALID_ARG;
  if (sim->d.N == 0) return MPM_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int g = sim->grid_g2p;
  const SimDev &d = sim->d;
  if (d.material == MPM_J_FLUID) k_read_particles<MPM_J_FLUID><<<g, 64, 0, st>>>(d, sim->cur, x, v, C, F_or_J, nullptr);
  else if (d.material == MPM_SAND) k_read_particles<MPM_SAND><<<g, 64, 0, st>>>(d, sim->cur, x, v, C, F_or_J, nullptr);
  else if (d.material == MPM_SNOW) k_read_particles<MPM_SNOW><<<g, 64, 0, st>>>(d, sim->cur, x, v, C, F_or_J, nullptr);
  else k_read_particles<MPM_FIXED_COROTATED><<<g, 64, 0, st>>>(d, sim->cur, x, v, C, F_or_J, nullptr);
  return hipGetLastError() == hipSuccess ? mark(sim, st) : MPM_ERR_HIP;
}

int mpm_run_noalloc(const mpm_params *params, int64_t n_particles, float *x, float *v, float *C, float *F_or_J,
                    const float *E_p, int32_t n_steps, uint32_t *status, void *stream) {
  if (!valid_params(params) || n_particles < 0 || n_steps < 0) return MPM_ERR_INVALID_ARG;
  if (params->material == MPM_SNOW) return MPM_ERR_INVALID_ARG;  // (its plastic state has no output here)
  if (n_particles > 0 && !x) return MPM_ERR_INVALID_ARG;
  const size_t need = mpm_workspace_bytes(params, n_particles);
  if (need == 0) return MPM_ERR_INVALID_ARG;
  if (need > (size_t)MPM_NOALLOC_SCRATCH_BYTES) return MPM_ERR_TOO_LARGE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MPM_ERR_HIP;
  void *base = nullptr;
  int rc = noalloc_scratch(dev, &base);
  if (rc != MPM_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // The state of a handle, on the stack: no graphs, no event, no private
  // stream; the steps are launched eagerly, as the graphs would run them.
  mpm_sim sim;
  layout(params, n_particles, E_p != nullptr, static_cast<char *>(base), &sim.d);
  const SimDev &d = sim.d;
  if ((rc = launch_shapes(&sim)) != MPM_OK) return rc;
  // every word the run reads is written first: all of the scratch it uses
  // starts from the fill kernels of init_state, whatever an earlier call left
  if ((rc = init_state(&sim, x, v, C, F_or_J, E_p, st)) != MPM_OK) return rc;
  if (d.N > 0) {
    for (int32_t k = 0; k < n_steps; ++k) {
      if ((rc = enqueue_step(&sim, st, sim.steps, 0, true, true)) != MPM_OK) return rc;
      sim.cur ^= 1;
      sim.steps += 1;
    }
    const int g = sim.grid_g2p;
    if (d.material == MPM_J_FLUID) k_read_particles<MPM_J_FLUID><<<g, 64, 0, st>>>(d, sim.cur, x, v, C, F_or_J, nullptr);
    else if (d.material == MPM_SAND) k_read_particles<MPM_SAND><<<g, 64, 0, st>>>(d, sim.cur, x, v, C, F_or_J, nullptr);
    else k_read_particles<MPM_FIXED_COROTATED><<<g, 64, 0, st>>>(d, sim.cur, x, v, C, F_or_J, nullptr);
  }
  if (status) k_copy_u32<<<1, 64, 0, st>>>(status, d.status, MPM_STATUS_WORDS);
  return hipGetLastError() == hipSuccess ? MPM_OK : MPM_ERR_HIP;
}

int mpm_read_plastic_state(mpm_sim *sim, float *alpha, void *stream) {
  if (!sim || !alpha || sim->d.material != MPM_SNOW) return MPM_ERR_INVALID_ARG;
  if (sim->d.N == 0) return MPM_OK;
  k_read_particles<MPM_SNOW><<<sim->grid_g2p, 64, 0, static_cast<hipStream_t>(stream)>>>(
      sim->d, sim->cur, nullptr, nullptr, nullptr, nullptr, alpha);
  return hipGetLastError() == hipSuccess ? mark(sim, static_cast<hipStream_t>(stream)) : MPM_ERR_HIP;
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
  return hipGetLastError() == hipSuccess ? mark(sim, st) : MPM_ERR_HIP;
}

int mpm_status(mpm_sim *sim, uint32_t *status_device, void *stream) {
  if (!sim || !status_device) return MPM_ERR_INVALID_ARG;
  if (hipMemcpyAsync(status_device, sim->d.status, sizeof(uint32_t) * MPM_STATUS_WORDS, hipMemcpyDeviceToDevice,
                     static_cast<hipStream_t>(stream)) != hipSuccess)
    return MPM_ERR_HIP;
  return mark(sim, static_cast<hipStream_t>(stream));
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
    case MPM_ERR_TOO_LARGE: return "the problem needs more memory than the static scratch of mpm_run_noalloc "
                                   "(MPM_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown error";
  }
}

}  // extern "C"
