/*
 * mpm.h -- C ABI of the MI355X MLS-MPM library (libmpm.so).
 *
 * One explicit MLS-MPM time step of the material point method: particles
 * are sorted by grid block, scattered to a background grid (P2G), the grid
 * momentum is updated (gravity, sticky walls), and the grid velocities are
 * gathered back to the particles (G2P) with the APIC affine matrix, the
 * deformation-gradient update and the fixed-corotated stress.  These are the
 * phases named in "Principles towards Real-Time Simulation of Material Point
 * Method on Modern GPUs" (rebuild-mapping and particle sorting, then P2G,
 * grid update and G2P, in its discussion of essential and non-essential
 * phases).
 *
 * The interface follows that page's single-GPU principles: all device memory
 * is handed over once at creation and never reallocated (its memory
 * reallocation principle); stepping is asynchronous, with no host-device
 * synchronisation inside a step (its CPU-GPU synchronisation principle); and
 * a whole step is replayed as one captured HIP graph (its principle of few
 * kernel launches per step).
 *
 * Conventions for every call:
 *   - Pointers documented as "device" must point to memory of the current
 *     HIP device.  "host" pointers are read only during the call.
 *   - `stream` is a hipStream_t passed as void*; NULL means the legacy
 *     default stream.  Every device-side effect is enqueued on it and is
 *     complete once the caller synchronises that stream.
 *   - Return value: MPM_OK (0) or a negative MPM_ERR_* code.  Argument errors
 *     are detected on the host before anything is enqueued and leave the
 *     simulation untouched.  No C++ exception crosses this interface.
 *   - A handle is not thread-safe; distinct handles are independent.
 *
 * Domain and grid: the domain is [0,1]^3, with grid_n nodes per axis at
 * x_i = i*dx, dx = 1/grid_n.  Dense grid outputs use linear index
 * i + n*(j + n*k) for node (i,j,k), i along x.  Particle positions are kept
 * in [2dx, (n-2)dx] per component so that every 3x3x3 stencil lies inside
 * the grid.
 */
#ifndef MPM_H
#define MPM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ---- */
#define MPM_OK 0
#define MPM_ERR_INVALID_ARG (-1) /* a NULL, negative or out-of-range argument */
#define MPM_ERR_WORKSPACE (-2)   /* workspace missing, too small or misaligned */
#define MPM_ERR_HIP (-3)         /* a HIP runtime call failed */
#define MPM_ERR_STATE (-4)       /* the handle is not usable (e.g. graph missing) */
#define MPM_ERR_TOO_LARGE (-5)   /* mpm_run_noalloc: the problem needs more than its static scratch */

/* Bytes of the static scratch of mpm_run_noalloc.  The library holds one
 * array of this size in the memory of every device it runs on, from the
 * first call there until the process ends: enough for the page's real-time
 * scenes (55,000 particles on a 64^3 grid need 54 MiB). */
#define MPM_NOALLOC_SCRATCH_BYTES (64u << 20)

/* ---- materials ---- */
#define MPM_FIXED_COROTATED 0 /* elastic solid, state F (3x3) */
#define MPM_J_FLUID 1         /* weakly compressible fluid, state J (scalar) */
#define MPM_SAND 2            /* Drucker-Prager sand, state F (3x3, elastic part) */
#define MPM_SNOW 3            /* non-associative Cam-clay snow, state F (3x3, elastic part)
                                 and the log plastic volume ln J_P (scalar) */

/* ---- status word bits (see mpm_status) ---- */
#define MPM_STATUS_NONFINITE 0x1u  /* a NaN or Inf appeared in particle velocity, C or position */
#define MPM_STATUS_CLAMPED 0x2u    /* a position component was clamped into [2dx,(n-2)dx] */
#define MPM_STATUS_INVERTED 0x4u   /* det F <= 0 (or J <= 0) met in the stress evaluation */
#define MPM_STATUS_BAD_INPUT 0x8u  /* non-finite or out-of-domain input at creation (it was clamped) */
#define MPM_STATUS_NO_CONVERGE 0x10u /* the polar iteration hit its iteration cap */
#define MPM_STATUS_WORDS 8         /* [0] flags, [1] clamped position components, [2] inverted count,
                                      [3] non-finite count, [4..7] reserved (0) */

typedef struct mpm_sim mpm_sim;

/* Scalar parameters of a simulation.
 *   struct_size : sizeof(mpm_params), for forward compatibility.
 *   grid_n      : nodes per axis, 8 <= grid_n <= 1024.
 *   dt          : time step (> 0).
 *   gravity     : acceleration added to every grid velocity, per axis.
 *   wall_nodes  : sticky-wall thickness: all velocity components are zeroed
 *                 on nodes with any index < wall_nodes or >= grid_n - wall_nodes
 *                 (0 <= wall_nodes <= grid_n/2).
 *   material    : MPM_FIXED_COROTATED, MPM_J_FLUID, MPM_SAND (Drucker-
 *                 Prager plasticity in Hencky strain with a constant friction
 *                 angle, projected after every deformation-gradient update:
 *                 the page merges the SVD, the plasticity projection and the
 *                 stress into the particle phase of P2G) or MPM_SNOW (the
 *                 non-associative Cam-clay model of Wolper et al. 2019, which
 *                 the page names for its snow scene with bulk modulus,
 *                 Poisson ratio, M, beta and xi: yield ellipse (1 + 2 beta)
 *                 q^2 + M^2 (p + beta p0)(p - p0) <= 0 in the pressure p and
 *                 shear measure q of the Hencky stress, hardening p0 = K
 *                 sinh(xi max(-a, 0)) with the log plastic volume a, projected
 *                 as MPM_SAND is; E > 0).
 *   E           : Young's modulus (bulk modulus K for MPM_J_FLUID), >= 0;
 *                 used when no per-particle modulus is given.
 *   nu          : Poisson ratio, 0 <= nu < 0.5 (ignored for MPM_J_FLUID).
 *   rho, p_vol  : density and initial particle volume (> 0); particle mass
 *                 is rho * p_vol.
 *   friction_deg: MPM_SAND only: friction angle in degrees, 0 < friction_deg < 90.
 *   snow_M, snow_beta, snow_xi, snow_alpha0: the snow material's
 *                 critical-state slope M > 0 (the page's friction
 *                 coefficient), cohesion beta >= 0, hardening xi >= 0 and the
 *                 log plastic volume ln J_P every particle starts with
 *                 (finite); read only for the snow material. */
typedef struct {
  uint32_t struct_size;
  int32_t grid_n;
  float dt;
  float gravity[3];
  int32_t wall_nodes;
  int32_t material;
  float E;
  float nu;
  float rho;
  float p_vol;
  float friction_deg;
  float snow_M;
  float snow_beta;
  float snow_xi;
  float snow_alpha0;
} mpm_params;

/* Bytes of device workspace a simulation of n_particles needs (0 when the
 * parameters are invalid).  Pure host computation.  The page's second
 * single-GPU principle (reducing memory reallocation once the simulation
 * starts; its Fig. 3 shows reallocation outlasting the kernels of a small
 * scene): the whole need is known before the first step, so the caller hands
 * the memory over once, at creation. */
size_t mpm_workspace_bytes(const mpm_params *params, int64_t n_particles);

/* Create a simulation and upload its initial state (the particle set of the
 * page's problem statement: material points carried across a background
 * grid by explicit steps).
 *   params      : host, read during the call.
 *   n_particles : 0 <= n < 2^28, and the particle buffers' slot capacity
 *                 n + 31 min(n, ceil(grid_n / 4)^3), rounded up to 64, below
 *                 2^29 (each 4^3-cell bin's slots start on a 32-particle
 *                 boundary; component offsets inside the 9-component fields
 *                 are 32-bit).  Larger requests return MPM_ERR_INVALID_ARG
 *                 (and mpm_workspace_bytes returns 0).
 *   x0          : device, (N,3) float32 row-major positions (required if N > 0).
 *   v0          : device, (N,3) velocities, or NULL for zero.
 *   C0          : device, (N,3,3) row-major APIC affine matrices, or NULL for zero.
 *   F0          : device, (N,3,3) deformation gradients for MPM_FIXED_COROTATED
 *                 and MPM_SAND (its elastic part, used as given until the
 *                 first update), or (N) volume ratios J for MPM_J_FLUID; NULL
 *                 for I (or 1).
 *   E_p         : device, (N) per-particle Young's modulus, or NULL for params->E;
 *                 must be NULL for MPM_SNOW (MPM_ERR_INVALID_ARG otherwise), whose
 *                 particles carry their log plastic volume instead.
 *   workspace   : device, at least mpm_workspace_bytes(params, N) bytes,
 *                 256-byte aligned, owned by the caller, and must outlive the
 *                 handle.  The library never allocates device memory.
 *   stream      : initialisation kernels are enqueued on it; the inputs may
 *                 be released once it has completed.
 *   out         : host, receives the handle.
 * Inputs with a non-finite or out-of-domain position are clamped into the
 * domain and raise MPM_STATUS_BAD_INPUT; this is reported through
 * mpm_status, without a host synchronisation. */
int mpm_create(const mpm_params *params, int64_t n_particles, const float *x0, const float *v0,
               const float *C0, const float *F0, const float *E_p, void *workspace,
               size_t workspace_bytes, void *stream, mpm_sim **out);

/* Advance n_steps >= 0 explicit steps, enqueued asynchronously on `stream`
 * (captured graphs of 8 steps, then single steps: per step key/bucket sort,
 * P2G, grid update, G2P: the phases of the page's pipeline, with its
 * principles of few kernels per step and no CPU-GPU synchronisation, Fig. 4).
 * No host synchronisation, no allocation.  One
 * exception: the first call after the fused host-scheduled interval changed
 * (mpm_set_sort_policy with fused steps on) waits on the host for this
 * handle's earlier work before it replaces the graphs of the old interval. */
int mpm_step(mpm_sim *sim, int32_t n_steps, void *stream);

/* Sort policy: the free zone of the page's non-essential-phase discussion
 * (the particle-to-bin mapping is rebuilt only when needed).
 *   max_interval : 0 or 1 = sort every step (the default); k > 1 = sort at
 *                  least every k steps.
 *   mover_budget : between those sorts, sort as soon as more than this many
 *                  particles are outside the bin of their chunk (counted on
 *                  the device by G2P; the decision is taken on the device at
 *                  the start of each step, without a host synchronisation).
 * Between sorts each chunk keeps its particles, and a particle that left its
 * chunk's bin is deposited and gathered through the grid directly (global
 * atomics and loads) instead of the chunk's LDS window.  The results equal
 * those of sorting every step up to the order of float additions.  Enqueued
 * on `stream`, it applies from the next step on.  Negative arguments return
 * MPM_ERR_INVALID_ARG. */
int mpm_set_sort_policy(mpm_sim *sim, int32_t max_interval, int64_t mover_budget, void *stream);

/* Fused steps: the page's fused G2P2G kernel (the G2P of one step and the
 * P2G of the next in one pass over the particles).  enable = 1: from the
 * next mpm_step on, a step whose successor does not sort (see
 * mpm_set_sort_policy) runs its G2P fused with the successor's P2G, so that
 * between sorts the state carried from step to step is x, F (or J) and the
 * modulus only.  The successor's sort decision is then taken one step
 * earlier, on the movers counted by the step before.  With a power-of-two
 * max_interval K <= 32 and a mover budget of at least the particle count,
 * the sorts follow the step number instead (step n sorts when n mod K = 0,
 * after one step that sorts or not by the policy), and a step after a
 * fused pass launches the fused kernel alone.  enable = 0 (the default):
 * separate P2G and G2P kernels.  Under the default policy (sort every step)
 * both settings run the same work.  The results equal those of separate
 * kernels up to the order of float additions; mpm_read_particles and
 * mpm_read_grid read the same state.  The first mpm_step in a new setting
 * captures its graphs (host work, no device allocation).  A host-side
 * setting: no stream.  enable outside {0, 1} returns MPM_ERR_INVALID_ARG. */
int mpm_set_fused_steps(mpm_sim *sim, int32_t enable);

/* Copy the particle state after the last step, in creation order, into
 * caller-owned device arrays (the Lagrangian half of the page's problem
 * statement, its introduction: material points that the explicit steps carry
 * across the background grid; asynchronous, as its CPU-GPU synchronisation
 * principle asks, Fig. 4): x (N,3), v (N,3), C (N,3,3), F_or_J (N,3,3)
 * for the elastic material, sand and snow (for sand and snow the elastic part
 * after the step's plasticity projection) or (N) for the fluid.  Any output
 * may be NULL.  Asynchronous on `stream`. */
int mpm_read_particles(mpm_sim *sim, float *x, float *v, float *C, float *F_or_J, void *stream);

/* For callers that cannot allocate: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  One call does what
 * mpm_create, mpm_step(n_steps), mpm_read_particles and mpm_status do on a
 * handle, with the same kernels, and allocates nothing: no device memory
 * (no hipMalloc or hipFree), no host memory, no stream, event or graph.  Its
 * workspace is the library's static scratch (MPM_NOALLOC_SCRATCH_BYTES on
 * each device) instead of a caller's: a problem for which
 * mpm_workspace_bytes(params, n_particles) exceeds it returns
 * MPM_ERR_TOO_LARGE before anything is enqueued.  The steps are launched one
 * kernel at a time (no graphs), each sorting, as mpm_step does by default.
 *   params, n_particles : as for mpm_create; the snow material is refused
 *                 (MPM_ERR_INVALID_ARG: its plastic state has no output here).
 *   x, v, C, F_or_J : device, caller-owned, the particle state in creation
 *                 order, read at the start and overwritten with the state after
 *                 n_steps steps (layouts of mpm_create and mpm_read_particles).
 *                 x is required when n_particles > 0; a NULL v, C or F_or_J
 *                 starts at zero (I, 1) and is not written back.
 *   E_p         : device, (N) per-particle Young's modulus, or NULL.
 *   n_steps     : >= 0.
 *   status      : device, MPM_STATUS_WORDS words of this run's status (as
 *                 mpm_status), or NULL.
 *   stream      : everything is enqueued on it, asynchronously.
 * Every call on one device uses that device's one scratch array and starts by
 * clearing all of it that the run reads (the array keeps the last call's
 * contents): calls that overlap on one device, on different streams or from
 * different threads, race and must be serialised by the caller. */
int mpm_run_noalloc(const mpm_params *params, int64_t n_particles, float *x, float *v, float *C, float *F_or_J,
                    const float *E_p, int32_t n_steps, uint32_t *status, void *stream);

/* Snow only: copy each particle's log plastic volume a = ln J_P after the last
 * step (after its plasticity projection, as mpm_read_particles reads F), in
 * creation order, into the caller-owned device array alpha (N).  The snow
 * model's hardening state (the page's snow scene; Wolper et al. 2019).
 * Before any step: params->snow_alpha0.  MPM_ERR_INVALID_ARG for a NULL
 * alpha or another material.  Asynchronous on `stream`. */
int mpm_read_plastic_state(mpm_sim *sim, float *alpha, void *stream);

/* Copy the grid state of the last step into caller-owned dense device arrays
 * (the Eulerian half of the page's problem statement, its introduction, after
 * the nodal computations of its multi-GPU reduction discussion: updating
 * nodal velocities and resolving collisions):
 * mass (n^3) and momentum (n^3 x 3) = m_i * v_i after gravity and walls.
 * Nodes the last step did not touch are 0.  Either output may be NULL.
 * Before any step both are all zero.  Asynchronous on `stream`. */
int mpm_read_grid(mpm_sim *sim, float *mass, float *momentum, void *stream);

/* Copy the MPM_STATUS_WORDS uint32 status words (flags, counters since
 * creation) into a caller-owned device array.  Asynchronous on `stream`.
 * Anomalies are recorded on the device and read when the caller chooses,
 * instead of being checked on the host inside a step: the page's CPU-GPU
 * synchronisation principle (a host check stalls the GPU in a pipeline
 * bubble, Fig. 4). */
int mpm_status(mpm_sim *sim, uint32_t *status_device, void *stream);

/* Steps taken since creation: a host-side counter, so the caller learns it
 * without reading anything back from the device (the page's CPU-GPU
 * synchronisation principle, Fig. 4). */
int64_t mpm_steps_taken(const mpm_sim *sim);

/* Number of kernel slots of a step (scan tiles, scan bins, scatter, P2G, G2P;
 * with fused steps the last slot is the G2P2G kernel, and a step between
 * host-scheduled sorts launches that slot alone), and the name of slot k:
 * the kernels the page's third single-GPU principle counts (minimising the
 * kernels executed within one time step). */
int32_t mpm_num_kernels(void);
const char *mpm_kernel_name(int32_t k);

/* The launch configuration chosen at creation for the scene's size (the
 * page's kernel-count principle and its mapping of particles to thread
 * blocks): out[0] = particles per chunk (64, 128 or 256), out[1] = P2G
 * accumulation windows per wavefront (2, or 8 for a small scene), out[2] =
 * kernels of the step's sort (1: the small-scene sort that scans and scatters
 * in one kernel; 2: a one-workgroup scan and the scatter; 3: tile totals,
 * scan and scatter).  Host-only, caller-owned out (3 entries).
 * MPM_ERR_INVALID_ARG for a NULL argument. */
int mpm_launch_config(const mpm_sim *sim, int32_t *out);

/* Measurement helper, for per-kernel time breakdowns like those of the page's
 * ablation study (§6.2): run n_steps steps eagerly (the same kernels and launch
 * shapes as the graph), bracketing every kernel with HIP events on `stream`,
 * then synchronise `stream` and add each kernel's elapsed milliseconds into
 * kernel_ms[k] (host, mpm_num_kernels() entries, caller-initialised); a
 * slot the step does not launch adds about 0.  Unlike mpm_step, every step
 * stores v and C. */
int mpm_step_profiled(mpm_sim *sim, int32_t n_steps, void *stream, float *kernel_ms);

/* Release the handle and its graphs (not the caller's workspace): memory is
 * returned only when the simulation ends, never during it (the page's memory
 * reallocation principle, Fig. 3).  Blocks the host until every operation
 * this handle enqueued (steps, policy changes, readbacks, status copies) has
 * completed on the device, whatever stream it was enqueued on, so the caller
 * may free the workspace and the output arrays once this returns; the
 * streams themselves need not exist any more.  NULL is ignored. */
void mpm_destroy(mpm_sim *sim);

/* Static description of a return code.  Argument errors are found on the
 * host before anything is enqueued, so reporting them needs no device round
 * trip (the page's CPU-GPU synchronisation principle, Fig. 4). */
const char *mpm_error_string(int code);

#ifdef __cplusplus
}
#endif
#endif /* MPM_H */
