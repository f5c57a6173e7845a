/*
 * pk.h - C ABI of the persistent-kernel Jacobi engine for AMD MI355X (gfx950).
 *
 * The engine advances one 2-D field by 5-point Jacobi sweeps of
 * -Lap(u) = f (Laplace when f is absent) on a regular grid with Dirichlet data
 * on the outer ring ("Persistent Kernels: Bridging GPU-CPU Execution", section
 * "The problem (another PDE solver)" and its "Derivation"; Jacobi as a
 * separate result matrix per iteration: section "Implementation details and
 * correctness"). One sweep replaces every interior node by
 *     0.25 * (((W + E) + (S + N)) + b),   b = (T)((h*h) * f),
 * in the element type T, IEEE round-to-nearest, no contraction, subnormals kept.
 *
 * In PK_PERSISTENT mode the engine launches one co-resident (cooperative)
 * kernel at create time and drives it through a task ring in fine-grained
 * pinned host memory: "Persistent Kernels", sections "What if this launch and
 * execution overhead didn't exist?" and "Base implementation"; sweeps are
 * separated by a grid-wide barrier made of an arrival counter and a
 * generation word with release/acquire ordering ("Grid-Wide Barriers and
 * Persistent Work Queues", section "The barrier is a counter and a
 * generation"). The grid is sized once from the occupancy query ("@persistent"
 * page, section "What it promises"), and a grid that is not co-resident is
 * refused rather than run ("Grid-Wide Barriers", section "The residency
 * requirement"). PK_LAUNCH mode runs the same sweep body as one ordinary
 * kernel launch per sweep, with the same block count, as the baseline the
 * first page compares against (section "Comparing the kernels").
 *
 * Conventions
 *   - Every call returns PK_OK (0) or a negative PK_E* status; nothing aborts
 *     or throws across this interface.
 *   - Host arrays are row-major ny x nx of the engine's element type (float
 *     for PK_F32, double for PK_F64): element (i, j) is at [i * nx + j], row i
 *     is y = i*h, column j is x = j*h, row ny-1 is the top edge (y = 1).
 *   - Host arrays passed in are borrowed for the duration of the call only.
 *   - An engine is used from one host thread at a time. At most one
 *     PK_PERSISTENT engine per device: its cooperative kernel holds the CUs
 *     it was sized for until PK_EXIT or pk_destroy. While it runs, do not make
 *     the host wait on other GPU work queued on the same device.
 */
#ifndef PK_H
#define PK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define PK_OK 0
#define PK_EINVAL (-1)    /* bad argument                                           */
#define PK_ENOMEM (-2)    /* device or pinned host allocation failed                */
#define PK_ELAUNCH (-3)   /* kernel launch failed, or cooperative grid not resident */
#define PK_EDEVICE (-4)   /* HIP runtime error, or the device reported a fault      */
#define PK_EBUSY (-5)     /* task ring full, or tasks still in flight               */
#define PK_ESTATE (-6)    /* call not valid in the engine's mode or state           */
#define PK_ETIMEDOUT (-7) /* pk_wait gave up; the engine is poisoned from then on   */

/* ---- element types, modes, layouts ------------------------------------- */
#define PK_F32 0
#define PK_F64 1

#define PK_PERSISTENT 0 /* one co-resident launch driven through the task ring */
#define PK_LAUNCH 1     /* one kernel launch per sweep (baseline)               */

/* Work layout of the persistent sweeping tasks.
 * STREAM: passes of up to pass_sweeps sweeps stream the field through HBM once
 *   each: the field is cut into units (a band of rows x a 64-lane column strip,
 *   16-byte row loads), one per wave, and each wave marches its unit keeping
 *   every sweep level of the pass in registers.
 * RESIDENT: each block keeps its band of rows (plus halo rows) in LDS for the
 *   whole task; only the halo rows go through HBM, once every halo_depth sweeps
 *   (the wider-halo scheme of "Persistent Kernels", "Reflections and next
 *   steps", "Fewer handshakes", with exact Jacobi semantics).
 * REGISTER: as RESIDENT (same bands, halos and exchanges, same results), but
 *   each block's rows live in VGPRs: a wave holds up to 4 consecutive rows of
 *   one 64-lane column strip (one 16-byte vector per lane per row); only
 *   wave-boundary rows and columns go through LDS. Needs rows of at most
 *   (threads / 64) x 64 vectors and band + 2 x halo_depth <= 4 x the waves of
 *   a column strip.
 * AUTO: the tile (RESIDENT or REGISTER) with the lower modelled time per sweep
 *   when one fits (block count and halo depth from the cost model), else
 *   STREAM.                                                                 */
#define PK_LAYOUT_AUTO 0
#define PK_LAYOUT_STREAM 1
#define PK_LAYOUT_RESIDENT 2
#define PK_LAYOUT_REGISTER 3

/* ---- tasks -------------------------------------------------------------- */
#define PK_SWEEP 1    /* n Jacobi sweeps (n >= 0)                                   */
#define PK_RESIDUAL 2 /* R = sqrt(sum over interior of rho^2),                      */
                      /*   rho = (((W+E)+(S+N)) + b) - 4u, all in double. With a   */
                      /*   SWEEP task queued after it, an fp64 streaming engine at  */
                      /*   depth 12 may sum it inside a pass that runs on into that  */
                      /*   task (pk_info.tasks_fused): the same R, fields and done  */
                      /*   records; the field a fused SWEEP task ends with is then  */
                      /*   never stored                                              */
#define PK_EXIT 3     /* the persistent kernel returns; the engine stays readable   */
#define PK_BARRIER 4  /* n grid barriers and nothing else (persistent only; timing) */
#define PK_STAMP 5    /* n rounds of the barrier visibility check (persistent only):*/
                      /*   each block stamps its slot, barrier, then checks that a  */
                      /*   neighbour's and a remote block's slots carry the stamp;  */
                      /*   pk_result.errors counts mismatches                       */
#define PK_SWEEP_RB 6 /* n red-black Gauss-Seidel iterations ("Persistent Kernels",  */
                      /*   "Implementation details and correctness", Figure 3):     */
                      /*   first every interior node with i + j even (red), then    */
                      /*   every one with i + j odd (black), each by the same       */
                      /*   formula as a Jacobi sweep from its neighbours' current   */
                      /*   values. Equal to the in-place iteration; computed as two */
                      /*   half-sweeps into the other buffer, so `cur` flips as for */
                      /*   SWEEP. n <= PK_TASK_N_MAX / 2.                          */
                      /*   sweeps_done counts iterations.                           */
#define PK_SWEEP_UNTIL 7 /* Jacobi sweeps until the residual reaches a tolerance:   */
                      /*   submitted with pk_submit_until (see there), not pk_submit */
#define PK_BLOCKSYNC 8 /* n rounds of the block-level step of a tile sub-sweep and   */
                      /*   nothing else (persistent only; timing): each wave writes  */
                      /*   LDS, the block barrier, each wave reads a neighbour's     */
                      /*   value. Its time per round is the synchronization floor of */
                      /*   one sub-sweep                                             */

/* ---- option flags ------------------------------------------------------- */
/* Debug only: the grid barrier drops its release/acquire ordering (relaxed
 * atomics, no fences). Every wait still ends and every access stays in bounds;
 * only the visibility of other blocks' writes is no longer guaranteed, so the
 * field is expected to diverge from the oracle. A negative control.          */
#define PK_DBG_BROKEN_BARRIER 0x1u
/* Debug only: thread 0 of every block records device wall-clock events (task
 * begin and end, arrival at and departure from each grid barrier or neighbour
 * sync, the start of each tile period, wave 0's tagged-halo polls) in a ring of
 * its own, read with pk_trace_read after the kernel has left: where a task's
 * time goes, computing or waiting for the slowest block ("Grid-Wide Barriers and
 * Persistent Work Queues", "What the barrier buys"). Persistent mode only. */
#define PK_DBG_TRACE 0x2u

/* Grid barrier construction (both are an arrival counter plus a generation
 * word with release/acquire ordering).
 * FLAT: every block adds to one counter; the last one bumps the generation.
 * TWO_LEVEL: blocks add to the counter of their XCD group (block b mod 8);
 *   the last of each group adds to a top counter; the last of those bumps one
 *   generation word per group. Arrivals then contend 8 ways instead of G ways.
 * XCD: TWO_LEVEL grouped by the XCD each block runs on (read from the
 *   hardware at launch), with the L2 write-back done once per XCD instead of
 *   once per block: every wave waits for its own stores before its block
 *   arrives and the last block of an XCD writes that XCD's L2 back once; each
 *   block still does its own acquire.
 * AUTO: XCD from 16 blocks up (TWO_LEVEL under PK_DBG_BROKEN_BARRIER),
 *   FLAT below.                                                              */
#define PK_BARRIER_AUTO 0
#define PK_BARRIER_FLAT 1
#define PK_BARRIER_TWO_LEVEL 2
#define PK_BARRIER_XCD 3

/* Halo exchange of the tile layouts (RESIDENT, REGISTER) between the sweeps of one task
 * (after every halo_depth sweeps, each block publishes its edge rows to device
 * memory and reloads its neighbours').
 * BARRIER: a grid barrier between publish and reload.
 * NEIGHBOR: point-to-point. Each block release-stores its exchange count to a
 *   flag of its own (one 128-B line per block) and acquires the flags of the
 *   two blocks whose bands border its own: blocks wait for their neighbours
 *   only, never for the slowest block of the grid ("Persistent Kernels",
 *   "Reflections and next steps", GPU-side scheduling on neighbour step
 *   counters; "Grid-Wide Barriers and Persistent Work Queues", "What the
 *   barrier buys", on every block waiting for the slowest). A block is at most
 *   one exchange ahead of a neighbour, which the two device buffers allow.
 *   The last exchange of every task is still a grid barrier, so a task ends
 *   with the whole field in device memory.
 * TAGGED (REGISTER layout only): no barrier and no flag. Every published
 *   32-bit half of a halo value travels in one 64-bit word together with the
 *   exchange number, stored and loaded as relaxed device-scope atomics into
 *   one of two buffers (by exchange parity); a reader loads its halo words
 *   until every one carries the current number. A word is written whole or
 *   not at all, so a matching tag proves its value; no cache write-back or
 *   invalidation is needed. A block publishes exchange e + 2 into the buffer
 *   of exchange e only after it has read its neighbours' exchange e + 1,
 *   which they publish only after reading e. The last exchange of every task
 *   is a grid barrier, as above.
 * AUTO: the cheaper of the kinds the layout supports by the cost model, or
 *   BARRIER under PK_DBG_BROKEN_BARRIER.
 * STREAM (persistent), between the passes of one task: BARRIER, a grid
 *   barrier after every pass. NEIGHBOR: after a full-depth pass followed by
 *   another, neighbour counters kept per XCD: every block arrives at its XCD's
 *   counter, the XCD's last block writes the XCD's L2 back once and publishes
 *   the pass count, and each block waits only for the XCDs that run the blocks
 *   whose units border its own (up and down by the halo's reach in bands, left
 *   and right by one strip; looked up once at launch); the other passes, and
 *   the last pass of every task, end with the grid barrier. AUTO: NEIGHBOR from
 *   16 blocks on (BARRIER under PK_DBG_BROKEN_BARRIER). TAGGED is refused.   */
#define PK_EXCHANGE_AUTO 0
#define PK_EXCHANGE_BARRIER 1
#define PK_EXCHANGE_NEIGHBOR 2
#define PK_EXCHANGE_TAGGED 3

typedef struct pk_opts {
    int dtype;             /* PK_F32 or PK_F64                                       */
    double h;              /* grid spacing; 0 => 1/(nx-1), which requires nx == ny  */
    int mode;              /* PK_PERSISTENT or PK_LAUNCH                             */
    int layout;            /* PK_LAYOUT_*; PK_LAUNCH always streams                  */
    int threads;           /* threads per block, multiple of 64, <= 1024; 0 = auto;  */
                           /* the persistent STREAM kernel takes at most 512         */
    int max_blocks;        /* grid size in blocks; 0 = automatic. STREAM uses it as */
                           /* given (PK_ELAUNCH if that grid cannot be co-resident),*/
                           /* the tiles as an upper bound (one band per block)    */
    int halo_depth;        /* RESIDENT, REGISTER: sweeps per halo exchange; 0 = auto*/
    unsigned flags;        /* PK_DBG_* flags                                         */
    void* stream;          /* hipStream_t to use; NULL => the engine makes its own  */
                           /* non-blocking stream (the persistent kernel must not   */
                           /* sit on a stream that other work waits behind)         */
    double idle_timeout_s; /* the persistent kernel leaves by itself after this     */
                           /* long without a task; 0 => 120 s                       */
    int barrier;           /* PK_BARRIER_*                                           */
    int pass_sweeps;       /* STREAM: sweeps per pass, 1..8 or 12 (else            */
                           /* PK_EINVAL): each wave carries k levels of its band in */
                           /* registers, so the field crosses HBM and the blocks    */
                           /* meet once per k sweeps; 0 = 12 where u, u' and b      */
                           /* exceed the 256 MiB Infinity Cache, else 8, shallower  */
                           /* where the field passes 4 GiB and its rows are so long */
                           /* that a unit's rows (its band and 2 (k + 1) halo rows) */
                           /* would pass the 4 GiB a pass addresses (pk_info        */
                           /* reports it); an explicit depth whose window cannot    */
                           /* fit is PK_EINVAL. A task's last                       */
                           /* pass is at most 8 deep (12 -> 4 + 8), as are         */
                           /* red-black passes, except an fp64 pass of 12 that runs */
                           /* on into a queued SWEEP task (see PK_RESIDUAL)         */
    int band_rows;         /* STREAM passes: rows per band (a unit is a band x one  */
                           /* strip, one per wave); 0 = automatic                   */
    int exchange;          /* PK_EXCHANGE_* (tiles; STREAM: BARRIER or NEIGHBOR)   */
    int reserved[4];       /* must be zero                                           */
} pk_opts;

#define PK_TASK_N_MAX 0x0FFFFFFF /* largest n of one task */

typedef struct pk_task {
    int kind; /* PK_SWEEP, PK_SWEEP_RB, PK_RESIDUAL, PK_EXIT, PK_BARRIER,  */
              /* PK_STAMP or PK_BLOCKSYNC (PK_SWEEP_UNTIL: pk_submit_until)  */
    int n;    /* count for SWEEP, SWEEP_RB, BARRIER, STAMP and BLOCKSYNC;   */
              /* ignored otherwise                                         */
} pk_task;

typedef struct pk_result {
    double residual;     /* PK_RESIDUAL: R; otherwise 0                               */
    int64_t sweeps_done; /* sweeps applied to the field when this task ended          */
    double device_us;    /* task time on the device clock (persistent), else 0        */
    int64_t errors;      /* PK_STAMP: mismatches seen; otherwise 0                    */
    int kind;            /* the task's kind                                           */
    int status;          /* PK_OK, or PK_EDEVICE if the device flagged a fault        */
} pk_result;

typedef struct pk_info {
    int nx, ny, dtype, mode, layout;
    int pitch;              /* device row stride in elements (rows are 256-B aligned)  */
    int grid_blocks;        /* blocks in the grid (both modes use the same count)       */
    int threads;            /* threads per block                                         */
    int blocks_per_cu_max;  /* occupancy query result for the persistent kernel          */
    int cus;                /* compute units on the device                               */
    int halo_depth;         /* RESIDENT, REGISTER: sweeps per exchange; 0 otherwise      */
    int band_rows;          /* rows per band (tiles: per block; STREAM: per unit)        */
    int strips;             /* STREAM: column strips                                     */
    int barrier;            /* PK_BARRIER_FLAT, _TWO_LEVEL or _XCD                       */
    int pass_sweeps;        /* STREAM: sweeps per pass                                   */
    int exchange;           /* PK_EXCHANGE_BARRIER, _NEIGHBOR or _TAGGED; LAUNCH: 0      */
    size_t lds_bytes;       /* dynamic LDS per block                                     */
    double kernel_ms;       /* PERSISTENT: launch-to-exit time of the kernel (HIP        */
                            /* events on its stream), valid after EXIT; LAUNCH: total   */
                            /* device time of the last pk_run_launch_per_iter batch     */
    int64_t sweeps_done;
    int64_t tasks_done;
    int64_t kernel_launches; /* launches made so far (persistent: 1)                     */
    int64_t tasks_carried;   /* PERSISTENT: tasks that started without a poll and a      */
                             /* broadcast barrier: the previous task's barrier carried */
                             /* them (the host had queued them ahead)                   */
    int wall_clock_khz;      /* rate of the device wall clock that task times and the   */
                             /* trace count in                                           */
    int trace_capacity;      /* PK_DBG_TRACE: events each block's ring holds; else 0   */
    int64_t tasks_fused;     /* PERSISTENT, STREAM: tasks that ran sweeps of a later    */
                             /* SWEEP task: a SWEEP task whose last pass ran on into   */
                             /* the SWEEP task two slots later (the RESIDUAL between   */
                             /* them summed inside that pass), or a RESIDUAL task that */
                             /* ran the next SWEEP task's first pass and summed its    */
                             /* level 0 (the host had queued them ahead)                */
} pk_info;

typedef struct pk_engine pk_engine;

/* Fill *o with the defaults (PK_F32, h = 0, PK_PERSISTENT, PK_LAYOUT_AUTO, ...):
 * every sizing choice left to the engine, which sizes the grid once from the
 * occupancy query ("@persistent" page, section "What it promises"). o may be
 * NULL (no-op). */
void pk_opts_default(pk_opts* o);

/* Create an engine for an nx x ny field (nx, ny >= 3): the grid of
 * "Persistent Kernels", "The problem (another PDE solver)", with h the node
 * spacing, and two device buffers for Jacobi ("Implementation details and
 * correctness": the update goes into a separate matrix).
 *   bc  - host array: the outer ring is the fixed Dirichlet data, the interior
 *         is the initial guess; copied into both device buffers.
 *   src - host array of f for -Lap(u) = f, or NULL for Laplace; b = (T)(h*h*f)
 *         is computed on the device once.
 * In PK_PERSISTENT mode the cooperative kernel is launched before returning, once,
 * with a grid sized from the occupancy query ("@persistent" page, "What it
 * promises"; "Grid-Wide Barriers", "The residency requirement").
 * Errors: PK_EINVAL (sizes, opts, NULL bc or out, h <= 0 when required; rows
 * longer than 1 GiB; a field taller than 4 GiB of its rows whose rows are too
 * long for a pass's 4 GiB window, about 850 MB even at a depth of 1),
 * PK_ENOMEM, PK_ELAUNCH (grid not co-resident / launch refused), PK_EDEVICE.
 * On error *out is left unchanged and nothing stays allocated. */
int pk_create(int nx, int ny, const void* bc, const void* src, const pk_opts* o,
              pk_engine** out);

/* Queue a task; tasks run in FIFO order. *ticket (may be NULL) receives the
 * task's sequence number (1, 2, ...). Does not block. The host writes the task
 * into the next slot of a ring in pinned host memory and the device's single
 * poller takes it ("Persistent Kernels", "Base implementation" for the
 * host-to-device task flags, "Thread synchronization" for one poller per
 * grid, and "Reflections and next steps", point 3, for a done word written only
 * after the work: here every slot carries a sequence number, so no early
 * acknowledgement is possible). A task travels to the
 * device as one 64-bit word, so n is at most PK_TASK_N_MAX (2^28 - 1): split
 * longer runs into several SWEEP tasks.
 * Errors: PK_EINVAL (unknown kind, n < 0 or > PK_TASK_N_MAX, persistent-only
 * kind in PK_LAUNCH mode), PK_EBUSY (ring full: wait on an older ticket first), PK_ESTATE
 * (after EXIT, or on a poisoned engine). */
int pk_submit(pk_engine* e, pk_task t, uint64_t* ticket);

/* Queue a PK_SWEEP_UNTIL task: Jacobi sweeps with an in-kernel stop on a
 * residual threshold ("Persistent Kernels", "Reflections and next steps",
 * GPU-side scheduling; "Grid-Wide Barriers and Persistent Work Queues", "What
 * the barrier buys": the convergence check as a grid reduction whose result
 * every block sees). The task computes R (as PK_RESIDUAL) of the current
 * field; while R > tol and fewer than max_sweeps sweeps are done, it runs
 * min(check_every, sweeps left) sweeps and computes R again. Every block sums
 * the per-block partials in the same fixed order, so all blocks take the same
 * decision without a further broadcast. pk_result.residual is the last R,
 * sweeps_done the running total. In PK_LAUNCH mode the same loop runs on the
 * host, synchronously, inside this call (each check waits for the GPU).
 * Errors: PK_EINVAL (max_sweeps < 0 or > PK_TASK_N_MAX, check_every < 1,
 * tol < 0 or not a number), otherwise as pk_submit. */
int pk_submit_until(pk_engine* e, int max_sweeps, int check_every, double tol, uint64_t* ticket);

/* Busy-poll (no sleep) until ticket has completed, at most timeout_s seconds
 * (<= 0 => 60 s). r (may be NULL) receives that task's result. The host spins
 * on the device's completion word without sleeping ("Persistent Kernels",
 * "Tuning sleep duration": a sleeping host adds tens of microseconds per task).
 * Errors: PK_EINVAL (ticket never issued), PK_ETIMEDOUT (poisons the engine:
 * a persistent kernel cannot be pre-empted, so only pk_destroy remains, which
 * then leaks rather than free memory the kernel may still use), PK_EDEVICE. */
int pk_wait(pk_engine* e, uint64_t ticket, double timeout_s, pk_result* r);

/* Copy the current field (ny x nx, ring included, row-major, the engine's
 * element type) into the caller-owned dst of at least ny*nx*elem bytes.
 * While the persistent kernel runs this is an in-kernel copy task into pinned
 * host memory (no DMA is queued behind the resident kernel): the device hands
 * results to the host through mapped host memory while it keeps running, as
 * in the CUDA persistent-thread page, sections "Device Communication" and
 * "Task Dispatch" (the ping-pong buffer the host reads while the kernel
 * stays resident).
 * Errors: PK_EINVAL (dst NULL, bytes too small), PK_EBUSY (tasks in flight),
 * PK_ESTATE (poisoned), PK_EDEVICE. */
int pk_readback(pk_engine* e, void* dst, size_t bytes);

/* PK_LAUNCH engines only: advance the field by n sweeps as n kernel launches
 * with the engine's block count, back to back (sync_each = 0) or with a
 * stream synchronize after each launch (sync_each = 1): the standard-launch
 * baselines of "Persistent Kernels", sections "Sketching out the experiment"
 * (same block count for both kernels) and "Comparing the kernels" (queued
 * launches, and a synchronization after every launch). *elapsed_us (may be
 * NULL) receives the host wall time from the first launch until the last
 * sweep finished. Errors: PK_ESTATE (persistent engine: its kernel holds the
 * CUs, extra launches could not run), PK_EBUSY (tasks in flight), PK_EINVAL. */
int pk_run_launch_per_iter(pk_engine* e, int n, int sync_each, double* elapsed_us);

/* PK_LAUNCH engines only: the HIP-graph form of the per-launch baseline
 * ("Persistent Kernels", "Reflections and next steps", the stronger baseline
 * that records a standard kernel's launch sequence once and replays it). The
 * n sweep launches are recorded once into a graph (stream capture on the
 * engine's stream) and the graph is replayed reps times, advancing the field
 * by n * reps sweeps. *elapsed_us (may be NULL) receives the host wall time
 * of the replays, from the first graph launch until the last sweep finished;
 * recording and instantiation are not included. Errors: PK_EINVAL (n < 1,
 * reps < 1), PK_ESTATE (persistent engine, or poisoned), PK_EDEVICE. */
int pk_run_graph_per_iter(pk_engine* e, int n, int reps, double* elapsed_us);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): n Jacobi sweeps and,
 * if residual is not NULL, the residual R of the result, on the caller's own
 * device buffers, with the kernels, grid and results (bit for bit) of a
 * PK_LAUNCH engine created with default options running the tasks SWEEP n and
 * RESIDUAL. Allocates nothing and never synchronizes: the launches are queued
 * on `stream` (NULL: the null stream) and the call returns.
 *   dtype       PK_F32 or PK_F64 (element type T below)
 *   nx, ny      field size (>= 3); pitch: row stride in elements, at least nx
 *               rounded up to 16 bytes, rows 16-byte aligned
 *   u0, u1      device arrays of ny x pitch T, 16-byte aligned. u0 holds the
 *               field (the outer ring is the Dirichlet data); u1 must hold the
 *               same ring, its interior is overwritten. Sweep k reads u[k % 2]
 *               and writes u[(k + 1) % 2]: the result is in u0 for even n, in
 *               u1 for odd n
 *   b           NULL (Laplace), or a device array like u0 holding the scaled
 *               source (T)((h*h) * f) (only interior nodes are read)
 *   residual    NULL, or a device-accessible double (device memory or mapped
 *               pinned host memory) that receives R of the final field
 * Scratch: one partial sum per block of the residual, in a fixed array of the
 * library (PK_NOALLOC_MAX_BLOCKS = 1024 doubles) per GPU. Calls that overlap
 * on one GPU (other streams, other host threads) race on it; each call writes
 * every partial it reads, so nothing carries over from an earlier call.
 * Errors: PK_EINVAL (sizes, pitch, alignment, n < 0, u0 == u1, or a plan whose
 * block count exceeds the scratch), PK_ELAUNCH (kernel not resident),
 * PK_EDEVICE (HIP error while queueing). */
int pk_sweep_noalloc(int dtype, int nx, int ny, int pitch, void* u0, void* u1, const void* b, int n,
                     double* residual, void* stream);

/* Engine geometry and counters: the grid the occupancy query allowed ("@persistent"
 * page, "What it promises"), the layout chosen, and the kernel time measured on the
 * device ("Persistent Kernels", "Sketching out the experiment").
 * Errors: PK_EINVAL (NULL e or info). */
int pk_get_info(pk_engine* e, pk_info* info);

/* PK_DBG_TRACE engines, once the persistent kernel has left (after PK_EXIT):
 * copy the device trace into dst. Layout, per block in block order: a uint64
 * count of the events the block recorded, then trace_capacity records of
 * {uint64 time (device wall clock, pk_info.wall_clock_khz), uint32 kind,
 * uint32 aux}; event e sits in record e % trace_capacity, so when count exceeds
 * the capacity the ring holds the latest events. Kinds: 1 task begin, 2 task end
 * (aux = task kind), 3 arrival at and 4 departure from a grid barrier (aux 0)
 * or neighbour sync (aux 1), 5 and 6 wave 0 starts and ends polling tagged halo
 * words, 7 a tile period starts (aux = its sweeps). *needed (may be NULL)
 * receives the bytes; dst NULL only asks for them. The measurement behind
 * "Grid-Wide Barriers and Persistent Work Queues", "What the barrier buys"
 * (every block waits for the slowest). Errors: PK_ESTATE (no trace, launch
 * mode), PK_EBUSY (the kernel is still running), PK_EINVAL (bytes too small),
 * PK_EDEVICE. */
int pk_trace_read(pk_engine* e, void* dst, size_t bytes, size_t* needed);

/* Stop the kernel (EXIT, bounded wait) and free everything. NULL is a no-op.
 * The kernel leaves only when it reads the EXIT task, so destroy first asks
 * for it through the ring ("Persistent Kernels", "Base implementation": the
 * host's stop task ends the persistent loop). If the kernel does not leave,
 * device memory is deliberately leaked and PK_ETIMEDOUT returned. */
int pk_destroy(pk_engine* e);

/* Static string for a status code (never NULL). Errors travel as status codes,
 * never as an abort of the process (the CUDA persistent-thread page, "Code
 * Implementation", aborts on any runtime error; a library cannot). */
const char* pk_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* PK_H */
