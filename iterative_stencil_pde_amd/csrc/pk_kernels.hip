// Kernels of the Jacobi engine for gfx950 and the host-side wrappers that
// launch them. The persistent kernel is launched once per engine; the sweep,
// residual and source kernels serve the launch-per-sweep baseline and setup.
#include <hip/hip_runtime.h>
#include <math.h>

#include "pk_device.h"
#include "pk_launch.h"
#include "pk_shared.h"
#include "../../include/pk.h"

using namespace pkd;

namespace {

// ---------------------------------------------------------------------------
// LDS-resident SWEEP task. Block (logical) L owns interior rows [r0, r1) and
// keeps rows [r0 - m, r1 + m) in LDS (two ping-pong buffers, plus b). Each
// period of up to m sweeps runs entirely in LDS: sub-sweep s recomputes the
// owned rows widened by the number of sub-sweeps still to come, so after the
// period the owned rows hold exact Jacobi values (a wider halo traded for
// redundant edge work, "Persistent Kernels", "Reflections and next steps",
// "Fewer handshakes"). Then the block publishes its m edge rows on each side
// (all its rows after the last period) into the other global buffer, the grid
// barrier orders those stores, and the block reads its neighbours' edge rows
// as its new halo. Alternating global buffers by exchange keeps a fast block
// from overwriting rows a slow neighbour still reads.
// ---------------------------------------------------------------------------
template <typename T, bool HAS_B>
__device__ void resident_sweep_task(const pk_kargs& a, int n, int& cur, BarrierCtx& bc, T* lds) {
    constexpr int W = VecW<T>::W;
    const int lb = logical_block(a.xcd_remap, a.grid);
    const int ny = a.ny;
    const int r0 = 1 + lb * a.res_band_rows;
    const int r1 = min(ny - 1, r0 + a.res_band_rows);
    const int m = a.res_halo;
    const int e0 = max(0, r0 - m);
    const int e1 = min(ny, r1 + m);
    const int lp = a.lds_pitch;
    const int nv = lp / W;
    const size_t p = static_cast<size_t>(a.pitch);
    T* A = lds;
    T* B = lds + static_cast<size_t>(a.res_ext_rows) * lp;
    T* Bt = lds + 2 * static_cast<size_t>(a.res_ext_rows) * lp;
    const int tid = static_cast<int>(threadIdx.x), nt = static_cast<int>(blockDim.x);

    {   // the task's starting tile, from the buffer that holds the whole field
        const T* g = static_cast<const T*>(a.u[cur]);
        const T* gb = static_cast<const T*>(a.b);
        const int tot = (e1 - e0) * nv;
        for (int idx = tid; idx < tot; idx += nt) {
            const int rr = idx / nv, col = (idx % nv) * W;
            const size_t go = static_cast<size_t>(e0 + rr) * p + col;
            const Vec<T> x = vload(g + go);
            vstore(A + rr * lp + col, x);
            vstore(B + rr * lp + col, x);
            if (HAS_B) vstore(Bt + rr * lp + col, vload(gb + go));
        }
    }
    __syncthreads();

    T* S = A;
    T* D = B;
    int remaining = n;
    while (remaining > 0) {
        const int sc = min(m, remaining);
        for (int s = 1; s <= sc; ++s) {
            const int lo = (r0 == 1) ? 1 : r0 - (sc - s);
            const int hi = (r1 == ny - 1) ? ny - 1 : r1 + (sc - s);
            resident_rows<T, HAS_B>(S, D, Bt, lo - e0, hi - e0, nv, lp, a.nx);
            __syncthreads();
            T* t = S;
            S = D;
            D = t;
        }
        remaining -= sc;
        const int mn = min(m, remaining);

        {   // publish: edge rows for the neighbours, or every owned row at the end
            T* g = static_cast<T*>(a.u[cur ^ 1]);
            int top_end, bot_begin;
            if (remaining == 0) {
                top_end = r1;
                bot_begin = r1;
            } else {
                top_end = (r0 > 1) ? min(r1, r0 + mn) : r0;
                bot_begin = (r1 < ny - 1) ? max(top_end, r1 - mn) : r1;
            }
            const int ntop = top_end - r0, nbot = r1 - bot_begin;
            const int tot = (ntop + nbot) * nv;
            for (int idx = tid; idx < tot; idx += nt) {
                const int k = idx / nv, col = (idx % nv) * W;
                const int rr = (k < ntop) ? r0 + k : bot_begin + (k - ntop);
                vstore(g + static_cast<size_t>(rr) * p + col, vload(S + (rr - e0) * lp + col));
            }
        }
        grid_barrier(bc, bc.broken);
        cur ^= 1;
        if (remaining > 0) {  // the neighbours' edge rows become this block's halo
            const T* g = static_cast<const T*>(a.u[cur]);
            const int above = (r0 > 1) ? mn : 0;
            const int below = (r1 < ny - 1) ? mn : 0;
            const int tot = (above + below) * nv;
            for (int idx = tid; idx < tot; idx += nt) {
                const int k = idx / nv, col = (idx % nv) * W;
                const int rr = (k < above) ? r0 - above + k : r1 + (k - above);
                vstore(S + (rr - e0) * lp + col, vload(g + static_cast<size_t>(rr) * p + col));
            }
            __syncthreads();
        }
    }
}

// Copy the field (unpadded rows) into the pinned host staging buffer.
template <typename T>
__device__ void readback_task(const pk_kargs& a, int cur) {
    const T* g = static_cast<const T*>(a.u[cur]);
    T* h = static_cast<T*>(a.staging);
    const int lane = threadIdx.x & 63;
    const int wpb = static_cast<int>(blockDim.x) >> 6;
    const int gw = static_cast<int>(blockIdx.x) * wpb + (static_cast<int>(threadIdx.x) >> 6);
    const int nw = a.grid * wpb;
    for (int r = gw; r < a.ny; r += nw) {
        const T* src = g + static_cast<size_t>(r) * a.pitch;
        T* dst = h + static_cast<size_t>(r) * a.nx;
        for (int c = lane; c < a.nx; c += 64) dst[c] = src[c];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");  // system scope: host-visible first
}

// Barrier visibility check: every block stamps its 64-word slot with the
// round number, crosses the barrier, and reads the slots of its neighbour and
// of a pseudo-random remote block; each word must carry this round's stamp.
// Slots alternate by round parity so a fast block never overwrites a slot that
// a slow block is still checking (the stamp/validate pattern of the ping-pong
// example on the persistent-thread page, "Task Dispatch").
__device__ int64_t stamp_task(const pk_kargs& a, int n, uint32_t& round, BarrierCtx& bc,
                              double* s_red) {
    int64_t errs = 0;
    const int g = a.grid;
    for (int k = 0; k < n; ++k) {
        const uint32_t s = ++round;
        uint32_t* base = a.stamp + static_cast<size_t>(s & 1u) * g * 64;
        if (threadIdx.x < 64) base[blockIdx.x * 64 + threadIdx.x] = s;
        grid_barrier(bc, bc.broken);
        if (threadIdx.x < 64) {
            const int nb = (static_cast<int>(blockIdx.x) + 1) % g;
            const uint32_t hsh = (s * 2654435761u) ^ (blockIdx.x * 40503u + 977u);
            const int rb = static_cast<int>(hsh % static_cast<uint32_t>(g));
            const uint32_t v1 = base[nb * 64 + threadIdx.x];
            const uint32_t v2 = base[rb * 64 + threadIdx.x];
            errs += (v1 != s) + (v2 != s);
        }
    }
    const double tot = block_sum(static_cast<double>(errs), s_red);
    if (threadIdx.x == 0 && tot > 0)
        __hip_atomic_fetch_add(&a.st->stamp_errors, static_cast<uint64_t>(tot), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    grid_barrier(bc);
    int64_t total = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        total = static_cast<int64_t>(__hip_atomic_load(&a.st->stamp_errors, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT));
        __hip_atomic_store(&a.st->stamp_errors, uint64_t(0), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    return total;
}

// ---------------------------------------------------------------------------
// The persistent kernel: launched once, loops over host tasks until EXIT.
// Block 0 lane 0 is the only thread that touches the host mailbox: it polls
// `tail` with relaxed system-scope loads, acquires once a task is there, and
// writes the task into device memory; the grid barrier that follows hands it
// to every block (one poller and a broadcast instead of per-block flags,
// "Persistent Kernels", "Thread synchronization"). The answer is written only
// after the task's last barrier and released before `done_seq` moves, so the
// host never sees "done" ahead of the work ("Reflections", point 3).
// ---------------------------------------------------------------------------
template <typename T, bool HAS_B, int LAYOUT>
__global__ void __launch_bounds__(1024) pk_persistent(pk_kargs a) {
    extern __shared__ __align__(16) unsigned char pk_lds[];
    __shared__ double s_red[16];
    __shared__ int s_kind, s_n, s_exit;
    __shared__ unsigned long long s_seq;

    BarrierCtx bc;
    bc.st = a.st;
    bc.grid = static_cast<uint32_t>(a.grid);
    bc.epoch = 0;
    bc.spin_ticks = a.spin_ticks;
    bc.broken = (a.flags & PK_DBG_BROKEN_BARRIER) != 0;
    bc.two_level = a.barrier_kind == PK_BARRIER_TWO_LEVEL;
    bc.xcd = false;
    bc.faulted = false;
    bc.xg = 0;
    bc.xmembers = 1;
    bc.xgroups = 1;
    if (a.barrier_kind == PK_BARRIER_XCD && a.grid > 1 && !bc.broken) {
        // count the blocks on each XCD (one flat barrier, generation 1), then
        // switch to the XCD barrier, whose counters start from zero
        if (threadIdx.x == 0) {
            bc.xg = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 7u;  // hwreg(HW_REG_XCC_ID, 0, 4)
            __hip_atomic_fetch_add(&a.st->xmembers[bc.xg].v, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        grid_barrier(bc);
        if (threadIdx.x == 0) {
            bc.xmembers = __hip_atomic_load(&a.st->xmembers[bc.xg].v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            bc.xgroups = 0;
            for (int k = 0; k < 8; ++k)
                bc.xgroups += __hip_atomic_load(&a.st->xmembers[k].v, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT) > 0u ? 1u : 0u;
        }
        bc.epoch = 0;
        bc.xcd = true;
    }

    const bool leader = (blockIdx.x == 0) && (threadIdx.x == 0);
    int cur = a.cur0;
    int64_t sweeps = 0;
    uint64_t next_seq = 1;
    uint32_t stamp_round = 0;
    pk_mailbox* mail = a.mail;

    for (;;) {
        if (leader) {
            uint32_t fault = __hip_atomic_load(&a.st->fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            int kind = PK_EXIT, nn = 0;
            if (!bc.faulted && fault == 0) {
                const uint64_t t0 = wall_clock64();
                bool idle = false;
                while (__hip_atomic_load(&mail->tail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) <
                       next_seq) {
                    __builtin_amdgcn_s_sleep(1);
                    if (wall_clock64() - t0 > a.idle_ticks) {
                        idle = true;
                        break;
                    }
                }
                if (idle) {
                    __hip_atomic_store(&a.st->fault, static_cast<uint32_t>(PK_FAULT_IDLE_TIMEOUT),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                } else {
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");  // the slot the host released
                    const pk_slot* sl = &mail->slot[next_seq % PK_RING];
                    const uint64_t sseq =
                        __hip_atomic_load(&sl->seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                    kind = __hip_atomic_load(&sl->kind, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                    nn = __hip_atomic_load(&sl->n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                    if (sseq != next_seq) {
                        kind = PK_EXIT;
                        __hip_atomic_store(&a.st->fault, static_cast<uint32_t>(PK_FAULT_BAD_TASK),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            }
            a.st->task_seq = next_seq;
            a.st->task_kind = kind;
            a.st->task_n = nn;
        }
        grid_barrier(bc);
        if (threadIdx.x == 0) {
            s_kind = __hip_atomic_load(&a.st->task_kind, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_n = __hip_atomic_load(&a.st->task_n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_seq = __hip_atomic_load(&a.st->task_seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t f = __hip_atomic_load(&a.st->fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_exit = (bc.faulted || f != 0 || s_kind == PK_EXIT) ? 1 : 0;
        }
        __syncthreads();
        const int kind = s_kind, n = s_n;
        const uint64_t seq = s_seq;
        const uint64_t t_begin = leader ? wall_clock64() : 0;

        if (s_exit) {
            if (leader) {
                const uint32_t f = __hip_atomic_load(&a.st->fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint32_t code = (f != 0) ? f : (bc.faulted ? PK_FAULT_BARRIER_TIMEOUT : 0u);
                if (kind == PK_EXIT && code == 0) {
                    pk_done_rec* d = &mail->done[seq % PK_RING];
                    d->kind = PK_EXIT;
                    d->status = PK_OK;
                    d->residual = 0.0;
                    d->sweeps_done = sweeps;
                    d->t_begin = t_begin;
                    d->t_end = t_begin;
                    d->errors = 0;
                    d->cur = cur;
                    d->seq = seq;
                    __hip_atomic_store(&mail->done_seq, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
                }
                __hip_atomic_store(&mail->fault, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                __hip_atomic_store(&mail->exited, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
            }
            break;
        }

        double res = 0.0;
        int64_t errs = 0;
        int status = PK_OK;
        if (kind == PK_SWEEP) {
            if constexpr (LAYOUT == PK_LAYOUT_RESIDENT) {
                resident_sweep_task<T, HAS_B>(a, n, cur, bc, reinterpret_cast<T*>(pk_lds));
            } else {
                for (int s = 0; s < n;) {
                    const int k = min(a.pass_sweeps, n - s);
                    stream_pass<T, HAS_B>(a, static_cast<const T*>(a.u[cur]), static_cast<T*>(a.u[cur ^ 1]), k);
                    grid_barrier(bc, bc.broken);
                    cur ^= 1;
                    s += k;
                }
            }
            sweeps += n;
        } else if (kind == PK_RESIDUAL) {
            const double part = stream_residual_block<T, HAS_B>(a, static_cast<const T*>(a.u[cur]), s_red);
            if (threadIdx.x == 0) a.partials[blockIdx.x] = part;
            grid_barrier(bc);
            if (blockIdx.x == 0) {
                const double tot = sum_partials(a.partials, a.grid);
                if (threadIdx.x == 0) res = sqrt(tot);
            }
        } else if (kind == PK_TASK_READBACK) {
            readback_task<T>(a, cur);
            grid_barrier(bc);
        } else if (kind == PK_BARRIER) {
            for (int s = 0; s < n; ++s) grid_barrier(bc);
        } else if (kind == PK_STAMP) {
            errs = stamp_task(a, n, stamp_round, bc, s_red);
        } else {
            status = PK_EINVAL;
        }
        if (leader) {
            pk_done_rec* d = &mail->done[seq % PK_RING];
            d->kind = kind;
            d->status = bc.faulted ? PK_EDEVICE : status;
            d->residual = res;
            d->sweeps_done = sweeps;
            d->t_begin = t_begin;
            d->t_end = wall_clock64();
            d->errors = errs;
            d->cur = cur;
            d->seq = seq;
            __hip_atomic_store(&mail->done_seq, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
            next_seq = seq + 1;
        }
    }
}

// ---- launch-per-sweep baseline and setup kernels ----------------------------
template <typename T, bool HAS_B>
__global__ void __launch_bounds__(1024) pk_sweep_launch(pk_kargs a, int src) {
    stream_sweep<T, HAS_B>(a, static_cast<const T*>(a.u[src]), static_cast<T*>(a.u[src ^ 1]));
}

template <typename T, bool HAS_B>
__global__ void __launch_bounds__(1024) pk_residual_launch(pk_kargs a, int src) {
    __shared__ double s_red[16];
    const double part = stream_residual_block<T, HAS_B>(a, static_cast<const T*>(a.u[src]), s_red);
    if (threadIdx.x == 0) a.partials[blockIdx.x] = part;
}

__global__ void __launch_bounds__(64) pk_residual_finalize(const double* partials, int grid,
                                                           double* out) {
    const double tot = sum_partials(partials, grid);
    if (threadIdx.x == 0) *out = sqrt(tot);
}

// b = (T)((h*h) * f) on every node, pitched.
template <typename T>
__global__ void __launch_bounds__(256) pk_scale_source(const T* f, T* b, int nx, int ny, int pitch,
                                                       double hh) {
    const size_t total = static_cast<size_t>(ny) * pitch;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
         i += static_cast<size_t>(gridDim.x) * blockDim.x) {
        const int c = static_cast<int>(i % pitch);
        b[i] = (c < nx) ? static_cast<T>(hh * static_cast<double>(f[i])) : T(0);
    }
}

template <typename T>
const void* persistent_fn(bool has_b, int layout) {
    if (layout == PK_LAYOUT_RESIDENT)
        return has_b ? reinterpret_cast<const void*>(&pk_persistent<T, true, PK_LAYOUT_RESIDENT>)
                     : reinterpret_cast<const void*>(&pk_persistent<T, false, PK_LAYOUT_RESIDENT>);
    return has_b ? reinterpret_cast<const void*>(&pk_persistent<T, true, PK_LAYOUT_STREAM>)
                 : reinterpret_cast<const void*>(&pk_persistent<T, false, PK_LAYOUT_STREAM>);
}

template <typename T>
const void* sweep_fn(bool has_b) {
    return has_b ? reinterpret_cast<const void*>(&pk_sweep_launch<T, true>)
                 : reinterpret_cast<const void*>(&pk_sweep_launch<T, false>);
}

}  // namespace

// ---- host-side entry points used by the runtime ------------------------------
const void* pkk_persistent_fn(int dtype, bool has_b, int layout) {
    return dtype == PK_F64 ? persistent_fn<double>(has_b, layout) : persistent_fn<float>(has_b, layout);
}

const void* pkk_sweep_fn(int dtype, bool has_b) {
    return dtype == PK_F64 ? sweep_fn<double>(has_b) : sweep_fn<float>(has_b);
}

hipError_t pkk_launch_sweep(int dtype, bool has_b, const pk_kargs& a, int threads, int src,
                            hipStream_t s) {
    const dim3 g(a.grid), b(threads);
    if (dtype == PK_F64) {
        if (has_b) hipLaunchKernelGGL((pk_sweep_launch<double, true>), g, b, 0, s, a, src);
        else hipLaunchKernelGGL((pk_sweep_launch<double, false>), g, b, 0, s, a, src);
    } else {
        if (has_b) hipLaunchKernelGGL((pk_sweep_launch<float, true>), g, b, 0, s, a, src);
        else hipLaunchKernelGGL((pk_sweep_launch<float, false>), g, b, 0, s, a, src);
    }
    return hipGetLastError();
}

hipError_t pkk_launch_residual(int dtype, bool has_b, const pk_kargs& a, int threads, int src,
                               double* out, hipStream_t s) {
    const dim3 g(a.grid), b(threads);
    if (dtype == PK_F64) {
        if (has_b) hipLaunchKernelGGL((pk_residual_launch<double, true>), g, b, 0, s, a, src);
        else hipLaunchKernelGGL((pk_residual_launch<double, false>), g, b, 0, s, a, src);
    } else {
        if (has_b) hipLaunchKernelGGL((pk_residual_launch<float, true>), g, b, 0, s, a, src);
        else hipLaunchKernelGGL((pk_residual_launch<float, false>), g, b, 0, s, a, src);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(pk_residual_finalize, dim3(1), dim3(64), 0, s, a.partials, a.grid, out);
    return hipGetLastError();
}

hipError_t pkk_launch_scale_source(int dtype, const void* f, void* b, int nx, int ny, int pitch,
                                   double hh, hipStream_t s) {
    const size_t total = static_cast<size_t>(ny) * pitch;
    const size_t want = (total + 255) / 256;
    const unsigned blocks = static_cast<unsigned>(want < 4096 ? want : 4096);
    if (dtype == PK_F64)
        hipLaunchKernelGGL(pk_scale_source<double>, dim3(blocks), dim3(256), 0, s,
                           static_cast<const double*>(f), static_cast<double*>(b), nx, ny, pitch, hh);
    else
        hipLaunchKernelGGL(pk_scale_source<float>, dim3(blocks), dim3(256), 0, s,
                           static_cast<const float*>(f), static_cast<float*>(b), nx, ny, pitch, hh);
    return hipGetLastError();
}
