// Device building blocks of the Jacobi engine (gfx950, wave64).
//
// The update every sweep applies to an interior node, in the element type T:
//     new = 0.25 * (((W + E) + (S + N)) + b)
// ("Persistent Kernels: Bridging GPU-CPU Execution", "The problem" and its
// "Derivation", with the source taken as -Lap(u) = f so b = +h*h*f; the order
// of the additions is fixed so that every implementation rounds alike).
// W/E are the neighbours in the same row, S/N the rows i-1 / i+1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pk_shared.h"

namespace pkd {

// ---------------------------------------------------------------------------
// 16-byte vectors: four floats or two doubles per lane, so one wave moves
// 1 KiB of a row per load instruction (global_load_dwordx4).
// ---------------------------------------------------------------------------
template <typename T>
struct VecW {
    static constexpr int W = 16 / sizeof(T);
};

// The compiler's vector type of one 16-byte vector (elements indexed as v[k]).
template <typename T>
using NativeVec = T __attribute__((ext_vector_type(VecW<T>::W)));

template <typename T>
struct alignas(16) Vec {
    NativeVec<T> v;
};

template <typename T>
__device__ __forceinline__ Vec<T> vzero() {
    Vec<T> r;
#pragma unroll
    for (int k = 0; k < VecW<T>::W; ++k) r.v[k] = T(0);
    return r;
}

template <typename T>
__device__ __forceinline__ Vec<T> vload(const T* p) {
    return *reinterpret_cast<const Vec<T>*>(p);
}

template <typename T>
__device__ __forceinline__ void vstore(T* p, const Vec<T>& x) {
    *reinterpret_cast<Vec<T>*>(p) = x;
}

// The same for device (global) memory, through address-space-1 pointers: the
// field pointers are chosen at run time (u[cur]), so the compiler cannot infer
// their address space and would otherwise emit flat loads and stores.
template <typename T>
__device__ __forceinline__ Vec<T> gload(const T* p) {
    Vec<T> r;
    r.v = *((__attribute__((address_space(1))) const NativeVec<T>*)(p));
    return r;
}

// Wait for this wave's outstanding vector memory operations (vmcnt(0)).
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Buffer access: a resource descriptor (base, size in bytes) in scalar
// registers, a per-lane byte offset and a wave-uniform byte offset. The lane
// offset stays in one register for a whole march and the row offset is scalar,
// so a row load needs no 64-bit address arithmetic and no address register
// that a later instruction could overwrite while the load is in flight.
// Descriptor word 3 is the data-format word of the gfx9 family (32-bit format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

template <typename T>
__device__ __forceinline__ Vec<T> bload(__amdgpu_buffer_rsrc_t r, uint32_t lane_off, uint32_t row_off) {
    Vec<T> x;
    x.v = __builtin_bit_cast(NativeVec<T>, __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, row_off, 0));
    return x;
}

template <typename T>
__device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, uint32_t lane_off, uint32_t row_off,
                                       const Vec<T>& x) {
    using U = unsigned int __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(U, x.v), r, lane_off, row_off, 0);
}

template <typename T>
__device__ __forceinline__ void gstore(T* p, const Vec<T>& x) {
    *((__attribute__((address_space(1))) NativeVec<T>*)(p)) = x.v;
}

template <typename T>
__device__ __forceinline__ T gload1(const T* p) {
    return *((__attribute__((address_space(1))) const T*)(p));
}

// ---------------------------------------------------------------------------
// Tagged halo words: a 16-byte vector travels as four 64-bit words, each a
// 32-bit quarter of the data (low half) and the exchange tag (high half),
// stored and loaded as relaxed device-scope atomics. A 64-bit atomic access is
// whole, so a word whose tag matches carries that exchange's data. Quarter k
// of the vectors of a row lies in plane k (`plane` words apart), so the lanes
// of a wave touch consecutive words in every access.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void tag_store(uint64_t* p, int plane, const Vec<T>& x, uint32_t tag) {
    const NativeVec<T> v = x.v;
    const uint32_t* h = reinterpret_cast<const uint32_t*>(&v);
    const uint64_t hi = static_cast<uint64_t>(tag) << 32;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        __hip_atomic_store(p + static_cast<size_t>(k) * plane, hi | h[k], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Loads the four words; true when every one carries `tag` (x is then the data).
template <typename T>
__device__ __forceinline__ bool tag_load(const uint64_t* p, int plane, Vec<T>& x, uint32_t tag) {
    uint64_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        w[k] = __hip_atomic_load(const_cast<uint64_t*>(p + static_cast<size_t>(k) * plane), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    NativeVec<T> v;
    uint32_t* h = reinterpret_cast<uint32_t*>(&v);
    bool ok = true;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        h[k] = static_cast<uint32_t>(w[k]);
        ok = ok && static_cast<uint32_t>(w[k] >> 32) == tag;
    }
    x.v = v;
    return ok;
}

// ---------------------------------------------------------------------------
// Whole-wave lane shifts (DPP wave_shr:1 / wave_shl:1). Lane l receives the
// value of lane l-1 (from_lower) or l+1 (from_upper); the lane with no source
// (0 or 63) keeps `edge`, which the caller loads from memory for exactly that
// lane. This gives each lane its W/E neighbour across the 16-byte vectors.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int dpp_from_lower_i(int edge, int v) {
    return __builtin_amdgcn_update_dpp(edge, v, 0x138, 0xf, 0xf, false);
}
__device__ __forceinline__ int dpp_from_upper_i(int edge, int v) {
    return __builtin_amdgcn_update_dpp(edge, v, 0x130, 0xf, 0xf, false);
}

__device__ __forceinline__ float from_lower(float edge, float v) {
    return __int_as_float(dpp_from_lower_i(__float_as_int(edge), __float_as_int(v)));
}
__device__ __forceinline__ float from_upper(float edge, float v) {
    return __int_as_float(dpp_from_upper_i(__float_as_int(edge), __float_as_int(v)));
}
__device__ __forceinline__ double from_lower(double edge, double v) {
    const long long e = __double_as_longlong(edge), x = __double_as_longlong(v);
    const int lo = dpp_from_lower_i(static_cast<int>(e), static_cast<int>(x));
    const int hi = dpp_from_lower_i(static_cast<int>(e >> 32), static_cast<int>(x >> 32));
    return __longlong_as_double((static_cast<long long>(hi) << 32) |
                                static_cast<long long>(static_cast<unsigned>(lo)));
}
__device__ __forceinline__ double from_upper(double edge, double v) {
    const long long e = __double_as_longlong(edge), x = __double_as_longlong(v);
    const int lo = dpp_from_upper_i(static_cast<int>(e), static_cast<int>(x));
    const int hi = dpp_from_upper_i(static_cast<int>(e >> 32), static_cast<int>(x >> 32));
    return __longlong_as_double((static_cast<long long>(hi) << 32) |
                                static_cast<long long>(static_cast<unsigned>(lo)));
}

// Per-lane bit blend: `keep_val` where the mask word is all ones, else
// `new_val`, as one v_bfi_b32 per 32 bits (written out: the optimiser would
// otherwise turn the choice into a select, and that into a branch around the
// arithmetic, or split it into two logic operations).
__device__ __forceinline__ uint32_t lane_mask(bool b) { return b ? 0xffffffffu : 0u; }
__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b) {
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(mask), "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float blend(uint32_t mask, float keep_val, float new_val) {
    return __uint_as_float(bfi(mask, __float_as_uint(keep_val), __float_as_uint(new_val)));
}
__device__ __forceinline__ double blend(uint32_t mask, double keep_val, double new_val) {
    const unsigned long long k = static_cast<unsigned long long>(__double_as_longlong(keep_val));
    const unsigned long long x = static_cast<unsigned long long>(__double_as_longlong(new_val));
    const uint32_t lo = bfi(mask, static_cast<uint32_t>(k), static_cast<uint32_t>(x));
    const uint32_t hi = bfi(mask, static_cast<uint32_t>(k >> 32), static_cast<uint32_t>(x >> 32));
    return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}

// The same lane shifts where the lane with no source (0 or 63) may receive
// anything (here zero): its result is not used. Without an old value to keep,
// the compiler can fold the shift into the add that consumes it.
__device__ __forceinline__ float from_lower_any(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x138, 0xf, 0xf, true));
}
__device__ __forceinline__ float from_upper_any(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x130, 0xf, 0xf, true));
}
__device__ __forceinline__ double from_lower_any(double v) {
    const long long x = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(x), 0x138, 0xf, 0xf, true);
    const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(x >> 32), 0x138, 0xf, 0xf, true);
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<long long>(static_cast<unsigned>(lo)));
}
__device__ __forceinline__ double from_upper_any(double v) {
    const long long x = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(x), 0x130, 0xf, 0xf, true);
    const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(x >> 32), 0x130, 0xf, 0xf, true);
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<long long>(static_cast<unsigned>(lo)));
}

// ---------------------------------------------------------------------------
// The stencil on one lane's vector. `col` is the first column of the vector;
// columns 0 and nx-1 (the Dirichlet ring) and padding columns >= nx keep
// their value. west_of_first / east_of_last are columns col-1 and col+W of
// the same row. In stencil(), `edge` holds, for lane 0, column col-1 and, for
// lane 63, column col+W; the other lanes get theirs by DPP.
// ---------------------------------------------------------------------------
template <typename T, bool HAS_B>
__device__ __forceinline__ Vec<T> stencil_we(const Vec<T>& s, const Vec<T>& m, const Vec<T>& n,
                                             const Vec<T>& b, T west_of_first, T east_of_last,
                                             int col, int nx) {
    constexpr int W = VecW<T>::W;
    Vec<T> o;
#pragma unroll
    for (int k = 0; k < W; ++k) {
        const T w = (k == 0) ? west_of_first : m.v[k - 1];
        const T e = (k == W - 1) ? east_of_last : m.v[k + 1];
        T t = (w + e) + (s.v[k] + n.v[k]);
        if (HAS_B) t = t + b.v[k];
        const int c = col + k;
        const bool ring = (c == 0) || (c >= nx - 1);
        o.v[k] = ring ? m.v[k] : T(0.25) * t;
    }
    return o;
}

// W/E neighbours of the end elements passed in (stencil_we) or taken by DPP
// from the adjacent lanes (stencil).
template <typename T, bool HAS_B>
__device__ __forceinline__ Vec<T> stencil(const Vec<T>& s, const Vec<T>& m, const Vec<T>& n,
                                          const Vec<T>& b, T edge, int col, int nx) {
    constexpr int W = VecW<T>::W;
    return stencil_we<T, HAS_B>(s, m, n, b, from_lower(edge, m.v[W - 1]), from_upper(edge, m.v[0]),
                                col, nx);
}

// Red-black half-sweeps ("Persistent Kernels", "Implementation details and
// correctness", Figure 3): node (i, j) is red when i + j is even; a half-sweep
// of colour `parity` updates only the nodes of that colour and keeps the rest.
// A vector starts at an even column, so in row `row` the updated elements are
// those whose index k has k mod 2 == (row + parity) mod 2.
template <typename T>
__device__ __forceinline__ Vec<T> rb_keep(const Vec<T>& o, const Vec<T>& m, int row, int parity) {
    constexpr int W = VecW<T>::W;
    const int rp = (row + parity) & 1;
    Vec<T> r;
#pragma unroll
    for (int k = 0; k < W; ++k) r.v[k] = ((k & 1) == rp) ? o.v[k] : m.v[k];
    return r;
}

// rho^2 summed over the interior nodes of one vector, in double:
//     rho = (((W + E) + (S + N)) + b) - 4u.
template <typename T, bool HAS_B>
__device__ __forceinline__ double rho2(const Vec<T>& s, const Vec<T>& m, const Vec<T>& n,
                                       const Vec<T>& b, T edge, int col, int nx) {
    constexpr int W = VecW<T>::W;
    const T west_of_first = from_lower(edge, m.v[W - 1]);
    const T east_of_last = from_upper(edge, m.v[0]);
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < W; ++k) {
        const double w = static_cast<double>((k == 0) ? west_of_first : m.v[k - 1]);
        const double e = static_cast<double>((k == W - 1) ? east_of_last : m.v[k + 1]);
        double t = (w + e) + (static_cast<double>(s.v[k]) + static_cast<double>(n.v[k]));
        if (HAS_B) t = t + static_cast<double>(b.v[k]);
        const double r = t - 4.0 * static_cast<double>(m.v[k]);
        const int c = col + k;
        const bool ring = (c == 0) || (c >= nx - 1);
        acc += ring ? 0.0 : r * r;
    }
    return acc;
}

// A store kept on its own: a relaxed atomic store is neither merged with the
// stores beside it into one wide store (whose register tuple the compiler then
// keeps live, and spills, across the task loop) nor made to wait for its own
// completion, as a volatile store is. For records written field by field by one
// thread (task completions, trace events); what orders them is the release
// that publishes the record.
template <typename V>
struct Same {
    using type = V;
};
template <typename V>
__device__ __forceinline__ void put(V* p, typename Same<V>::type v, int scope = __HIP_MEMORY_SCOPE_SYSTEM) {
    if constexpr (sizeof(V) == 8)
        __hip_atomic_store(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                           scope);
    else
        __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __builtin_bit_cast(uint32_t, v), __ATOMIC_RELAXED,
                           scope);
}

// ---------------------------------------------------------------------------
// Grid-wide barrier: an arrival counter plus a generation word
// ("Grid-Wide Barriers and Persistent Work Queues", "The barrier is a counter
// and a generation"; the "@persistent" page, "grid_barrier"). The counter only
// ever grows: generation g completes when it reaches (g+1) * G, so there is no
// reset and no reset race ("Failure modes that only appear at this scale").
//   - each thread of the block arrives at a block barrier first;
//   - lane 0 adds 1 to the counter with release ordering (agent scope), so
//     the block's stores are visible before it is counted;
//   - the block that brings the counter to (g+1) * G stores g+1 into the
//     generation word with release ordering; the others spin on it with
//     relaxed loads and then issue one acquire fence, so the loads after the
//     barrier see every block's stores (spin relaxed, acquire once:
//     "Persistent Kernels", "Reflections and next steps", point 2);
//   - a final block barrier releases the block's other threads.
// The grid must be co-resident (cooperative launch). A wait that exceeds
// `spin_ticks` of the device wall clock marks the engine faulted and stops
// waiting from then on, so every wave still reaches the end of the kernel.
// `relaxed` (negative control only, set for the barriers between sweeps and
// stamp rounds of an engine created with PK_DBG_BROKEN_BARRIER) drops the
// release/acquire ordering: the same atomics, relaxed, and no fence. Every
// block still runs the same number of barriers and every wait still ends;
// only the visibility of other blocks' writes is no longer ordered. The task
// broadcast and the other barriers always keep their ordering, so all blocks
// agree on what to run.
// ---------------------------------------------------------------------------
struct BarrierCtx {
    pk_dev_state* st;
    uint32_t grid;
    uint32_t epoch;      // generations completed (identical in every block)
    uint64_t spin_ticks;
    bool broken;         // engine flag: data barriers run relaxed (negative control)
    bool two_level;      // per-XCD-group counters under a top counter
    bool xcd;            // groups by hardware XCD, cache maintenance once per XCD
    bool faulted;        // thread 0's view; broadcast at task boundaries
    // XCD barrier: thread 0's view of its groups, in the block's shared memory
    // (values live across every task would otherwise hold vector registers)
    struct XcdState* xs;
    uint32_t nbr_epoch;  // neighbour exchanges completed (identical in every block)
    uint64_t tag_epoch;  // tagged exchanges completed (identical in every block)
    uint32_t nbar;       // grid barriers passed (identical in every block)
    // task carry: leader-only state in the block's shared memory (registers
    // live across every pass cost the streaming kernels spills), except the
    // read-ahead slot word, which must stay a register for its load to be in
    // flight while the task runs
    struct CarryState* carry;
    uint64_t carry_word;
    // device trace (thread 0's view), in the block's shared memory: the state
    // is touched only when an event is recorded, so it takes no registers
    struct TraceState* trace;
    // streaming passes under neighbour counters, in the block's shared memory
    // (kernel arguments read inside the task loop would be kept in registers
    // across every pass)
    struct PassNbr* pn;
};

// Neighbour counters between streaming passes: whether the passes use them
// (the same in every block), and the XCDs a block waits for after a pass, one bit
// each: its own and those that run the blocks whose units border its own.
struct PassNbr {
    uint32_t on;
    uint32_t mask;
};

// XCD barrier groups as thread 0 sees them: this block's XCD, the blocks on it,
// and the XCDs with at least one block.
struct XcdState {
    uint32_t g;
    uint32_t members;
    uint32_t groups;
};

// This block's trace ring (null when the trace is off) and its event count.
struct TraceState {
    unsigned char* ring;
    uint64_t count;
};

// Appends one event to the block's trace ring (thread 0 only; a no-op when the
// trace is off).
__device__ __forceinline__ void trace_event(BarrierCtx& bc, uint32_t kind, uint32_t aux = 0) {
    if (threadIdx.x != 0) return;
    TraceState* ts = bc.trace;
    if (!ts->ring) return;
    // field by field (put): merged into one 16-byte store, the record's registers
    // were kept, and spilled, across the tile loops
    pk_trace_rec* r = reinterpret_cast<pk_trace_rec*>(ts->ring + 8) + (ts->count % PK_TRACE_CAP);
    put(&r->t, wall_clock64(), __HIP_MEMORY_SCOPE_AGENT);
    put(&r->kind, kind, __HIP_MEMORY_SCOPE_AGENT);
    put(&r->aux, aux, __HIP_MEMORY_SCOPE_AGENT);
    ts->count += 1;
    put(reinterpret_cast<uint64_t*>(ts->ring), ts->count, __HIP_MEMORY_SCOPE_AGENT);
}

// Task carry state of the leader (block 0, thread 0), in shared memory: the
// task read ahead once at task start (seq), when (t0), and whether it still
// waits to be compared (pending); `age` is how long a bus read takes.
struct CarryState {
    uint64_t seq;
    uint64_t t0;
    uint64_t age;
    int pending;
    uint64_t t_task;  // start of the task under way (its done record's t_begin)
};

// Leader only, before it arrives at an ordered grid barrier: if the task read
// ahead has been published by the host, hand it on through the barrier. It is
// compared at the first ordered barrier at least `age` after the read was
// issued (so the read has returned and stalls nothing: loads complete in order,
// and the barrier's own atomics would wait behind it). The stores are ordered
// before the barrier's arrival, so every block sees them after the barrier.
// One try per task: a task not yet published goes the ordinary way (poll,
// broadcast barrier).
__device__ __forceinline__ void carry_at_barrier(BarrierCtx& bc) {
    CarryState* cs = bc.carry;
    if (!cs->pending || wall_clock64() - cs->t0 < cs->age) return;
    cs->pending = 0;
    const uint64_t w = bc.carry_word;
    const uint64_t seq = cs->seq;
    if (static_cast<uint32_t>(w >> 32) != static_cast<uint32_t>(seq)) return;
    pk_carry* c = &bc.st->carry[seq & 1];
    __hip_atomic_store(&c->kind, static_cast<int32_t>((w >> 28) & 0xF), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&c->n, static_cast<int32_t>(w & PK_TASK_N_MAX), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&c->seq, seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Lane 0 spins until *gen reaches `target` (relaxed loads, bounded in time).
__device__ __forceinline__ void spin_until(BarrierCtx& bc, uint32_t* gen, uint32_t target) {
    if (bc.faulted) return;
    const uint64_t t0 = wall_clock64();
    while (static_cast<int32_t>(__hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                                target) < 0) {
        __builtin_amdgcn_s_sleep(1);
        if (wall_clock64() - t0 > bc.spin_ticks) {
            bc.faulted = true;
            __hip_atomic_store(&bc.st->fault, static_cast<uint32_t>(PK_FAULT_BARRIER_TIMEOUT),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
    }
}

__device__ __forceinline__ uint32_t arrive(uint32_t* ctr, bool relaxed) {
    return relaxed ? __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                   : __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}


// XCD-grouped barrier (PK_BARRIER_XCD). A wave's stores are in its XCD's L2
// once its vmcnt reaches 0 (the vector L1 is write-through), and an agent-scope
// release fence writes back the whole L2 of the XCD it runs on. So the release
// can be done once per XCD instead of once per block:
//   every wave: vmcnt(0) (its stores have reached the XCD's L2);
//   lane 0: relaxed add to its XCD's counter; the last block of the XCD issues
//     the release fence (one L2 write-back covering every block of that XCD)
//     and adds to the top counter; the last XCD stores the top generation and
//     the generation word of every XCD;
//   every block then waits for its XCD's generation and issues its own acquire
//     fence: the L2 invalidate must stay per block, because it is also what
//     invalidates the block's own CU L1 (a workgroup-scope invalidate does not
//     touch the L1 outside thread-group-split mode).
// Blocks are grouped by the XCD they actually run on, read from the hardware
// at launch, so placement does not affect correctness.
__device__ __forceinline__ void xcd_barrier(BarrierCtx& bc) {
    if (threadIdx.x == 0) carry_at_barrier(bc);
    wait_vm();
    __syncthreads();
    trace_event(bc, PK_TR_SYNC_ARRIVE, 0);
    if (threadIdx.x == 0) {
        const uint32_t target = bc.epoch + 1;
        pk_dev_state* st = bc.st;
        const uint32_t g = bc.xs->g;
        const uint32_t old = __hip_atomic_fetch_add(&st->xgrp_count[g].v, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        bool released = false;
        if (old == target * bc.xs->members - 1u) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            const uint32_t old2 = __hip_atomic_fetch_add(&st->xtop_count, 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            if (old2 == target * bc.xs->groups - 1u) {
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
                for (uint32_t k = 0; k < 8; ++k)
                    __hip_atomic_store(&st->xgrp_gen[k].v, target, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                released = true;
            }
        }
        if (!released) spin_until(bc, &st->xgrp_gen[g].v, target);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    trace_event(bc, PK_TR_SYNC_LEAVE, 0);
    bc.epoch += 1;
    __syncthreads();
}

// Point-to-point halo sync between the blocks of neighbouring bands. Every
// wave waits for its own stores (the edge rows just published), the block
// meets, and thread 0 publishes the new exchange count on the block's flag
// with agent-scope release, then acquires the flags of logical blocks lb-d and
// lb+d for d = 1..dist (bounded spins): all blocks whose bands its halo reaches. Blocks meet only their neighbours ("Persistent
// Kernels", "Reflections and next steps", GPU-side scheduling).
__device__ __forceinline__ void neighbor_sync(BarrierCtx& bc, uint32_t* nbr, int lb, int dist) {
    wait_vm();
    __syncthreads();
    const uint32_t target = bc.nbr_epoch + 1;
    trace_event(bc, PK_TR_SYNC_ARRIVE, 1);
    if (threadIdx.x == 0 && !bc.faulted) {
        __hip_atomic_store(nbr + static_cast<size_t>(lb) * PK_NBR_WORDS, target, __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_AGENT);
        // every block whose band the halo reaches: dist bands on each side
        for (int d = 1; d <= dist; ++d) {
            if (lb - d >= 0) spin_until(bc, nbr + static_cast<size_t>(lb - d) * PK_NBR_WORDS, target);
            if (lb + d < static_cast<int>(bc.grid))
                spin_until(bc, nbr + static_cast<size_t>(lb + d) * PK_NBR_WORDS, target);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    trace_event(bc, PK_TR_SYNC_LEAVE, 1);
    bc.nbr_epoch = target;
    __syncthreads();
}

// Point-to-point sync between two streaming passes of the same unit
// decomposition, by neighbour counters kept per XCD. Unit u runs on logical
// block u mod G; a pass reads the halo rows and overlap columns that the units
// next to its own (bands within the halo's reach, strips one either side, both
// halves of a split edge unit) wrote in the pass before, and overwrites what
// they read then. At launch every block notes the XCDs that run the blocks
// holding those units, and its own (`pn->mask`: a block that did not wait for
// its own XCD could arrive at the XCD's counter for the next pass before the
// rest of its XCD arrived for this one, and the last-arrival test would fail). After a pass every wave waits for its stores
// to reach its XCD's L2, thread 0 adds 1 to its XCD's arrival counter, and the
// XCD's last block writes the L2 back once (agent-scope release) and publishes
// the pass count for the XCD; the block then waits only for the XCDs in its mask
// (wave 0, one lane per XCD, one round of loads per poll, bounded in time) and
// acquires. A block is at most one pass ahead of any block it reads from, which
// the two field buffers allow. Blocks meet their neighbours' XCDs, never the
// whole grid ("Persistent Kernels", "Reflections and next steps", GPU-side
// scheduling on neighbour step counters; "Grid-Wide Barriers and Persistent Work
// Queues", "What the barrier buys", on every block waiting for the slowest).
__device__ __forceinline__ void pass_neighbor_sync(BarrierCtx& bc, uint32_t mask) {
    wait_vm();
    __syncthreads();
    const uint32_t target = bc.nbr_epoch + 1;
    trace_event(bc, PK_TR_SYNC_ARRIVE, 1);
    if (threadIdx.x < 64) {  // wave 0
        const int lane = static_cast<int>(threadIdx.x);
        pk_dev_state* st = bc.st;
        bool faulted = __shfl(static_cast<int>(bc.faulted), 0, 64) != 0;
        if (lane == 0 && !faulted) {
            const uint32_t g = bc.xs->g;
            const uint32_t old = __hip_atomic_fetch_add(&st->xpass_count[g].v, 1u, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
            if (old == target * bc.xs->members - 1u) {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                __hip_atomic_store(&st->xpass_gen[g].v, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        const bool watch = lane < 8 && ((mask >> lane) & 1u);
        if (!faulted) {
            const uint64_t t0 = wall_clock64();
            for (;;) {
                const bool ok = !watch ||
                                static_cast<int32_t>(__hip_atomic_load(&st->xpass_gen[lane & 7].v, __ATOMIC_RELAXED,
                                                                       __HIP_MEMORY_SCOPE_AGENT) -
                                                     target) >= 0;
                if (__all(ok)) break;
                __builtin_amdgcn_s_sleep(1);
                if (wall_clock64() - t0 > bc.spin_ticks) {
                    faulted = true;
                    if (lane == 0)
                        __hip_atomic_store(&st->fault, static_cast<uint32_t>(PK_FAULT_BARRIER_TIMEOUT),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        if (lane == 0) bc.faulted = faulted;
    }
    trace_event(bc, PK_TR_SYNC_LEAVE, 1);
    bc.nbr_epoch = target;
    __syncthreads();
}

__device__ __forceinline__ void grid_barrier(BarrierCtx& bc, bool relaxed = false) {
    bc.nbar += 1;
    if (bc.xcd && !relaxed && bc.grid > 1) {
        xcd_barrier(bc);
        return;
    }
    if (threadIdx.x == 0 && !relaxed) carry_at_barrier(bc);
    __syncthreads();
    trace_event(bc, PK_TR_SYNC_ARRIVE, 0);
    if (threadIdx.x == 0 && bc.grid > 1) {
        const uint32_t target = bc.epoch + 1;
        pk_dev_state* st = bc.st;
        if (!bc.two_level) {
            const uint32_t old = arrive(&st->bar_count, relaxed);
            if (old == target * bc.grid - 1u) {
                if (!relaxed) __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
                __hip_atomic_store(&st->bar_gen, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                spin_until(bc, &st->bar_gen, target);
            }
        } else {
            const uint32_t g = blockIdx.x & 7u;
            const uint32_t members = (bc.grid - g + 7u) >> 3;   // blocks in group g
            const uint32_t groups = bc.grid < 8u ? bc.grid : 8u;
            bool released = false;
            const uint32_t old = arrive(&st->grp_count[g].v, relaxed);
            if (old == target * members - 1u) {                  // last of its group
                if (!relaxed) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                const uint32_t old2 = arrive(&st->top_count, relaxed);
                if (old2 == target * groups - 1u) {              // last of all
                    if (!relaxed) __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
                    for (uint32_t k = 0; k < groups; ++k)
                        __hip_atomic_store(&st->grp_gen[k].v, target, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    released = true;
                }
            }
            if (!released) spin_until(bc, &st->grp_gen[g].v, target);
        }
        if (!relaxed) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    trace_event(bc, PK_TR_SYNC_LEAVE, 0);
    bc.epoch += 1;
    __syncthreads();
}

// Hardware dispatch places block b on XCD (b mod 8). With remapping, logical
// block numbers [x*G/8, (x+1)*G/8) all live on XCD x, so neighbouring work
// (and the halo rows it shares) stays inside one XCD's L2.
// Wave index in the block, in a scalar register: the compiler's divergence
// analysis treats threadIdx.x >> 6 as per-lane, which would put every loop
// driven by it into vector registers under exec masks.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
}

// threadIdx.x as a value the compiler must read afresh where it is used: the
// per-lane addresses of the rarely run tasks (readback, stamp rounds) are then
// formed inside those tasks, not hoisted out of the task loop and kept, or
// spilled, across every other task.
__device__ __forceinline__ int thread_id_here() {
    int t = static_cast<int>(threadIdx.x);
    asm volatile("" : "+v"(t));
    return t;
}

__device__ __forceinline__ int logical_block(int remap, int grid) {
    const int b = static_cast<int>(blockIdx.x);
    if (!remap) return b;
    const int per = grid >> 3;
    return (b & 7) * per + (b >> 3);
}

// Global wave number for unit assignment, wave-major across blocks: unit u goes
// to wave (u / G) of logical block (u mod G), so every block (every CU) gets
// work even when there are fewer units than waves, and consecutive units sit on
// consecutive logical blocks, i.e. on one XCD.
__device__ __forceinline__ int unit_wave(const pk_kargs& a) {
    return wave_id() * a.grid + logical_block(a.xcd_remap, a.grid);
}

// ---------------------------------------------------------------------------
// Fixed-order double reductions (bitwise reproducible for a given grid).
// ---------------------------------------------------------------------------
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Sum over the block; the result is valid in thread 0.
__device__ __forceinline__ double block_sum(double v, double* s_red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_sum(v);
    if (lane == 0) s_red[wave] = v;
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x == 0) {
        const int nw = blockDim.x >> 6;
        for (int w = 0; w < nw; ++w) t += s_red[w];
    }
    __syncthreads();
    return t;
}

// ---------------------------------------------------------------------------
// Streaming sweep. A unit is a band of interior rows x one strip of 64 lanes
// x W columns. The wave walks down its band keeping rows i-1, i, i+1 in
// registers (the column-march of "Persistent Kernels", "Cache-line aware
// tiling and iteration", with a 16-byte vector per lane instead of one
// column per thread) and issues CH rows of loads before computing them.
// ---------------------------------------------------------------------------
template <typename T, bool HAS_B, int CH>
__device__ __forceinline__ void stream_unit(const T* __restrict__ src, T* __restrict__ dst,
                                            const T* __restrict__ bsrc, int nx, int pitch, int c0,
                                            int r_begin, int r_end, int parity) {
    constexpr int W = VecW<T>::W;
    const int lane = threadIdx.x & 63;
    const int col = c0 + lane * W;
    const bool act = col < nx;
    const int hcol = (lane == 0) ? c0 - 1 : c0 + 64 * W;
    const bool hact = (lane == 0) ? (c0 > 0) : ((lane == 63) && (c0 + 64 * W < nx));
    const size_t p = static_cast<size_t>(pitch);

    Vec<T> up = act ? gload(src + static_cast<size_t>(r_begin - 1) * p + col) : vzero<T>();
    Vec<T> mid = act ? gload(src + static_cast<size_t>(r_begin) * p + col) : vzero<T>();
    T mh = hact ? gload1(src + static_cast<size_t>(r_begin) * p + hcol) : T(0);

    for (int r = r_begin; r < r_end; r += CH) {
        Vec<T> dn[CH];
        Vec<T> bb[CH];
        T dh[CH];
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int rl = min(r + k + 1, r_end);  // r_end itself is a valid row
            dn[k] = act ? gload(src + static_cast<size_t>(rl) * p + col) : vzero<T>();
            dh[k] = hact ? gload1(src + static_cast<size_t>(rl) * p + hcol) : T(0);
            if (HAS_B) {
                const int rb = min(r + k, r_end - 1);
                bb[k] = act ? gload(bsrc + static_cast<size_t>(rb) * p + col) : vzero<T>();
            } else {
                bb[k] = vzero<T>();
            }
        }
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            Vec<T> o = stencil<T, HAS_B>(up, mid, dn[k], bb[k], mh, col, nx);
            if (parity >= 0) o = rb_keep(o, mid, r + k, parity);  // wave-uniform
            if (act && r + k < r_end) gstore(dst + static_cast<size_t>(r + k) * p + col, o);
            up = mid;
            mid = dn[k];
            mh = dh[k];
        }
    }
}

template <typename T, bool HAS_B>
__device__ __forceinline__ double stream_unit_residual(const T* __restrict__ src,
                                                       const T* __restrict__ bsrc, int nx,
                                                       int pitch, int c0, int r_begin, int r_end) {
    constexpr int W = VecW<T>::W;
    constexpr int CH = 4;
    const int lane = threadIdx.x & 63;
    const int col = c0 + lane * W;
    const bool act = col < nx;
    const int hcol = (lane == 0) ? c0 - 1 : c0 + 64 * W;
    const bool hact = (lane == 0) ? (c0 > 0) : ((lane == 63) && (c0 + 64 * W < nx));
    const size_t p = static_cast<size_t>(pitch);

    Vec<T> up = act ? gload(src + static_cast<size_t>(r_begin - 1) * p + col) : vzero<T>();
    Vec<T> mid = act ? gload(src + static_cast<size_t>(r_begin) * p + col) : vzero<T>();
    T mh = hact ? gload1(src + static_cast<size_t>(r_begin) * p + hcol) : T(0);
    double acc = 0.0;
    for (int r = r_begin; r < r_end; r += CH) {
        Vec<T> dn[CH];
        Vec<T> bb[CH];
        T dh[CH];
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int rl = min(r + k + 1, r_end);
            dn[k] = act ? gload(src + static_cast<size_t>(rl) * p + col) : vzero<T>();
            dh[k] = hact ? gload1(src + static_cast<size_t>(rl) * p + hcol) : T(0);
            if (HAS_B) {
                const int rb = min(r + k, r_end - 1);
                bb[k] = act ? gload(bsrc + static_cast<size_t>(rb) * p + col) : vzero<T>();
            } else {
                bb[k] = vzero<T>();
            }
        }
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            if (r + k < r_end) {  // wave-uniform: short bands skip the rows past their end
                const double q = rho2<T, HAS_B>(up, mid, dn[k], bb[k], mh, col, nx);
                if (act) acc += q;
            }
            up = mid;
            mid = dn[k];
            mh = dh[k];
        }
    }
    return acc;
}

// One sweep over all units, src -> dst; parity >= 0: one red-black half-sweep
// of that colour (the other colour is copied).
template <typename T, bool HAS_B>
__device__ __forceinline__ void stream_sweep(const pk_kargs& a, const T* __restrict__ src,
                                             T* __restrict__ dst, int parity = -1) {
    constexpr int W = VecW<T>::W;
    const int gw = unit_wave(a);
    const int nw = a.grid * (static_cast<int>(blockDim.x) >> 6);
    const int units = a.strips * a.bands;
    const T* bsrc = static_cast<const T*>(a.b);
    for (int u = gw; u < units; u += nw) {
        const int strip = u % a.strips, band = u / a.strips;
        const int r_begin = 1 + band * a.band_rows;
        const int r_end = min(a.ny - 1, r_begin + a.band_rows);
        if (r_begin >= r_end) continue;
        // rows of loads in flight per wave: fewer when b doubles the traffic
        constexpr int CH = (HAS_B || sizeof(T) == 8) ? 4 : 8;
        stream_unit<T, HAS_B, CH>(src, dst, bsrc, a.nx, a.pitch, strip * 64 * W, r_begin, r_end,
                                  parity);
    }
}

// ---------------------------------------------------------------------------
// K sweeps per pass (temporal blocking in the column march). Level 0 is the
// field in src; level j row i is the stencil of level j-1 rows i-1, i, i+1.
// At step t the wave loads level-0 row t and computes level j row t-j for
// j = 1..K (t+j when marching up); each level keeps its last two rows in
// registers (the third operand is the row the level below produced at this
// step), and level K's row is stored when it lies in the unit's band [r0, r1).
// The band therefore reads K halo rows above and below, and the field is read
// and written once per K sweeps. Ring rows keep their value at every level (the
// middle row of the previous level), ring and padding columns likewise (the
// stencil's mask).
//
// Only the rows a stored row depends on are computed: level j needs rows
// [r0 - (K - j), r1 + (K - j)), which it reaches at step 2j, so during the
// first 2K steps the levels above step / 2 are skipped (their rows would fall
// outside that range).
//
// Columns: the strip's lanes 0..ov-1 and 64-ov..63 overlap the neighbouring
// strips and are never stored. Their outer neighbours may hold anything, so
// wrong values spread inward one column per level; after K <= ov * W levels
// they have not reached a stored lane. A strip stores (64 - 2 ov) * W columns
// starting at c0 + ov * W. Results equal K single sweeps bit for bit: every
// stored value is the same expression on the same operands.
//
// Ring handling (MODE):
//   PASS_CHECKED: every level checks whether its row is a ring row (kept) and
//     every element whether it is a ring or padding column (kept).
//   PASS_COLS, PASS_EDGE, PASS_INNER: for units whose rows meet a ring row only
//     during the first 2K steps of the march (the first band marches down from
//     the top ring, the last band up from the bottom ring, and no band ends
//     within K rows of the far ring). The ring-row check runs only in those
//     steps, as a branch-free blend. PASS_INNER also leaves out the column
//     check, for units whose columns [c0, c0 + 64 W) are all interior.
//     PASS_EDGE_LO / PASS_EDGE_HI, for a Laplace unit that holds one of the two
//     ring columns when nx is a multiple of W: column 0 is then element 0 of its lane
//     and column nx - 1 element W - 1 of its lane, and no stored lane holds a
//     padding column, so the march keeps just that one element (one per-lane
//     blend a level) instead of checking every element: padding and outside
//     columns feed only the ring columns, which are kept.
//     (The edge strips' waves finish last and hold up the pass: with them on
//     the INNER march's cost, 4096^2 ran 14% faster; with one blend a level,
//     4.48 -> 4.22 us per sweep.)
//
// RES: the pass also sums rho^2 of its result (the residual of the field it
// stores, as a RESIDUAL task would compute it, element by element the same
// expression): a level K+1 that computes rho of level K's rows instead of a
// stencil, accumulated in double per lane over the band's rows and the strip's
// stored lanes, so every interior node counts once. The unit then reaches K+1
// halo rows and needs K+1 overlap columns.
// TAP: the pass also sums rho^2 of an intermediate level, h0 (0..K-1: the field
// after h0 of its K sweeps, h0 = 0 the field it reads), from the operands of
// level h0 + 1's stencil, over the same rows and lanes as RES: a residual taken
// inside a pass whose later levels run on (a RESIDUAL task between two SWEEP
// tasks, computed in the pass that crosses from one to the other).
//
// Memory: rows go in chunks of CH, loaded one chunk ahead of their use. With
// DEFER, a chunk's level-K rows are stored at the start of the next chunk
// (before its loads): faster where stores are a large share of the traffic
// (fp64, or with b); otherwise each row is stored as soon as it is computed.
// ---------------------------------------------------------------------------
enum { PASS_CHECKED = 0, PASS_COLS = 1, PASS_INNER = 2, PASS_EDGE_LO = 3, PASS_EDGE_HI = 4 };

// rho^2 of one vector summed in double over its interior elements, from the
// vector (m), its row neighbours (s, n), its W/E neighbours by DPP and b
// (overlap lanes are not summed, so their outer neighbours may be anything)
template <typename T, bool HAS_B, bool COLS>
__device__ __forceinline__ double pass_rho2(const Vec<T>& s, const Vec<T>& m, const Vec<T>& n,
                                            const Vec<T>& b, int col, int nx) {
    constexpr int W = VecW<T>::W;
    const T west = from_lower_any(m.v[W - 1]), east = from_upper_any(m.v[0]);
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < W; ++k) {
        const double w = static_cast<double>((k == 0) ? west : m.v[k - 1]);
        const double e = static_cast<double>((k == W - 1) ? east : m.v[k + 1]);
        double t = (w + e) + (static_cast<double>(s.v[k]) + static_cast<double>(n.v[k]));
        if (HAS_B) t = t + static_cast<double>(b.v[k]);
        const double r = t - 4.0 * static_cast<double>(m.v[k]);
        if constexpr (COLS) {
            const int c = col + k;
            acc += (c == 0 || c >= nx - 1) ? 0.0 : r * r;
        } else {
            acc += r * r;
        }
    }
    return acc;
}

template <typename T, bool HAS_B, bool COLS>
__device__ __forceinline__ Vec<T> pass_stencil(const Vec<T>& s, const Vec<T>& m, const Vec<T>& n,
                                               const Vec<T>& b, int col, int nx) {
    constexpr int W = VecW<T>::W;
    // lanes 0 and 63 are overlap lanes (never stored): their outer neighbours
    // may be anything, so the shifts need no edge value
    const T west = from_lower_any(m.v[W - 1]), east = from_upper_any(m.v[0]);
    if constexpr (COLS) return stencil_we<T, HAS_B>(s, m, n, b, west, east, col, nx);
    Vec<T> o;
#pragma unroll
    for (int k = 0; k < W; ++k) {
        const T w = (k == 0) ? west : m.v[k - 1];
        const T e = (k == W - 1) ? east : m.v[k + 1];
        T t = (w + e) + (s.v[k] + n.v[k]);
        if (HAS_B) t = t + b.v[k];
        o.v[k] = T(0.25) * t;
    }
    return o;
}

// keep_val where mask is all ones, else new_val, element by element
template <typename T>
__device__ __forceinline__ Vec<T> vblend(uint32_t mask, const Vec<T>& keep_val, const Vec<T>& new_val) {
    Vec<T> r;
#pragma unroll
    for (int k = 0; k < VecW<T>::W; ++k) r.v[k] = blend(mask, keep_val.v[k], new_val.v[k]);
    return r;
}

template <bool V>
struct HeadSteps {
    static constexpr bool value = V;
};

// A step's slot in a level's three-row ring (the step number mod 3).
template <int P>
struct RingSlot {
    static constexpr int value = P;
};

template <typename T, bool HAS_B, int K, int DIR, bool RB, int MODE, bool RES, bool TAP = false>
__device__ __forceinline__ double stream_pass_unit(const T* __restrict__ src, T* __restrict__ dst,
                                                   const T* __restrict__ bsrc, int nx, int ny,
                                                   int pitch, int c0, int ov, int r0, int r1, int h0) {
    constexpr int dir = DIR;
    constexpr int W = VecW<T>::W;
    constexpr int L = K + (RES ? 1 : 0);  // levels of the march (the last one rho with RES)
    // ROT: each level keeps its last three rows in a ring indexed by the step
    // number mod 3, and the march takes three rows a chunk, so every ring slot is
    // known at compile time and no row moves from one register to another (the
    // two-row form copies every level's rows at every step). One row more per
    // level: only where no b delay line shares the register file.
    constexpr bool ROT = !HAS_B;
    constexpr int CH = ROT ? 3 : ((HAS_B || L >= 3) ? 2 : 4);  // rows per chunk
    constexpr int HEAD = (2 * L + CH - 1) / CH * CH;  // steps taken with the head's level checks
    constexpr bool DEFER = sizeof(T) == 8 || (HAS_B && L <= PK_SHALLOW_PASS + 1);
    constexpr bool COLS = MODE == PASS_CHECKED || MODE == PASS_COLS;  // every element checked
    const int lane = threadIdx.x & 63;
    const int col = c0 + lane * W;
    const bool act = col >= 0 && col < nx;
    const bool store_lane = act && lane >= ov && lane < 64 - ov;
    // Loads are unconditional, at addresses clamped into the unit's rows and the
    // row's vectors: rows outside the field read a ring row, lanes outside it a
    // vector of the same row. Neither value reaches a stored element: ring rows
    // keep their value at every level, rows beyond them feed only ring rows, and
    // a lane outside the field borders a ring column, which keeps its value.
    // The buffer descriptors cover rows [w0, w1), every row the unit reads or
    // writes (the planner keeps them within 4 GiB).
    const int w0 = max(0, r0 - L), w1 = min(ny, r1 + L);
    const size_t p = static_cast<size_t>(pitch);
    const uint32_t row_bytes = static_cast<uint32_t>(p * sizeof(T));
    const uint32_t win_bytes = static_cast<uint32_t>(w1 - w0) * row_bytes;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + static_cast<size_t>(w0) * p, win_bytes);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dst + static_cast<size_t>(w0) * p, win_bytes);
    const __amdgpu_buffer_rsrc_t rbs = make_rsrc(HAS_B ? bsrc + static_cast<size_t>(w0) * p : src, win_bytes);
    // PASS_EDGE_LO: the lane holding column 0 (element 0); PASS_EDGE_HI: the lane
    // holding column nx - 1 (element W - 1)
    const uint32_t ring_lane = lane_mask(MODE == PASS_EDGE_LO ? col == 0 : col + W - 1 == nx - 1);
    const uint32_t lbyte = static_cast<uint32_t>(min(max(col, 0), pitch - W)) * sizeof(T);
    const uint32_t sbyte = static_cast<uint32_t>(max(col, 0)) * sizeof(T);  // stored lanes have col >= 0
    const int b_lo = max(w0, 1), b_hi = min(w1, ny - 1) - 1;  // b rows: interior rows of the window

    // two-row form: level j rows x-1 and x, x the last row it received;
    // ROT: level j's rows of the last three steps, the row of step q in slot q mod 3
    Vec<T> ra[ROT ? 1 : L], rm[ROT ? 1 : L];
    Vec<T> hr[ROT ? L : 1][3];
    Vec<T> bq[L];         // bq[j] = b row of the level j+1 row computed at this step
    double acc = 0.0;     // RES: this lane's rho^2
#pragma unroll
    for (int j = 0; j < L; ++j) {
        if constexpr (ROT) {
            hr[j][0] = hr[j][1] = hr[j][2] = vzero<T>();
        } else {
            ra[j] = rm[j] = vzero<T>();
        }
        bq[j] = vzero<T>();
    }
    // dir = +1 marches down from r0 - L, dir = -1 marches up from r1 - 1 + L
    const int nsteps = (r1 - r0) + 2 * L;
    const int t_first = dir > 0 ? r0 - L : r1 - 1 + L;
    const auto load_chunk = [&](int q, Vec<T>* u, Vec<T>* b) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int t = t_first + dir * (q + c);
            u[c] = bload<T>(rs, lbyte, static_cast<uint32_t>(min(max(t, w0), w1 - 1) - w0) * row_bytes);
            if (HAS_B)
                b[c] = bload<T>(rbs, lbyte, static_cast<uint32_t>(min(max(t - dir, b_lo), b_hi) - w0) * row_bytes);
            else
                b[c] = vzero<T>();
        }
    };
    // level K row of step q, stored if it lies in the band
    const auto store_row = [&](int q, const Vec<T>& x) {
        const int row = t_first + dir * q - dir * K;
        if (row >= r0 && row < r1) {  // wave-uniform
            const uint32_t roff = static_cast<uint32_t>(row - w0) * row_bytes;
            if (store_lane) bstore<T>(rd, sbyte, roff, x);
        }
    };
    Vec<T> out[CH];  // DEFER: a chunk's level-K rows, stored at the start of the next chunk
    // One step: level-0 row u (and its b row); returns level K's row. In the first
    // 2L steps (head) only levels j <= q / 2 are computed: a higher level's row at
    // this step lies outside the rows any stored row (or summed rho) depends on.
    // slot_c (ROT): q mod 3.
    const auto step = [&](int q, const Vec<T>& u, const Vec<T>& b, auto head_c, auto slot_c) -> Vec<T> {
        constexpr bool head = decltype(head_c)::value;
        constexpr int P = decltype(slot_c)::value;
        const int t = t_first + dir * q;
#pragma unroll
        for (int j = L - 1; j > 0; --j) bq[j] = bq[j - 1];
        bq[0] = b;
        Vec<T> inc = u;  // row t of level 0, then level j's new row
        Vec<T> outK = u;
#pragma unroll
        for (int j = 1; j <= L; ++j) {
            // level j-1's rows of steps t-2 and t-1 (inc is its row of step t)
            const Vec<T> up = ROT ? hr[ROT ? j - 1 : 0][(P + 1) % 3] : ra[ROT ? 0 : j - 1];
            const Vec<T> mid = ROT ? hr[ROT ? j - 1 : 0][(P + 2) % 3] : rm[ROT ? 0 : j - 1];
            const auto keep = [&](const Vec<T>& x) {  // level j-1 moves on by one row
                if constexpr (ROT) {
                    hr[j - 1][P] = x;
                } else {
                    ra[j - 1] = mid;
                    rm[j - 1] = x;
                }
            };
            if constexpr (TAP) {
                // rho of level h0's row t - dir j (the field after h0 of the pass's
                // sweeps), from the operands of level h0 + 1's stencil at this step
                const int row = t - dir * j;
                if (j == h0 + 1 && (!head || 2 * j <= q) && row >= r0 && row < r1) {  // wave-uniform
                    const double r2 = pass_rho2<T, HAS_B, MODE != PASS_INNER>(up, mid, inc, bq[j - 1], col, nx);
                    if (store_lane) acc += r2;
                }
            }
            if (RES && j == L) {  // rho of level K's row t - dir L, if it is a band row
                const int row = t - dir * j;
                if ((!head || 2 * j <= q) && row >= r0 && row < r1) {  // wave-uniform
                    const double r2 = pass_rho2<T, HAS_B, COLS>(up, mid, inc, bq[j - 1], col, nx);
                    if (store_lane) acc += r2;
                }
                keep(inc);
                continue;
            }
            if (!head || 2 * j <= q) {  // wave-uniform
                const int row = t - dir * j;  // level j row computed at this step
                // level j-1 rows row-1, row, row+1 (dir = -1: row+1, row, row-1)
                Vec<T> o = pass_stencil<T, HAS_B, COLS>(up, mid, inc, bq[j - 1], col, nx);
                if constexpr (MODE == PASS_EDGE_LO) o.v[0] = blend(ring_lane, mid.v[0], o.v[0]);
                if constexpr (MODE == PASS_EDGE_HI) o.v[W - 1] = blend(ring_lane, mid.v[W - 1], o.v[W - 1]);
                if (RB) o = rb_keep(o, mid, row, (h0 + j - 1) & 1);
                const bool ring = row <= 0 || row >= ny - 1;  // ring rows (and beyond) keep their value
                if (MODE == PASS_CHECKED) {
                    if (ring) o = mid;
                } else if (head) {
                    o = vblend(lane_mask(ring), mid, o);
                }
                keep(inc);
                inc = o;
            } else {  // a row outside every stored row's reach: shift only
                keep(inc);
            }
            if (j == K) outK = inc;
        }
        return outK;
    };
    const auto run = [&](int q_begin, int q_end, auto head_c) {
        Vec<T> ld[CH], lb[CH];  // the chunk being computed
        load_chunk(q_begin, ld, lb);
        // nothing may be in flight when a loop is entered: the compiler's wait
        // analysis merges the loop's entry with its back edge, and loads pending
        // at entry would make it wait for every prefetch right after issuing it
        wait_vm();
        for (int q0 = q_begin; q0 < q_end; q0 += CH) {
            if (DEFER && q0 > 0) {
#pragma unroll
                for (int c = 0; c < CH; ++c) store_row(q0 - CH + c, out[c]);
            }
            Vec<T> nld[CH], nlb[CH];
            // always issued (past the end it reads clamped rows that nothing uses)
            load_chunk(q0 + CH, nld, nlb);
            // whole chunks: a step past the last computes rows beyond the band's
            // halo, which are never stored
            if constexpr (ROT) {  // q0 is a multiple of 3: the ring slots are 0, 1, 2
                const Vec<T> x0 = step(q0, ld[0], lb[0], head_c, RingSlot<0>{});
                if (DEFER) out[0] = x0;
                else store_row(q0, x0);
                const Vec<T> x1 = step(q0 + 1, ld[1], lb[1], head_c, RingSlot<1>{});
                if (DEFER) out[1] = x1;
                else store_row(q0 + 1, x1);
                const Vec<T> x2 = step(q0 + 2, ld[2], lb[2], head_c, RingSlot<2>{});
                if (DEFER) out[2] = x2;
                else store_row(q0 + 2, x2);
            } else {
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    const Vec<T> x = step(q0 + c, ld[c], lb[c], head_c, RingSlot<0>{});
                    if (DEFER) out[c] = x;
                    else store_row(q0 + c, x);
                }
            }
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                ld[c] = nld[c];
                lb[c] = nlb[c];
            }
        }
    };
    run(0, HEAD, HeadSteps<true>{});
    run(HEAD, nsteps, HeadSteps<false>{});
    if (DEFER) {
        // the last chunk computed
        const int q_last = nsteps > HEAD ? HEAD + ((nsteps - HEAD - 1) / CH) * CH : HEAD - CH;
#pragma unroll
        for (int c = 0; c < CH; ++c) store_row(q_last + c, out[c]);
    }
    return acc;
}

// The units of a pass: band b x strip s is unit b * strips + s. The units of
// the two edge strips hold a ring column, and even with the march's cheapest
// ring handling they finish last, holding up the pass; where the grid has a
// spare wave for each, they are split into the top and the bottom half of their
// band, the bottom halves numbered after all other units (2 b for strip 0,
// 2 b + 1 for the last strip). 8192^2 fp64 Poisson (1975 units for 2048 waves):
// 31.0-31.5 against 31.9-32.3 us per sweep.
__device__ __forceinline__ bool pass_split_edges(int strips, int pbands, int waves) {
    return strips >= 2 && (strips + 2) * pbands <= waves;
}

// Band, strip and half (0: the whole band, or an edge unit's top half; 1: its
// bottom half) of unit u of a pass with `units` = strips x pbands regular units.
__device__ __forceinline__ void pass_unit_place(int u, int strips, int units, int& band, int& strip, int& half) {
    if (u < units) {
        band = u / strips;
        strip = u - band * strips;
        half = 0;
    } else {
        band = (u - units) >> 1;
        strip = ((u - units) & 1) ? strips - 1 : 0;
        half = 1;
    }
}

// One unit of a Jacobi pass in a given ring mode, marching down or up.
template <typename T, bool HAS_B, int K, int MODE, bool TAP>
__device__ __forceinline__ double pass_unit_dir(int dir, const T* __restrict__ src, T* __restrict__ dst,
                                                const T* __restrict__ bsrc, int nx, int ny, int pt, int c0,
                                                int ov, int r0, int r1, int h0) {
    return dir > 0 ? stream_pass_unit<T, HAS_B, K, 1, false, MODE, false, TAP>(src, dst, bsrc, nx, ny, pt, c0, ov, r0, r1, h0)
                   : stream_pass_unit<T, HAS_B, K, -1, false, MODE, false, TAP>(src, dst, bsrc, nx, ny, pt, c0, ov, r0, r1, h0);
}

// One pass of k sweeps (a depth PK_PASS_DEPTH_OK accepts) over all units, src -> dst.
// h0 >= 0: the k levels are red-black half-sweeps, level j of colour (h0+j-1) mod 2
// (RB), or the level whose rho^2 is summed (TAP).
// RES, TAP: also this lane's rho^2 of the result, or of level h0 (returned; 0 otherwise).
template <typename T, bool HAS_B, int K, bool RB, bool RES, bool TAP = false>
__device__ __forceinline__ double stream_pass_k(const pk_kargs& a, const T* __restrict__ src,
                                                T* __restrict__ dst, int h0) {
    constexpr int W = VecW<T>::W;
    constexpr int L = K + (RES ? 1 : 0);
    const int ov = (L + W - 1) / W;
    const int stride = (64 - 2 * ov) * W;  // stored columns per strip
    const int strips = (a.nx + stride - 1) / stride;
    const int gw = unit_wave(a);
    const int nw = a.grid * (static_cast<int>(blockDim.x) >> 6);
    const int units = strips * a.pbands;
    const bool split = pass_split_edges(strips, a.pbands, nw);
    const int total = units + (split ? 2 * a.pbands : 0);
    const T* bsrc = static_cast<const T*>(a.b);
    double acc = 0.0;
    for (int u = gw; u < total; u += nw) {
        int band, strip, half;
        pass_unit_place(u, strips, units, band, strip, half);
        int r0 = 1 + band * a.pband_rows;
        int r1 = min(a.ny - 1, r0 + a.pband_rows);
        if (split && (strip == 0 || strip == strips - 1)) {
            const int rm = r0 + (r1 - r0 + 1) / 2;
            if (half) r0 = rm;
            else r1 = rm;
        }
        if (r0 >= r1) continue;
        const int c0 = strip * stride - ov * W;
        // the first band marches down from the top ring, the last up from the
        // bottom ring; the others march down (march_down: HBM-bound passes) or
        // alternate, so that neighbouring bands read the halo rows they share at
        // about the same time (and hit in the XCD's L2)
        const int dir = band == 0 ? 1
                        : (band == a.pbands - 1 ? -1 : (a.march_down || !(band & 1) ? 1 : -1));
        // the march meets a ring row only in its first 2L steps unless the band
        // ends within L rows of the far ring (a single band, or a short last band)
        const bool rows_late = dir > 0 ? r1 + L > a.ny : r0 < L;
        const bool lo = c0 < 1, hi = c0 + 64 * W > a.nx - 1;  // the unit holds ring column 0 / nx - 1
        const int nx = a.nx, ny = a.ny, pt = a.pitch;
        // red-black passes, the last pass of a task (RES) and passes of fewer than
        // PK_SHALLOW_PASS sweeps (a task's passes are all as deep as the engine's
        // depth but its last one or two) take the checked march
        if constexpr (RB || RES || K < PK_SHALLOW_PASS) {
            if (dir > 0) acc += stream_pass_unit<T, HAS_B, K, 1, RB, PASS_CHECKED, RES>(src, dst, bsrc, nx, ny, pt, c0, ov, r0, r1, h0);
            else acc += stream_pass_unit<T, HAS_B, K, -1, RB, PASS_CHECKED, RES>(src, dst, bsrc, nx, ny, pt, c0, ov, r0, r1, h0);
        } else {
            double r;
            if (rows_late)
                r = pass_unit_dir<T, HAS_B, K, PASS_CHECKED, TAP>(dir, src, dst, bsrc, nx, ny, pt, c0, ov, r0, r1, h0);
            else if (!HAS_B && lo != hi && nx % W == 0) {  // (with b the register file is full at depth 12)
                if (lo)
                    r = pass_unit_dir<T, HAS_B, K, PASS_EDGE_LO, TAP>(dir, src, dst, bsrc, nx, ny, pt, c0, ov, r0, r1, h0);
                else
                    r = pass_unit_dir<T, HAS_B, K, PASS_EDGE_HI, TAP>(dir, src, dst, bsrc, nx, ny, pt, c0, ov, r0, r1, h0);
            } else if (lo || hi)
                r = pass_unit_dir<T, HAS_B, K, PASS_COLS, TAP>(dir, src, dst, bsrc, nx, ny, pt, c0, ov, r0, r1, h0);
            else
                r = pass_unit_dir<T, HAS_B, K, PASS_INNER, TAP>(dir, src, dst, bsrc, nx, ny, pt, c0, ov, r0, r1, h0);
            if constexpr (TAP) acc += r;
        }
    }
    return acc;
}

// One pass of k sweeps; res (Jacobi only): also returns this lane's rho^2 of
// the result (the residual march of the last pass of a task); tap >= 0 (Jacobi,
// fp64, k = PK_MAX_PASS): returns this lane's rho^2 of the field after `tap` of
// the pass's sweeps instead.
template <typename T, bool HAS_B>
__device__ __forceinline__ double stream_pass(const pk_kargs& a, const T* __restrict__ src,
                                              T* __restrict__ dst, int k, int h0, bool res, int tap = -1) {
    if constexpr (sizeof(T) == 8) {  // (the fp32 kernels do not fuse tasks)
        if (tap >= 0) return stream_pass_k<T, HAS_B, PK_MAX_PASS, false, false, true>(a, src, dst, tap);
    }
    // red-black passes are their own instances: the colour mask stays out of the
    // Jacobi march
    if (h0 >= 0) {
        switch (k) {
            case 2: stream_pass_k<T, HAS_B, 2, true, false>(a, src, dst, h0); break;
            case 3: stream_pass_k<T, HAS_B, 3, true, false>(a, src, dst, h0); break;
            case 4: stream_pass_k<T, HAS_B, 4, true, false>(a, src, dst, h0); break;
            case 5: stream_pass_k<T, HAS_B, 5, true, false>(a, src, dst, h0); break;
            case 6: stream_pass_k<T, HAS_B, 6, true, false>(a, src, dst, h0); break;
            case 7: stream_pass_k<T, HAS_B, 7, true, false>(a, src, dst, h0); break;
            case 8: stream_pass_k<T, HAS_B, 8, true, false>(a, src, dst, h0); break;
            default: stream_sweep<T, HAS_B>(a, src, dst, h0); break;
        }
        return 0.0;
    }
    if (res) {
        switch (k) {
            case 1: return stream_pass_k<T, HAS_B, 1, false, true>(a, src, dst, h0);
            case 2: return stream_pass_k<T, HAS_B, 2, false, true>(a, src, dst, h0);
            case 3: return stream_pass_k<T, HAS_B, 3, false, true>(a, src, dst, h0);
            case 4: return stream_pass_k<T, HAS_B, 4, false, true>(a, src, dst, h0);
            case 5: return stream_pass_k<T, HAS_B, 5, false, true>(a, src, dst, h0);
            case 6: return stream_pass_k<T, HAS_B, 6, false, true>(a, src, dst, h0);
            case 7: return stream_pass_k<T, HAS_B, 7, false, true>(a, src, dst, h0);
            default: return stream_pass_k<T, HAS_B, 8, false, true>(a, src, dst, h0);
        }
    }
    switch (k) {
        case 2: stream_pass_k<T, HAS_B, 2, false, false>(a, src, dst, h0); break;
        case 3: stream_pass_k<T, HAS_B, 3, false, false>(a, src, dst, h0); break;
        case 4: stream_pass_k<T, HAS_B, 4, false, false>(a, src, dst, h0); break;
        case 5: stream_pass_k<T, HAS_B, 5, false, false>(a, src, dst, h0); break;
        case 6: stream_pass_k<T, HAS_B, 6, false, false>(a, src, dst, h0); break;
        case 7: stream_pass_k<T, HAS_B, 7, false, false>(a, src, dst, h0); break;
        case 8: stream_pass_k<T, HAS_B, 8, false, false>(a, src, dst, h0); break;
        case PK_MAX_PASS: stream_pass_k<T, HAS_B, PK_MAX_PASS, false, false>(a, src, dst, h0); break;
        default: stream_sweep<T, HAS_B>(a, src, dst, -1); break;
    }
    return 0.0;
}

// Per-block sum of rho^2 over the same units; valid in thread 0.
template <typename T, bool HAS_B>
__device__ __forceinline__ double stream_residual_block(const pk_kargs& a, const T* __restrict__ src,
                                                        double* s_red) {
    constexpr int W = VecW<T>::W;
    const int gw = unit_wave(a);
    const int nw = a.grid * (static_cast<int>(blockDim.x) >> 6);
    const int units = a.strips * a.bands;
    const T* bsrc = static_cast<const T*>(a.b);
    double acc = 0.0;
    for (int u = gw; u < units; u += nw) {
        const int strip = u % a.strips, band = u / a.strips;
        const int r_begin = 1 + band * a.band_rows;
        const int r_end = min(a.ny - 1, r_begin + a.band_rows);
        if (r_begin >= r_end) continue;
        acc += stream_unit_residual<T, HAS_B>(src, bsrc, a.nx, a.pitch, strip * 64 * W, r_begin,
                                              r_end);
    }
    return block_sum(acc, s_red);
}

// Fixed-order total of the per-block partials, by the first wave of a block;
// the result is valid in thread 0.
__device__ __forceinline__ double sum_partials(const double* partials, int grid) {
    // the lane's address is formed here, not hoisted out of the task loop and
    // kept (or spilled) across every other task
    const int t = thread_id_here();
    const int lane = t & 63;
    double v = 0.0;
    if (t < 64)
        for (int k = lane; k < grid; k += 64) v += partials[k];
    return wave_sum(v);
}

// ---------------------------------------------------------------------------
// LDS-resident sweep rows.
//
// A row of the tile holds nv = lp / W vectors. Work goes out per wave in items
// of 64 lanes: a row narrower than 64 vectors shares an item with 64 / sw - 1
// others (sw = the power of two >= nv), a wider row is cut into segs segments
// of 64 vectors. Each wave keeps one segment for the whole task (segs <= waves
// per block) and walks the row groups with a stride, so a lane's column, its
// ring mask and whether it reads an edge neighbour from LDS are fixed per task.
//
// All of this is set up once per task (TileMap): the CU's scalar unit is
// shared by all its waves, so scalar set-up repeated per sub-sweep by every
// wave costs as much as the stencil itself on small tiles.
// ---------------------------------------------------------------------------
template <typename T>
struct TileMap {
    static constexpr int W = VecW<T>::W;
    int nv, lp, nx;
    int lsw;       // log2 of the lanes per row within an item (<= 6)
    int lrpi;      // log2 of the rows per item (6 - lsw)
    int segs;      // segments per row
    int seg0;      // this wave's first segment
    int seg_step;  // next segment of this wave (more segments than waves only)
    int g0, g_step;  // this wave's first row group and group stride
    bool active;   // the wave has work
    int sub;       // this lane's row within an item
    int lsub;      // this lane's vector within its row segment
};

template <typename T>
__device__ __forceinline__ TileMap<T> tile_map(int nv, int lp, int nx) {
    TileMap<T> t;
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const int wave = wave_id();
    const int nwv = static_cast<int>(blockDim.x) >> 6;
    int lsw = 0;
    while ((1 << lsw) < nv && lsw < 6) ++lsw;
    t.nv = nv;
    t.lp = lp;
    t.nx = nx;
    t.lsw = lsw;
    t.lrpi = 6 - lsw;
    t.segs = (nv + (1 << lsw) - 1) >> lsw;
    const int per = t.segs < nwv ? t.segs : nwv;  // segments handled at once
    const int wps = nwv / per;                    // waves per segment
    t.active = wave < wps * per;
    t.seg0 = wave % t.segs;
    t.seg_step = per;
    t.g0 = wave / t.segs;
    t.g_step = wps;
    t.sub = lane >> lsw;
    t.lsub = lane & ((1 << lsw) - 1);
    return t;
}

// Rows [lo, hi) of D from S (LDS row stride lp elements; Bt holds b).
// RB: a red-black half-sweep; node colour from the global row (local row +
// q_row) and column, updated when it equals `parity`.
// ONE: rows of one segment (at most 64 vectors): no lane ever needs an edge
// element from LDS (a row's end lanes border ring or padding columns, which
// keep their values), so the lane shifts take no edge value.
template <typename T, bool HAS_B, bool RB, bool ONE>
__device__ __forceinline__ void resident_rows(const T* S, T* D, const T* Bt, int lo, int hi,
                                              const TileMap<T>& t, int q_row = 0, int parity = 0) {
    constexpr int W = VecW<T>::W;
    if (!t.active) return;
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const int lp = t.lp;
    const int groups = (hi - lo + (1 << t.lrpi) - 1) >> t.lrpi;
    for (int seg = t.seg0; seg < t.segs; seg += t.seg_step) {
        const int v = (seg << t.lsw) + t.lsub;
        const bool vact = v < t.nv;
        const int col = (vact ? v : (seg << t.lsw)) * W;
        // a lane's W/E neighbour comes by DPP from the adjacent lane; the lanes
        // at the ends of a 64-wide segment read it from LDS unless it can only
        // reach a ring or padding column (rows of one segment never need it)
        const bool need_w = lane == 0 && col > 0;
        const bool need_e = lane == 63 && col + W < lp;
        bool keep[W];
#pragma unroll
        for (int k = 0; k < W; ++k) keep[k] = (col + k == 0) || (col + k >= t.nx - 1);
        for (int g = t.g0; g < groups; g += t.g_step) {
            const int r = lo + (g << t.lrpi) + t.sub;
            const bool act = vact && r < hi;
            const int rr = r < hi ? r : hi - 1;
            const int o0 = rr * lp + col;
            const T* p = S + o0;
            const Vec<T> m = vload(p);
            const Vec<T> s = vload(p - lp);
            const Vec<T> n = vload(p + lp);
            const Vec<T> bb = HAS_B ? vload(Bt + o0) : vzero<T>();
            T west, east;
            if constexpr (ONE) {
                west = from_lower_any(m.v[W - 1]);
                east = from_upper_any(m.v[0]);
            } else {
                T ew = T(0), ee = T(0);
                if (need_w) ew = p[-1];
                if (need_e) ee = p[W];
                west = from_lower(ew, m.v[W - 1]);
                east = from_upper(ee, m.v[0]);
            }
            Vec<T> o;
#pragma unroll
            for (int k = 0; k < W; ++k) {
                const T w = (k == 0) ? west : m.v[k - 1];
                const T e = (k == W - 1) ? east : m.v[k + 1];
                T x = (w + e) + (s.v[k] + n.v[k]);
                if (HAS_B) x = x + bb.v[k];
                o.v[k] = keep[k] ? m.v[k] : T(0.25) * x;
            }
            if (RB) o = rb_keep(o, m, rr + q_row, parity);
            if (act) vstore(D + o0, o);
        }
    }
}

}  // namespace pkd
