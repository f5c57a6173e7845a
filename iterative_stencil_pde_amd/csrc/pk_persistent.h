// The persistent kernel of the Jacobi engine for gfx950, as a template. Each
// layout's instances are compiled in a translation unit of their own
// (pk_kern_stream_f32.hip, pk_kern_stream_f64.hip, pk_kern_resident.hip,
// pk_kern_register_f32.hip, pk_kern_register_f64.hip), which builds them in parallel and lets each
// instance carry only its own layout's code.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "pk_device.h"
#include "pk_launch.h"
#include "pk_shared.h"
#include "../../include/pk.h"

using namespace pkd;

namespace {

// The periods of a tile task of n sweeps with halo depth m: the fewest periods
// of at most m sweeps (P = ceil(n / m)), as even as possible: the first n mod P
// have n / P + 1 sweeps, the rest n / P (the same number of exchanges as
// periods of m, and narrower trapezoids). Every block computes the same
// sequence; its two divisions happen once a task, not once a period (an integer
// division is a few dozen instructions, on the scalar unit that the CU's waves
// share).
struct Periods {
    int count, q, r;
    __device__ __forceinline__ Periods(int n, int m) {
        count = n > 0 ? (n - 1) / m + 1 : 0;
        q = count > 0 ? n / count : 0;
        r = count > 0 ? n - q * count : 0;
    }
    // sweeps of period k (0-based), 0 past the last
    __device__ __forceinline__ int len(int k) const { return k < count ? q + (k < r ? 1 : 0) : 0; }
};

// The same sequence from the sweeps still to come: the LDS tile's form (its
// single-block plan measured ~4% slower with the schedule above, although it
// computes one period a task either way).
__device__ __forceinline__ int period_len(int remaining, int m) {
    if (remaining <= 0) return 0;
    const int periods = (remaining - 1) / m + 1;
    return (remaining - 1) / periods + 1;
}

// Interior rows of band L when the interior is split into `grid` bands of
// q or q+1 rows (the first `rem` bands get the extra row).
__device__ __forceinline__ int band_begin(const pk_kargs& a, int L) {
    return 1 + L * a.res_q + min(L, a.res_rem);
}

// ---------------------------------------------------------------------------
// Register-tile SWEEP task (PK_LAYOUT_REGISTER). Same bands, halos, sub-sweep
// row ranges, publish / exchange / reload protocol as the LDS-resident task
// below (so the same results, bit for bit), but the tile rows live in VGPRs:
// the waves form cw column groups (64 lanes x W columns each) times rw row
// groups, and a lane holds one 16-byte vector of each of its RT consecutive
// rows (and of b). A sub-sweep updates the active rows in place, marching
// down the wave's rows with the old value of the row above in a register, so
// the stencil reads nothing from memory; W/E come from DPP lane shifts. Only
// what crosses a wave boundary goes through LDS: each wave's first and last
// row, and its first and last column. The instruction count per row is about
// half that of the LDS tile, whose sub-sweeps are bound by vector issue.
// ---------------------------------------------------------------------------
constexpr int PK_REG_RMAX = 4;  // rows per wave

// Exchange slot of one wave for one sub-sweep parity: its first row, its last
// row, its first column (element 0 of lane 0, one per row) and its last column
// (element W-1 of lane 63).
template <typename T>
struct RegSlot {
    static constexpr int W = VecW<T>::W;
    static constexpr int size = 2 * 64 * W + 2 * PK_REG_RMAX;
    static constexpr int top = 0, bottom = 64 * W, first_col = 2 * 64 * W,
                         last_col = 2 * 64 * W + PK_REG_RMAX;
};

// ONE: a single column strip (cw == 1): lane 0's W neighbour and lane 63's E
// neighbour can only belong to ring or padding columns, which keep their
// values, so the lane shifts need no edge values.
// ALN: nx is a multiple of the vector width, so column 0 is element 0 of its
// lane, column nx - 1 element W - 1 of its lane, and every other lane holds
// interior columns or padding only; padding lanes are never published, so their
// values do not matter and only those two elements need keeping (two blends a
// row instead of W).
template <typename T, bool HAS_B, bool RB, int RT, bool ONE, bool ALN, bool TRACE>
__device__ __forceinline__ void reg_sweep_rows(const pk_kargs& a, int n, int& cur, BarrierCtx& bc, T* lds) {
    constexpr int W = VecW<T>::W;
    using S = RegSlot<T>;
    static_assert(RT <= PK_REG_RMAX, "rows per wave");
    const int lb = logical_block(a.xcd_remap, a.grid);
    const int ny = a.ny, nx = a.nx;
    const int r0 = band_begin(a, lb), r1 = band_begin(a, lb + 1);
    const int m = a.res_halo;
    const int e0 = max(0, r0 - m), e1 = min(ny, r1 + m);
    const int nwv = static_cast<int>(blockDim.x) >> 6;
    const int wave = wave_id(), lane = static_cast<int>(threadIdx.x) & 63;
    const int cw = a.reg_cw;
    const int rw = nwv / cw;
    const int cg = wave % cw, rg = wave / cw;
    const bool wave_live = rg < rw;  // wave-uniform
    const int col = (cg * 64 + lane) * W;
    const bool lane_live = wave_live && col < nx;
    const int row_base = e0 + rg * RT;
    const size_t p = static_cast<size_t>(a.pitch);
    const bool has_left = cg > 0, has_right = cg + 1 < cw;  // wave-uniform
    uint32_t keep[W];  // ring (and, unless ALN, padding) columns keep their value
#pragma unroll
    for (int k = 0; k < W; ++k)
        keep[k] = ALN ? lane_mask((k == 0 && col == 0) || (k == W - 1 && col + k == nx - 1))
                      : lane_mask((col + k == 0) || (col + k >= nx - 1));

    Vec<T> u[RT], bb[RT];
    {
        const T* g = static_cast<const T*>(a.u[cur]);
        const T* gb = static_cast<const T*>(a.b);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const int row = row_base + r;
            const bool ok = lane_live && row < e1;
            u[r] = ok ? gload(g + static_cast<size_t>(row) * p + col) : vzero<T>();
            if (HAS_B) bb[r] = ok ? gload(gb + static_cast<size_t>(row) * p + col) : vzero<T>();
        }
    }
    // this wave's LDS slot in the parity-0 half; the parity-1 half follows
    T* const slot0 = lds + static_cast<size_t>(wave) * S::size;
    const size_t half = static_cast<size_t>(nwv) * S::size;
    int par = 0;
    int remaining = n;
    const Periods periods(n, m);
    int period = 0;  // the period under way
    while (remaining > 0) {
        const int sc = periods.len(period);
        if constexpr (TRACE) trace_event(bc, PK_TR_PERIOD, static_cast<uint32_t>(sc));
        // The rows of sub-sweep s (as in the LDS tile) are [max(1, r0 - (sc - s)),
        // min(ny - 1, r1 + (sc - s))): a row at distance d above the band takes
        // part up to sub-sweep sc - d, the row d below its last row up to
        // sc - 1 - d, the band's rows in all, ring rows in none. Wave-uniform.
        int last_s[RT];
        int last_any = 0;
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const int row = row_base + r;
            int l;
            if (!wave_live || row < 1 || row >= ny - 1) l = 0;
            else if (row < r0) l = sc - (r0 - row);
            else if (row < r1) l = sc;
            else l = sc - 1 - (row - r1);
            last_s[r] = __builtin_amdgcn_readfirstlane(l);
            last_any = max(last_any, last_s[r]);
        }
        // sub-sweep s with this wave's LDS slot of its parity
        const auto sub_sweep = [&](int s, T* mine) {
            // red-black: the colour of this sub-sweep
            const int parity = (n - remaining + s - 1) & 1;
            if (wave_live) {
                vstore(mine + S::top + lane * W, u[0]);
                vstore(mine + S::bottom + lane * W, u[RT - 1]);
                if (cw > 1 && (lane == 0 || lane == 63)) {
                    const bool first = lane == 0;
                    T* dst = mine + (first ? S::first_col : S::last_col);
#pragma unroll
                    for (int r = 0; r < RT; ++r) dst[r] = first ? u[r].v[0] : u[r].v[W - 1];
                }
            }
            __syncthreads();
            // wave-uniform: which of this wave's rows take part; with 4 rows a wave,
            // a bit mask from this sub-sweep's row range measured faster
            uint32_t act = 0;
            if constexpr (RT != 2) {
                const int lo = max(1, r0 - (sc - s));
                const int hi = min(ny - 1, r1 + (sc - s));
                const int first = max(0, lo - row_base), last = min(RT, hi - row_base);
                act = (wave_live && first < last) ? ((1u << last) - (1u << first)) : 0u;
            }
            const auto row_on = [&](int r) { return RT == 2 ? s <= last_s[r] : (act & (1u << r)) != 0u; };
            if (RT == 2 ? s <= last_any : act != 0u) {
                // The first row of row group 0 and the last of row group rw - 1 never
                // take part (the tile spans band + 2m rows and a sub-sweep at most
                // band + 2(m - 1), or they are ring rows), so those groups read their
                // own slot instead of a missing neighbour's: no branch, never used.
                const Vec<T> above = vload(mine - (rg > 0 ? static_cast<size_t>(cw) * S::size : 0) + S::bottom + lane * W);
                const Vec<T> below = vload(mine + (rg + 1 < rw ? static_cast<size_t>(cw) * S::size : 0) + S::top + lane * W);
                // outside neighbours of lanes 0 and 63 for every row
                T edge[RT];
#pragma unroll
                for (int r = 0; r < RT; ++r) edge[r] = T(0);
                if (ONE) {
                } else if (lane == 0 && has_left) {
                    const T* src = mine - S::size + S::last_col;
#pragma unroll
                    for (int r = 0; r < RT; ++r) edge[r] = src[r];
                } else if (lane == 63 && has_right) {
                    const T* src = mine + S::size + S::first_col;
#pragma unroll
                    for (int r = 0; r < RT; ++r) edge[r] = src[r];
                }
                Vec<T> prev = above;
#pragma unroll
                for (int r = 0; r < RT; ++r) {
                    const Vec<T> old = u[r];
                    const int row = row_base + r;
                    if (row_on(r)) {  // wave-uniform
                        const Vec<T> nxt = (r + 1 < RT) ? u[r + 1 < RT ? r + 1 : r] : below;
                        T west, east;
                        if constexpr (ONE) {
                            west = from_lower_any(old.v[W - 1]);
                            east = from_upper_any(old.v[0]);
                        } else {
                            west = from_lower(edge[r], old.v[W - 1]);
                            east = from_upper(edge[r], old.v[0]);
                        }
                        Vec<T> o;
#pragma unroll
                        for (int k = 0; k < W; ++k) {
                            const T w = (k == 0) ? west : old.v[k - 1];
                            const T ea = (k == W - 1) ? east : old.v[k + 1];
                            T x = (w + ea) + (prev.v[k] + nxt.v[k]);
                            if (HAS_B) x = x + bb[r].v[k];
                            if (!ALN || k == 0 || k == W - 1)
                                o.v[k] = blend(keep[k], old.v[k], T(0.25) * x);
                            else
                                o.v[k] = T(0.25) * x;
                        }
                        if (RB) o = rb_keep(o, old, row, parity);
                        u[r] = o;
                    }
                    prev = old;
                }
            }
        };
        // two sub-sweeps an iteration: no slot select or register rotation between them
        T* const mine0 = par ? slot0 + half : slot0;
        T* const mine1 = par ? slot0 : slot0 + half;
        for (int s = 1; s <= sc; s += 2) {
            sub_sweep(s, mine0);
            if (s < sc) sub_sweep(s + 1, mine1);
        }
        par ^= sc & 1;
        remaining -= sc;
        const int mn = periods.len(++period);  // the next period, 0 at the end
        // rows to publish: edge rows for the neighbours, or every owned row at the end
        int top_end, bot_begin;
        if (remaining == 0) {
            top_end = r1;
            bot_begin = r1;
        } else {
            top_end = (r0 > 1) ? min(r1, r0 + mn) : r0;
            bot_begin = (r1 < ny - 1) ? max(top_end, r1 - mn) : r1;
        }
        // rows to reload: the neighbours' edge rows (interior rows only: the ring
        // never changes)
        const int above = min(mn, r0 - 1);
        const int below = min(mn, ny - 1 - r1);
        if (remaining > 0 && a.exchange == PK_EXCHANGE_TAGGED) {
            // the tag of exchange e: never 0 (the buffers start zeroed) and never
            // equal to the tag of exchange e - 2, the previous use of the buffer
            const uint32_t tag = static_cast<uint32_t>(bc.tag_epoch % 0xFFFFFFFFull) + 1u;
            uint64_t* tb = a.tag + static_cast<size_t>(bc.tag_epoch & 1u) * ny * a.tag_pitch;
            const int vi = cg * 64 + lane;   // this lane's vector: word vi of each plane
            const int plane = a.tag_pitch / 4;
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const int row = row_base + r;
                const bool out = (row >= r0 && row < top_end) || (row >= bot_begin && row < r1);
                if (lane_live && out) tag_store(tb + static_cast<size_t>(row) * a.tag_pitch + vi, plane, u[r], tag);
            }
            uint32_t need = 0;  // halo rows of this wave, a bit per row (wave-uniform)
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const int row = row_base + r;
                if ((row >= r0 - above && row < r0) || (row >= r1 && row < r1 + below)) need |= 1u << r;
            }
            if (!wave_live) need = 0;
            if (TRACE && wave == 0 && need) trace_event(bc, PK_TR_TAG_WAIT, static_cast<uint32_t>(bc.tag_epoch));
            if (need && !bc.faulted) {
                // load every halo word of the wave until all carry this exchange's tag
                // (straight into the rows: their old values are not needed again)
                const uint64_t t0 = wall_clock64();
                for (;;) {
                    bool ok = true;
#pragma unroll
                    for (int r = 0; r < RT; ++r) {
                        if ((need & (1u << r)) && lane_live)
                            ok = tag_load(tb + static_cast<size_t>(row_base + r) * a.tag_pitch + vi, plane, u[r],
                                          tag) && ok;
                    }
                    if (__ballot(!ok) == 0) break;
                    // a fault elsewhere is read only once the poll has waited far
                    // longer than an exchange takes (1/65536 of the limit, ~30 us at
                    // 2 s): read after every miss, it put a second memory round trip
                    // in front of the next poll
                    const uint64_t waited = wall_clock64() - t0;
                    const bool late =
                        waited > a.tag_ticks ||
                        (waited > (a.tag_ticks >> 16) &&
                         __hip_atomic_load(&a.st->fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u);
                    if (late) {  // a fault elsewhere, or a tag that never comes: give up
                        bc.faulted = true;
                        if (lane == 0)
                            __hip_atomic_store(&a.st->fault, static_cast<uint32_t>(PK_FAULT_BARRIER_TIMEOUT),
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            if (TRACE && wave == 0 && need) trace_event(bc, PK_TR_TAG_DONE, static_cast<uint32_t>(bc.tag_epoch));
            bc.tag_epoch += 1;
            continue;  // the field buffers are untouched until the task's last exchange
        }
        {   // publish into the other field buffer
            T* g = static_cast<T*>(a.u[cur ^ 1]);
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const int row = row_base + r;
                const bool out = (row >= r0 && row < top_end) || (row >= bot_begin && row < r1);
                if (lane_live && out) gstore(g + static_cast<size_t>(row) * p + col, u[r]);
            }
        }
        if (remaining > 0 && a.exchange == PK_EXCHANGE_NEIGHBOR)
            neighbor_sync(bc, a.nbr, lb, a.res_dist);
        else
            grid_barrier(bc, bc.broken);
        cur ^= 1;
        if (remaining > 0) {  // the neighbours' edge rows become this block's halo
            const T* g = static_cast<const T*>(a.u[cur]);
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const int row = row_base + r;
                const bool halo = (row >= r0 - above && row < r0) || (row >= r1 && row < r1 + below);
                if (lane_live && halo) u[r] = gload(g + static_cast<size_t>(row) * p + col);
            }
        }
    }
}

// Rows per wave (RT, 2 or 4) are chosen per engine and compiled into the
// kernel instance it runs: each instance holds one row count's registers.
template <typename T, bool HAS_B, bool RB, int RT, bool TRACE>
__device__ __forceinline__ void reg_sweep_task(const pk_kargs& a, int n, int& cur, BarrierCtx& bc, T* lds) {
    const bool aln = a.nx % VecW<T>::W == 0;
    if (a.reg_cw == 1) {
        if (aln)
            reg_sweep_rows<T, HAS_B, RB, RT, true, true, TRACE>(a, n, cur, bc, lds);
        else
            reg_sweep_rows<T, HAS_B, RB, RT, true, false, TRACE>(a, n, cur, bc, lds);
    } else {
        if (aln)
            reg_sweep_rows<T, HAS_B, RB, RT, false, true, TRACE>(a, n, cur, bc, lds);
        else
            reg_sweep_rows<T, HAS_B, RB, RT, false, false, TRACE>(a, n, cur, bc, lds);
    }
}

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
// n sub-sweeps: Jacobi sweeps, or (RB) red-black half-sweeps, red first.
template <typename T, bool HAS_B, bool RB, bool TRACE>
__device__ __forceinline__ void resident_sweep_task(const pk_kargs& a, int n, int& cur, BarrierCtx& bc, T* lds) {
    constexpr int W = VecW<T>::W;
    const int lb = logical_block(a.xcd_remap, a.grid);
    const int ny = a.ny;
    const int r0 = band_begin(a, lb);
    const int r1 = band_begin(a, lb + 1);
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
        constexpr int U = 4;  // loads in flight per thread
        for (int base = tid; base < tot; base += U * nt) {
            Vec<T> x[U], xb[U];
            int dst[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int idx = base + u * nt;
                dst[u] = -1;
                if (idx < tot) {
                    const int rr = idx / nv, col = (idx % nv) * W;
                    const size_t go = static_cast<size_t>(e0 + rr) * p + col;
                    x[u] = gload(g + go);
                    if (HAS_B) xb[u] = gload(gb + go);
                    dst[u] = rr * lp + col;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (dst[u] < 0) continue;
                vstore(A + dst[u], x[u]);
                vstore(B + dst[u], x[u]);
                if (HAS_B) vstore(Bt + dst[u], xb[u]);
            }
        }
    }
    __syncthreads();

    T* S = A;
    T* D = B;
    const TileMap<T> tm = tile_map<T>(nv, lp, a.nx);
    int remaining = n;
    while (remaining > 0) {
        const int sc = period_len(remaining, m);
        if constexpr (TRACE) trace_event(bc, PK_TR_PERIOD, static_cast<uint32_t>(sc));
        for (int s = 1; s <= sc; ++s) {
            // rows of this sub-sweep: the owned band widened by the sub-sweeps
            // still to come, within the interior (a halo deeper than the
            // neighbouring band reaches back to the ring)
            const int lo = max(1, r0 - (sc - s));
            const int hi = min(ny - 1, r1 + (sc - s));
            // colour of this half-sweep: half-sweeps done so far in the task, mod 2
            const int parity = (n - remaining + s - 1) & 1;
            if (tm.segs == 1)
                resident_rows<T, HAS_B, RB, true>(S, D, Bt, lo - e0, hi - e0, tm, e0, parity);
            else
                resident_rows<T, HAS_B, RB, false>(S, D, Bt, lo - e0, hi - e0, tm, e0, parity);
            __syncthreads();
            T* t = S;
            S = D;
            D = t;
        }
        remaining -= sc;
        const int mn = period_len(remaining, m);  // the next period, 0 at the end

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
                gstore(g + static_cast<size_t>(rr) * p + col, vload(S + (rr - e0) * lp + col));
            }
        }
        if (remaining > 0 && a.exchange == PK_EXCHANGE_NEIGHBOR)
            neighbor_sync(bc, a.nbr, lb, a.res_dist);
        else
            grid_barrier(bc, bc.broken);
        cur ^= 1;
        if (remaining > 0) {  // the neighbours' edge rows become this block's halo
            const T* g = static_cast<const T*>(a.u[cur]);
            const int above = min(mn, r0 - 1);       // interior rows only: row 0 is ring
            const int below = min(mn, ny - 1 - r1);
            const int tot = (above + below) * nv;
            // several loads in flight per thread before the LDS stores: each
            // one is a trip to memory (the release/acquire pair of the
            // barrier leaves these rows in no cache)
            constexpr int U = 4;
            for (int base = tid; base < tot; base += U * nt) {
                Vec<T> x[U];
                int dst[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int idx = base + u * nt;
                    dst[u] = -1;
                    if (idx < tot) {
                        const int k = idx / nv, col = (idx % nv) * W;
                        const int rr = (k < above) ? r0 - above + k : r1 + (k - above);
                        x[u] = gload(g + static_cast<size_t>(rr) * p + col);
                        dst[u] = (rr - e0) * lp + col;
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (dst[u] >= 0) vstore(S + dst[u], x[u]);
            }
            __syncthreads();
        }
    }
}

// Copy the field (unpadded rows) into the pinned host staging buffer.
template <typename T>
__device__ __forceinline__ void readback_task(const pk_kargs& a, int cur) {
    const T* g = static_cast<const T*>(a.u[cur]);
    T* h = static_cast<T*>(a.staging);
    const int lane = thread_id_here() & 63;
    const int wpb = static_cast<int>(blockDim.x) >> 6;
    const int gw = static_cast<int>(blockIdx.x) * wpb + wave_id();
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
__device__ __forceinline__ int64_t stamp_task(const pk_kargs& a, int n, uint32_t& round, BarrierCtx& bc,
                              double* s_red) {
    int64_t errs = 0;
    const int g = a.grid;
    const int tid = thread_id_here();
    for (int k = 0; k < n; ++k) {
        const uint32_t s = ++round;
        uint32_t* base = a.stamp + static_cast<size_t>(s & 1u) * g * 64;
        if (tid < 64) base[blockIdx.x * 64 + tid] = s;
        grid_barrier(bc, bc.broken);
        if (tid < 64) {
            const int nb = (static_cast<int>(blockIdx.x) + 1) % g;
            const uint32_t hsh = (s * 2654435761u) ^ (blockIdx.x * 40503u + 977u);
            const int rb = static_cast<int>(hsh % static_cast<uint32_t>(g));
            const uint32_t v1 = base[nb * 64 + tid];
            const uint32_t v2 = base[rb * 64 + tid];
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

// A task's completion record, field by field (the leader only; the release
// store of done_seq that follows publishes it to the host).
__device__ __forceinline__ void write_done(pk_done_rec* d, uint64_t seq, int kind, int status, double residual,
                                           int64_t sweeps, uint64_t t_begin, uint64_t t_end, int64_t errors,
                                           int cur, int carried) {
    put(&d->kind, kind);
    put(&d->status, status);
    put(&d->residual, residual);
    put(&d->sweeps_done, sweeps);
    put(&d->t_begin, t_begin);
    put(&d->t_end, t_end);
    put(&d->errors, errors);
    put(&d->cur, cur);
    put(&d->carried, carried);
    put(&d->seq, seq);
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
// Residual state shared by the sweeping tasks (identical in every block): the
// round count picks the half of `partials` a round uses; `ready` says that the
// last streaming pass already wrote this round's partials (of the field as it
// is now), so the next residual only sums them.
struct ResidualState {
    uint32_t round;
    bool ready;
};

// Task fusion across a RESIDUAL task (streaming layout), in the block's shared
// memory (read at task boundaries only): the SWEEP task two slots after task
// `from_seq` starts with `pre` of its sweeps already applied by that task's last
// pass; `dec` is the decision for the task under way, as read after the grid
// barrier that published it.
struct FuseState {
    uint64_t from_seq;
    uint64_t cur_seq;  // the task under way (thread 0's copy)
    int pre;
    int dec;
};

// Depth of the next streaming pass with `left` sweeps (or red-black
// half-sweeps) to go: the engine's depth, or `left` when fewer. A depth the
// kernel does not carry (9..11) runs 8 first. A task's last Jacobi pass also
// sums the residual with one level more, so it is at most PK_SHALLOW_PASS deep:
// a 12-sweep tail runs as 4 + 8. Red-black passes are at most PK_SHALLOW_PASS
// deep. Every block computes the same sequence.
__device__ __forceinline__ int pass_depth(int depth, int left, bool rb) {
    int k = min(depth, left);
    if (k > PK_SHALLOW_PASS && (rb || !PK_PASS_DEPTH_OK(k))) k = PK_SHALLOW_PASS;
    if (k == left && k > PK_SHALLOW_PASS) k = left - PK_SHALLOW_PASS;
    return k;
}

// Leader only, before the grid barrier ahead of a task's last P or fewer
// sweeps: whether the two tasks after the SWEEP task fs->cur_seq are a RESIDUAL
// and a SWEEP of at least `need` sweeps, both already published by the host; the
// decision (the task's sequence number, or 0) goes to a device word that the
// barrier publishes.
__device__ __forceinline__ void fuse_decide(const pk_kargs& a, FuseState* fs, int need) {
    const uint64_t seq = *reinterpret_cast<volatile unsigned long long*>(&fs->cur_seq);
    const pk_mailbox* mail = a.mail;
    const uint64_t w1 = __hip_atomic_load(&mail->slot[(seq + 1) % PK_RING].word, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_SYSTEM);
    const uint64_t w2 = __hip_atomic_load(&mail->slot[(seq + 2) % PK_RING].word, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_SYSTEM);
    const bool ok = static_cast<uint32_t>(w1 >> 32) == static_cast<uint32_t>(seq + 1) &&
                    static_cast<int>((w1 >> 28) & 0xF) == PK_RESIDUAL &&
                    static_cast<uint32_t>(w2 >> 32) == static_cast<uint32_t>(seq + 2) &&
                    static_cast<int>((w2 >> 28) & 0xF) == PK_SWEEP && static_cast<int>(w2 & PK_TASK_N_MAX) >= need;
    __hip_atomic_store(&a.st->fuse_seq, ok ? seq : 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Leader only, at the start of a RESIDUAL task of a field no pass has summed:
// whether the next task is a SWEEP of at least PK_MAX_PASS sweeps, already
// published by the host (the decision, as for fuse_decide, through a barrier).
__device__ __forceinline__ void fuse_decide_next(const pk_kargs& a, uint64_t seq) {
    const uint64_t w = __hip_atomic_load(&a.mail->slot[(seq + 1) % PK_RING].word, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_SYSTEM);
    const bool ok = static_cast<uint32_t>(w >> 32) == static_cast<uint32_t>(seq + 1) &&
                    static_cast<int>((w >> 28) & 0xF) == PK_SWEEP && static_cast<int>(w & PK_TASK_N_MAX) >= PK_MAX_PASS;
    __hip_atomic_store(&a.st->fuse_seq, ok ? seq : 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// n sub-sweeps of the field in u[cur] in the engine's layout (cur flips):
// Jacobi sweeps, or (rb) red-black half-sweeps, red first.
// fusable (streaming layout, fp64): a plain SWEEP task (fs->cur_seq) that may
// run its last pass on into a later SWEEP task; run_ahead (n = 0): run the next
// task's first pass with the residual of its level 0; returns the sweeps of that
// later task applied here (0 if none). The fp32 kernels leave fusion out: its code cost
// their passes 10% (4096^2 fp32 Laplace, 4.48 against 4.08 us per sweep) in
// register pressure, and the fp32 workloads that stream run one long task.
template <typename T, bool HAS_B, int LAYOUT, int RT, bool TRACE>
__device__ __forceinline__ int sweeps_task(const pk_kargs& a, int n, bool rb, int& cur, BarrierCtx& bc,
                                           T* lds, ResidualState& rs, double* s_red, bool fusable,
                                           FuseState* fs, bool run_ahead = false) {
    int ahead = 0;
    if constexpr (LAYOUT == PK_LAYOUT_RESIDENT) {
        if (rb)
            resident_sweep_task<T, HAS_B, true, TRACE>(a, n, cur, bc, lds);
        else
            resident_sweep_task<T, HAS_B, false, TRACE>(a, n, cur, bc, lds);
    } else if constexpr (LAYOUT == PK_LAYOUT_REGISTER) {
        if (rb)
            reg_sweep_task<T, HAS_B, true, RT, TRACE>(a, n, cur, bc, lds);
        else
            reg_sweep_task<T, HAS_B, false, RT, TRACE>(a, n, cur, bc, lds);
    } else {
        // Fusion: where the task's last t <= P sweeps are followed by a RESIDUAL
        // and a SWEEP of at least P - t sweeps (t = P: at least P; the leader
        // reads their slots just before the grid barrier ahead of those sweeps),
        // they run as one P-deep pass: the task's own t, then the first P - t of
        // that later SWEEP task, summing rho^2 of level t on the way (a tap), the
        // RESIDUAL's value; a tail of exactly P runs as a pass of its own first,
        // and the tap is then at level 0 of the later task's first pass. The field
        // the task ends with is never stored; every stored value is still the
        // same expression on the same operands.
        const int P = a.pass_sweeps;
        const bool fz = sizeof(T) == 8 && fusable && !rb && !bc.broken && P == PK_MAX_PASS;
        // (run_ahead: n = 0, a RESIDUAL task running the next task's first pass)
        bool fused = run_ahead;  // the leader's decision for the tail (uniform)
        int s = 0;
        while (s < n) {
            const int left = n - s;
            int k;
            if (fz && left > P) k = P;
            else k = pass_depth(P, left, rb);
            // the last Jacobi pass of a task also sums rho^2 of its result, so a
            // RESIDUAL that follows need not read the field again ("Grid-Wide
            // Barriers", "What the barrier buys": the convergence check as a
            // reduction at the barrier); not under the negative control
            const bool res = s + k >= n && !rb && !bc.broken;
            const double acc = stream_pass<T, HAS_B>(a, static_cast<const T*>(a.u[cur]),
                                                     static_cast<T*>(a.u[cur ^ 1]), k, rb ? (s & 1) : -1, res);
            if (res) {
                const double p = block_sum(acc, s_red);
                if (threadIdx.x == 0) a.partials[static_cast<size_t>(rs.round & 1u) * a.grid + blockIdx.x] = p;
            }
            // the barrier ahead of the task's last P or fewer sweeps decides whether
            // they fuse (the leader publishes the decision before arriving)
            const int rest = n - (s + k);
            const bool decide = fz && rest > 0 && rest <= P;
            if (decide && blockIdx.x == 0 && threadIdx.x == 0) fuse_decide(a, fs, rest < P ? P - rest : P);
            // between two full-depth passes (the same units), neighbour counters may
            // stand in for the grid barrier; a task's last pass, and the passes next
            // to a shallower one, end with the barrier (it also orders the partials
            // before any read)
            if (__builtin_amdgcn_readfirstlane(bc.pn->on) && k == P && !res && s + k < n &&
                pass_depth(P, n - s - k, rb) == P && (rb || s + k + P < n))
                pass_neighbor_sync(bc, __builtin_amdgcn_readfirstlane(bc.pn->mask));
            else
                grid_barrier(bc, bc.broken);
            cur ^= 1;
            rs.ready = res;
            s += k;
            if (decide) {
                if (threadIdx.x == 0)
                    fs->dec = __hip_atomic_load(&a.st->fuse_seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                              *reinterpret_cast<volatile unsigned long long*>(&fs->cur_seq);
                __syncthreads();
                fused = fs->dec != 0;
                __syncthreads();
                if (fused) break;
            }
        }
        if (fused) {
            // the fused tail: this task's last t sweeps and the later task's first
            // P - t in one pass, rho^2 of level t summed for the RESIDUAL between.
            // A tail of exactly P runs as a pass of its own, and the later task's
            // first P sweeps then tap level 0 (the field this task ends with).
            int t = n - s;
            if (t == P) {
                stream_pass<T, HAS_B>(a, static_cast<const T*>(a.u[cur]), static_cast<T*>(a.u[cur ^ 1]), P, -1,
                                      false);
                grid_barrier(bc, bc.broken);
                cur ^= 1;
                t = 0;
            }
            const double acc = stream_pass<T, HAS_B>(a, static_cast<const T*>(a.u[cur]),
                                                     static_cast<T*>(a.u[cur ^ 1]), P, -1, false, t);
            const double p = block_sum(acc, s_red);
            if (threadIdx.x == 0) a.partials[static_cast<size_t>(rs.round & 1u) * a.grid + blockIdx.x] = p;
            grid_barrier(bc, bc.broken);  // also orders the partials before any read
            cur ^= 1;
            rs.ready = true;
            ahead = P - t;
        }
    }
    if (rb && n > 0) rs.ready = false;  // the field changed, no partials of it
    return ahead;
}

// One residual round: each block's partial goes to the half of `partials` of
// this round's parity, a grid barrier, then the sum in a fixed order (blocks in
// order, the same code everywhere, so bitwise the same in every block). Only
// the blocks that ask (all) read the partials back. Rounds alternate halves: a
// block writes round r + 2 only after passing round r + 1's barrier, which every
// reader of round r reaches only after its reads. Returns R in every thread of
// a block that asked (0 elsewhere).
// When the last streaming pass already wrote this round's partials (rs.ready),
// the round only sums them: that pass's grid barrier ordered them.
template <typename T, bool HAS_B>
__device__ __forceinline__ double residual_round(const pk_kargs& a, int cur, BarrierCtx& bc,
                                                 ResidualState& rs, double* s_red, bool all) {
    double* part = a.partials + static_cast<size_t>(rs.round & 1u) * a.grid;
    rs.round += 1;
    if (!rs.ready) {
        const double p = stream_residual_block<T, HAS_B>(a, static_cast<const T*>(a.u[cur]), s_red);
        if (threadIdx.x == 0) part[blockIdx.x] = p;
        grid_barrier(bc);
    }
    rs.ready = false;
    double r = 0.0;
    if (all || blockIdx.x == 0) {
        const double tot = sum_partials(part, a.grid);
        if (threadIdx.x == 0) s_red[0] = sqrt(tot);
        __syncthreads();
        r = s_red[0];
        __syncthreads();
    }
    return r;
}

// The streaming kernel's passes keep up to 12 levels of the march in registers:
// blocks of at most 512 threads give it 256 VGPRs per lane.
// (Two waves per SIMD already keep its vector unit busy: 768-thread blocks, which
// the fp32 Laplace passes would fit, measured slower, 6.5 against 5.3 us per
// 4096^2 sweep, with shorter bands and more halo rows.)
template <typename T, bool HAS_B, int LAYOUT>
struct PkMaxThreads {
    static constexpr int value = LAYOUT == PK_LAYOUT_STREAM ? 512 : 1024;
};

// RT: rows per wave of the register layout (0 in the other layouts).
// TRACE: the tile layouts' per-period and tag-poll events are compiled in
// (task and synchronization events are in every instance, behind a run-time
// check); an engine made with PK_DBG_TRACE runs this instance. The events
// inside the tile loops cost the untraced instances about 3 % per sweep on a
// 256^2 grid, so they live only here.
template <typename T, bool HAS_B, int LAYOUT, int RT, bool TRACE>
__global__ void __launch_bounds__((PkMaxThreads<T, HAS_B, LAYOUT>::value)) pk_persistent(pk_kargs a) {
    extern __shared__ __align__(16) unsigned char pk_lds[];
    __shared__ double s_red[16];
    __shared__ int s_kind, s_n, s_exit, s_carried, s_every;
    __shared__ double s_tol;
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
    bc.nbr_epoch = 0;
    bc.tag_epoch = 0;
    bc.nbar = 0;
    __shared__ CarryState s_carry;
    if (threadIdx.x == 0) {
        s_carry.seq = 0;
        s_carry.t0 = 0;
        s_carry.age = a.carry_age_ticks;
        s_carry.pending = 0;
        s_carry.t_task = 0;
    }
    __shared__ XcdState s_xcd;
    if (threadIdx.x == 0) {
        s_xcd.g = 0;
        s_xcd.members = 1;
        s_xcd.groups = 1;
    }
    __syncthreads();
    bc.carry = &s_carry;
    bc.xs = &s_xcd;
    bc.carry_word = 0;
    __shared__ TraceState s_trace;
    if (threadIdx.x == 0) {
        s_trace.ring = a.trace ? a.trace + static_cast<size_t>(blockIdx.x) * PK_TRACE_BLOCK_BYTES : nullptr;
        s_trace.count = 0;
    }
    bc.trace = &s_trace;
    __shared__ PassNbr s_pn;
    __shared__ FuseState s_fuse;
    if (threadIdx.x == 0) {
        s_pn.on = 0;
        s_pn.mask = 0;
        s_fuse.from_seq = 0;
        s_fuse.cur_seq = 0;
        s_fuse.pre = 0;
        s_fuse.dec = 0;
    }
    bc.pn = &s_pn;
    // neighbour counters between streaming passes (more than one block)
    const bool pass_nbr = LAYOUT == PK_LAYOUT_STREAM && a.pass_nbr_dist > 0 && a.grid > 1 && !bc.broken;
    if ((a.barrier_kind == PK_BARRIER_XCD || pass_nbr) && a.grid > 1 && !bc.broken) {
        // count the blocks on each XCD (one grid barrier of the flat or two-level
        // kind); the XCD barrier's counters start from zero after it. Under pass
        // neighbour counters each block also notes its XCD beside its flag.
        const int lb = logical_block(a.xcd_remap, a.grid);
        if (threadIdx.x == 0) {
            s_xcd.g = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 7u;  // hwreg(HW_REG_XCC_ID, 0, 4)
            __hip_atomic_fetch_add(&a.st->xmembers[s_xcd.g].v, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (pass_nbr)
                __hip_atomic_store(a.nbr + static_cast<size_t>(lb) * PK_NBR_WORDS + 1, s_xcd.g, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        grid_barrier(bc);
        if (threadIdx.x == 0) {
            s_xcd.members = __hip_atomic_load(&a.st->xmembers[s_xcd.g].v, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
            uint32_t groups = 0;
            for (int k = 0; k < 8; ++k)
                groups += __hip_atomic_load(&a.st->xmembers[k].v, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) > 0u ? 1u : 0u;
            s_xcd.groups = groups;
        }
        if (pass_nbr && threadIdx.x < 64) {
            // the XCDs of the blocks holding the units next to this block's units in
            // a full-depth pass (see pass_neighbor_sync): for each unit of the
            // block, lane i looks up one neighbour (band d, strip e) and, where that
            // is a split edge unit, the block of its bottom half too
            const int lane = static_cast<int>(threadIdx.x), dist = a.pass_nbr_dist, g = a.grid;
            const int S = a.pass_nbr_strips, NB = a.pbands, units = S * NB;
            const bool split = pass_split_edges(S, NB, g * (static_cast<int>(blockDim.x) >> 6));
            const int total = units + (split ? 2 * NB : 0);
            const int d = lane / 3 - dist, e = lane % 3 - 1;
            uint32_t mask = 0;
            for (int u = lb; u < total; u += g) {
                int band, strip, half;
                pass_unit_place(u, S, units, band, strip, half);
                const int b2 = band + d, s2 = strip + e;
                uint32_t x0 = 8, x1 = 8;
                if (lane < 3 * (2 * dist + 1) && b2 >= 0 && b2 < NB && s2 >= 0 && s2 < S) {
                    const int q0 = (b2 * S + s2) % g;
                    if (q0 != lb)
                        x0 = __hip_atomic_load(a.nbr + static_cast<size_t>(q0) * PK_NBR_WORDS + 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                    if (split && (s2 == 0 || s2 == S - 1)) {
                        const int q1 = (units + 2 * b2 + (s2 == 0 ? 0 : 1)) % g;
                        if (q1 != lb)
                            x1 = __hip_atomic_load(a.nbr + static_cast<size_t>(q1) * PK_NBR_WORDS + 1,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
                for (uint32_t k = 0; k < 8; ++k)
                    if (__any(x0 == k || x1 == k)) mask |= 1u << k;
            }
            // and its own XCD: a block must not arrive at its XCD's counter for the
            // next pass before every block of that XCD has arrived for this one (the
            // last-arrival test counts arrivals pass by pass)
            if (lane == 0) {
                s_pn.on = 1;
                s_pn.mask = mask | (1u << s_xcd.g);
            }
        }
        if (a.barrier_kind == PK_BARRIER_XCD) {
            bc.epoch = 0;
            bc.xcd = true;
        }
    }

    const bool leader = (blockIdx.x == 0) && (threadIdx.x == 0);
    int cur = a.cur0;
    int64_t sweeps = 0;
    uint64_t next_seq = 1;
    bool may_carry = false;  // the last task passed an ordered barrier (uniform)
    ResidualState rs{0u, false};  // residual rounds so far (uniform) and ready partials
    uint32_t stamp_round = 0;
    pk_mailbox* mail = a.mail;

    for (;;) {
        // Fast path: the previous task's last ordered barrier carried this task
        // in (the leader had read it ahead); every block reads the same carry
        // word after that barrier, so all take the same path.
        // One round of loads: the carry's sequence, kind and count (all written
        // before the barrier that carried it, so read together and kept only if
        // the sequence matches) and the fault flag; one after another they were
        // three memory round trips at every task start.
        if (threadIdx.x == 0) {
            s_carried = 0;
            uint64_t cs = 0;
            int32_t ck = PK_EXIT, cn = 0;
            if (may_carry) {
                const pk_carry* c = &a.st->carry[next_seq & 1];
                cs = __hip_atomic_load(&c->seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ck = __hip_atomic_load(&c->kind, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                cn = __hip_atomic_load(&c->n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            const uint32_t f = __hip_atomic_load(&a.st->fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (may_carry && cs == next_seq) {
                s_carried = 1;
                s_kind = ck;
                s_n = cn;
                s_seq = next_seq;
                s_exit = (bc.faulted || f != 0 || ck == PK_EXIT) ? 1 : 0;
            }
        }
        __syncthreads();
        if (!s_carried) {
            if (leader) {
                uint32_t fault = __hip_atomic_load(&a.st->fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                int kind = PK_EXIT, nn = 0;
                if (!bc.faulted && fault == 0) {
                    const uint64_t t0 = wall_clock64();
                    bool idle = false;
                    // the slot word carries the whole task: poll it until its
                    // sequence half is the one expected (one bus read per poll)
                    const uint64_t* slot = &mail->slot[next_seq % PK_RING].word;
                    uint64_t w = 0;
                    for (;;) {
                        w = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                        if (static_cast<uint32_t>(w >> 32) == static_cast<uint32_t>(next_seq)) break;
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
                        kind = static_cast<int>((w >> 28) & 0xF);
                        nn = static_cast<int>(w & PK_TASK_N_MAX);
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
        }
        const int kind = s_kind, n = s_n;
        const uint64_t seq = s_seq;
        if (leader) s_carry.t_task = wall_clock64();
        const uint32_t nbar0 = bc.nbar;
        // read the next slot ahead for work tasks (not for the timing tasks, and
        // not for empty sweeps, whose only barrier comes at once)
        const bool work = ((kind == PK_SWEEP || kind == PK_SWEEP_RB) && n > 0) || kind == PK_RESIDUAL ||
                          kind == PK_SWEEP_UNTIL || kind == PK_TASK_READBACK;
        if (leader && !bc.broken && work) {
            s_carry.seq = seq + 1;
            s_carry.t0 = wall_clock64();
            s_carry.pending = 1;
            bc.carry_word = __hip_atomic_load(&mail->slot[(seq + 1) % PK_RING].word, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_SYSTEM);
        }

        trace_event(bc, PK_TR_TASK_BEGIN, static_cast<uint32_t>(kind));
        if (s_exit) {
            if (leader) {
                const uint32_t f = __hip_atomic_load(&a.st->fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint32_t code = (f != 0) ? f : (bc.faulted ? PK_FAULT_BARRIER_TIMEOUT : 0u);
                if (kind == PK_EXIT && code == 0) {
                    write_done(&mail->done[seq % PK_RING], seq, PK_EXIT, PK_OK, 0.0, sweeps, s_carry.t_task,
                               s_carry.t_task, 0, cur, s_carried);
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
        int fused_task = 0;  // the task ran sweeps of a later SWEEP task (fused)
        if (kind == PK_SWEEP || kind == PK_SWEEP_RB || kind == PK_RESIDUAL || kind == PK_SWEEP_UNTIL) {
            // The sweeping tasks share one loop (one copy of the sweep and
            // residual code in the kernel): an optional residual check, then up
            // to `every` sweeps, until the budget is spent or R <= tol.
            const bool rb = kind == PK_SWEEP_RB;
            const bool until = kind == PK_SWEEP_UNTIL;
            const bool check = until || kind == PK_RESIDUAL;
            // a SWEEP task may start with some of its sweeps already applied by
            // the fused last pass of the SWEEP task two slots before it
            const int pre = (kind == PK_SWEEP && s_fuse.from_seq + 2 == seq) ? s_fuse.pre : 0;
            const int budget = kind == PK_RESIDUAL ? 0 : n - pre;
            double tol = -1.0;  // R >= 0: never stops a plain residual
            int every = budget;
            if (until) {
                // parameters: each block acquires the slot word the host released
                // after writing them, then reads them
                if (threadIdx.x == 0) {
                    (void)__hip_atomic_load(&mail->slot[seq % PK_RING].word, __ATOMIC_ACQUIRE,
                                            __HIP_MEMORY_SCOPE_SYSTEM);
                    const pk_param* prm = &mail->param[seq % PK_RING];
                    s_tol = __hip_atomic_load(&prm->tol, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                    s_every = __hip_atomic_load(&prm->every, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                }
                __syncthreads();
                tol = s_tol;
                every = s_every;
            }
            // A RESIDUAL of a field no pass has summed, with a SWEEP of at least a
            // pass queued right after it: that SWEEP task's first pass runs here (as
            // the tail of a SWEEP task fused into it does, through the one call of
            // sweeps_task below) and sums the residual of its level 0, the field as
            // it is now, instead of a pass that only reads the field; the SWEEP task
            // then starts with those sweeps applied.
            bool run_ahead = false;
            if constexpr (LAYOUT == PK_LAYOUT_STREAM && sizeof(T) == 8) {
                if (kind == PK_RESIDUAL && !rs.ready && !bc.broken && a.pass_sweeps == PK_MAX_PASS) {
                    if (leader) fuse_decide_next(a, seq);
                    grid_barrier(bc);
                    if (threadIdx.x == 0)
                        s_fuse.dec = __hip_atomic_load(&a.st->fuse_seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                                     *reinterpret_cast<volatile unsigned long long*>(&s_seq);
                    __syncthreads();
                    run_ahead = s_fuse.dec != 0;
                    __syncthreads();
                }
            }
            {
                int done = 0;
                for (;;) {  // the same decisions in every block
                    if (check && !run_ahead) {
                        res = residual_round<T, HAS_B>(a, cur, bc, rs, s_red, until);
                        if (res <= tol) break;
                    }
                    if (!run_ahead && done >= budget) break;
                    const int k = run_ahead ? 0 : min(every, budget - done);
                    // red-black: k iterations = 2k half-sweeps, each computed into
                    // the other buffer with the other colour copied (the in-place
                    // result: a node never reads its own colour)
                    const bool fusable = LAYOUT == PK_LAYOUT_STREAM && sizeof(T) == 8 && kind == PK_SWEEP;
                    if (fusable && threadIdx.x == 0)
                        s_fuse.cur_seq = *reinterpret_cast<volatile unsigned long long*>(&s_seq);
                    const int ahead = sweeps_task<T, HAS_B, LAYOUT, RT, TRACE>(
                        a, rb ? 2 * k : k, rb, cur, bc, reinterpret_cast<T*>(pk_lds), rs, s_red, fusable, &s_fuse,
                        run_ahead);
                    if (ahead > 0) {  // uniform: a later SWEEP task is ahead by that much
                        fused_task = 1;
                        __syncthreads();
                        if (threadIdx.x == 0) {
                            // the task two slots after this SWEEP task, or the one right
                            // after this RESIDUAL (copied from shared memory here: a
                            // register copy of the sequence made for this store was
                            // kept, and spilled, across the task)
                            s_fuse.from_seq = *reinterpret_cast<volatile unsigned long long*>(&s_seq) -
                                              (kind == PK_RESIDUAL ? 1u : 0u);
                            s_fuse.pre = ahead;
                        }
                    }
                    if (run_ahead) {  // then the residual round sums what that pass summed
                        run_ahead = false;
                        continue;
                    }
                    done += k;
                }
                sweeps += done + pre;
            }
        } else if (kind == PK_TASK_READBACK) {
            readback_task<T>(a, cur);
            grid_barrier(bc);
        } else if (kind == PK_BARRIER) {
            for (int s = 0; s < n; ++s) grid_barrier(bc);
        } else if (kind == PK_STAMP) {
            errs = stamp_task(a, n, stamp_round, bc, s_red);
        } else if (kind == PK_BLOCKSYNC) {
            // the block-level step of every tile sub-sweep and nothing else: each
            // wave writes to LDS, the block meets, each wave reads its neighbour's
            // value (slots alternate by round, as the tiles' exchange slots do)
            const int wv = wave_id();
            double v = static_cast<double>(wv);
            for (int r = 0; r < n; ++r) {
                if ((threadIdx.x & 63) == 0) s_red[(r & 1) * 8 + (wv & 7)] = v;
                __syncthreads();
                v += s_red[(r & 1) * 8 + ((wv + 1) & 7)];
            }
            if (v < 0.0) errs = 1;  // never: keeps the loop's result in use
        } else {
            status = PK_EINVAL;
        }
        // A carry is published only at an ordered barrier of the task before the
        // one it carries. The leader therefore writes carry[(seq + 1) & 1] only
        // after every block has passed either that barrier or, on the ordinary
        // path, the broadcast barrier of this task, i.e. after every block read
        // carry[(seq - 1) & 1], the same word. A task without a barrier carries
        // nothing, so the next one starts the ordinary way.
        trace_event(bc, PK_TR_TASK_END, static_cast<uint32_t>(kind));
        if (leader) s_carry.pending = 0;  // never publish it outside its task
        may_carry = !bc.broken && bc.nbar != nbar0;
        if (leader) {
            write_done(&mail->done[seq % PK_RING], seq, kind, bc.faulted ? PK_EDEVICE : status, res, sweeps,
                       s_carry.t_task, wall_clock64(), errs, cur, s_carried | (fused_task << 1));
            __hip_atomic_store(&mail->done_seq, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
        }
        next_seq = seq + 1;
    }
}

}  // namespace
