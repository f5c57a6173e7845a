// Host runtime of the Jacobi engine: argument checks, grid planning from the
// occupancy query, device buffers, the pinned mailbox, the cooperative launch,
// task submission and completion, and the launch-per-sweep baseline.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstdint>
#include <cstring>
#include <functional>
#include <new>
#include <vector>

#include "../../include/pk.h"
#include "pk_launch.h"
#include "pk_ring.h"
#include "pk_shared.h"

namespace {

enum EngineState { RUNNING = 0, EXITED = 1, POISONED = 2 };

struct Plan {
    int layout = PK_LAYOUT_STREAM;
    int threads = 1024;
    int grid = 1;
    int strips = 1, bands = 1, band_rows = 1;
    int res_q = 0, res_rem = 0, res_halo = 0, res_ext_rows = 0, lds_pitch = 0;
    int res_dist = 1;  // bands the tile's halo reaches on each side
    int reg_cw = 1, reg_rows = 0;
    size_t lds_bytes = 0;
    int xcd_remap = 0;
    int barrier_kind = PK_BARRIER_FLAT;
    int exchange = 0;  // tiles: PK_EXCHANGE_*; persistent STREAM: between passes; LAUNCH: 0
    int pass_sweeps = 1;
    int pband_rows = 1, pbands = 1;
    int march_down = 0;
    int pass_nbr_strips = 0, pass_nbr_dist = 0;  // STREAM passes under PK_EXCHANGE_NEIGHBOR
    int occ = 0;  // blocks per CU allowed by the occupancy query
};

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Stream geometry for a given grid: one unit (band x strip) per wave where the
// field is large enough, never less than `min_rows` rows per band.
void stream_geometry(Plan& p, int nx, int ny, int esize, int min_rows) {
    const int W = 16 / esize;
    p.strips = ceil_div(nx, 64 * W);
    const int interior = ny - 2;
    const int nw = p.grid * (p.threads / 64);
    int bands = std::max(1, nw / p.strips);
    // bands of at most min_rows rows where the waves allow (254 rows make 64 bands
    // of 4 rather than 51 of 5: the residual's march loads 4 rows a round)
    bands = std::min(bands, std::max(1, ceil_div(interior, std::max(1, min_rows))));
    p.band_rows = ceil_div(interior, bands);
    p.bands = ceil_div(interior, p.band_rows);
}

}  // namespace

struct pk_engine {
    int nx = 0, ny = 0, dtype = PK_F32, esize = 4, pitch = 0;
    size_t pitch_bytes = 0;
    int mode = PK_PERSISTENT;
    bool has_b = false;
    double h = 0.0;
    unsigned flags = 0;
    Plan plan;
    int cus = 0;
    int wclk_khz = 100000;  // device wall clock rate
    void* d_u[2] = {nullptr, nullptr};
    void* d_b = nullptr;
    pk_dev_state* d_st = nullptr;
    double* d_partials = nullptr;
    uint32_t* d_stamp = nullptr;
    uint32_t* d_nbr = nullptr;
    uint64_t* d_tag = nullptr;  // tagged halo words (PK_EXCHANGE_TAGGED only)
    unsigned char* d_trace = nullptr;  // PK_DBG_TRACE: grid x PK_TRACE_BLOCK_BYTES
    pk_mailbox* h_mail = nullptr;
    pk_mailbox* d_mail = nullptr;
    void* h_staging = nullptr;
    void* d_staging = nullptr;
    double* h_lres = nullptr;  // launch mode: residual results (pinned, mapped)
    double* d_lres = nullptr;
    hipStream_t stream = nullptr;
    bool own_stream = false;
    hipEvent_t ev_start = nullptr, ev_end = nullptr;
    hipEvent_t ev_ticket[PK_RING] = {};
    pk_kargs ka{};
    int state = RUNNING;
    bool launched = false;
    pkr::HostRing ring;
    // launch mode bookkeeping
    int cur = 0;
    int64_t sweeps_done = 0;
    int64_t launches = 0;
    double last_batch_ms = 0.0;
    std::vector<pk_result> lresults;  // by ticket
};

namespace {

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Opt-in diagnostics on stderr (environment variable PK_DEBUG set).
void debug_msg(const char* what, hipError_t e) {
    static const bool on = std::getenv("PK_DEBUG") != nullptr;
    if (on) std::fprintf(stderr, "pk: %s: %s\n", what, hipGetErrorString(e));
}

int map_err(hipError_t e) {
    if (e == hipSuccess) return PK_OK;
    if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) return PK_ENOMEM;
    return PK_EDEVICE;
}

void release(pk_engine* e) {
    if (!e) return;
    for (auto& ev : e->ev_ticket)
        if (ev) (void)hipEventDestroy(ev);
    if (e->ev_start) (void)hipEventDestroy(e->ev_start);
    if (e->ev_end) (void)hipEventDestroy(e->ev_end);
    if (e->d_u[0]) (void)hipFree(e->d_u[0]);
    if (e->d_u[1]) (void)hipFree(e->d_u[1]);
    if (e->d_b) (void)hipFree(e->d_b);
    if (e->d_st) (void)hipFree(e->d_st);
    if (e->d_partials) (void)hipFree(e->d_partials);
    if (e->d_stamp) (void)hipFree(e->d_stamp);
    if (e->d_nbr) (void)hipFree(e->d_nbr);
    if (e->d_tag) (void)hipFree(e->d_tag);
    if (e->d_trace) (void)hipFree(e->d_trace);
    if (e->h_mail) (void)hipHostFree(e->h_mail);
    if (e->h_staging) (void)hipHostFree(e->h_staging);
    if (e->h_lres) (void)hipHostFree(e->h_lres);
    if (e->own_stream && e->stream) (void)hipStreamDestroy(e->stream);
    delete e;
}

// ---------------------------------------------------------------------------
// Planning of the tile layouts (RESIDENT in LDS, REGISTER in VGPRs): one band of
// interior rows per block, bands of q or q+1 rows, halo depth m, tile height
// ext = band + 2m (the halo may reach past the adjacent bands, m > q: every
// block then publishes min(band, 2m) rows and reloads 2m).
// Estimated time per sweep = sub-sweep + exchange / m, with costs fitted to
// measured configurations on MI355X (one block of 16 waves per CU; 256^2 and
// 1024^2, block counts that are multiples of 8, halos up to 20 rows; rms error
// about 0.05 us per sweep). With A = band + m - 1, the rows of an average
// sub-sweep:
//   LDS sub-sweep: 0.31 us + 0.30 us per work item (a 64-lane row segment)
//     per wave;
//   exchange with the grid barrier:   2.48 us + 0.0105 us per block;
//   exchange with neighbour flags:    1.39 us + 0.0034 us per KB moved + 0.020 us per block
//     + 0.29 us per further band the halo reaches (one more pair of flags to poll;
//     every block also writes its XCD's L2 back on its own).
// The register tile, from 606 configurations (256^2 fp32 Poisson, 512^2 and
// 1024^2 Laplace; rms error 0.08 us per sweep), with r rows per wave:
//   sub-sweep: 0.36 us (+ 0.11 with several column strips) + 0.033 us per row
//     segment per SIMD (ceil(A / r) r x strips / 4: the waves go round the 4
//     SIMDs of the CU);
//   exchange with the grid barrier:   2.38 us + 0.019 us per KB moved + 0.0086 us per block;
//   exchange with neighbour flags:    0.91 us + 0.046 us per KB + 0.015 us per block
//     + 0.32 us per further band;
//   exchange with tagged words:       0.72 us + 0.048 us per KB of field rows moved
//     + 0.0028 us per block + 0.08 us per further band (the words are twice
//     the data, uncached).
// ---------------------------------------------------------------------------
struct TilePlan {
    int g = 0, q = 0, rem = 0, m = 0, ext = 0, rows = 0, cw = 1;
    int exchange = PK_EXCHANGE_BARRIER;
    size_t lds = 0;
    double cost = 1e30;
};

// dist: bands the halo reaches on each side (neighbour flags polled per side)
double exchange_estimate_us(int exchange, int g, double kb, int dist, bool register_tile) {
    if (register_tile) {
        if (exchange == PK_EXCHANGE_TAGGED) return 0.720 + 0.0479 * kb + 0.0028 * g + 0.081 * (dist - 1);
        if (exchange == PK_EXCHANGE_NEIGHBOR) return 0.913 + 0.0458 * kb + 0.0147 * g + 0.321 * (dist - 1);
        return 2.38 + 0.0189 * kb + 0.0086 * g;
    }
    return exchange == PK_EXCHANGE_NEIGHBOR ? 1.39 + 0.0034 * kb + 0.020 * g + 0.286 * (dist - 1)
                                            : 2.48 + 0.0105 * g;
}

constexpr int kRegRows = 4;  // rows per wave held in registers (PK_REG_RMAX)
constexpr int kMaxHalo = 64;  // deepest LDS-tile halo the planner considers
constexpr uint64_t kInfinityCacheBytes = 256ull << 20;  // the MI355X's last-level cache

// One candidate block count g for the LDS (register == false) or register tile.
// `exchanges` lists the exchange kinds to consider (LDS tile only).
TilePlan tile_candidate(int nx, int ny, int esize, bool has_b, int nwv, size_t lds_max, int g,
                        int want_m, bool register_tile, int exchanges) {
    TilePlan t;
    const int W = 16 / esize;
    const int interior = ny - 2;
    if (g < 1 || g > interior) return t;
    const int q = interior / g, rem = interior % g;
    const int band_max = q + (rem ? 1 : 0);
    const int nvec = (nx + W - 1) / W;
    const int lp = nvec * W;
    int m_hi = g == 1 ? (1 << 20) : kMaxHalo;
    if (want_m > 0) m_hi = std::min(m_hi, want_m);
    auto ext_of = [&](int m) { return g == 1 ? ny : std::min(ny, band_max + 2 * m); };
    t.g = g;
    t.q = q;
    t.rem = rem;
    // tile rows a block can hold, time per sub-sweep of `rows` rows on average
    int max_rows = 0;
    std::function<double(double, int)> sub_us;
    std::function<int(int)> reg_rows;
    if (register_tile) {
        // cw column groups of 64 lanes x rw row groups of waves, kRegRows rows each
        const int cw = (nvec + 63) / 64;
        if (cw > nwv) return TilePlan{};
        const int rw = nwv / cw;
        max_rows = rw * kRegRows;
        t.cw = cw;
        t.lds = static_cast<size_t>(2) * nwv * (2 * 64 * W + 2 * kRegRows) * esize;
        if (t.lds > lds_max) return TilePlan{};
        reg_rows = [rw](int ext) { return (ext + rw - 1) / rw <= 2 ? 2 : kRegRows; };
        // the waves go round the CU's 4 SIMDs, so the active row segments of a
        // sub-sweep spread over them; column groups add an edge exchange. The
        // cost grows with the rows updated, not in whole waves (measured after
        // the sub-sweep loop lost its per-row scalar work: 256^2 Poisson at 64
        // blocks, m = 12 beat 11, 13 and 14 in every scan, which bounds the
        // 2-row slope to 0.018 .. 0.038; 1024^2 at 256 blocks, m = 6 beat 5,
        // which rounding to whole 4-row waves had ranked the other way)
        sub_us = [cw](double rows, int r) {
            return 0.362 + (cw > 1 ? 0.109 : 0.0) + (r == 2 ? 0.025 : 0.0334) * rows * cw / 4.0;
        };
    } else {
        const size_t row_bytes = static_cast<size_t>(lp) * esize * (has_b ? 3 : 2);
        max_rows = static_cast<int>(lds_max / row_bytes);
        // work items per row: rows narrower than 64 vectors share a wave
        int sw = 1;
        while (sw < nvec && sw < 64) sw *= 2;
        const int rpi = 64 / sw;
        const int segs = (nvec + sw - 1) / sw;
        sub_us = [rpi, segs, nwv](double rows, int) {
            const double items = std::ceil(rows / rpi) * segs;
            return 0.311 + 0.295 * items / nwv;
        };
        t.lds = row_bytes;  // per tile row, scaled below
    }
    if (ext_of(1) > max_rows && !(g == 1 && ny <= max_rows)) return TilePlan{};
    if (g == 1) {
        if (ny > max_rows) return TilePlan{};
        t.m = 1 << 20;
        t.ext = ny;
        t.rows = register_tile ? reg_rows(ny) : 0;
        if (!register_tile) t.lds *= static_cast<size_t>(ny);
        t.cost = sub_us(interior, t.rows);
        return t;
    }
    // an explicit halo depth is taken as given (the deepest that fits, if less);
    // otherwise every depth is costed
    int m_lo = 1;
    if (want_m > 0) {
        int mf = std::min(m_hi, ny);
        while (mf > 1 && ext_of(mf) > max_rows) --mf;
        m_lo = mf;
    }
    for (int m = m_lo; m <= std::min(m_hi, ny); ++m) {
        if (ext_of(m) > max_rows) break;
        // bytes per exchange: min(band, 2m) rows published, 2m rows reloaded (the
        // fit used 2m + 2m, so count their mean twice)
        const double kb = (std::min(q, 2 * m) + 2.0 * m) * lp * esize / 1024.0;
        const int dist = (m + q - 1) / q;  // bands the halo reaches on each side
        const int r = register_tile ? reg_rows(ext_of(m)) : 0;
        for (int x = PK_EXCHANGE_BARRIER; x <= PK_EXCHANGE_TAGGED; ++x) {
            if (!(exchanges & (1 << x))) continue;
            const double c = sub_us(band_max + m - 1.0, r) + exchange_estimate_us(x, g, kb, dist, register_tile) / m;
            if (c < t.cost) {
                t.cost = c;
                t.m = m;
                t.exchange = x;
                t.rows = r;
            }
        }
    }
    if (t.m == 0) return TilePlan{};
    t.ext = ext_of(t.m);
    if (!register_tile) t.lds *= static_cast<size_t>(t.ext);
    return t;
}

// Best tile plan over block counts (or the given one).
TilePlan best_tile(int nx, int ny, int esize, bool has_b, int nwv, size_t lds_max, int cus,
                   int want_g, int want_m, bool register_tile, int exchanges) {
    TilePlan best;
    const int interior = ny - 2;
    const int lo = want_g > 0 ? want_g : 1;
    const int hi = want_g > 0 ? want_g : std::min(cus, interior);
    TilePlan single;
    for (int g = lo; g <= hi; ++g) {
        // from 8 blocks up, only multiples of 8: then consecutive bands sit on one
        // XCD (measured ~0.1 us per sweep faster than neighbouring counts)
        if (want_g <= 0 && g >= 8 && g % 8 != 0) continue;
        const TilePlan t = tile_candidate(nx, ny, esize, has_b, nwv, lds_max, g, want_m, register_tile,
                                          exchanges);
        if (t.g == 1) single = t;
        if (t.g && t.cost < best.cost) best = t;
    }
    // one block needs no synchronisation at all; the fit (made on multi-block
    // tiles) overrates its sub-sweeps: 64^2 measured 0.52 us with one block
    // against 0.58 with the seven the model preferred
    if (want_g <= 0 && single.g == 1 && single.cost <= 1.2 * best.cost) best = single;
    return best;
}

// Choose layout, block size and grid. Both modes share the result, so the
// launch-per-sweep baseline uses the same block count as the persistent kernel
// ("Persistent Kernels", "Sketching out the experiment").
int plan_engine(pk_engine* e, const pk_opts& o, const hipDeviceProp_t& prop) {
    Plan p;
    p.threads = o.threads ? o.threads : 1024;
    const int W = 16 / e->esize;
    const int interior = e->ny - 2;
    const size_t lds_max = prop.sharedMemPerBlock > 1024 ? prop.sharedMemPerBlock - 1024 : 0;
    const int nwv = p.threads / 64;

    bool tiled = false;
    if (e->mode == PK_PERSISTENT && o.layout != PK_LAYOUT_STREAM) {
        TilePlan reg, lds;
        // exchange kinds each tile may use (bit per PK_EXCHANGE_* value); tagged
        // words are the register tile's only
        const int exchanges = o.exchange != PK_EXCHANGE_AUTO ? (1 << o.exchange)
                              : (o.flags & PK_DBG_BROKEN_BARRIER) ? (1 << PK_EXCHANGE_BARRIER)
                              : ((1 << PK_EXCHANGE_BARRIER) | (1 << PK_EXCHANGE_NEIGHBOR) |
                                 (1 << PK_EXCHANGE_TAGGED));
        if (o.layout == PK_LAYOUT_AUTO || o.layout == PK_LAYOUT_REGISTER)
            reg = best_tile(e->nx, e->ny, e->esize, e->has_b, nwv, lds_max, e->cus, o.max_blocks,
                            o.halo_depth, true, exchanges);
        if ((o.layout == PK_LAYOUT_AUTO || o.layout == PK_LAYOUT_RESIDENT) &&
            (exchanges & ~(1 << PK_EXCHANGE_TAGGED)))
            lds = best_tile(e->nx, e->ny, e->esize, e->has_b, nwv, lds_max, e->cus, o.max_blocks,
                            o.halo_depth, false, exchanges & ~(1 << PK_EXCHANGE_TAGGED));
        // one block needs no synchronisation at all: the single-block LDS tile
        // keeps its 1.2x preference against the register tile too
        const bool use_reg = reg.g && (!lds.g || (lds.g == 1 ? reg.cost * 1.2 < lds.cost : reg.cost <= lds.cost));
        const TilePlan& t = use_reg ? reg : lds;
        if (t.g) {
            p.layout = use_reg ? PK_LAYOUT_REGISTER : PK_LAYOUT_RESIDENT;
            p.grid = t.g;
            p.res_q = t.q;
            p.res_rem = t.rem;
            p.res_halo = t.m;
            p.res_dist = (t.g == 1 || t.q < 1) ? 1 : (t.m + t.q - 1) / t.q;
            p.res_ext_rows = t.ext;
            p.reg_cw = t.cw;
            p.reg_rows = t.rows;
            p.lds_pitch = static_cast<int>(round_up(static_cast<size_t>(e->nx), W));
            p.lds_bytes = t.lds;
            p.exchange = t.exchange;
            tiled = true;
        } else if (o.layout == PK_LAYOUT_RESIDENT || o.layout == PK_LAYOUT_REGISTER) {
            return PK_EINVAL;  // asked for, but the bands do not fit
        }
    }
    if (!tiled) {
        if (o.exchange == PK_EXCHANGE_TAGGED) return PK_EINVAL;  // the register tile's only
        p.layout = PK_LAYOUT_STREAM;
        // the persistent streaming kernel's blocks are as large as its register
        // budget allows (its passes keep up to 12 levels of the march in registers)
        if (e->mode == PK_PERSISTENT) {
            hipFuncAttributes fa{};
            if (hipFuncGetAttributes(&fa, pkk_persistent_fn(e->dtype, e->has_b, PK_LAYOUT_STREAM, 0, false)) != hipSuccess)
                return PK_EDEVICE;
            p.threads = std::min(p.threads, fa.maxThreadsPerBlock / 64 * 64);
        }
        const int wpb = p.threads / 64;
        // enough blocks for one wave per unit of >= 4 rows, at most one block per CU
        const int strips = ceil_div(e->nx, 64 * W);
        const int units = strips * std::max(1, interior / 4);
        int g = std::min(e->cus, ceil_div(units, wpb));
        if (o.max_blocks > 0) g = o.max_blocks;  // an explicit grid, checked below
        p.grid = std::max(1, g);
    }
    p.xcd_remap = (p.grid >= 8 && p.grid % 8 == 0) ? 1 : 0;
    p.barrier_kind = o.barrier != PK_BARRIER_AUTO ? o.barrier
                     : (p.grid >= 16 && !(o.flags & PK_DBG_BROKEN_BARRIER) ? PK_BARRIER_XCD
                        : (p.grid >= 16 ? PK_BARRIER_TWO_LEVEL : PK_BARRIER_FLAT));
    stream_geometry(p, e->nx, e->ny, e->esize, 4);
    // passes of k sweeps (stream layout, persistent only): about one unit per
    // wave, bands at least 4 k rows tall (each band re-reads 2 k halo rows).
    // Default depth: a deeper pass reads and writes the field fewer times per
    // sweep but recomputes more overlap rows and columns, so it pays where the
    // pass is bound by memory traffic, i.e. where the arrays it streams (u, u'
    // and b) do not fit the 256 MiB Infinity Cache (8192^2 fp64 Poisson: 41.7 us
    // per sweep at 8, 31.9 at 12); where they fit, the pass is bound by vector
    // issue and 8 is fastest (4096^2 fp32: 4.54 us at 8, 5.28 at 12).
    p.pass_sweeps = 1;
    if (e->mode == PK_PERSISTENT && p.layout == PK_LAYOUT_STREAM) {
        const uint64_t streamed = static_cast<uint64_t>(e->pitch_bytes) * e->ny * (e->has_b ? 3 : 2);
        const bool hbm = streamed > kInfinityCacheBytes;
        p.pass_sweeps = o.pass_sweeps > 0 ? o.pass_sweeps : (hbm ? PK_MAX_PASS : PK_SHALLOW_PASS);
        // rows so long that a unit's window at that depth (2 (k + 1) halo rows and
        // at least one band row, addressed with 32-bit byte offsets) would pass
        // 4 GiB where the field itself is taller than that: the deepest depth
        // whose window fits (checked again below)
        const uint64_t fit = 0xFFFFFFFFull / e->pitch_bytes;
        if (o.pass_sweeps == 0 && static_cast<uint64_t>(e->ny) > fit) {
            while (p.pass_sweeps > 1 && fit < static_cast<uint64_t>(2 * (p.pass_sweeps + 1) + 1))
                p.pass_sweeps = p.pass_sweeps == PK_MAX_PASS ? PK_SHALLOW_PASS : p.pass_sweeps - 1;
        }
        // march direction: where the passes stream from HBM, every band but the
        // last marches down (8192^2 fp64 Poisson: 31.8 -> 30.9 us per sweep);
        // where the arrays sit in the Infinity Cache, neighbouring bands march in
        // opposite directions and meet on the halo rows they share, in L2
        // (4096^2: 4.15 against 4.18 us with all bands down)
        p.march_down = hbm ? 1 : 0;
        // how a task's passes meet: neighbour counters per XCD (auto from 16
        // blocks on; 4096^2 fp32: 4.10 against 4.24 us per sweep with a grid
        // barrier after every pass, 8192^2 fp64 Poisson: the same), else the
        // grid barrier (the negative control keeps the barrier it weakens)
        p.exchange = o.exchange == PK_EXCHANGE_NEIGHBOR || o.exchange == PK_EXCHANGE_BARRIER ? o.exchange
                     : (p.grid >= 16 && !(o.flags & PK_DBG_BROKEN_BARRIER) ? PK_EXCHANGE_NEIGHBOR
                                                                              : PK_EXCHANGE_BARRIER);
    }
    {
        const int k = p.pass_sweeps;
        const int ov = (k + W - 1) / W;
        const int strips_k = ceil_div(e->nx, (64 - 2 * ov) * W);
        const int nw = p.grid * (p.threads / 64);
        int bands = std::max(1, nw / strips_k);
        bands = std::min(bands, std::max(1, interior / (4 * k)));
        p.pband_rows = o.band_rows > 0 ? std::min(o.band_rows, interior) : ceil_div(interior, bands);
        // a pass addresses a unit's rows (band + 2L halo rows, L <= k + 1 levels:
        // a task's last pass also sums the residual, and never past the field's
        // own rows) through 32-bit byte offsets: where the field is taller than
        // 4 GiB of rows, shorter bands for very wide rows, and refuse what cannot fit
        const uint64_t lim = 0xFFFFFFFFull / e->pitch_bytes;
        if (static_cast<uint64_t>(e->ny) > lim) {
            if (lim < static_cast<uint64_t>(2 * (k + 1) + 1)) return PK_EINVAL;
            p.pband_rows = static_cast<int>(std::min<uint64_t>(p.pband_rows, lim - 2 * (k + 1)));
        }
        p.pbands = ceil_div(interior, p.pband_rows);
        // neighbour counters between two full-depth passes: the units of such a
        // pass and the bands its k-row halo reaches; beyond PK_PASS_NBR_DIST bands
        // (very short bands) the passes keep the grid barrier
        if (p.layout == PK_LAYOUT_STREAM && p.exchange == PK_EXCHANGE_NEIGHBOR) {
            const int dist = ceil_div(k, p.pband_rows);
            if (dist <= PK_PASS_NBR_DIST) {
                p.pass_nbr_strips = strips_k;
                p.pass_nbr_dist = dist;
            }
        }
    }

    // occupancy of the kernel that will be resident, at its LDS footprint
    const void* fn = e->mode == PK_PERSISTENT ? pkk_persistent_fn(e->dtype, e->has_b, p.layout, p.reg_rows, (e->flags & PK_DBG_TRACE) != 0)
                                              : pkk_sweep_fn(e->dtype, e->has_b);
    if (p.lds_bytes > 0)
        (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  static_cast<int>(p.lds_bytes));
    int occ = 0;
    const hipError_t oe = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, p.threads, p.lds_bytes);
    if (oe != hipSuccess) {
        debug_msg("occupancy query", oe);
        return PK_EDEVICE;
    }
    p.occ = occ;
    if (occ < 1 || (e->mode == PK_PERSISTENT && p.grid > occ * e->cus)) {
        if (std::getenv("PK_DEBUG"))
            std::fprintf(stderr, "pk: grid of %d blocks x %d threads (%zu B LDS) not co-resident: "
                         "%d per CU x %d CUs\n", p.grid, p.threads, p.lds_bytes, occ, e->cus);
        return PK_ELAUNCH;
    }
    e->plan = p;
    return PK_OK;
}

void fill_kargs(pk_engine* e) {
    pk_kargs& a = e->ka;
    const Plan& p = e->plan;
    a.u[0] = e->d_u[0];
    a.u[1] = e->d_u[1];
    a.b = e->d_b;
    a.nx = e->nx;
    a.ny = e->ny;
    a.pitch = e->pitch;
    a.cur0 = 0;
    a.strips = p.strips;
    a.bands = p.bands;
    a.band_rows = p.band_rows;
    a.res_q = p.res_q;
    a.res_rem = p.res_rem;
    a.reg_cw = p.reg_cw;
    a.reg_rows = p.reg_rows;
    a.res_halo = p.res_halo;
    a.res_dist = p.res_dist;
    a.res_ext_rows = p.res_ext_rows;
    a.lds_pitch = p.lds_pitch;
    a.layout = p.layout;
    a.grid = p.grid;
    a.xcd_remap = p.xcd_remap;
    a.barrier_kind = p.barrier_kind;
    a.pass_sweeps = p.pass_sweeps;
    a.pband_rows = p.pband_rows;
    a.march_down = p.march_down;
    a.pass_nbr_strips = p.pass_nbr_strips;
    a.pass_nbr_dist = p.pass_nbr_dist;
    a.pbands = p.pbands;
    a.flags = e->flags;
    a.st = e->d_st;
    a.mail = e->d_mail;
    a.partials = e->d_partials;
    a.staging = e->d_staging;
    a.stamp = e->d_stamp;
    a.nbr = e->d_nbr;
    a.exchange = p.exchange;
    a.tag = e->d_tag;
    a.tag_pitch = 4 * (e->pitch * e->esize / 16);
    a.trace = e->d_trace;
}

bool poll_exited(void* ctx) {
    auto* e = static_cast<pk_engine*>(ctx);
    return __atomic_load_n(&e->h_mail->exited, __ATOMIC_ACQUIRE) != 0;
}

}  // namespace

extern "C" {

void pk_opts_default(pk_opts* o) {
    if (!o) return;
    std::memset(o, 0, sizeof(*o));
    o->dtype = PK_F32;
    o->mode = PK_PERSISTENT;
    o->layout = PK_LAYOUT_AUTO;
}

const char* pk_strerror(int s) {
    switch (s) {
        case PK_OK: return "ok";
        case PK_EINVAL: return "invalid argument";
        case PK_ENOMEM: return "out of memory";
        case PK_ELAUNCH: return "launch failed or grid not co-resident";
        case PK_EDEVICE: return "device or runtime error";
        case PK_EBUSY: return "busy: ring full or tasks in flight";
        case PK_ESTATE: return "not valid in the engine's mode or state";
        case PK_ETIMEDOUT: return "timed out; engine poisoned";
        default: return "unknown status";
    }
}

int pk_create(int nx, int ny, const void* bc, const void* src, const pk_opts* opts,
              pk_engine** out) {
    if (!out || !bc || nx < 3 || ny < 3) return PK_EINVAL;
    pk_opts o;
    if (opts) o = *opts;
    else pk_opts_default(&o);
    if (o.dtype != PK_F32 && o.dtype != PK_F64) return PK_EINVAL;
    if (o.mode != PK_PERSISTENT && o.mode != PK_LAUNCH) return PK_EINVAL;
    if (o.layout < PK_LAYOUT_AUTO || o.layout > PK_LAYOUT_REGISTER) return PK_EINVAL;
    if (o.threads != 0 && (o.threads < 64 || o.threads > 1024 || o.threads % 64 != 0)) return PK_EINVAL;
    if (o.max_blocks < 0 || o.halo_depth < 0 || o.idle_timeout_s < 0) return PK_EINVAL;
    if (o.pass_sweeps < 0 || (o.pass_sweeps > 0 && !PK_PASS_DEPTH_OK(o.pass_sweeps)) || o.band_rows < 0)
        return PK_EINVAL;
    if (o.flags & ~(PK_DBG_BROKEN_BARRIER | PK_DBG_TRACE)) return PK_EINVAL;
    if ((o.flags & PK_DBG_TRACE) && o.mode != PK_PERSISTENT) return PK_EINVAL;
    if (o.barrier < PK_BARRIER_AUTO || o.barrier > PK_BARRIER_XCD) return PK_EINVAL;
    // the negative control relaxes the flat/two-level barriers; the XCD barrier keeps
    // separate counters, so the two are not combined
    if ((o.flags & PK_DBG_BROKEN_BARRIER) && o.barrier == PK_BARRIER_XCD) return PK_EINVAL;
    if (o.exchange < PK_EXCHANGE_AUTO || o.exchange > PK_EXCHANGE_TAGGED) return PK_EINVAL;
    // the negative control weakens the grid barrier only
    if ((o.flags & PK_DBG_BROKEN_BARRIER) && o.exchange >= PK_EXCHANGE_NEIGHBOR) return PK_EINVAL;
    // tagged words: the register tile only
    if (o.exchange == PK_EXCHANGE_TAGGED && o.layout != PK_LAYOUT_AUTO && o.layout != PK_LAYOUT_REGISTER)
        return PK_EINVAL;
    for (int r : o.reserved)
        if (r != 0) return PK_EINVAL;
    double h = o.h;
    if (h == 0.0) {
        if (nx != ny) return PK_EINVAL;
        h = 1.0 / (nx - 1);
    }
    if (!(h > 0.0)) return PK_EINVAL;
    const int esize = o.dtype == PK_F64 ? 8 : 4;
    if (static_cast<int64_t>(nx) * esize > (int64_t(1) << 30)) return PK_EINVAL;

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PK_EDEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return PK_EDEVICE;

    pk_engine* e = new (std::nothrow) pk_engine();
    if (!e) return PK_ENOMEM;
    e->nx = nx;
    e->ny = ny;
    e->dtype = o.dtype;
    e->esize = esize;
    e->mode = o.mode;
    e->has_b = src != nullptr;
    e->h = h;
    e->flags = o.flags;
    e->cus = prop.multiProcessorCount;
    e->pitch_bytes = round_up(static_cast<size_t>(nx) * esize, 256);
    e->pitch = static_cast<int>(e->pitch_bytes / esize);

    int rc = plan_engine(e, o, prop);
    if (rc != PK_OK) { release(e); return rc; }

    hipError_t he;
    const size_t fbytes = e->pitch_bytes * static_cast<size_t>(ny);
#define PK_TRY(expr)                                 \
    do {                                             \
        he = (expr);                                 \
        if (he != hipSuccess) {                      \
            rc = map_err(he);                        \
            release(e);                              \
            return rc;                               \
        }                                            \
    } while (0)

    if (o.stream) {
        e->stream = static_cast<hipStream_t>(o.stream);
    } else {
        PK_TRY(hipStreamCreateWithFlags(&e->stream, hipStreamNonBlocking));
        e->own_stream = true;
    }
    PK_TRY(hipMalloc(&e->d_u[0], fbytes));
    PK_TRY(hipMalloc(&e->d_u[1], fbytes));
    PK_TRY(hipMemsetAsync(e->d_u[0], 0, fbytes, e->stream));
    PK_TRY(hipMemsetAsync(e->d_u[1], 0, fbytes, e->stream));
    const size_t hrow = static_cast<size_t>(nx) * esize;
    PK_TRY(hipMemcpy2DAsync(e->d_u[0], e->pitch_bytes, bc, hrow, hrow, ny, hipMemcpyHostToDevice, e->stream));
    PK_TRY(hipMemcpy2DAsync(e->d_u[1], e->pitch_bytes, bc, hrow, hrow, ny, hipMemcpyHostToDevice, e->stream));
    if (src) {
        void* d_f = nullptr;
        PK_TRY(hipMalloc(&e->d_b, fbytes));
        PK_TRY(hipMalloc(&d_f, fbytes));
        he = hipMemsetAsync(d_f, 0, fbytes, e->stream);
        if (he == hipSuccess)
            he = hipMemcpy2DAsync(d_f, e->pitch_bytes, src, hrow, hrow, ny, hipMemcpyHostToDevice, e->stream);
        if (he == hipSuccess)
            he = pkk_launch_scale_source(e->dtype, d_f, e->d_b, nx, ny, e->pitch, h * h, e->stream);
        if (he == hipSuccess) he = hipStreamSynchronize(e->stream);
        (void)hipFree(d_f);
        if (he != hipSuccess) { rc = map_err(he); release(e); return rc; }
    }
    PK_TRY(hipMalloc(reinterpret_cast<void**>(&e->d_st), sizeof(pk_dev_state)));
    PK_TRY(hipMemsetAsync(e->d_st, 0, sizeof(pk_dev_state), e->stream));
    PK_TRY(hipMalloc(reinterpret_cast<void**>(&e->d_partials), sizeof(double) * 2 * e->plan.grid));
    PK_TRY(hipMalloc(reinterpret_cast<void**>(&e->d_stamp), sizeof(uint32_t) * 2 * 64 * e->plan.grid));
    PK_TRY(hipMemsetAsync(e->d_stamp, 0, sizeof(uint32_t) * 2 * 64 * e->plan.grid, e->stream));
    const size_t nbr_bytes = sizeof(uint32_t) * PK_NBR_WORDS * e->plan.grid;
    PK_TRY(hipMalloc(reinterpret_cast<void**>(&e->d_nbr), nbr_bytes));
    PK_TRY(hipMemsetAsync(e->d_nbr, 0, nbr_bytes, e->stream));
    if (e->plan.exchange == PK_EXCHANGE_TAGGED) {
        // two parities x ny rows x 4 words per 16-byte vector; tag 0 is never current
        const size_t tag_bytes = sizeof(uint64_t) * 2 * static_cast<size_t>(ny) * 4 * (e->pitch * e->esize / 16);
        PK_TRY(hipMalloc(reinterpret_cast<void**>(&e->d_tag), tag_bytes));
        PK_TRY(hipMemsetAsync(e->d_tag, 0, tag_bytes, e->stream));
    }
    if (e->flags & PK_DBG_TRACE) {
        const size_t tb = static_cast<size_t>(PK_TRACE_BLOCK_BYTES) * e->plan.grid;
        PK_TRY(hipMalloc(reinterpret_cast<void**>(&e->d_trace), tb));
        PK_TRY(hipMemsetAsync(e->d_trace, 0, tb, e->stream));
    }
    PK_TRY(hipHostMalloc(reinterpret_cast<void**>(&e->h_mail), sizeof(pk_mailbox),
                         hipHostMallocCoherent | hipHostMallocMapped));
    std::memset(e->h_mail, 0, sizeof(pk_mailbox));
    PK_TRY(hipHostGetDevicePointer(reinterpret_cast<void**>(&e->d_mail), e->h_mail, 0));
    PK_TRY(hipEventCreate(&e->ev_start));
    PK_TRY(hipEventCreate(&e->ev_end));
    if (e->mode == PK_PERSISTENT) {
        PK_TRY(hipHostMalloc(&e->h_staging, static_cast<size_t>(nx) * ny * esize,
                             hipHostMallocCoherent | hipHostMallocMapped));
        PK_TRY(hipHostGetDevicePointer(&e->d_staging, e->h_staging, 0));
    } else {
        PK_TRY(hipHostMalloc(reinterpret_cast<void**>(&e->h_lres), sizeof(double) * PK_RING,
                             hipHostMallocCoherent | hipHostMallocMapped));
        PK_TRY(hipHostGetDevicePointer(reinterpret_cast<void**>(&e->d_lres), e->h_lres, 0));
        for (auto& ev : e->ev_ticket) PK_TRY(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
    }
    fill_kargs(e);
    int wclk_khz = 0;
    if (hipDeviceGetAttribute(&wclk_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || wclk_khz <= 0)
        wclk_khz = 100000;
    e->wclk_khz = wclk_khz;
    const double idle_s = o.idle_timeout_s > 0 ? o.idle_timeout_s : 120.0;
    e->ka.idle_ticks = static_cast<uint64_t>(idle_s * wclk_khz * 1000.0);
    e->ka.spin_ticks = static_cast<uint64_t>((idle_s + 10.0) * wclk_khz * 1000.0);
    // a read of host memory over the bus takes ~1-2 us; compare a read-ahead
    // task slot only 2.5 us after issuing it
    e->ka.carry_age_ticks = static_cast<uint64_t>(2.5e-6 * wclk_khz * 1000.0);
    // a neighbour's halo words arrive within microseconds of each other's; 2 s
    // without them means a fault
    e->ka.tag_ticks = static_cast<uint64_t>(2.0 * wclk_khz * 1000.0);
    PK_TRY(hipStreamSynchronize(e->stream));
    e->ring.attach(e->h_mail);

    if (e->mode == PK_PERSISTENT) {
        const void* fn = pkk_persistent_fn(e->dtype, e->has_b, e->plan.layout, e->plan.reg_rows,
                                           (e->flags & PK_DBG_TRACE) != 0);
        void* args[] = {&e->ka};
        PK_TRY(hipEventRecord(e->ev_start, e->stream));
        he = hipLaunchCooperativeKernel(fn, dim3(e->plan.grid), dim3(e->plan.threads), args,
                                        static_cast<unsigned>(e->plan.lds_bytes), e->stream);
        if (he != hipSuccess) {
            debug_msg("cooperative launch", he);
            (void)hipStreamSynchronize(e->stream);
            release(e);
            return PK_ELAUNCH;
        }
        e->launched = true;
        e->launches = 1;
        (void)hipEventRecord(e->ev_end, e->stream);
    }
#undef PK_TRY
    *out = e;
    return PK_OK;
}

int pk_submit(pk_engine* e, pk_task t, uint64_t* ticket) {
    if (!e) return PK_EINVAL;
    if (e->state != RUNNING) return PK_ESTATE;
    const bool known = t.kind == PK_SWEEP || t.kind == PK_SWEEP_RB || t.kind == PK_RESIDUAL ||
                       t.kind == PK_EXIT || t.kind == PK_BARRIER || t.kind == PK_STAMP ||
                       t.kind == PK_BLOCKSYNC;
    if (!known || t.n < 0 || t.n > PK_TASK_N_MAX) return PK_EINVAL;
    // red-black runs 2n half-sweeps
    if (t.kind == PK_SWEEP_RB && t.n > PK_TASK_N_MAX / 2)
        return PK_EINVAL;
    if (e->mode == PK_LAUNCH) {
        if (t.kind == PK_BARRIER || t.kind == PK_STAMP || t.kind == PK_BLOCKSYNC) return PK_EINVAL;
        const uint64_t seq = e->lresults.size() + 1;
        hipEvent_t& ev = e->ev_ticket[seq % PK_RING];
        if (seq > PK_RING) {  // the slot's previous ticket must be finished
            const hipError_t q = hipEventQuery(ev);
            if (q == hipErrorNotReady) return PK_EBUSY;
            if (q != hipSuccess) return PK_EDEVICE;
            pk_result& old = e->lresults[seq - PK_RING - 1];
            if (old.kind == PK_RESIDUAL) old.residual = e->h_lres[(seq - PK_RING) % PK_RING];
        }
        pk_result r{};
        r.kind = t.kind;
        hipError_t he = hipSuccess;
        if (t.kind == PK_SWEEP || t.kind == PK_SWEEP_RB) {
            // red-black: one launch per half-sweep, red (parity 0) first
            const int launches = t.kind == PK_SWEEP_RB ? 2 * t.n : t.n;
            for (int s = 0; s < launches && he == hipSuccess; ++s) {
                he = pkk_launch_sweep(e->dtype, e->has_b, e->ka, e->plan.threads, e->cur,
                                      t.kind == PK_SWEEP_RB ? (s & 1) : -1, e->stream);
                e->cur ^= 1;
                ++e->launches;
            }
            e->sweeps_done += t.n;
        } else if (t.kind == PK_RESIDUAL) {
            he = pkk_launch_residual(e->dtype, e->has_b, e->ka, e->plan.threads, e->cur,
                                     e->d_lres + seq % PK_RING, e->stream);
            e->launches += 2;
        } else if (t.kind == PK_EXIT) {
            e->state = EXITED;
        }
        if (he == hipSuccess) he = hipEventRecord(ev, e->stream);
        if (he != hipSuccess) { e->state = POISONED; return PK_EDEVICE; }
        r.sweeps_done = e->sweeps_done;
        e->lresults.push_back(r);
        if (ticket) *ticket = seq;
        return PK_OK;
    }
    if (__atomic_load_n(&e->h_mail->exited, __ATOMIC_ACQUIRE)) {
        e->state = EXITED;  // the kernel left by itself (idle timeout or fault)
        return PK_ESTATE;
    }
    uint64_t seq = 0;
    const int rc = e->ring.publish(t.kind, t.n, &seq);
    if (rc != PK_OK) return rc;
    if (t.kind == PK_EXIT) e->state = EXITED;
    if (ticket) *ticket = seq;
    return PK_OK;
}

int pk_submit_until(pk_engine* e, int max_sweeps, int check_every, double tol, uint64_t* ticket) {
    if (!e) return PK_EINVAL;
    if (e->state != RUNNING) return PK_ESTATE;
    if (max_sweeps < 0 || max_sweeps > PK_TASK_N_MAX || check_every < 1 || !(tol >= 0.0)) return PK_EINVAL;
    if (e->mode == PK_LAUNCH) {
        // the same loop on the host; every check waits for the GPU
        if (hipStreamSynchronize(e->stream) != hipSuccess) { e->state = POISONED; return PK_EDEVICE; }
        const uint64_t seq = e->lresults.size() + 1;
        if (seq > PK_RING) {  // the event and residual slot of an older ticket are reused
            pk_result& old = e->lresults[seq - PK_RING - 1];
            if (old.kind == PK_RESIDUAL) old.residual = e->h_lres[(seq - PK_RING) % PK_RING];
        }
        double* slot = e->d_lres + seq % PK_RING;
        auto residual = [&](double* out) -> hipError_t {
            hipError_t he = pkk_launch_residual(e->dtype, e->has_b, e->ka, e->plan.threads, e->cur, slot,
                                                e->stream);
            e->launches += 2;
            if (he == hipSuccess) he = hipStreamSynchronize(e->stream);
            if (he == hipSuccess) *out = e->h_lres[seq % PK_RING];
            return he;
        };
        double rres = 0.0;
        int done = 0;
        hipError_t he = residual(&rres);
        while (he == hipSuccess && !(rres <= tol) && done < max_sweeps) {
            const int k = std::min(check_every, max_sweeps - done);
            for (int s = 0; s < k && he == hipSuccess; ++s) {
                he = pkk_launch_sweep(e->dtype, e->has_b, e->ka, e->plan.threads, e->cur, -1, e->stream);
                e->cur ^= 1;
                ++e->launches;
            }
            done += k;
            if (he == hipSuccess) he = residual(&rres);
        }
        if (he == hipSuccess) he = hipEventRecord(e->ev_ticket[seq % PK_RING], e->stream);
        if (he != hipSuccess) { e->state = POISONED; return PK_EDEVICE; }
        e->sweeps_done += done;
        pk_result r{};
        r.kind = PK_SWEEP_UNTIL;
        r.residual = rres;
        r.sweeps_done = e->sweeps_done;
        e->lresults.push_back(r);
        if (ticket) *ticket = seq;
        return PK_OK;
    }
    if (__atomic_load_n(&e->h_mail->exited, __ATOMIC_ACQUIRE)) {
        e->state = EXITED;
        return PK_ESTATE;
    }
    pk_param prm{};
    prm.tol = tol;
    prm.every = check_every;
    uint64_t seq = 0;
    const int rc = e->ring.publish(PK_SWEEP_UNTIL, max_sweeps, &seq, &prm);
    if (rc != PK_OK) return rc;
    if (ticket) *ticket = seq;
    return PK_OK;
}

int pk_wait(pk_engine* e, uint64_t ticket, double timeout_s, pk_result* r) {
    if (!e) return PK_EINVAL;
    if (e->state == POISONED) return PK_ESTATE;
    if (timeout_s <= 0) timeout_s = 60.0;
    if (e->mode == PK_LAUNCH) {
        if (ticket == 0 || ticket > e->lresults.size()) return PK_EINVAL;
        const uint64_t latest = e->lresults.size();
        // events are reused every PK_RING tickets; a later ticket done implies this one
        const auto t0 = std::chrono::steady_clock::now();
        if (latest - ticket < PK_RING) {
            hipEvent_t ev = e->ev_ticket[ticket % PK_RING];
            for (;;) {
                const hipError_t q = hipEventQuery(ev);
                if (q == hipSuccess) break;
                if (q != hipErrorNotReady) { e->state = POISONED; return PK_EDEVICE; }
                const double el = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
                if (el > timeout_s) { e->state = POISONED; return PK_ETIMEDOUT; }
            }
            pk_result& res = e->lresults[ticket - 1];
            if (res.kind == PK_RESIDUAL) res.residual = e->h_lres[ticket % PK_RING];
        }
        if (r) *r = e->lresults[ticket - 1];
        return PK_OK;
    }
    pkr::DoneInfo d{};
    const int rc = e->ring.wait(ticket, timeout_s, &d, poll_exited, e);
    if (rc == PK_ETIMEDOUT) e->state = POISONED;
    if (rc != PK_OK) return rc;
    if (r) {
        r->residual = d.residual;
        r->sweeps_done = d.sweeps_done;
        r->errors = d.errors;
        r->kind = d.kind;
        r->status = d.status;
        r->device_us = d.t_end >= d.t_begin ? (d.t_end - d.t_begin) * 1000.0 / e->wclk_khz : 0.0;
    }
    return d.status == PK_OK ? PK_OK : d.status;
}

int pk_readback(pk_engine* e, void* dst, size_t bytes) {
    if (!e || !dst) return PK_EINVAL;
    if (e->state == POISONED) return PK_ESTATE;
    const size_t need = static_cast<size_t>(e->nx) * e->ny * e->esize;
    if (bytes < need) return PK_EINVAL;
    const size_t hrow = static_cast<size_t>(e->nx) * e->esize;
    const bool gone = e->mode == PK_PERSISTENT && __atomic_load_n(&e->h_mail->exited, __ATOMIC_ACQUIRE);
    if (e->mode == PK_PERSISTENT && e->state == RUNNING && !gone) {
        if (e->ring.in_flight() != 0) return PK_EBUSY;
        uint64_t seq = 0;
        int rc = e->ring.publish(PK_TASK_READBACK, 0, &seq);
        if (rc != PK_OK) return rc;
        pkr::DoneInfo d{};
        rc = e->ring.wait(seq, 120.0, &d, poll_exited, e);
        if (rc == PK_ETIMEDOUT) e->state = POISONED;
        if (rc != PK_OK) return rc;
        if (d.status != PK_OK) return d.status;
        std::memcpy(dst, e->h_staging, need);
        return PK_OK;
    }
    int cur = e->cur;
    if (e->mode == PK_PERSISTENT) {
        // the kernel has left: wait for it to drain, then an ordinary copy is safe;
        // the field is in the buffer the last completed task reported
        if (hipEventSynchronize(e->ev_end) != hipSuccess) return PK_EDEVICE;
        e->ring.harvest();
        cur = e->ring.last_cur();
    }
    hipError_t he = hipMemcpy2DAsync(dst, hrow, e->d_u[cur], e->pitch_bytes, hrow, e->ny,
                                      hipMemcpyDeviceToHost, e->stream);
    if (he == hipSuccess) he = hipStreamSynchronize(e->stream);
    return map_err(he);
}

int pk_run_launch_per_iter(pk_engine* e, int n, int sync_each, double* elapsed_us) {
    if (!e || n < 0) return PK_EINVAL;
    if (e->mode != PK_LAUNCH) return PK_ESTATE;
    if (e->state != RUNNING) return PK_ESTATE;
    if (hipStreamSynchronize(e->stream) != hipSuccess) return PK_EDEVICE;
    hipError_t he = hipEventRecord(e->ev_start, e->stream);
    const auto t0 = std::chrono::steady_clock::now();
    for (int s = 0; s < n && he == hipSuccess; ++s) {
        he = pkk_launch_sweep(e->dtype, e->has_b, e->ka, e->plan.threads, e->cur, -1, e->stream);
        e->cur ^= 1;
        ++e->launches;
        if (he == hipSuccess && sync_each) he = hipStreamSynchronize(e->stream);
    }
    if (he == hipSuccess) he = hipEventRecord(e->ev_end, e->stream);
    if (he == hipSuccess) he = hipStreamSynchronize(e->stream);
    const auto t1 = std::chrono::steady_clock::now();
    if (he != hipSuccess) { e->state = POISONED; return PK_EDEVICE; }
    e->sweeps_done += n;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, e->ev_start, e->ev_end) == hipSuccess) e->last_batch_ms = ms;
    if (elapsed_us) *elapsed_us = std::chrono::duration<double, std::micro>(t1 - t0).count();
    return PK_OK;
}

int pk_run_graph_per_iter(pk_engine* e, int n, int reps, double* elapsed_us) {
    if (!e || n < 1 || reps < 1) return PK_EINVAL;
    if (e->mode != PK_LAUNCH || e->state != RUNNING) return PK_ESTATE;
    if (hipStreamSynchronize(e->stream) != hipSuccess) return PK_EDEVICE;
    // a graph of n sweeps reads u[c] and leaves the field in u[c ^ (n & 1)]:
    // with n odd the replays alternate between the two starting buffers
    const int variants = (n & 1) ? 2 : 1;
    hipGraphExec_t exec[2] = {nullptr, nullptr};
    hipError_t he = hipSuccess;
    for (int v = 0; v < variants && he == hipSuccess; ++v) {
        hipGraph_t graph = nullptr;
        he = hipStreamBeginCapture(e->stream, hipStreamCaptureModeThreadLocal);
        const int c0 = e->cur ^ v;
        for (int s = 0; s < n && he == hipSuccess; ++s)
            he = pkk_launch_sweep(e->dtype, e->has_b, e->ka, e->plan.threads, c0 ^ (s & 1), -1, e->stream);
        const hipError_t ce = hipStreamEndCapture(e->stream, &graph);
        if (he == hipSuccess) he = ce;
        if (he == hipSuccess) he = hipGraphInstantiate(&exec[v], graph, nullptr, nullptr, 0);
        if (graph) (void)hipGraphDestroy(graph);
    }
    double us = 0.0;
    if (he == hipSuccess) {
        he = hipEventRecord(e->ev_start, e->stream);
        const auto t0 = std::chrono::steady_clock::now();
        for (int r = 0; r < reps && he == hipSuccess; ++r) he = hipGraphLaunch(exec[variants == 2 ? (r & 1) : 0], e->stream);
        if (he == hipSuccess) he = hipEventRecord(e->ev_end, e->stream);
        if (he == hipSuccess) he = hipStreamSynchronize(e->stream);
        us = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
    }
    for (auto& x : exec)
        if (x) (void)hipGraphExecDestroy(x);
    if (he != hipSuccess) {
        debug_msg("graph baseline", he);
        e->state = POISONED;
        return PK_EDEVICE;
    }
    const int64_t total = static_cast<int64_t>(n) * reps;
    if (total & 1) e->cur ^= 1;
    e->sweeps_done += total;
    e->launches += total;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, e->ev_start, e->ev_end) == hipSuccess) e->last_batch_ms = ms;
    if (elapsed_us) *elapsed_us = us;
    return PK_OK;
}

int pk_sweep_noalloc(int dtype, int nx, int ny, int pitch, void* u0, void* u1, const void* b, int n,
                     double* residual, void* stream) {
    if (dtype != PK_F32 && dtype != PK_F64) return PK_EINVAL;
    const int esize = dtype == PK_F64 ? 8 : 4;
    const int W = 16 / esize;
    if (nx < 3 || ny < 3 || n < 0 || !u0 || !u1 || u0 == u1) return PK_EINVAL;
    // rows are read and written as whole 16-byte vectors
    if (pitch < (nx + W - 1) / W * W || (static_cast<int64_t>(pitch) * esize) % 16 != 0) return PK_EINVAL;
    if (static_cast<int64_t>(nx) * esize > (int64_t(1) << 30)) return PK_EINVAL;
    if ((reinterpret_cast<uintptr_t>(u0) | reinterpret_cast<uintptr_t>(u1) | reinterpret_cast<uintptr_t>(b)) % 16)
        return PK_EINVAL;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PK_EDEVICE;
    double* part = nullptr;
    if (pkk_noalloc_scratch(dev, &part) != hipSuccess) return PK_EDEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return PK_EDEVICE;
    // the plan of a PK_LAUNCH engine with default options (same grid, same
    // geometry, so the same results bit for bit); nothing here allocates
    pk_engine e;
    e.nx = nx;
    e.ny = ny;
    e.dtype = dtype;
    e.esize = esize;
    e.mode = PK_LAUNCH;
    e.has_b = b != nullptr;
    e.cus = prop.multiProcessorCount;
    e.pitch = pitch;
    e.pitch_bytes = static_cast<size_t>(pitch) * esize;
    pk_opts o;
    pk_opts_default(&o);
    o.dtype = dtype;
    o.mode = PK_LAUNCH;
    const int rc = plan_engine(&e, o, prop);
    if (rc != PK_OK) return rc;
    if (e.plan.grid > PK_NOALLOC_MAX_BLOCKS) return PK_EINVAL;  // more partials than the scratch holds
    pk_kargs a{};
    a.u[0] = u0;
    a.u[1] = u1;
    a.b = b;
    a.nx = nx;
    a.ny = ny;
    a.pitch = pitch;
    a.strips = e.plan.strips;
    a.bands = e.plan.bands;
    a.band_rows = e.plan.band_rows;
    a.grid = e.plan.grid;
    a.xcd_remap = e.plan.xcd_remap;
    a.pass_sweeps = 1;
    a.partials = part;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t he = hipSuccess;
    int cur = 0;
    for (int k = 0; k < n && he == hipSuccess; ++k, cur ^= 1)
        he = pkk_launch_sweep(dtype, e.has_b, a, e.plan.threads, cur, -1, st);
    if (he == hipSuccess && residual)
        he = pkk_launch_residual(dtype, e.has_b, a, e.plan.threads, cur, residual, st);
    if (he != hipSuccess) {
        debug_msg("pk_sweep_noalloc", he);
        return PK_EDEVICE;
    }
    return PK_OK;
}

int pk_get_info(pk_engine* e, pk_info* info) {
    if (!e || !info) return PK_EINVAL;
    std::memset(info, 0, sizeof(*info));
    info->nx = e->nx;
    info->ny = e->ny;
    info->dtype = e->dtype;
    info->mode = e->mode;
    info->layout = e->plan.layout;
    info->pitch = e->pitch;
    info->grid_blocks = e->plan.grid;
    info->threads = e->plan.threads;
    info->blocks_per_cu_max = e->plan.occ;
    info->cus = e->cus;
    const bool tiled = e->plan.layout == PK_LAYOUT_RESIDENT || e->plan.layout == PK_LAYOUT_REGISTER;
    info->halo_depth = tiled ? e->plan.res_halo : 0;
    info->band_rows = tiled ? e->plan.res_q + (e->plan.res_rem ? 1 : 0)
                      : (e->plan.pass_sweeps > 1 ? e->plan.pband_rows : e->plan.band_rows);
    info->strips = e->plan.strips;
    info->lds_bytes = e->plan.lds_bytes;
    info->barrier = e->plan.barrier_kind;
    info->pass_sweeps = e->plan.pass_sweeps;
    info->exchange = e->plan.exchange;
    info->kernel_launches = e->launches;
    info->wall_clock_khz = e->wclk_khz;
    info->trace_capacity = e->d_trace ? PK_TRACE_CAP : 0;
    if (e->mode == PK_PERSISTENT) {
        info->sweeps_done = e->ring.sweeps_seen();
        info->tasks_done = static_cast<int64_t>(e->ring.done_seen());
        info->tasks_carried = static_cast<int64_t>(e->ring.carried_seen());
        info->tasks_fused = static_cast<int64_t>(e->ring.fused_seen());
        // once the kernel has said it is leaving, its end event completes promptly
        if (__atomic_load_n(&e->h_mail->exited, __ATOMIC_ACQUIRE) &&
            hipEventSynchronize(e->ev_end) == hipSuccess) {
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, e->ev_start, e->ev_end) == hipSuccess) info->kernel_ms = ms;
        }
    } else {
        info->sweeps_done = e->sweeps_done;
        info->tasks_done = static_cast<int64_t>(e->lresults.size());
        info->kernel_ms = e->last_batch_ms;
    }
    return PK_OK;
}

int pk_trace_read(pk_engine* e, void* dst, size_t bytes, size_t* needed) {
    if (!e) return PK_EINVAL;
    if (!e->d_trace) return PK_ESTATE;
    const size_t need = static_cast<size_t>(PK_TRACE_BLOCK_BYTES) * e->plan.grid;
    if (needed) *needed = need;
    if (!dst) return PK_OK;
    if (bytes < need) return PK_EINVAL;
    if (!__atomic_load_n(&e->h_mail->exited, __ATOMIC_ACQUIRE)) return PK_EBUSY;
    if (hipEventSynchronize(e->ev_end) != hipSuccess) return PK_EDEVICE;  // the kernel has drained
    hipError_t he = hipMemcpyAsync(dst, e->d_trace, need, hipMemcpyDeviceToHost, e->stream);
    if (he == hipSuccess) he = hipStreamSynchronize(e->stream);
    return map_err(he);
}

int pk_destroy(pk_engine* e) {
    if (!e) return PK_OK;
    if (e->mode == PK_PERSISTENT && e->launched) {
        const bool exited = __atomic_load_n(&e->h_mail->exited, __ATOMIC_ACQUIRE) != 0;
        if (!exited) {
            if (e->state == RUNNING) {
                uint64_t seq = 0;
                // make room, then ask the kernel to leave
                int rc = e->ring.publish(PK_EXIT, 0, &seq);
                const auto t0 = std::chrono::steady_clock::now();
                while (rc == PK_EBUSY) {
                    e->ring.harvest();
                    rc = e->ring.publish(PK_EXIT, 0, &seq);
                    if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(30)) break;
                }
                e->state = EXITED;
            }
            const auto t0 = std::chrono::steady_clock::now();
            while (__atomic_load_n(&e->h_mail->exited, __ATOMIC_ACQUIRE) == 0) {
                if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(30)) {
                    // the kernel may still run: leak its memory rather than free it
                    return PK_ETIMEDOUT;
                }
            }
        }
        (void)hipEventSynchronize(e->ev_end);
    } else if (e->mode == PK_LAUNCH) {
        (void)hipStreamSynchronize(e->stream);
    }
    release(e);
    return PK_OK;
}

}  // extern "C"
