// Memory layouts shared by the host runtime and the device kernels.
//
// Host<->device mailbox (fine-grained, coherent pinned host memory, mapped on
// the device). The host publishes a task as one 64-bit slot word (sequence
// number, kind and count together, one atomic store); one device thread
// (block 0, lane 0) polls the next slot's word, so a single read over the bus
// both notices the task and delivers it. The device answers by filling
// `done[seq % PK_RING]` and then moving `done_seq`. Every
// word that one side polls sits on its own 128-byte line, so the writer of one
// flag never invalidates the line of another (the first page's flag-padding
// point, "Reflections and next steps").
#pragma once

#include <stdint.h>

#define PK_RING 64u
// Streaming pass depths (sweeps per pass) the kernel carries: 1..8 and 12.
// Passes that also sum the residual, and red-black passes, are at most
// PK_SHALLOW_PASS deep.
#define PK_MAX_PASS 12
#define PK_SHALLOW_PASS 8
#define PK_PASS_DEPTH_OK(k) ((k) >= 1 && ((k) <= PK_SHALLOW_PASS || (k) == PK_MAX_PASS))
#define PK_LINE 128

// Internal task kinds (the public ones are in pk.h); kinds fit in 4 bits.
#define PK_TASK_READBACK 15

// Device trace (PK_DBG_TRACE): thread 0 of every block appends events to a
// ring of PK_TRACE_CAP records of its own; the count of events ever written
// (which may exceed the capacity: the ring then holds the latest) precedes them.
#define PK_TRACE_CAP 8192
enum PkTraceKind : uint32_t {
    PK_TR_TASK_BEGIN = 1,   // aux = task kind
    PK_TR_TASK_END = 2,     // aux = task kind
    PK_TR_SYNC_ARRIVE = 3,  // a grid barrier (aux 0) or neighbour sync (aux 1): the block's work is done
    PK_TR_SYNC_LEAVE = 4,   // every block it waits for has arrived
    PK_TR_TAG_WAIT = 5,     // wave 0 starts polling its tagged halo words
    PK_TR_TAG_DONE = 6,     // they all carry the current exchange number
    PK_TR_PERIOD = 7,       // a tile period (up to halo_depth sub-sweeps) starts; aux = its sweeps
};
struct pk_trace_rec {
    uint64_t t;  // device wall clock
    uint32_t kind;
    uint32_t aux;
};
// bytes of one block's trace: its event count, then its ring
#define PK_TRACE_BLOCK_BYTES (8u + PK_TRACE_CAP * 16u)

// Device fault codes (pk_dev_state::fault).
#define PK_FAULT_BARRIER_TIMEOUT 1u
#define PK_FAULT_IDLE_TIMEOUT 2u

// Slot word: bits 63..32 the low half of the sequence number, 31..28 the
// kind, 27..0 the count (PK_TASK_N_MAX, from pk.h, is the largest count).
#ifndef PK_TASK_N_MAX
#define PK_TASK_N_MAX 0x0FFFFFFF
#endif

struct alignas(PK_LINE) pk_slot {
    uint64_t word;
};

static inline uint64_t pk_slot_pack(uint64_t seq, int kind, int n) {
    return ((seq & 0xFFFFFFFFull) << 32) | (static_cast<uint64_t>(kind & 0xF) << 28) |
           static_cast<uint64_t>(n & PK_TASK_N_MAX);
}
static inline uint32_t pk_slot_seq(uint64_t w) { return static_cast<uint32_t>(w >> 32); }
static inline int pk_slot_kind(uint64_t w) { return static_cast<int>((w >> 28) & 0xF); }
static inline int pk_slot_n(uint64_t w) { return static_cast<int>(w & PK_TASK_N_MAX); }

struct alignas(PK_LINE) pk_done_rec {
    uint64_t seq;
    int32_t kind;
    int32_t status;
    double residual;
    int64_t sweeps_done;
    uint64_t t_begin;  // device wall clock ticks
    uint64_t t_end;
    int64_t errors;
    int32_t cur;  // buffer index that holds the whole field after this task (after
                  // its last pass, where that pass ran on into a later task)
    int32_t carried;  // bit 0: the task was handed on by the previous task's barrier;
                      // bit 1: it ran sweeps of a later SWEEP task (fused)
};

// Parameters of a PK_SWEEP_UNTIL task, written by the host before it releases
// the task's slot word.
struct alignas(PK_LINE) pk_param {
    double tol;
    int32_t every;
    int32_t pad;
};

struct pk_mailbox {
    alignas(PK_LINE) uint64_t done_seq;  // device writes: last completed seq
    alignas(PK_LINE) uint32_t exited;    // device writes 1 when the kernel leaves
    alignas(PK_LINE) uint32_t fault;     // device writes a PK_FAULT_* code
    pk_slot slot[PK_RING];
    pk_param param[PK_RING];
    pk_done_rec done[PK_RING];
};

// Device-memory state of one engine; zeroed once before the kernel starts.
// The barrier's two words live on separate lines: arrivals hammer `count`
// while waiters poll `gen`.
struct alignas(256) pk_word256 {
    uint32_t v;
};

// A task handed on by the leader inside the previous task's barrier, so the
// next task needs no broadcast barrier of its own; indexed by seq & 1.
struct alignas(PK_LINE) pk_carry {
    uint64_t seq;
    int32_t kind;
    int32_t n;
};

struct pk_dev_state {
    // The words every task touches come first, within the 4 KiB that a global
    // instruction reaches from a scalar base with its immediate offset: no
    // per-word 64-bit address has to be kept in vector registers.
    alignas(PK_LINE) uint64_t task_seq;    // task broadcast (written by the leader)
    int32_t task_kind;
    int32_t task_n;
    pk_carry carry[2];
    alignas(PK_LINE) uint32_t fault;       // device-side fault, read by every block
    alignas(PK_LINE) uint64_t stamp_errors;
    alignas(PK_LINE) uint32_t bar_count;   // arrivals, monotonically increasing
    alignas(PK_LINE) uint32_t bar_gen;     // completed barrier generations
    alignas(256) uint32_t top_count;
    alignas(256) uint32_t xtop_count;
    alignas(256) uint32_t xtop_gen;
    // two-level barrier: one arrival counter and one generation word per XCD
    // group (block b belongs to group b mod 8), and the top-level counter above
    pk_word256 grp_count[8];
    pk_word256 grp_gen[8];
    // XCD barrier: groups are the XCDs the blocks actually run on (hardware
    // XCC id), with one L2 write-back and one L2 invalidate per XCD, and the
    // top-level counter and generation above
    pk_word256 xmembers[8];
    pk_word256 xgrp_count[8];
    pk_word256 xgrp_gen[8];
    // streaming passes under neighbour counters: arrivals per XCD, and the passes
    // whose stores the XCD has written back
    pk_word256 xpass_count[8];
    pk_word256 xpass_gen[8];
    // a streaming SWEEP task whose last pass runs on into the SWEEP task two
    // slots later, summing the RESIDUAL task between them inside that pass: the
    // leader's decision (the task's sequence, 0 for none), published through the
    // grid barrier before that pass
    alignas(PK_LINE) uint64_t fuse_seq;
};

// Kernel arguments (passed by value).
// Words per neighbour-exchange flag: one 128-byte line per block, so a
// block's store does not touch the line its neighbours poll. (Word 1 holds the
// block's XCD when the streaming passes use neighbour counters.)
#define PK_NBR_WORDS 32
// Streaming passes synchronised by neighbour counters: bands a pass's halo may
// reach on each side (the 3 (2 d + 1) neighbouring blocks are looked up at launch
// by the 64 lanes of one wave); deeper reaches (bands shorter than a tenth of the
// pass depth) keep the grid barrier.
#define PK_PASS_NBR_DIST 10

struct pk_kargs {
    void* u[2];            // the two field buffers (ny rows x pitch elements)
    const void* b;         // scaled source h*h*f (pitched), or null for Laplace
    int nx, ny, pitch;     // pitch in elements
    int cur0;              // buffer index holding the field at launch
    // stream geometry: unit = (band, strip); strip = 64 lanes x vector width
    int strips, bands, band_rows;
    // passes of several sweeps: rows per band and bands (strips depend on k)
    int pass_sweeps;       // sweeps per pass in the stream layout (1 = a pass per sweep)
    int pband_rows, pbands;
    int march_down;        // passes: every band but the last marches down (else directions alternate)
    int pass_nbr_strips;   // passes synchronised by neighbour counters: strips of a full-depth pass
    int pass_nbr_dist;     // and the bands its halo reaches on each side (0: grid barrier after every pass)
    // resident and register geometry: one band per block, the interior split
    // into bands of res_q or res_q + 1 rows (the first res_rem bands are longer)
    int res_q, res_rem;
    int reg_cw, reg_rows;  // register layout: column waves, rows per wave
    int res_halo;          // sweeps per halo exchange
    int res_dist;          // bands a halo reaches on each side: ceil(halo / shortest band)
    int res_ext_rows;      // LDS rows per buffer
    int lds_pitch;         // LDS row stride in elements
    int layout;            // PK_LAYOUT_STREAM or PK_LAYOUT_RESIDENT
    int grid;              // blocks in the grid
    int xcd_remap;         // 1: map consecutive logical blocks onto one XCD
    int barrier_kind;      // PK_BARRIER_FLAT or PK_BARRIER_TWO_LEVEL
    uint32_t flags;
    uint64_t idle_ticks;   // wall-clock ticks without a task before leaving
    uint64_t spin_ticks;   // wall-clock ticks a barrier may wait before faulting
    uint64_t carry_age_ticks;  // wall-clock ticks after which a read-ahead task slot has arrived
    pk_dev_state* st;
    pk_mailbox* mail;      // device-visible address of the host mailbox
    double* partials;      // residual partials: 2 x grid doubles (alternating rounds)
    void* staging;         // readback target (pinned host, device-visible)
    uint32_t* stamp;       // 2 x grid x 64 words for the visibility check
    uint32_t* nbr;         // neighbour exchange flags, PK_NBR_WORDS words per block
    int exchange;          // tiles: PK_EXCHANGE_BARRIER, _NEIGHBOR or _TAGGED; STREAM
                           // (persistent): _BARRIER or _NEIGHBOR between passes
    uint64_t* tag;         // tagged halo words: 2 parities x ny rows x tag_pitch words
    int tag_pitch;         // words per row: 4 planes of one word per 16-byte vector
    uint64_t tag_ticks;    // longest wait for a tagged halo word (device clock ticks)
    unsigned char* trace;  // PK_DBG_TRACE: grid x PK_TRACE_BLOCK_BYTES, or null
};
