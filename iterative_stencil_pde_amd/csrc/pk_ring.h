// Host side of the task mailbox: publish sequence-numbered task slots, harvest
// completion records, busy-poll for a ticket. No HIP calls, so the protocol can
// be exercised on the CPU against a thread that plays the device.
//
// Protocol (see pk_shared.h for the layout):
//   host:   store slot[s % RING] = pack(s, kind, n) (one 64-bit word).
//   device: poll slot[s % RING] until its sequence half equals s, run the
//           task, write done[s % RING], release-store done_seq = s.
// A slot is reused only after its previous task's record has been harvested,
// so neither side ever overwrites something the other still needs. Sequence
// numbers replace IDLE/DONE toggles, so there is no early acknowledgement
// ("Persistent Kernels", "Reflections and next steps", point 3), and the host
// polls without sleeping ("Tuning sleep duration": a sleep costs ~50 us of
// timer slack).
#pragma once

#include <chrono>
#include <cstdint>
#include <vector>

#include "../../include/pk.h"
#include "pk_shared.h"

namespace pkr {

struct DoneInfo {
    uint64_t seq = 0;
    int kind = 0;
    int status = 0;
    double residual = 0.0;
    int64_t sweeps_done = 0;
    uint64_t t_begin = 0, t_end = 0;
    int64_t errors = 0;
    int cur = 0;
    int carried = 0;
};

inline void cpu_relax() {
#if defined(__x86_64__)
    __builtin_ia32_pause();
#endif
}

class HostRing {
public:
    void attach(pk_mailbox* m) {
        m_ = m;
        next_ = 1;
        harvested_ = 0;
        carried_ = 0;
        fused_ = 0;
        done_.assign(1, DoneInfo{});
    }

    // Publish a task. PK_EBUSY when PK_RING tasks are already in flight.
    int publish(int kind, int n, uint64_t* seq, const pk_param* prm = nullptr) {
        harvest();
        if (next_ - 1 - harvested_ >= PK_RING) return PK_EBUSY;
        if (prm) m_->param[next_ % PK_RING] = *prm;  // ordered before the slot's release
        __atomic_store_n(&m_->slot[next_ % PK_RING].word, pk_slot_pack(next_, kind, n),
                         __ATOMIC_RELEASE);
        if (seq) *seq = next_;
        ++next_;
        return PK_OK;
    }

    // Copy every newly completed record out of the mailbox.
    void harvest() {
        const uint64_t d = __atomic_load_n(&m_->done_seq, __ATOMIC_ACQUIRE);
        while (harvested_ < d && harvested_ + 1 < next_) {
            const uint64_t s = harvested_ + 1;
            const pk_done_rec& r = m_->done[s % PK_RING];
            DoneInfo x;
            x.seq = r.seq;
            x.kind = r.kind;
            x.status = (r.seq == s) ? r.status : PK_EDEVICE;
            x.residual = r.residual;
            x.sweeps_done = r.sweeps_done;
            x.t_begin = r.t_begin;
            x.t_end = r.t_end;
            x.errors = r.errors;
            x.cur = r.cur;
            x.carried = r.carried & 1;
            carried_ += (r.carried & 1) ? 1 : 0;
            fused_ += (r.carried & 2) ? 1 : 0;
            done_.push_back(x);
            harvested_ = s;
        }
    }

    // Busy-poll until `ticket` completes. `exited(ctx)` reports that the device
    // side has stopped answering for good.
    int wait(uint64_t ticket, double timeout_s, DoneInfo* out, bool (*exited)(void*), void* ctx) {
        if (ticket == 0 || ticket >= next_) return PK_EINVAL;
        const auto t0 = std::chrono::steady_clock::now();
        unsigned spins = 0;
        for (;;) {
            harvest();
            if (harvested_ >= ticket) break;
            if (exited && exited(ctx)) {
                harvest();
                if (harvested_ >= ticket) break;
                return PK_EDEVICE;
            }
            if ((++spins & 1023u) == 0) {
                const double el = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
                if (el > timeout_s) return PK_ETIMEDOUT;
            }
            cpu_relax();
        }
        if (out) *out = done_[ticket];
        return PK_OK;
    }

    uint64_t in_flight() {
        harvest();
        return next_ - 1 - harvested_;
    }
    uint64_t done_seen() const { return harvested_; }
    uint64_t issued() const { return next_ - 1; }
    int64_t sweeps_seen() const { return harvested_ ? done_[harvested_].sweeps_done : 0; }
    int last_cur() const { return harvested_ ? done_[harvested_].cur : 0; }
    uint64_t carried_seen() const { return carried_; }
    uint64_t fused_seen() const { return fused_; }

private:
    pk_mailbox* m_ = nullptr;
    uint64_t next_ = 1;
    uint64_t harvested_ = 0;
    uint64_t carried_ = 0;
    uint64_t fused_ = 0;
    std::vector<DoneInfo> done_;  // index = ticket
};

}  // namespace pkr
