// Host side of the task mailbox (pk_ring.h) against a CPU thread that plays the
// device: it polls `tail`, acquires, reads the slot, "runs" the task (a SWEEP
// adds n to a sweep counter, a RESIDUAL returns a value derived from the
// ticket), writes the completion record and releases `done_seq`, exactly as the
// persistent kernel's leader does. Built and run by tests/test_host_protocol.py,
// under ThreadSanitizer and AddressSanitizer. Exit status 0 = all checks passed.
#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "../../iterative_stencil_pde_amd/csrc/pk_ring.h"
#include "../../iterative_stencil_pde_amd/csrc/pk_shared.h"

namespace {

int failures = 0;
#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            std::fprintf(stderr, "CHECK failed line %d: %s\n", __LINE__, #c); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

struct FakeDevice {
    pk_mailbox* m;
    int stall_after = -1;   // stop answering after this many tasks (never exits)
    int exit_after = -1;    // leave (exited = 1) after this many tasks
    int delay_us = 0;       // per task
    std::atomic<bool> stop{false};
    int64_t sweeps = 0;

    void run() {
        uint64_t next = 1;
        int handled = 0;
        while (!stop.load(std::memory_order_relaxed)) {
            const uint64_t w = __atomic_load_n(&m->slot[next % PK_RING].word, __ATOMIC_ACQUIRE);
            if (pk_slot_seq(w) != static_cast<uint32_t>(next)) {
                std::this_thread::yield();
                continue;
            }
            if (handled == stall_after) {
                while (!stop.load(std::memory_order_relaxed)) std::this_thread::yield();
                return;
            }
            if (handled == exit_after) {
                __atomic_store_n(&m->exited, 1u, __ATOMIC_RELEASE);
                return;
            }
            const uint64_t seq = next;
            const int kind = pk_slot_kind(w), n = pk_slot_n(w);
            if (delay_us) std::this_thread::sleep_for(std::chrono::microseconds(delay_us));
            pk_done_rec& d = m->done[next % PK_RING];
            if (kind == PK_SWEEP) sweeps += n;
            d.kind = kind;
            d.status = PK_OK;
            d.residual = kind == PK_RESIDUAL ? 1.0 / static_cast<double>(seq) : 0.0;
            d.sweeps_done = sweeps;
            d.errors = 0;
            d.cur = static_cast<int32_t>(sweeps & 1);
            d.seq = seq;
            __atomic_store_n(&m->done_seq, next, __ATOMIC_RELEASE);
            ++next;
            ++handled;
        }
    }
};

bool exited_fn(void* ctx) {
    auto* m = static_cast<pk_mailbox*>(ctx);
    return __atomic_load_n(&m->exited, __ATOMIC_ACQUIRE) != 0;
}

void test_fifo_wraparound() {
    auto* m = new pk_mailbox();
    std::memset(m, 0, sizeof(*m));
    pkr::HostRing ring;
    ring.attach(m);
    FakeDevice dev;
    dev.m = m;
    std::thread t(&FakeDevice::run, &dev);
    const int ntask = 5 * PK_RING + 7;  // wraps the ring several times
    std::vector<uint64_t> tickets;
    int64_t expect = 0;
    for (int k = 0; k < ntask; ++k) {
        uint64_t s = 0;
        const int kind = (k % 3 == 2) ? PK_RESIDUAL : PK_SWEEP;
        int rc;
        while ((rc = ring.publish(kind, k, &s)) == PK_EBUSY) {
            pkr::DoneInfo d;
            CHECK(ring.wait(tickets[tickets.size() - PK_RING], 5.0, &d, exited_fn, m) == PK_OK);
        }
        CHECK(rc == PK_OK);
        CHECK(s == static_cast<uint64_t>(k + 1));
        tickets.push_back(s);
    }
    for (int k = 0; k < ntask; ++k) {
        pkr::DoneInfo d;
        CHECK(ring.wait(tickets[k], 5.0, &d, exited_fn, m) == PK_OK);
        const int kind = (k % 3 == 2) ? PK_RESIDUAL : PK_SWEEP;
        if (kind == PK_SWEEP) expect += k;
        CHECK(d.seq == tickets[k] && d.kind == kind && d.status == PK_OK);
        CHECK(d.sweeps_done == expect);
        if (kind == PK_RESIDUAL) CHECK(d.residual == 1.0 / static_cast<double>(tickets[k]));
    }
    CHECK(ring.in_flight() == 0);
    CHECK(ring.done_seen() == static_cast<uint64_t>(ntask));
    CHECK(ring.wait(0, 1.0, nullptr, exited_fn, m) == PK_EINVAL);
    CHECK(ring.wait(ntask + 1, 1.0, nullptr, exited_fn, m) == PK_EINVAL);
    dev.stop = true;
    t.join();
    delete m;
}

void test_ring_full_is_busy() {
    auto* m = new pk_mailbox();
    std::memset(m, 0, sizeof(*m));
    pkr::HostRing ring;
    ring.attach(m);
    // no device thread yet: exactly PK_RING tasks fit
    uint64_t s = 0;
    for (unsigned k = 0; k < PK_RING; ++k) CHECK(ring.publish(PK_SWEEP, 1, &s) == PK_OK);
    CHECK(ring.publish(PK_SWEEP, 1, &s) == PK_EBUSY);
    CHECK(ring.in_flight() == PK_RING);
    FakeDevice dev;
    dev.m = m;
    std::thread t(&FakeDevice::run, &dev);
    pkr::DoneInfo d;
    CHECK(ring.wait(PK_RING, 5.0, &d, exited_fn, m) == PK_OK);
    CHECK(d.sweeps_done == PK_RING);
    CHECK(ring.publish(PK_SWEEP, 1, &s) == PK_OK && s == PK_RING + 1);
    CHECK(ring.wait(s, 5.0, &d, exited_fn, m) == PK_OK);
    dev.stop = true;
    t.join();
    delete m;
}

void test_stalled_device_times_out() {
    auto* m = new pk_mailbox();
    std::memset(m, 0, sizeof(*m));
    pkr::HostRing ring;
    ring.attach(m);
    FakeDevice dev;
    dev.m = m;
    dev.stall_after = 2;
    std::thread t(&FakeDevice::run, &dev);
    uint64_t a = 0, b = 0, c = 0;
    CHECK(ring.publish(PK_SWEEP, 1, &a) == PK_OK);
    CHECK(ring.publish(PK_SWEEP, 1, &b) == PK_OK);
    CHECK(ring.publish(PK_SWEEP, 1, &c) == PK_OK);
    pkr::DoneInfo d;
    CHECK(ring.wait(b, 5.0, &d, exited_fn, m) == PK_OK);
    const auto t0 = std::chrono::steady_clock::now();
    CHECK(ring.wait(c, 0.2, &d, exited_fn, m) == PK_ETIMEDOUT);
    const double el = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    CHECK(el >= 0.2 && el < 2.0);
    dev.stop = true;
    t.join();
    delete m;
}

void test_exited_device_is_an_error() {
    auto* m = new pk_mailbox();
    std::memset(m, 0, sizeof(*m));
    pkr::HostRing ring;
    ring.attach(m);
    FakeDevice dev;
    dev.m = m;
    dev.exit_after = 3;
    std::thread t(&FakeDevice::run, &dev);
    uint64_t s[5];
    for (auto& x : s) CHECK(ring.publish(PK_RESIDUAL, 0, &x) == PK_OK);
    pkr::DoneInfo d;
    CHECK(ring.wait(s[2], 5.0, &d, exited_fn, m) == PK_OK);  // completed before it left
    CHECK(ring.wait(s[3], 5.0, &d, exited_fn, m) == PK_EDEVICE);
    t.join();
    delete m;
}

void test_slow_device_keeps_order() {
    auto* m = new pk_mailbox();
    std::memset(m, 0, sizeof(*m));
    pkr::HostRing ring;
    ring.attach(m);
    FakeDevice dev;
    dev.m = m;
    dev.delay_us = 50;
    std::thread t(&FakeDevice::run, &dev);
    uint64_t last = 0;
    for (int k = 0; k < 3 * PK_RING; ++k) {
        uint64_t s = 0;
        while (ring.publish(PK_SWEEP, 2, &s) == PK_EBUSY) {
            pkr::DoneInfo d;
            CHECK(ring.wait(ring.done_seen() + 1, 5.0, &d, exited_fn, m) == PK_OK);
        }
        last = s;
    }
    pkr::DoneInfo d;
    CHECK(ring.wait(last, 10.0, &d, exited_fn, m) == PK_OK);
    CHECK(d.sweeps_done == 2 * 3 * PK_RING);
    CHECK(ring.last_cur() == 0 && ring.sweeps_seen() == 2 * 3 * PK_RING);
    dev.stop = true;
    t.join();
    delete m;
}

}  // namespace

int main() {
    test_fifo_wraparound();
    test_ring_full_is_busy();
    test_stalled_device_times_out();
    test_exited_device_is_an_error();
    test_slow_device_keeps_order();
    if (failures) {
        std::fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("host protocol: all checks passed\n");
    return 0;
}
