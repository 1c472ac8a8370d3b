// Host run of the grid barrier's arrival and wait protocol
// (combine_group_limited_amd/csrc/barrier_protocol.hpp) with one thread per
// block and sequentially consistent atomics.  Prints one line per scenario:
// "<name> ok" or "<name> FAIL <reason>".
#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "barrier_protocol.hpp"

using namespace cgl;

struct HostAtomics {
    uint32_t load(uint32_t* p) const { return __atomic_load_n(p, __ATOMIC_SEQ_CST); }
    void store(uint32_t* p, uint32_t v) const { __atomic_store_n(p, v, __ATOMIC_SEQ_CST); }
    uint32_t fetch_add(uint32_t* p, uint32_t v) const { return __atomic_fetch_add(p, v, __ATOMIC_SEQ_CST); }
    void pause() const { std::this_thread::yield(); }
};

constexpr int kWords = 1024;

static bool at_rest(const uint32_t* ws) {
    if (ws[0] != 0 || ws[kBarrierGiveUpWord] != 0) return false;
    for (int c = 0; c < kBarrierGroups; ++c)
        if (ws[kBarrierGroupStride * (1 + c)] != 0) return false;
    return true;
}

// One launch: blocks in `present` run `nbar` barriers; result[b] counts the
// barriers block b got through.  arrivals[i] counts blocks that reached
// barrier i; a block that got through checks that all nb had reached it.
static bool launch(uint32_t* ws, int nb, const std::vector<int>& present, int nbar, uint32_t spin,
                   std::vector<int>& passed, std::string& why) {
    std::vector<std::atomic<int>> arrivals(nbar);
    for (auto& a : arrivals) a = 0;
    std::atomic<int> early{0};
    passed.assign(nb, -1);
    std::vector<std::thread> th;
    for (int b : present)
        th.emplace_back([&, b] {
            HostAtomics op;
            const bool refused = barrier_refused(op, ws);
            int n = 0;
            for (int i = 0; i < nbar; ++i) {
                arrivals[i].fetch_add(1);
                if (!barrier_arrive_wait(op, ws, b, nb, spin, i == 0 && refused)) break;
                if (arrivals[i].load() != nb) early.fetch_add(1);
                ++n;
            }
            passed[b] = n;
        });
    for (auto& t : th) t.join();
    if (early.load()) {
        why = "a block got through a barrier before every block had reached it";
        return false;
    }
    return true;
}

static void report(const char* name, bool ok, const std::string& why) {
    std::printf("%s %s%s%s\n", name, ok ? "ok" : "FAIL", ok ? "" : " ", ok ? "" : why.c_str());
}

int main() {
    std::vector<uint32_t> mem(kWords, 0);
    uint32_t* ws = mem.data();
    std::vector<int> passed;
    std::string why;

    // 1. every block present: every barrier passes, workspace at rest after
    {
        bool ok = true;
        for (int nb : {1, 3, 8, 9, 37}) {
            std::vector<int> all(nb);
            for (int b = 0; b < nb; ++b) all[b] = b;
            for (int rep = 0; rep < 20 && ok; ++rep) {
                ok = launch(ws, nb, all, 4, 1u << 30, passed, why);
                for (int b = 0; b < nb && ok; ++b)
                    if (passed[b] != 4) ok = false, why = "a block stopped with every block present";
                if (ok && !at_rest(ws)) ok = false, why = "workspace not at rest after a launch";
            }
        }
        report("all_present", ok, why);
    }

    // 2. one block never runs: the others give up and count themselves; every
    // later launch on the workspace is refused (no arrivals, counters left as
    // they are) until the workspace is zeroed, after which launches pass
    {
        const int nb = 12;
        std::vector<int> some, all;
        for (int b = 0; b < nb; ++b) {
            all.push_back(b);
            if (b != 5) some.push_back(b);
        }
        bool ok = launch(ws, nb, some, 2, 2000, passed, why);
        for (int b : some)
            if (ok && passed[b] != 0) ok = false, why = "a block passed with one block missing";
        if (ok && ws[kBarrierGiveUpWord] != (uint32_t)some.size()) ok = false, why = "give-ups not counted";
        std::vector<uint32_t> before(mem);
        if (ok) ok = launch(ws, nb, all, 2, 1u << 30, passed, why);
        for (int b : all)
            if (ok && passed[b] != 0) ok = false, why = "a launch on a refused workspace passed a barrier";
        if (ok && before != mem) ok = false, why = "a refused launch changed the workspace";
        std::fill(mem.begin(), mem.end(), 0u);
        if (ok) ok = launch(ws, nb, all, 2, 1u << 30, passed, why);
        for (int b : all)
            if (ok && passed[b] != 2) ok = false, why = "no pass after the workspace was zeroed";
        if (ok && !at_rest(ws)) ok = false, why = "not at rest after the recovery launch";
        report("give_up_then_refused", ok, why);
    }

    // 3. a block that arrives after others gave up stops at once (it does not
    // wait out its own, here very long, poll limit)
    {
        std::fill(mem.begin(), mem.end(), 0u);
        const int nb = 6;
        HostAtomics op;
        std::vector<std::thread> th;
        std::atomic<int> fails{0};
        for (int b = 0; b < nb - 2; ++b)
            th.emplace_back([&, b] {
                if (barrier_arrive_wait(op, ws, b, nb, 1000, false)) fails.fetch_add(1);
            });
        for (auto& t : th) t.join();
        const auto t0 = std::chrono::steady_clock::now();
        const bool late = barrier_arrive_wait(op, ws, nb - 2, nb, 20000000u, false);
        const double s = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
        bool ok = fails.load() == 0 && !late && s < 1.0 && ws[kBarrierGiveUpWord] == (uint32_t)(nb - 1);
        report("late_block_stops", ok, "late block waited or passed");
    }
    return 0;
}
