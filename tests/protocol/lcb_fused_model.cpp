// Host model of the persistent IKBO-LCB launch's work protocol (ROCS Sec. 4.2.3: request and
// candidate tiles in one persistent schedule; the candidate epilogue waits on per-request-tile
// completion flags with release/acquire semantics), for ThreadSanitizer. Test infrastructure: it
// shares no code with the library; it restates the kernel's protocol with std::atomic.
//
// One host thread per workgroup. Shared state as in the kernel's sync words:
//   req_counter            request items (tile, split) claimed in ascending order
//   cand_counter[x]        candidate tiles of "XCD" x claimed in descending order from its range end
//   arrive[t], ready[t]    per request tile: splits arrived, result published
//   timed_out              a wait ran out; every later wait stops at once
// Data (plain, non-atomic, so TSan checks the ordering): partial[split][t] written by each split,
// z[t] written by the last split to arrive (the sum in split order), out[c] by candidate tiles.
// Orderings mirror the kernel, written as operations on the atomics themselves (ThreadSanitizer
// does not model standalone fences): the kernel's release fence before its arrival count and
// before its flag store become a release read-modify-write and a release store; its relaxed flag
// polls followed by agent-coherent loads of the guarded data become acquire loads here.
//
// usage: lcb_fused_model <workgroups> <request tiles> <splits> <candidate tiles> <publish 0|1>
//                        <wait bound in microseconds>
// Checks: every item claimed exactly once; z equals the split-order sum; with publish, every
// candidate output equals its expected value; without, every candidate output is the NaN marker;
// the program always ends. Exit 0 on success.
#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <thread>
#include <vector>

namespace {

constexpr int kXcds = 8;
constexpr long long kNanMark = -1;

struct Shared {
    int W, Q, S, T;
    bool publish;
    std::chrono::microseconds bound;
    std::atomic<int> req_counter{0};
    std::atomic<int> cand_counter[kXcds];
    std::vector<std::atomic<int>> arrive, ready, req_claims, cand_claims;
    std::atomic<int> timed_out{0};
    std::vector<std::vector<long long>> partial;   // [S][Q]
    std::vector<long long> z;                      // [Q]
    std::vector<long long> out;                    // [T]
    Shared(int w, int q, int s, int t, bool p, int bound_us)
        : W(w), Q(q), S(s), T(t), publish(p), bound(bound_us), arrive(q), ready(q), req_claims(q * s),
          cand_claims(t), partial(s, std::vector<long long>(q, 0)), z(q, 0), out(t, 0) {
        for (auto &c : cand_counter) c.store(0);
        for (auto &a : arrive) a.store(0);
        for (auto &r : ready) r.store(0);
        for (auto &c : req_claims) c.store(0);
        for (auto &c : cand_claims) c.store(0);
    }
};

long long partial_value(int t, int s) { return 1000LL * t + 7 * s + 1; }

long long expected_z(const Shared &sh, int t) {
    long long v = 0;
    for (int s = 0; s < sh.S; ++s) v += partial_value(t, s);
    return v;
}

long long expected_out(const Shared &sh, int c) {
    long long v = 3LL * c;                 // the tile's own main loop
    for (int t = 0; t < sh.Q; ++t) v += expected_z(sh, t);   // every request tile's Z columns
    return v;
}

void workgroup(Shared &sh, int id) {
    const int x = id % kXcds;
    const int per_xcd = (sh.T + kXcds - 1) / kXcds;
    const int c_beg = x * per_xcd, c_end = std::min(sh.T, c_beg + per_xcd);
    const int req_items = sh.Q * sh.S;
    for (;;) {
        const int r = sh.req_counter.fetch_add(1, std::memory_order_relaxed);
        if (r < req_items) {
            // request item: tile r / S, split r % S (splits of a tile are consecutive items)
            const int t = r / sh.S, s = r % sh.S;
            sh.req_claims[r].fetch_add(1, std::memory_order_relaxed);
            sh.partial[s][t] = partial_value(t, s);
            // the arrival count releases this split's partials and acquires the earlier splits'
            const int a = sh.arrive[t].fetch_add(1, std::memory_order_acq_rel);
            if (a == sh.S - 1) {
                long long v = 0;
                for (int k = 0; k < sh.S; ++k) v += sh.partial[k][t];   // split order
                sh.z[t] = v;
                if (sh.publish) sh.ready[t].store(1, std::memory_order_release);
            }
            continue;
        }
        const int k = sh.cand_counter[x].fetch_add(1, std::memory_order_relaxed);
        const int c = c_end - 1 - k;       // candidate tiles descending
        if (c < c_beg) break;
        sh.cand_claims[c].fetch_add(1, std::memory_order_relaxed);
        long long acc = 3LL * c;            // the main loop needs no request data
        const auto deadline = std::chrono::steady_clock::now() + sh.bound;
        bool ok = true;
        for (int t = 0; t < sh.Q && ok; ++t) {
            if (sh.timed_out.load(std::memory_order_relaxed)) ok = false;
            while (ok && sh.ready[t].load(std::memory_order_acquire) == 0) {
                if (std::chrono::steady_clock::now() > deadline || sh.timed_out.load(std::memory_order_relaxed)) {
                    ok = false;
                    sh.timed_out.store(1, std::memory_order_relaxed);
                } else {
                    std::this_thread::yield();
                }
            }
        }
        if (ok) {
            for (int t = 0; t < sh.Q; ++t) acc += sh.z[t];   // each ordered by its flag's acquire
            sh.out[c] = acc;
        } else {
            sh.out[c] = kNanMark;
        }
    }
}

}  // namespace

int main(int argc, char **argv) {
    if (argc != 7) {
        std::fprintf(stderr, "usage: %s W Q S T publish bound_us\n", argv[0]);
        return 2;
    }
    Shared sh(std::atoi(argv[1]), std::atoi(argv[2]), std::atoi(argv[3]), std::atoi(argv[4]), std::atoi(argv[5]) != 0,
              std::atoi(argv[6]));
    std::vector<std::thread> th;
    for (int w = 0; w < sh.W; ++w) th.emplace_back(workgroup, std::ref(sh), w);
    for (auto &t : th) t.join();
    int bad = 0;
    for (int i = 0; i < sh.Q * sh.S; ++i)
        if (sh.req_claims[i].load() != 1) ++bad;
    for (int c = 0; c < sh.T; ++c)
        if (sh.cand_claims[c].load() != 1) ++bad;
    for (int t = 0; t < sh.Q; ++t)
        if (sh.z[t] != expected_z(sh, t)) ++bad;
    for (int c = 0; c < sh.T; ++c) {
        if (sh.publish && sh.out[c] != expected_out(sh, c)) ++bad;
        if (!sh.publish && sh.out[c] != kNanMark) ++bad;
    }
    std::printf("model W=%d Q=%d S=%d T=%d publish=%d: %s\n", sh.W, sh.Q, sh.S, sh.T, (int)sh.publish,
                bad ? "FAILED" : "ok");
    return bad ? 1 : 0;
}
