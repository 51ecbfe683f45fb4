// kloop_sim.cpp -- replays, on the host, the order in which the matrix-core
// kernel runs the k steps of one tile, with the schedule functions the kernel
// itself uses (hpc_tiling_amd/csrc/kloop.hpp), and checks every run of 1 to
// 64 steps on rings of 2, 3 and 4 buffers, with direct loads off, with every
// step whole, and with a partial last step (loaded directly, its k tail
// masked, whenever direct loads are on).
//
// The replay follows the kernel's control flow: the prologue loads the first
// D = NS - 1 tiles and waits at a barrier; each step issues the load of the
// tile D ahead (direct or through VGPRs), runs its MFMA groups on ring buffer
// step % NS, reads the first fragments of the next step (before its barrier on
// rings of three or four buffers, after it on two), and ends with a barrier
// that completes every outstanding load except, on four-buffer rings after a
// load straight to LDS, the one just issued.  Checked:
//   * every step is computed exactly once, in order, on ring position
//     step % NS;
//   * every tile is loaded exactly once, before the step that reads it, into
//     a buffer whose previous tile is already consumed;
//   * a direct load is issued only for a whole k step (index < ndirect), and
//     every whole step is loaded directly; the partial last step is loaded
//     straight to LDS exactly when partial_step_direct says so; nothing past
//     the last step is loaded;
//   * a tile is complete (its loads waited for by a barrier) before any
//     fragment of it is read.
// Prints one line per failure and exits with 1 if there was any.
#include <cstdio>
#include <vector>

#include "kloop.hpp"

using namespace mi;

namespace {

// How a load is issued: whole steps directly, the partial step directly
// with its k tail masked (direct loads on) or through VGPRs.
constexpr int kIssueDirect = 0, kIssueMasked = 1, kIssueStaged = 2;

struct Replay {
    int nsteps, ndirect, ns, d;
    bool direct_on;
    std::vector<int> computed, loaded, ready_barrier, consumed_barrier;
    std::vector<int> in_flight;  // tiles whose direct loads have not been waited for
    std::vector<int> staged;     // tiles in VGPRs, stored to LDS before the next barrier
    int barriers = 0, last = -1, errors = 0;

    Replay(int n, int nd, int s, bool on)
        : nsteps(n), ndirect(nd), ns(s), d(s - 1), direct_on(on), computed(n, 0), loaded(n, 0),
          ready_barrier(n, -1), consumed_barrier(n, -1) {}

    void fail(const char *what, int at) {
        if (errors < 3)
            std::printf("FAIL nsteps=%d ndirect=%d ns=%d direct_on=%d at %d: %s\n", nsteps,
                        ndirect, ns, (int)direct_on, at, what);
        ++errors;
    }

    // `kind`: the schedule's kLoad* value; how it is issued follows the
    // kernel's rule (loads_directly).
    void load(int t, int kind) {
        if (t < 0 || t >= nsteps) return fail("load past the last step", t);
        if (kind == kLoadDirect && t >= ndirect) fail("direct load of a step that is not whole", t);
        if (kind == kLoadRegs && t < ndirect) fail("whole step staged through VGPRs", t);
        const int how = kind == kLoadDirect ? kIssueDirect
                        : loads_directly(kind, direct_on) ? kIssueMasked : kIssueStaged;
        if (how == kIssueMasked && t != nsteps - 1) fail("masked direct load of a middle step", t);
        if (direct_on && how == kIssueStaged) fail("staged load with direct loads on", t);
        if (++loaded[t] > 1) fail("tile loaded twice", t);
        // the buffer's previous tile must be consumed, and the barrier after
        // its last read passed
        const int prev = t - ns;
        if (prev >= 0 && (consumed_barrier[prev] < 0 || consumed_barrier[prev] > barriers))
            fail("ring buffer overwritten before its tile was consumed", t);
        if (how == kIssueStaged)
            staged.push_back(t);
        else
            in_flight.push_back(t);
    }

    // keep_newest: the barrier waits for all direct loads but the last issued.
    void barrier(bool keep_newest) {
        ++barriers;
        for (int t : staged) ready_barrier[t] = barriers;
        staged.clear();
        std::vector<int> keep;
        for (size_t i = 0; i < in_flight.size(); ++i) {
            if (keep_newest && i + 1 == in_flight.size())
                keep.push_back(in_flight[i]);
            else
                ready_barrier[in_flight[i]] = barriers;
        }
        in_flight = keep;
    }

    bool ready(int t) const { return ready_barrier[t] >= 0 && ready_barrier[t] <= barriers; }

    void read_first_fragment(int t) {
        // (the last step reads the next buffer too: stale and unused)
        if (t < nsteps && !ready(t)) fail("fragment read before the tile is complete", t);
    }

    void compute(int s, int cur) {
        if (s < 0 || s >= nsteps) return fail("step out of range", s);
        if (cur != s % ns) fail("wrong ring position", s);
        if (s != last + 1) fail("steps out of order", s);
        last = s;
        if (++computed[s] > 1) fail("step computed twice", s);
        if (!ready(s)) fail("step computed before its tile is complete", s);
    }

    // one_step of the kernel: `kind` is a kLoad* value (kLoadAuto decides).
    void one_step(int s, int kind, int cur) {
        const int ld = kind == kLoadAuto ? load_of(s + d, nsteps, ndirect) : kind;
        if (ld != kLoadNone) load(s + d, ld);
        compute(s, cur);
        if (d >= 2) read_first_fragment(s + 1);
        if (s < nsteps) consumed_barrier[s] = barriers + 1;
        barrier(keeps_load_in_flight(ns, ld, direct_on));
        if (d == 1) read_first_fragment(s + 1);
    }

    void run() {
        for (int t = 0; t < d && t < nsteps; ++t) load(t, load_of(t, nsteps, ndirect));
        barrier(d >= 3 && 2 < ndirect);
        read_first_fragment(0);

        const KLoop kl = kloop_schedule(nsteps, ndirect, ns);
        if (kl.steady_end % ns || kl.auto_end % ns || kl.auto_end < kl.steady_end)
            fail("phase bounds not whole ring rounds", kl.auto_end);
        int step = 0;
        for (; step < kl.steady_end; step += ns)
            for (int j = 0; j < ns; ++j) one_step(step + j, kLoadDirect, j);
        for (; step < kl.auto_end; step += ns)
            for (int j = 0; j < ns; ++j) one_step(step + j, kLoadAuto, j);
        if (ns == 2 || kl.tail == kTailDecided) {
            for (int i = 0; i < kTailMax; ++i)
                if (step + i < nsteps) one_step(step + i, kLoadAuto, i % ns);
        } else if (kl.tail < 0 || kl.tail >= kNumTailSequences) {
            fail("tail index out of range", kl.tail);
        } else {
            const TailSeq seq = kTailSequences[kl.tail];
            for (int i = 0; i < seq.r && i < kTailMax; ++i)
                one_step(step + i, load_of(i + d, seq.r, seq.nd), i % ns);
        }
        for (int s = 0; s < nsteps; ++s) {
            if (computed[s] != 1) fail("step not computed", s);
            if (loaded[s] != 1) fail("tile not loaded", s);
        }
    }
};

}  // namespace

int main() {
    int failures = 0, runs = 0;
    for (int ns = 2; ns <= 4; ++ns)
        for (int nsteps = 1; nsteps <= 64; ++nsteps) {
            // direct loads off; every step whole; the last step partial
            // (ndirect: whole steps, loadable directly)
            const int cases[3][2] = {{0, 0}, {nsteps, 1}, {nsteps - 1, 1}};
            for (const auto &c : cases) {
                Replay r(nsteps, c[0], ns, partial_step_direct(ns, c[1] != 0));
                r.run();
                failures += r.errors > 0;
                ++runs;
            }
        }
    std::printf("%d runs, %d failed\n", runs, failures);
    return failures ? 1 : 0;
}
