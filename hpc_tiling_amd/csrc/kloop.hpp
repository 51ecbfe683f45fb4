// kloop.hpp -- the order in which one workgroup runs the k steps of a tile
// (the "big iterations" over K of page "GEMM优化原理", section
// 基于 shared memory 计算, pipelined as in section "prefetch 和双缓冲").
//
// The tile of step s goes to LDS ring buffer s % NS (NS = 2 to 4 buffers) and
// is loaded D = NS - 1 steps ahead: the prologue loads steps 0 .. D-1, step s
// loads step s + D.  A load is direct (global -> LDS: the whole k steps,
// index < ndirect, and the partial last k step with its k tail masked) or
// staged through VGPRs (every step when direct loads cannot address the
// operands).  The steps run in three phases, each with its loads fixed at
// compile time where possible:
//   steady   [0, steady_end)           NS steps per iteration, every load
//                                      direct (each ring position a constant);
//   decided  [steady_end, auto_end)    NS steps per iteration, each step
//                                      deciding its load at run time;
//   tail     [auto_end, nsteps)        at most kTailMax steps: one of a few
//                                      fixed sequences (kTailSequences), or
//                                      decided step by step (kTailDecided).
// Plain constexpr functions (no device-only code), so that a host program can
// replay the schedule and check it.
#pragma once

namespace mi {

// What a step loads for the step D ahead.  kLoadRegs is the partial last k
// step (or any step when direct loads are off); on four-buffer rings with
// direct loads on it is loaded directly too, four bytes per lane, with the
// elements past the end of k sent out of the buffer's range (they land in LDS
// as zeros).
constexpr int kLoadNone = 0, kLoadDirect = 1, kLoadRegs = 2, kLoadAuto = 3;

constexpr int kTailMax = 5;       // steps left after the loops, at most
constexpr int kTailDecided = -1;  // tail: every remaining step decides its load

// How the tile of step t is loaded in a run of nsteps steps whose first
// ndirect are whole: not at all past the end, directly while whole, else
// through VGPRs.  The prologue loads t = 0 .. D-1 this way, and a deciding
// step s the tile t = s + D.
constexpr int load_of(int t, int nsteps, int ndirect) {
    return t >= nsteps ? kLoadNone : (t < ndirect ? kLoadDirect : kLoadRegs);
}

// Whether the partial last k step is loaded directly (with `direct_ok`: the
// operands are addressable by direct loads): only on four-buffer rings, where
// its load can stay in flight across the barrier of the step that issues it;
// on shorter rings that barrier waits for the load either way, and staging it
// through VGPRs costs fewer registers.
constexpr bool partial_step_direct(int ns, bool direct_ok) { return ns == 4 && direct_ok; }

// Whether a load of kind `load` goes straight to LDS (no VGPR staging):
// whole steps always, the partial step when `direct_on`
// (partial_step_direct).
constexpr bool loads_directly(int load, bool direct_on) {
    return load == kLoadDirect || (load == kLoadRegs && direct_on);
}

// Whether the barrier that ends a step may leave the load that step issued
// in flight: only on four-buffer rings, whose loads run three steps ahead,
// and only for loads that go straight to LDS (a staged tile is written to
// LDS from VGPRs before the barrier, so its load is complete by then).
constexpr bool keeps_load_in_flight(int ns, int load, bool direct_on) {
    return ns == 4 && loads_directly(load, direct_on);
}

// The fixed tail sequences: r remaining steps, the first nd of them whole.
// Tail step i loads step i + D as load_of(i + D, r, nd) would decide it.
struct TailSeq {
    int r, nd;
};
constexpr TailSeq kTailSequences[] = {{1, 0}, {1, 1}, {2, 1}, {2, 2}, {3, 2},
                                      {3, 3}, {4, 3}, {4, 4}, {5, 4}};
constexpr int kNumTailSequences = sizeof(kTailSequences) / sizeof(kTailSequences[0]);

// Index in kTailSequences of (r, nd), or kTailDecided when there is none.
constexpr int tail_index(int r, int nd) {
    for (int i = 0; i < kNumTailSequences; ++i)
        if (kTailSequences[i].r == r && kTailSequences[i].nd == nd) return i;
    return kTailDecided;
}

struct KLoop {
    int steady_end;  // multiple of ns
    int auto_end;    // multiple of ns, nsteps - kTailMax <= auto_end <= nsteps
    int tail;        // index in kTailSequences, or kTailDecided
};

// Ceiling of a / b for b > 0, 0 for a <= 0.
constexpr int ceil_pos(int a, int b) { return a > 0 ? (a + b - 1) / b : 0; }

// The schedule of `nsteps` k steps, `ndirect` of them (the leading ones)
// loadable directly (0 when direct loads are off), on a ring of `ns` buffers.
// The steady phase lasts while every load of an iteration is direct: the
// iteration starting at step s loads up to step s + ns - 1 + d.  A fixed tail
// sequence is used for rings of three or four buffers when one matches the
// remaining steps exactly (r steps, nd = ndirect - auto_end of them whole);
// two-buffer rings, and tails the list does not hold (no direct loads among
// several steps, say), decide step by step.
constexpr KLoop kloop_schedule(int nsteps, int ndirect, int ns) {
    const int d = ns - 1;
    KLoop k{0, 0, kTailDecided};
    k.steady_end = ns * ceil_pos(ndirect - (ns - 1 + d), ns);
    k.auto_end = k.steady_end + ns * ceil_pos(nsteps - kTailMax - k.steady_end, ns);
    const int r = nsteps - k.auto_end, nd = ndirect - k.auto_end;
    if (ns >= 3 && nd >= 0) k.tail = tail_index(r, nd);
    return k;
}

}  // namespace mi
