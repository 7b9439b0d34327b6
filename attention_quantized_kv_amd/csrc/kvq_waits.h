// kvq_waits.h -- the request order of the Q8_0/Q4_0 streaming kernel's ring
// and the s_waitcnt vmcnt counts that follow from it (attn_mfma_stream.hip).
// Pure constexpr arithmetic, compilable for the host as well, so that a CPU
// test can check every count against a simulation of the request stream.
#pragma once

namespace kvq {

// Ring slots of the streaming kernel per head_dim: a few KiB in flight per
// wave (the slots must divide the 3 * D / 64 code pieces of a chunk).  DEEP:
// waves with up to 8 rows (more of their requests land while they compute)
// and waves with two row tiles (about twice as long on each piece) ask for
// their pieces further ahead, where the LDS has room.
constexpr int stream_ring_slots(int D, bool deep = false) {
    return D == 256 ? (deep ? 6 : 4) : D == 128 ? (deep ? 6 : 3) : 3;
}

// Wait counts.  Per chunk a wave issues its requests in a fixed order: the
// QK step consumes code pieces 2p, 2p+1 (slice p, both tiles) and requests
// the pieces R places further on; then the next chunk's K scales; the PV
// step consumes piece 2KL+u and requests the one R further on; then the next
// chunk's V scales.  Piece J of chunk k was requested when piece J-R was
// consumed, so the number of requests issued after it by the time it is
// consumed is fixed; s_waitcnt vmcnt(that count) guarantees it has landed
// (requests complete in order).  The first chunk's requests go out in the
// same order before the loop, so it uses the same counts; the last chunk
// (nothing further requested) waits with 0.
template <int KL, int R>
struct Waits {
    static constexpr int NP = 3 * KL, NI = 3 * KL + 2;
    static constexpr int issue_pos(int j) { return j < 2 * KL ? j : j + 1; }          // slot of "consume j" in a chunk's requests
    static constexpr int event_pos(int J) { return J < 2 * KL ? 2 * (J / 2) : 2 * KL + 1 + (J - 2 * KL); }
    static constexpr int after(int J) {
        const int m = ((J - R) % NP + NP) % NP;
        return event_pos(J) - issue_pos(m) - 1 + (J < R ? NI : 0);
    }
    static constexpr int mn(int a, int b) { return a < b ? a : b; }
    // QK slice p (and, for p = 0, this chunk's K scales, issued at 2KL of the
    // chunk before)
    static constexpr int qk(int p) { return p == 0 ? mn(mn(after(0), after(1)), NI - 2 * KL - 1) : mn(after(2 * p), after(2 * p + 1)); }
    // PV slice u (and, for u = 0, this chunk's V scales, issued last in the chunk before)
    static constexpr int pv(int u) { return u == 0 ? mn(after(2 * KL), NI - KL - 1) : after(2 * KL + u); }
};

}  // namespace kvq
