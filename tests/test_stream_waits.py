"""The s_waitcnt vmcnt counts of the Q8_0/Q4_0 streaming kernel, checked on
the CPU against a simulation of its request stream.

Each wave of attn_mfma_stream.hip streams its chunks through a ring of R
one-KiB slots (R depends on head_dim, and is larger for waves with two row tiles) with direct-to-LDS loads and, before it reads a piece out of
LDS, waits until at most N of its vector-memory requests are outstanding
(requests complete in issue order).  N comes from the constexpr table
Waits<KL, R> in csrc/kvq_waits.h.  A count that is too high would let a wave
read a slot before its data has landed: silent, timing-dependent wrong output.

The simulation below is written from the kernel's issue order: the first
chunk's requests before the loop (in the order a previous chunk would have
issued them), then per chunk the QK slices (wait, read pieces 2p and 2p+1,
request the pieces R further on, of this chunk or of the next), the next
chunk's K scales, the PV slices (wait, read piece 2KL+u, request the one R
further on), the next chunk's V scales.  For every wait it counts the
requests issued after the newest request the read needs; the table's count
must not exceed it.  The table is extracted by compiling the header with g++.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "attention_quantized_kv_amd", "csrc", "kvq_waits.h")
HEAD_DIMS = (64, 128, 256)
DEEP = (0, 1)               # the deeper ring of waves with two row tiles
CASES = [(D, deep) for D in HEAD_DIMS for deep in DEEP]


def _table(tmp_path):
    src = tmp_path / "waits.cpp"
    src.write_text(f'#include "{HEADER}"\n#include <cstdio>\n' + r'''
template <int D, int DEEP> void dump() {
    constexpr int KL = D / 64, R = kvq::stream_ring_slots(D, DEEP != 0);
    using W = kvq::Waits<KL, R>;
    std::printf("%d %d %d", D, DEEP, R);
    for (int p = 0; p < KL; ++p) std::printf(" %d", W::qk(p));
    for (int u = 0; u < KL; ++u) std::printf(" %d", W::pv(u));
    std::printf("\n");
}
int main() { dump<64, 0>(); dump<64, 1>(); dump<128, 0>(); dump<128, 1>(); dump<256, 0>(); dump<256, 1>(); }
''')
    exe = str(tmp_path / "waits")
    subprocess.run(["g++", "-std=c++17", "-O0", "-o", exe, str(src)], check=True, capture_output=True)
    out = {}
    for line in subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split("\n"):
        if line.strip():
            f = [int(x) for x in line.split()]
            D, deep, R, KL = f[0], f[1], f[2], f[0] // 64
            out[(D, deep)] = (R, f[3:3 + KL], f[3 + KL:3 + 2 * KL])
    return out


def simulate(KL, R, qk, pv, n_chunks):
    """Returns [(what, table count, requests issued after the needed ones)]
    for every wait of a wave that streams n_chunks chunks."""
    NP = 3 * KL
    issued = []

    def after(item):
        return len(issued) - 1 - issued.index(item)

    # the first chunk, before the loop: the refills a previous chunk's reads
    # of pieces NP-R .. would have issued, K scales after the QK slices, V
    # scales last
    for J in range(2 * KL):
        if J + R >= NP:
            issued.append((0, "p", J + R - NP))
    issued.append((0, "ks"))
    for J in range(2 * KL, NP):
        if J + R >= NP:
            issued.append((0, "p", J + R - NP))
    issued.append((0, "vs"))

    waits = []
    for k in range(n_chunks):
        more = k + 1 < n_chunks

        def refill(J):
            jn = J + R
            if jn < NP:
                issued.append((k, "p", jn))
            elif more:
                issued.append((k + 1, "p", jn - NP))

        for p in range(KL):
            need = [(k, "p", 2 * p), (k, "p", 2 * p + 1)] + ([(k, "ks")] if p == 0 else [])
            waits.append((f"chunk {k} qk {p}", qk[p] if more else 0, min(after(x) for x in need)))
            refill(2 * p)
            refill(2 * p + 1)
        if more:
            issued.append((k + 1, "ks"))
        for u in range(KL):
            need = [(k, "p", 2 * KL + u)] + ([(k, "vs")] if u == 0 else [])
            waits.append((f"chunk {k} pv {u}", pv[u] if more else 0, min(after(x) for x in need)))
            refill(2 * KL + u)
        if more:
            issued.append((k + 1, "vs"))
    # every piece of every chunk was requested exactly once
    assert sorted(x for x in issued if x[1] == "p") == sorted((c, "p", j) for c in range(n_chunks) for j in range(NP))
    return waits


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_wait_counts_never_exceed_the_requests_issued_since(tmp_path):
    table = _table(tmp_path)
    assert sorted(table) == CASES
    for D, deep in CASES:
        R, qk, pv = table[(D, deep)]
        KL = D // 64
        assert (3 * KL) % R == 0 and R <= 3 * KL
        for n_chunks in range(1, 70):
            for what, count, margin in simulate(KL, R, qk, pv, n_chunks):
                assert 0 <= count <= margin, f"D={D} deep={deep} R={R} {n_chunks} chunks, {what}: waits for {count} " \
                                             f"but only {margin} requests follow the needed one"


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_wait_counts_are_tight_in_the_steady_state(tmp_path):
    """The table is exact: in every chunk but the last each count equals the
    requests issued since the needed one (a smaller count would only cost
    time, not correctness)."""
    table = _table(tmp_path)
    for D, deep in CASES:
        R, qk, pv = table[(D, deep)]
        for what, count, margin in simulate(D // 64, R, qk, pv, 8):
            if not what.startswith("chunk 7"):
                assert count == margin, f"D={D} deep={deep}: {what} waits for {count}, {margin} follow"


def test_simulation_catches_a_count_one_too_high():
    """The check is not vacuous: one more than a steady-state count fails."""
    KL, R = 4, 4
    base = simulate(KL, R, [99] * KL, [99] * KL, 3)
    exact = {w: m for w, _, m in base}
    qk = [exact[f"chunk 1 qk {p}"] for p in range(KL)]
    pv = [exact[f"chunk 1 pv {u}"] for u in range(KL)]
    assert all(c <= m for _, c, m in simulate(KL, R, qk, pv, 3))
    qk[2] += 1
    assert any(c > m for _, c, m in simulate(KL, R, qk, pv, 3))
