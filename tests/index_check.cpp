// Host-side replay of the kernels' index arithmetic (CPU only, no GPU calls).
//
// For many shapes it builds the library's own Plan and walks every thread of every
// reduction and elementwise kernel exactly as the kernels' loops do -- with the
// library's own ChannelWalk / FlatNCHWWalk helpers -- and checks that each access
// stays inside its buffer, that the walks agree with the direct index formulas,
// and that every element is visited exactly once.  Exit status 0 means all held.
#include <cstdio>
#include <algorithm>
#include <cstdlib>
#include <random>
#include <vector>

#include "device.hpp"
#include "fused.hpp"
#include "plan.hpp"

using namespace iabn;

static int failures = 0;
#define CHECK(cond, ...)                                                 \
    do {                                                                 \
        if (!(cond)) {                                                   \
            if (failures < 20) { std::printf("FAIL %s:%d ", __FILE__, __LINE__); \
                                 std::printf(__VA_ARGS__); std::printf("\n"); } \
            ++failures;                                                  \
        }                                                                \
    } while (0)

struct Shape { int64_t N, C, H, W; int layout, dtype; };

static void check_plan(const Shape& s, bool vec)
{
    const Plan pl = make_plan(s.N, s.C, s.H, s.W, s.layout, s.dtype, vec);
    const int V = pl.V;
    const int64_t numel = pl.numel, nvec = numel / V, C = pl.C, m = pl.m;
    if (numel == 0) return;
    CHECK(numel % V == 0, "numel %% V");
    CHECK(pl.P >= 1 && pl.unit >= 1, "P/unit");
    if (pl.layout == kNCHW)
        CHECK(pl.P * pl.unit >= m && (pl.P - 1) * pl.unit < m, "partials cover m exactly");
    CHECK(pl.reduce_blocks < (int64_t(1) << 31) && pl.apply_blocks < (int64_t(1) << 31), "grid");
    CHECK(pl.off_const == kWsHeaderBytes && pl.off_part_a >= kWsHeaderBytes + size_t(C) * 16, "const section");
    CHECK(pl.P_bwd >= 1 && (pl.layout == kNHWC || pl.P_bwd == pl.P), "backward partials");
    CHECK(pl.reduce_blocks_bwd < (int64_t(1) << 31), "backward grid");
    const int64_t Pmax = std::max(pl.P, pl.P_bwd);
    CHECK(pl.off_part_b >= pl.off_part_a + size_t(Pmax * C) * 4, "part a section");
    CHECK(pl.off_count >= pl.off_part_b + size_t(Pmax * C) * 4, "part b section");
    CHECK(pl.bytes >= pl.off_count + size_t(pl.P) * 4, "count section");
    CHECK(pl.off_part_a % 256 == 0 && pl.off_part_b % 256 == 0, "alignment");

    std::vector<uint8_t> seen(size_t(nvec), 0);
    // ---- reduction kernels (the statistics; NCHW backward sums share the tiling)
    if (pl.layout == kNCHW) {
        const int64_t HWv = pl.HW / V;
        CHECK(pl.HW % V == 0 && pl.unit % V == 0, "NCHW vector alignment");
        CHECK(pl.reduce_blocks == C * pl.P, "NCHW grid");
        for (int64_t b = 0; b < pl.reduce_blocks; ++b) {
            const int64_t c = b / pl.P, p = b - c * pl.P;
            CHECK(c * pl.HW < numel, "pivot");
            const int64_t j1 = std::min(p * pl.unit + pl.unit, m) / V;
            for (int t = 0; t < kThreads; ++t) {
                int64_t j = p * pl.unit / V + t;
                ChannelWalk w;
                w.init(j < j1 ? j : 0, c, C, HWv, kThreads);
                for (; j < j1; j += kThreads) {
                    const int64_t direct = ((j / HWv) * C + c) * HWv + j % HWv;
                    CHECK(w.addr == direct, "ChannelWalk b=%lld t=%d j=%lld", (long long)b, t,
                          (long long)j);
                    CHECK(w.addr >= 0 && w.addr < nvec, "reduce bounds");
                    if (w.addr >= 0 && w.addr < nvec) seen[size_t(w.addr)]++;
                    w.step();
                }
            }
        }
        for (int64_t i = 0; i < nvec; ++i)
            CHECK(seen[size_t(i)] == 1, "reduction visits vector %lld %d times", (long long)i,
                  int(seen[size_t(i)]));
    } else {
        // the statistics (P partials) and the backward sums (P_bwd) walk the same
        // row groups with their own grid
        auto walk = [&](int64_t P, int64_t blocks, const char* what) {
            std::fill(seen.begin(), seen.end(), 0);
            const int64_t Cv = C / V;
            CHECK(C % V == 0, "NHWC vector alignment");
            CHECK(kThreads % pl.tpr == 0, "tpr divides the workgroup");
            CHECK(pl.slices * pl.tpr >= Cv, "slices cover the row");
            CHECK(blocks == pl.slices * P, "NHWC grid (%s)", what);
            const int rpi = kThreads / pl.tpr;
            CHECK(pl.unit == (m + rpi - 1) / rpi, "row groups");
            CHECK(P <= pl.unit, "no empty partial (%s)", what);
            for (int64_t b = 0; b < blocks; ++b) {
                const int64_t p = b / pl.slices, sl = b - p * pl.slices;
                for (int t = 0; t < kThreads; ++t) {
                    const int rs = t / pl.tpr;
                    const int64_t col = sl * pl.tpr + (t - rs * pl.tpr);
                    if (col >= Cv) continue;
                    CHECK(p * C + col * V + V <= Pmax * C, "partial index (%s)", what);
                    for (int64_t g = p; g < pl.unit; g += P) {
                        const int64_t r = g * rpi + rs;
                        if (r >= m) continue;
                        const int64_t a = r * Cv + col;
                        CHECK(a >= 0 && a < nvec, "NHWC reduce bounds (%s)", what);
                        if (a >= 0 && a < nvec) seen[size_t(a)]++;
                    }
                    // LDS tree partners stay inside the workgroup
                    for (int st = rpi / 2; st >= 1; st >>= 1)
                        if (rs < st) CHECK(t + st * pl.tpr < kThreads, "LDS partner");
                }
            }
            for (int64_t i = 0; i < nvec; ++i)
                CHECK(seen[size_t(i)] == 1, "%s visits vector %lld %d times", what,
                      (long long)i, int(seen[size_t(i)]));
        };
        walk(pl.P, pl.reduce_blocks, "statistics");
        walk(pl.P_bwd, pl.reduce_blocks_bwd, "backward sums");
    }

    // ---- elementwise kernels (the grid for leaky ReLU and identity, and for ELU)
    CHECK(pl.apply_blocks_elu < (int64_t(1) << 31), "ELU grid");
    auto elementwise = [&](int64_t blocks) {
        std::fill(seen.begin(), seen.end(), 0);
        const int64_t stride = blocks * kThreads;
        if (pl.layout == kNCHW) {
            const int64_t HWv = pl.HW / V;
            for (int64_t t0 = 0; t0 < stride; ++t0) {
                int64_t v = t0;
                FlatNCHWWalk w;
                w.init(v < nvec ? v : 0, C, HWv, stride);
                for (; v < nvec; v += stride) {
                    CHECK(w.c == (v / HWv) % C, "FlatNCHWWalk v=%lld", (long long)v);
                    CHECK(w.c >= 0 && w.c < C, "channel bounds");
                    seen[size_t(v)]++;
                    w.step();
                }
            }
        } else {
            const int64_t Cv = C / V;
            if (pl.fixed_col) CHECK(stride % Cv == 0, "fixed channel group needs stride %% Cv == 0");
            for (int64_t t0 = 0; t0 < stride; ++t0) {
                if (t0 >= nvec) break;
                const int64_t c0 = (t0 % Cv) * V;
                CHECK(c0 + V - 1 < C, "channel group bounds");
                for (int64_t v = t0; v < nvec; v += stride) {
                    if (pl.fixed_col) CHECK((v % Cv) * V == c0, "fixed channel group");
                    seen[size_t(v)]++;
                }
            }
        }
        for (int64_t i = 0; i < nvec; ++i)
            CHECK(seen[size_t(i)] == 1, "elementwise visits vector %lld %d times", (long long)i,
                  int(seen[size_t(i)]));
    };
    elementwise(pl.apply_blocks);
    elementwise(pl.apply_blocks_elu);

    // ---- channel-resident NCHW kernels: every variant that could hold the channel
    if (pl.layout == kNCHW && pl.vec && numel * pl.esize < (int64_t(1) << 32)) {
        const int64_t HWv = pl.HW / V, Vc = m / V;
        struct Var { int T, NR; };
        std::vector<Var> vars;
#define IABN_ROW(ID, T, NR) vars.push_back({T, NR});
        IABN_FUSED_FWD_VARIANTS(IABN_ROW)
#undef IABN_ROW
#define IABN_ROW(ID, T, NRV, NRL, G, DYR) vars.push_back({T, NRV + NRL});
        IABN_FUSED_BWD_VARIANTS(IABN_ROW)
#undef IABN_ROW
        for (const Var& vv : vars) {
            if (int64_t(vv.T) * vv.NR < Vc) continue;           // the plan never picks it
            if (nvec > 20000000 && vv.T * vv.NR > 4 * Vc) continue;  // keep big shapes quick
            std::fill(seen.begin(), seen.end(), 0);
            for (int64_t c = 0; c < C; ++c)
                for (int t = 0; t < vv.T; ++t) {
                    ChannelWalk32 w;
                    w.init(uint32_t(t), uint32_t(c), uint32_t(C), uint32_t(HWv), uint32_t(vv.T));
                    for (int k = 0; k < vv.NR; ++k) {
                        const int64_t j = t + int64_t(k) * vv.T;
                        if (j < Vc) {
                            const int64_t direct = ((j / HWv) * C + c) * HWv + j % HWv;
                            CHECK(int64_t(w.off) == direct, "ChannelWalk32 c=%lld t=%d k=%d",
                                  (long long)c, t, k);
                            CHECK(int64_t(w.off) < nvec, "fused bounds");
                            CHECK((int64_t(w.off) << 4) < (int64_t(1) << 32), "byte offset");
                            if (int64_t(w.off) < nvec) seen[size_t(w.off)]++;
                        }
                        w.step();
                    }
                }
            for (int64_t i = 0; i < nvec; ++i)
                CHECK(seen[size_t(i)] == 1, "fused T=%d NR=%d visits %lld %d times", vv.T, vv.NR,
                      (long long)i, int(seen[size_t(i)]));
        }
    }

    // ---- channel-resident NCHW kernels in groups: the group the plan takes at 256
    // CUs, each member's share walked from its first vector
    {
        const NchwGroupChoice gc = fused_nchw_group_pick(pl, 256);
        if (gc.group > 1) {
            const int64_t HWv = pl.HW / V, Vc = m / V, G = gc.group;
            const int64_t share = (Vc + G - 1) / G;
            CHECK(C * G <= 256, "group grid within the CUs");
            CHECK((G - 1) * share < Vc, "every member holds vectors");
            const int64_t words = nhwc_exchange_words(C, G, C);
            CHECK(((C + 31) / 32) * 32 + (C - 1) * G * 4 + (G - 1) * 4 + 3 < words, "exchange words");
            for (const int var : {gc.fwd, gc.bwd}) {
                const int T = var == gc.fwd ? fused_fwd_threads(var) : fused_bwd_threads(var);
                int NR = 0;
                if (var == gc.fwd) {
#define IABN_ROW(ID, T_, NR_) if (ID == var) NR = NR_;
                    IABN_FUSED_FWD_VARIANTS(IABN_ROW)
#undef IABN_ROW
                } else {
#define IABN_ROW(ID, T_, NRV, NRL, G_, DYR) if (ID == var) NR = NRV + NRL;
                    IABN_FUSED_BWD_VARIANTS(IABN_ROW)
#undef IABN_ROW
                }
                CHECK(int64_t(T) * NR >= share, "variant holds the share");
                std::fill(seen.begin(), seen.end(), 0);
                for (int64_t c = 0; c < C; ++c)
                    for (int64_t j = 0; j < G; ++j) {
                        const int64_t v0 = j * share, v1 = std::min(Vc, v0 + share);
                        for (int t = 0; t < T; ++t) {
                            ChannelWalk32 w;
                            w.init(uint32_t(v0 + t), uint32_t(c), uint32_t(C), uint32_t(HWv),
                                   uint32_t(T));
                            for (int k = 0; k < NR; ++k) {
                                const int64_t v = v0 + t + int64_t(k) * T;
                                if (v < v1) {
                                    const int64_t direct = ((v / HWv) * C + c) * HWv + v % HWv;
                                    CHECK(int64_t(w.off) == direct, "group walk c=%lld j=%lld t=%d",
                                          (long long)c, (long long)j, t);
                                    CHECK((int64_t(w.off) << 4) < (int64_t(1) << 32), "byte offset");
                                    if (int64_t(w.off) < nvec) seen[size_t(w.off)]++;
                                }
                                w.step();
                            }
                        }
                    }
                for (int64_t i = 0; i < nvec; ++i)
                    CHECK(seen[size_t(i)] == 1, "grouped T=%d NR=%d G=%lld visits %lld %d times",
                          T, NR, (long long)G, (long long)i, int(seen[size_t(i)]));
            }
        }
    }

    // ---- channel-resident NCHW kernels on single elements (off the vector path)
    if (pl.layout == kNCHW && !pl.vec && numel * pl.esize < (int64_t(1) << 32)) {
        const int64_t HW = pl.HW;
        struct Var { int T, NR; };
        std::vector<Var> vars;
#define IABN_ROW(ID, T, NR) vars.push_back({T, NR});
        IABN_FUSED_SCALAR_VARIANTS(IABN_ROW)
#undef IABN_ROW
        for (const Var& vv : vars) {
            if (int64_t(vv.T) * vv.NR < m) continue;            // the plan never picks it
            if (numel > 20000000 && vv.T * vv.NR > 4 * m) continue;
            std::fill(seen.begin(), seen.end(), 0);
            for (int64_t c = 0; c < C; ++c)
                for (int t = 0; t < vv.T; ++t) {
                    ChannelWalk32 w;
                    w.init(uint32_t(t), uint32_t(c), uint32_t(C), uint32_t(HW), uint32_t(vv.T));
                    for (int k = 0; k < vv.NR; ++k) {
                        const int64_t j = t + int64_t(k) * vv.T;
                        if (j < m) {
                            const int64_t direct = ((j / HW) * C + c) * HW + j % HW;
                            CHECK(int64_t(w.off) == direct, "scalar walk c=%lld t=%d k=%d",
                                  (long long)c, t, k);
                            CHECK(int64_t(w.off) < numel, "scalar bounds");
                            CHECK(int64_t(w.off) * pl.esize < (int64_t(1) << 32), "byte offset");
                            if (int64_t(w.off) < numel) seen[size_t(w.off)]++;
                        }
                        w.step();
                    }
                }
            for (int64_t i = 0; i < numel; ++i)
                CHECK(seen[size_t(i)] == 1, "scalar T=%d NR=%d visits %lld %d times", vv.T, vv.NR,
                      (long long)i, int(seen[size_t(i)]));
        }
    }

    // ---- slice-resident NHWC kernels: every variant and group size the plan could
    // take (rows of each member fit; groups: slices % 8 == 0, no empty member)
    if (pl.layout == kNHWC && pl.vec && numel * pl.esize < (int64_t(1) << 32)) {
        const int64_t cv = C / V;
        struct Var { int T, LPR, NR; };
        std::vector<Var> vars;
#define IABN_ROW(ID, T, LPR, NR) vars.push_back({T, LPR, NR});
        IABN_FUSED_NHWC_VARIANTS(IABN_ROW)
#undef IABN_ROW
        for (const Var& vv : vars) {
            for (uint32_t G = 1; G <= 64; G *= 2) {
                const int64_t rps = vv.T / vv.LPR;
                if (cv % vv.LPR != 0) continue;
                const uint32_t slices = uint32_t(cv / vv.LPR);
                const int64_t mg = (m + G - 1) / G;
                if (rps * vv.NR < mg) continue;                       // never picked
                if (G > 1 && (slices % 8 != 0 || int64_t(G - 1) * mg >= m)) continue;
                const int64_t words = nhwc_exchange_words(slices, G, C);
                const uint32_t nch = uint32_t(V * vv.LPR);
                std::fill(seen.begin(), seen.end(), 0);
                std::vector<int> pair_seen(size_t(slices) * G, 0);
                for (uint32_t b = 0; b < slices * G; ++b) {
                    uint32_t sl, member;
                    nhwc_group_member(b, slices, G, sl, member);
                    CHECK(sl < slices && member < G, "slice map bounds");
                    if (sl >= slices || member >= G) continue;
                    pair_seen[size_t(sl) * G + member]++;
                    const uint32_t r0 = member * uint32_t(mg);
                    const uint32_t r1 = std::min(uint32_t(m), r0 + uint32_t(mg));
                    CHECK(r0 < r1, "member %u of %u has no rows", member, G);
                    if (G > 1) {
                        // epoch, and this member's tagged words for every channel
                        CHECK(int64_t(sl) < ((int64_t(slices) + 31) & ~int64_t(31)), "epoch");
                        const int64_t w0 = ((int64_t(slices) + 31) & ~int64_t(31)) +
                                           int64_t(sl) * G * nch * 4;
                        for (uint32_t j = 0; j < G; ++j)
                            CHECK(w0 + (int64_t(j) * nch + nch - 1) * 4 + 3 < words,
                                  "exchange words");
                    }
                    for (int t = 0; t < vv.T; ++t) {
                        const uint32_t lane = uint32_t(t) % uint32_t(vv.LPR);
                        const uint32_t rb = r0 + uint32_t(t) / uint32_t(vv.LPR);
                        const uint32_t col = sl * uint32_t(vv.LPR) + lane;
                        CHECK(col < cv, "slice column");
                        for (int k = 0; k < vv.NR; ++k) {
                            const uint32_t row = rb + uint32_t(k) * uint32_t(rps);
                            // the clamped load stays inside the member's rows
                            const uint32_t lrow = std::min(row, r1 - 1);
                            CHECK(lrow >= r0 && int64_t(lrow) * cv + col < nvec, "load bounds");
                            if (row < r1) {
                                const uint32_t idx = row * uint32_t(cv) + col;
                                CHECK(int64_t(idx) == int64_t(row) * cv + col, "32-bit index");
                                CHECK(int64_t(idx) < nvec, "slice bounds");
                                if (int64_t(idx) < nvec) seen[size_t(idx)]++;
                            }
                        }
                    }
                }
                for (size_t q = 0; q < pair_seen.size(); ++q)
                    CHECK(pair_seen[q] == 1, "slice/member %zu taken %d times", q, pair_seen[q]);
                for (int64_t i = 0; i < nvec; ++i)
                    CHECK(seen[size_t(i)] == 1, "slice T=%d LPR=%d NR=%d G=%u visits %lld %d times",
                          vv.T, vv.LPR, vv.NR, G, (long long)i, int(seen[size_t(i)]));
            }
        }
        // streamed slice kernels: every variant and group size 8..32, the forward's
        // and the backward's (resident rows, chunk) split
        struct SVar { int T, LPR, NR, L, U, streams; };
        std::vector<SVar> svars;
#define IABN_ROW(ID, T, LPR, NRF, LF, UF, NRB, LB, UB) \
    svars.push_back({T, LPR, NRF, LF, UF, 1}); svars.push_back({T, LPR, NRB, LB, UB, 2});
        IABN_STREAM_NHWC_VARIANTS(IABN_ROW)
#undef IABN_ROW
        for (const SVar& sv : svars) {
            CHECK(sv.L % sv.U == 0, "LDS rows are whole chunks");
            // the LDS rows (16 B per thread, row and stream) fit 160 KB beside the
            // scatter rows
            CHECK(size_t(sv.L) * sv.T * 16 * sv.streams <= size_t(136) * 1024, "LDS rows fit");
        }
        for (const SVar& sv : svars) {
            for (uint32_t G = 8; G <= 64; G *= 2) {
                if (cv % sv.LPR != 0) continue;
                const uint32_t slices = uint32_t(cv / sv.LPR);
                const int64_t mg = (m + G - 1) / G;
                if (int64_t(G - 1) * mg >= m) continue;
                const uint32_t RPS = uint32_t(sv.T / sv.LPR);
                std::fill(seen.begin(), seen.end(), 0);
                std::vector<int> pair_seen(size_t(slices) * G, 0);
                for (uint32_t b = 0; b < slices * G; ++b) {
                    uint32_t sl, member;
                    nhwc_stream_member(b, slices, sl, member);
                    CHECK(sl < slices && member < G, "stream map bounds");
                    if (sl >= slices || member >= G) continue;
                    CHECK(member % 8 == b % 8, "stream member on XCD b %% 8");
                    pair_seen[size_t(sl) * G + member]++;
                    const uint32_t r0 = member * uint32_t(mg);
                    const uint32_t r1 = std::min(uint32_t(m), r0 + uint32_t(mg));
                    CHECK(r0 < r1, "stream member %u has no rows", member);
                    const uint32_t nk = (r1 - r0 + RPS - 1) / RPS;
                    const uint32_t nchunk = nk > uint32_t(sv.NR) ? (nk - sv.NR + sv.U - 1) / sv.U : 0;
                    for (int t = 0; t < sv.T; ++t) {
                        const uint32_t lane = uint32_t(t) % uint32_t(sv.LPR);
                        const uint32_t rb = r0 + uint32_t(t) / uint32_t(sv.LPR);
                        const uint32_t col = sl * uint32_t(sv.LPR) + lane;
                        auto visit = [&](uint32_t row) {
                            const uint32_t lrow = std::min(row, r1 - 1);
                            CHECK(int64_t(lrow) * cv + col < nvec, "stream load bounds");
                            if (row < r1) {
                                const uint32_t idx = row * uint32_t(cv) + col;
                                CHECK(int64_t(idx) == int64_t(row) * cv + col, "stream 32-bit index");
                                if (int64_t(idx) < nvec) seen[size_t(idx)]++;
                            }
                        };
                        for (int k = 0; k < sv.NR; ++k) visit(rb + uint32_t(k) * RPS);
                        for (uint32_t c = 0; c < nchunk; ++c)
                            for (int u = 0; u < sv.U; ++u) visit(rb + (uint32_t(sv.NR) + c * sv.U + u) * RPS);
                    }
                }
                for (size_t q = 0; q < pair_seen.size(); ++q)
                    CHECK(pair_seen[q] == 1, "stream slice/member %zu taken %d times", q, pair_seen[q]);
                for (int64_t i = 0; i < nvec; ++i)
                    CHECK(seen[size_t(i)] == 1, "stream T=%d LPR=%d NR=%d U=%d G=%u visits %lld %d times",
                          sv.T, sv.LPR, sv.NR, sv.U, G, (long long)i, int(seen[size_t(i)]));
            }
        }
        // the plan's own choice obeys the group rules at the MI355X's 256 CUs
        const NhwcChoice ch = fused_nhwc_pick(pl, 256);
        if (ch.variant >= 0 && ch.group > 1) {
            int lpr = 0;
            switch (ch.variant) {
#define IABN_ROW(ID, T, LPR, NR) case ID: lpr = LPR; break;
                IABN_FUSED_NHWC_VARIANTS(IABN_ROW)
#undef IABN_ROW
            default: break;
            }
            CHECK(lpr > 0 && cv % lpr == 0 && (cv / lpr) % 8 == 0, "group slices");
            CHECK(lpr > 0 && (cv / lpr) * ch.group <= 256, "group grid within the CUs");
        }
    }
}

int main(int argc, char** argv)
{
    std::vector<Shape> shapes = {
        {2, 4, 8, 8, kNCHW, kF32},      {32, 256, 56, 56, kNCHW, kF32},
        {32, 64, 112, 112, kNCHW, kF32}, {32, 64, 112, 112, kNCHW, kBF16},
        {4, 16, 300, 300, kNCHW, kF32}, {3, 16, 100, 97, kNCHW, kF32}, {5, 8, 130, 128, kNCHW, kBF16},
        {2, 256, 512, 512, kNHWC, kBF16}, {16, 512, 28, 28, kNCHW, kF32},
        {64, 2048, 7, 7, kNHWC, kBF16},
        {4, 6, 16, 20, kNCHW, kF32}, {3, 5, 17, 19, kNCHW, kF32}, {4, 6, 16, 20, kNCHW, kBF16},
        {3, 5, 17, 19, kNCHW, kBF16}, {3, 24, 9, 11, kNHWC, kF32}, {2, 13, 10, 7, kNHWC, kF32},
        {2, 200, 12, 12, kNHWC, kF32}, {3, 24, 9, 11, kNHWC, kBF16}, {2, 13, 10, 7, kNHWC, kBF16},
        {2, 200, 12, 12, kNHWC, kBF16}, {2, 5, 1, 1, kNCHW, kF32}, {1, 1, 300, 301, kNCHW, kF32},
        {2, 4104, 3, 3, kNHWC, kBF16}, {2, 4104, 3, 3, kNHWC, kF32}, {2, 64, 3, 1, kNCHW, kF32},
        {3, 8, 1, 1, kNHWC, kBF16}, {8, 32, 28, 28, kNCHW, kF32}, {4, 64, 32, 32, kNHWC, kBF16},
        {4, 32, 14, 14, kNCHW, kF32}, {8, 512, 7, 7, kNHWC, kBF16}, {4, 64, 16, 16, kNCHW, kF32},
        {4, 64, 16, 16, kNHWC, kBF16}, {4, 32, 12, 12, kNCHW, kF32}, {4, 256, 12, 12, kNHWC, kBF16},
        {2, 16, 8, 8, kNCHW, kF32}, {2, 16, 8, 8, kNHWC, kBF16}, {2, 16, 8, 8, kNCHW, kBF16},
        {2, 16, 8, 8, kNHWC, kF32},      {64, 1024, 7, 7, kNHWC, kF32}, {32, 2048, 14, 14, kNHWC, kBF16},
        {2, 64, 1, 1, kNHWC, kBF16},     {5, 96, 11, 13, kNHWC, kBF16},   {3, 40, 7, 9, kNHWC, kF32},
        {32, 64, 7, 7, kNCHW, kF32},     {500, 3, 7, 7, kNCHW, kBF16},    {10, 5, 7, 7, kNCHW, kF32},
        {8, 512, 28, 28, kNHWC, kBF16},  {64, 256, 14, 14, kNHWC, kBF16}, {32, 512, 28, 28, kNHWC, kBF16},
        {32, 1024, 14, 14, kNHWC, kBF16}, {32, 256, 28, 28, kNHWC, kF32}, {7, 512, 9, 13, kNHWC, kBF16},
        {3, 1024, 11, 17, kNHWC, kF32},  {2, 256, 200, 200, kNHWC, kBF16}, {8, 256, 56, 56, kNHWC, kBF16},
        {5, 128, 99, 101, kNHWC, kF32},   {2, 64, 256, 260, kNHWC, kBF16},
        // one element per channel (the inference passes take m = 1)
        {1, 65536, 1, 1, kNCHW, kF32},   {1, 1, 1, 65536, kNCHW, kF32},   {1, 4096, 1, 1, kNHWC, kBF16},
    };
    std::mt19937_64 rng(12345);
    const int n_random = argc > 1 ? std::atoi(argv[1]) : 300;
    for (int i = 0; i < n_random; ++i) {
        Shape s;
        s.N = 1 + rng() % 9; s.C = 1 + rng() % 300; s.H = 1 + rng() % 17; s.W = 1 + rng() % 17;
        s.layout = int(rng() % 2); s.dtype = int(rng() % 2);
        if (s.N * s.H * s.W < 2) s.N = 2;
        shapes.push_back(s);
    }
    int checked = 0;
    for (const Shape& s : shapes) {
        check_plan(s, false);
        if (vec_shape_ok(s.C, s.H * s.W, s.layout, s.dtype)) check_plan(s, true);
        ++checked;
        if (failures) {
            std::printf("shape N=%lld C=%lld H=%lld W=%lld layout=%d dtype=%d\n", (long long)s.N,
                        (long long)s.C, (long long)s.H, (long long)s.W, s.layout, s.dtype);
            return 1;
        }
    }
    std::printf("OK %d shapes\n", checked);
    return 0;
}
