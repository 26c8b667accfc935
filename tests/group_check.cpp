// Host run of the group exchange (place_batchnorm_activation_amd/csrc/group.hpp)
// with one host thread per workgroup (tests/hostshim stands in for HIP).  It
// follows the kernels' call sequence -- read the slice's epoch, form the token,
// exchange, member 0 advances the epoch -- and checks, exit status 0 when all hold:
//  1. every member gets the sums over all members, added in member order (the
//     same bits in every member), for one- and two-level groups, several slices
//     at once and many calls in a row on one workspace; a workspace of garbage
//     and the words of earlier calls are never taken;
//  2. a partial whose four words are not all tagged with this call's token (a
//     torn or stale one) is not taken; once completed, it is;
//  3. a member that never publishes turns the others' sums into NaN after the
//     bounded wait, instead of a hang, and the waiting members record the
//     timeout in the workspace's status word; calls where every member arrives
//     leave the word as it was.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <thread>
#include <vector>

#include "group.hpp"

namespace iabn {
uint64_t process_salt() { return 0x5DEECE66DA3B1C27ull; }
}

using namespace iabn;

static int failures = 0;
#define CHECK(cond, ...)                                                   \
    do {                                                                   \
        if (!(cond)) {                                                     \
            ++failures;                                                    \
            std::printf("FAIL %s:%d: ", __FILE__, __LINE__);               \
            std::printf(__VA_ARGS__);                                      \
            std::printf("\n");                                             \
        }                                                                  \
    } while (0)

// Words of the exchange for `slices` slices of G members, one channel each.
static size_t words_needed(uint32_t slices, uint32_t G) { return ((slices + 31u) & ~31u) + size_t(slices) * G * 4; }

// Sums of member j of slice s in call k: distinct per call and of widely varied
// magnitude, so that only the member-order addition gives the expected bits.
static double part1(int k, uint32_t s, uint32_t j)
{
    return std::ldexp(1.0 + 0.1 * j + 0.01 * k + 0.001 * s, int((j * 7) % 40) - 20);
}
static double part2(int k, uint32_t s, uint32_t j)
{
    return std::ldexp(1.0 / (3.0 + j + k + s), int((j * 11) % 50) - 25);
}

// One member's side of one call (the kernels' order); absent: never publishes.
static void member_call(const SliceGroup& grp, uint32_t s, uint32_t slices, uint32_t j, int k,
                        double& o1, double& o2)
{
    threadIdx.x = 0;
    const uint64_t epoch = __hip_atomic_load(grp.xchg + s, __ATOMIC_RELAXED, 0);
    const uint64_t tok = group_token(grp, s, epoch);
    double s1 = part1(k, s, j), s2 = part2(k, s, j);
    group_sums<1, 1>(grp, s, slices, j, tok, true, s1, s2);
    if (j == 0) __hip_atomic_store(grp.xchg + s, epoch + 1, __ATOMIC_RELAXED, 0);
    o1 = s1;
    o2 = s2;
}

static void run_calls(uint32_t G, uint32_t slices, int calls, uint64_t garbage_seed)
{
    std::vector<uint64_t> ws(words_needed(slices, G));
    std::mt19937_64 rng(garbage_seed);
    for (auto& w : ws) w = rng();                   // whatever the workspace held
    uint64_t status = rng();
    const uint64_t status0 = status;
    SliceGroup grp{ws.data(), process_salt(), G, 1, &status};
    for (int k = 0; k < calls; ++k) {
        std::vector<double> o1(slices * G), o2(slices * G);
        std::vector<std::thread> th;
        for (uint32_t s = 0; s < slices; ++s)
            for (uint32_t j = 0; j < G; ++j)
                th.emplace_back(member_call, std::cref(grp), s, slices, j, k, std::ref(o1[s * G + j]),
                                std::ref(o2[s * G + j]));
        for (auto& t : th) t.join();
        for (uint32_t s = 0; s < slices; ++s) {
            double e1 = 0.0, e2 = 0.0;
            for (uint32_t j = 0; j < G; ++j) {
                e1 += part1(k, s, j);
                e2 += part2(k, s, j);
            }
            for (uint32_t j = 0; j < G; ++j) {
                CHECK(o1[s * G + j] == e1 && o2[s * G + j] == e2,
                      "G=%u slice %u member %u call %d: got (%.17g, %.17g), expected (%.17g, %.17g)", G, s, j, k,
                      o1[s * G + j], o2[s * G + j], e1, e2);
            }
        }
    }
    CHECK(status == status0, "G=%u: status word changed without a timeout", G);
}

// A partner whose words carry this call's tag on words 0-1 only: not taken until
// its last two words are written too.
static void torn_partial()
{
    const uint32_t G = 2, slices = 1;
    std::vector<uint64_t> ws(words_needed(slices, G), 0);
    uint64_t status = 0;
    SliceGroup grp{ws.data(), process_salt(), G, 1, &status};
    const uint64_t tok = group_token(grp, 0, 0);
    uint64_t* words = group_words(grp, 0, slices, 1);
    const uint32_t tlo = uint32_t(tok), thi = uint32_t(tok >> 32);
    const double v1 = 3.5, v2 = -7.25;
    const uint64_t b1 = uint64_t(__double_as_longlong(v1)), b2 = uint64_t(__double_as_longlong(v2));
    uint64_t* w = words + 1 * 4;                    // member 1's slot
    w[0] = tagged(tlo, uint32_t(b1 >> 32));
    w[1] = tagged(thi, uint32_t(b1));
    w[2] = tagged(tlo ^ 1u, uint32_t(b2 >> 32));    // stale tags
    w[3] = tagged(thi ^ 1u, uint32_t(b2));
    double r1 = 0, r2 = 0;
    std::thread reader([&] { group_fetch(words, 1, 1, 0, tok, r1, r2, &status); });
    std::this_thread::sleep_for(std::chrono::milliseconds(20));
    __hip_atomic_store(w + 2, tagged(tlo, uint32_t(b2 >> 32)), __ATOMIC_RELAXED, 0);
    __hip_atomic_store(w + 3, tagged(thi, uint32_t(b2)), __ATOMIC_RELAXED, 0);
    reader.join();
    CHECK(r1 == v1 && r2 == v2, "torn partial: got (%g, %g), expected (%g, %g)", r1, r2, v1, v2);
    CHECK(status == 0, "torn partial completed: status word set");

    // the same torn words, never completed: NaN after the bounded wait
    w[2] = tagged(tlo ^ 1u, uint32_t(b2 >> 32));
    w[3] = tagged(thi ^ 1u, uint32_t(b2));
    group_fetch(words, 1, 1, 0, tok, r1, r2, &status);
    CHECK(std::isnan(r1) && std::isnan(r2), "torn partial never completed: got (%g, %g)", r1, r2);
    CHECK(status == kExchangeTimeout, "torn partial never completed: status word not set");
}

// Member `absent` never runs: the members that wait on it end with NaN.
static void absent_member(uint32_t G, uint32_t absent)
{
    const uint32_t slices = 1;
    std::vector<uint64_t> ws(words_needed(slices, G), 0);
    uint64_t status = 0;
    SliceGroup grp{ws.data(), process_salt(), G, 1, &status};
    std::vector<double> o1(G, 0.0), o2(G, 0.0);
    std::vector<std::thread> th;
    for (uint32_t j = 0; j < G; ++j)
        if (j != absent)
            th.emplace_back(member_call, std::cref(grp), 0u, slices, j, 0, std::ref(o1[j]), std::ref(o2[j]));
    for (auto& t : th) t.join();
    for (uint32_t j = 0; j < G; ++j) {
        if (j == absent) continue;
        CHECK(std::isnan(o1[j]) && std::isnan(o2[j]), "G=%u absent %u: member %u got (%g, %g), expected NaN", G,
              absent, j, o1[j], o2[j]);
    }
    CHECK(status == kExchangeTimeout, "G=%u absent %u: status word not set (%llx)", G, absent,
          (unsigned long long)status);
}

int main()
{
    for (uint32_t G : {2u, 3u, 4u, 5u, 8u, 15u, 16u, 17u, 32u, 64u}) run_calls(G, G <= 8 ? 4 : 2, 6, 1000 + G);
    torn_partial();
    absent_member(4, 3);                            // one level
    absent_member(16, 5);                           // two levels: a member member 0 waits on
    absent_member(16, 0);                           // two levels: member 0 itself
    if (failures) {
        std::printf("FAILED %d checks\n", failures);
        return 1;
    }
    std::printf("OK\n");
    return 0;
}
