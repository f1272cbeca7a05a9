// Driver for the sanitizer build of the library's host-only code: the gather layout, the
// EPLB placement (balancedness, hierarchical rebalance, logical-to-physical table) and the
// status strings.  Built with -fsanitize=address,undefined -fno-sanitize-recover=all on the
// host side; it makes no GPU call.  Every argument check is driven to its error return, and
// every successful result is checked against properties any correct placement has.  An
// out-of-bounds access or undefined behaviour aborts; a failed property exits with status 2.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <vector>

#include "moe.h"

static int failures = 0;
#define EXPECT(c)                                                                 \
    do {                                                                          \
        if (!(c)) {                                                               \
            std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

static uint64_t rng_state = 0x243F6A8885A308D3ull;
static uint32_t rnd() {  // splitmix64, upper half
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return static_cast<uint32_t>((z ^ (z >> 31)) >> 32);
}

static void check_status_strings() {
    for (int s = -2; s <= 8; ++s) {
        const char* t = moe_status_string(static_cast<moe_status>(s));
        EXPECT(t != nullptr && std::strlen(t) > 0);
    }
    EXPECT(std::strstr(moe_version(), "gfx950") != nullptr);
}

static void check_layout_case(const std::vector<int32_t>& n, moe_pad_mode mode, int is_extend, int idle,
                              int bound) {
    const int W = static_cast<int>(n.size());
    moe_gather_layout_t L;
    std::memset(&L, 0xAB, sizeof L);
    const moe_status s = moe_gather_layout(n.data(), W, mode, is_extend, idle, bound, &L);
    EXPECT(s == MOE_OK);
    if (s != MOE_OK) return;
    EXPECT(L.num_replicas == W);
    EXPECT(L.mode == MOE_PAD_MAX_LEN || L.mode == MOE_PAD_SUM_LEN);
    if (mode != MOE_PAD_AUTO) EXPECT(L.mode == mode);
    EXPECT(L.offsets[0] == 0 && L.offsets[W] == L.rows);
    int64_t sum = 0;
    for (int i = 0; i < W; ++i) {
        EXPECT(L.sizes[i] == (bound > 0 ? bound : n[i]));
        EXPECT(L.offsets[i + 1] - L.offsets[i] >= (L.rows ? L.sizes[i] : 0));
        sum += L.sizes[i];
    }
    if (sum == 0) EXPECT(L.rows == 0);
    else if (L.mode == MOE_PAD_SUM_LEN) EXPECT(L.rows == sum);
}

static void check_layout() {
    const int widths[] = {1, 2, 3, 8, 33, MOE_MAX_REPLICAS};
    for (int W : widths)
        for (int rep = 0; rep < 4; ++rep) {
            std::vector<int32_t> n(W);
            int32_t mx = 0;
            for (int i = 0; i < W; ++i) {
                n[i] = (rnd() % 4 == 0) ? 0 : static_cast<int32_t>(rnd() % 5000);
                if (rep == 3) n[i] = 0;  // every replica idle
                mx = n[i] > mx ? n[i] : mx;
            }
            for (int m = MOE_PAD_AUTO; m <= MOE_PAD_SUM_LEN; ++m)
                for (int ext = 0; ext <= 1; ++ext)
                    for (int idle = 0; idle <= 1; ++idle) {
                        check_layout_case(n, static_cast<moe_pad_mode>(m), ext, idle, 0);
                        check_layout_case(n, static_cast<moe_pad_mode>(m), ext, idle, mx + 7);
                    }
        }
    moe_gather_layout_t L;
    int32_t n[3] = {4, 0, 9};
    EXPECT(moe_gather_layout(nullptr, 3, MOE_PAD_AUTO, 0, 0, 0, &L) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_gather_layout(n, 3, MOE_PAD_AUTO, 0, 0, 0, nullptr) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_gather_layout(n, 0, MOE_PAD_AUTO, 0, 0, 0, &L) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_gather_layout(n, MOE_MAX_REPLICAS + 1, MOE_PAD_AUTO, 0, 0, 0, &L) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_gather_layout(n, 3, static_cast<moe_pad_mode>(7), 0, 0, 0, &L) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_gather_layout(n, 3, MOE_PAD_AUTO, 0, 0, -1, &L) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_gather_layout(n, 3, MOE_PAD_AUTO, 0, 0, 8, &L) == MOE_ERR_INVALID_ARG);  // 9 > bound
    n[1] = -1;
    EXPECT(moe_gather_layout(n, 3, MOE_PAD_AUTO, 0, 0, 0, &L) == MOE_ERR_INVALID_ARG);
}

static void check_balancedness() {
    const int layers = 3, P = 24, gpus = 6;
    std::vector<int64_t> cnt(layers * P);
    for (auto& c : cnt) c = rnd() % 1000;
    for (int s = 0; s < P; ++s) cnt[2 * P + s] = 5;  // perfectly balanced layer
    std::vector<double> out(layers, -1.0);
    EXPECT(moe_eplb_balancedness(cnt.data(), layers, P, gpus, out.data()) == MOE_OK);
    for (int l = 0; l < layers; ++l) EXPECT(out[l] > 0.0 && out[l] <= 1.0);
    EXPECT(std::fabs(out[2] - 1.0) < 1e-12);
    EXPECT(moe_eplb_balancedness(cnt.data(), 0, P, gpus, out.data()) == MOE_OK);
    EXPECT(moe_eplb_balancedness(cnt.data(), layers, P, 5, out.data()) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_eplb_balancedness(nullptr, layers, P, gpus, out.data()) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_eplb_balancedness(cnt.data(), layers, 0, gpus, out.data()) == MOE_ERR_INVALID_ARG);
}

struct Placement {
    int L, E, P, groups, nodes, gpus;
};

static void check_rebalance(const Placement& c, bool zero_heavy) {
    const int L = c.L, E = c.E, P = c.P;
    std::vector<double> w(static_cast<size_t>(L) * E);
    for (auto& v : w) v = zero_heavy && (rnd() % 3 == 0) ? 0.0 : static_cast<double>(rnd() % 100000);
    std::vector<int32_t> phy2log(static_cast<size_t>(L) * P, -9), rank(static_cast<size_t>(L) * P, -9),
        cnt(static_cast<size_t>(L) * E, -9);
    EXPECT(moe_eplb_rebalance(w.data(), L, E, P, c.groups, c.nodes, c.gpus, phy2log.data(), rank.data(),
                              cnt.data()) == MOE_OK);
    const int e_node = E / c.nodes, p_node = P / c.nodes;
    for (int l = 0; l < L; ++l) {
        const int32_t* p2l = &phy2log[static_cast<size_t>(l) * P];
        const int32_t* rk = &rank[static_cast<size_t>(l) * P];
        const int32_t* lc = &cnt[static_cast<size_t>(l) * E];
        std::vector<int> seen(E, 0), node_of(E, -1);
        int total = 0, max_rep = 0;
        for (int e = 0; e < E; ++e) {
            EXPECT(lc[e] >= 1);
            total += lc[e];
            max_rep = lc[e] > max_rep ? lc[e] : max_rep;
        }
        EXPECT(total == P);
        for (int p = 0; p < P; ++p) {
            const int e = p2l[p];
            EXPECT(e >= 0 && e < E);
            if (e < 0 || e >= E) continue;
            EXPECT(rk[p] >= 0 && rk[p] < lc[e]);
            ++seen[e];
            const int nd = p / p_node;  // every replica of an expert stays on one node
            if (node_of[e] < 0) node_of[e] = nd;
            EXPECT(node_of[e] == nd);
        }
        for (int e = 0; e < E; ++e) EXPECT(seen[e] == lc[e]);
        std::vector<int> per_node(c.nodes, 0);
        for (int e = 0; e < E; ++e)
            if (node_of[e] >= 0) ++per_node[node_of[e]];
        for (int nd = 0; nd < c.nodes; ++nd) EXPECT(per_node[nd] == e_node);
        // the dispatch table of the layer
        std::vector<int32_t> phys_of(static_cast<size_t>(E) * max_rep, -9), n_rep(E, -9);
        EXPECT(moe_eplb_logical_to_physical(p2l, rk, P, E, max_rep, phys_of.data(), n_rep.data()) == MOE_OK);
        for (int e = 0; e < E; ++e) {
            EXPECT(n_rep[e] == lc[e]);
            for (int r = 0; r < max_rep; ++r) {
                const int32_t p = phys_of[static_cast<size_t>(e) * max_rep + r];
                if (r < lc[e]) EXPECT(p >= 0 && p < P && p2l[p] == e && rk[p] == r);
                else EXPECT(p == -1);
            }
        }
        if (max_rep > 1)
            EXPECT(moe_eplb_logical_to_physical(p2l, rk, P, E, max_rep - 1, phys_of.data(), n_rep.data()) ==
                   MOE_ERR_CAPACITY);
    }
}

static void check_rebalance_errors() {
    const int E = 8, P = 12;
    std::vector<double> w(E, 1.0);
    std::vector<int32_t> a(P), b(P), c(E);
    EXPECT(moe_eplb_rebalance(w.data(), 1, E, P, 3, 1, 1, a.data(), b.data(), c.data()) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_eplb_rebalance(w.data(), 1, E, P, 4, 3, 3, a.data(), b.data(), c.data()) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_eplb_rebalance(w.data(), 1, E, P, 4, 2, 3, a.data(), b.data(), c.data()) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_eplb_rebalance(w.data(), 1, E, P, 4, 1, 5, a.data(), b.data(), c.data()) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_eplb_rebalance(w.data(), 1, E, 4, 4, 1, 1, a.data(), b.data(), c.data()) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_eplb_rebalance(nullptr, 1, E, P, 4, 1, 1, a.data(), b.data(), c.data()) == MOE_ERR_INVALID_ARG);
    w[3] = -1.0;
    EXPECT(moe_eplb_rebalance(w.data(), 1, E, P, 4, 1, 1, a.data(), b.data(), c.data()) == MOE_ERR_INVALID_ARG);
    w[3] = std::numeric_limits<double>::quiet_NaN();
    EXPECT(moe_eplb_rebalance(w.data(), 1, E, P, 4, 1, 1, a.data(), b.data(), c.data()) == MOE_ERR_INVALID_ARG);
    w[3] = std::numeric_limits<double>::infinity();
    EXPECT(moe_eplb_rebalance(w.data(), 1, E, P, 4, 1, 1, a.data(), b.data(), c.data()) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_eplb_rebalance(w.data(), 0, E, P, 4, 1, 1, a.data(), b.data(), c.data()) == MOE_OK);

    // hand-made tables for the dispatch-table checks: 3 experts on 4 slots
    const int32_t p2l[4] = {0, 1, 2, 1}, rk[4] = {0, 0, 0, 1};
    int32_t phys_of[3 * 3], n_rep[3];  // room for max_rep up to 3
    EXPECT(moe_eplb_logical_to_physical(p2l, rk, 4, 3, 2, phys_of, n_rep) == MOE_OK);
    EXPECT(n_rep[1] == 2 && phys_of[1 * 2 + 1] == 3 && phys_of[0 * 2 + 1] == -1);
    EXPECT(moe_eplb_logical_to_physical(p2l, rk, 4, 3, 1, phys_of, n_rep) == MOE_ERR_CAPACITY);
    const int32_t dup[4] = {0, 0, 0, 0};  // replica 0 of expert 1 twice
    const int32_t p2l_dup[4] = {0, 1, 2, 1};
    EXPECT(moe_eplb_logical_to_physical(p2l_dup, dup, 4, 3, 2, phys_of, n_rep) == MOE_ERR_INVALID_ARG);
    const int32_t gap[4] = {0, 0, 0, 2};  // expert 1 has replicas 0 and 2
    EXPECT(moe_eplb_logical_to_physical(p2l, gap, 4, 3, 3, phys_of, n_rep) == MOE_ERR_INVALID_ARG);
    const int32_t none[4] = {0, 1, 1, 1}, rk_none[4] = {0, 0, 1, 2};  // expert 2 has no slot
    EXPECT(moe_eplb_logical_to_physical(none, rk_none, 4, 3, 3, phys_of, n_rep) == MOE_ERR_INVALID_ARG);
    const int32_t out_of_range[4] = {0, 1, 3, 1};
    EXPECT(moe_eplb_logical_to_physical(out_of_range, rk, 4, 3, 2, phys_of, n_rep) == MOE_ERR_INVALID_ARG);
    const int32_t neg_rank[4] = {0, 0, -1, 1};
    EXPECT(moe_eplb_logical_to_physical(p2l, neg_rank, 4, 3, 2, phys_of, n_rep) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_eplb_logical_to_physical(nullptr, rk, 4, 3, 2, phys_of, n_rep) == MOE_ERR_INVALID_ARG);
}

int main() {
    check_status_strings();
    check_layout();
    check_balancedness();
    const Placement cases[] = {
        {1, 8, 8, 1, 1, 1},       // no redundancy
        {2, 16, 24, 4, 2, 4},     // two nodes, eight redundant slots
        {1, 12, 12, 3, 1, 4},     // one node, one slot each
        {2, 256, 288, 8, 4, 32},  // 256 routed experts, 32 redundant slots, 4 nodes of 8 GPUs
        {1, 64, 128, 8, 8, 16},   // twice as many slots as experts
    };
    for (const Placement& c : cases) {
        check_rebalance(c, false);
        check_rebalance(c, true);
    }
    check_rebalance_errors();
    if (failures) {
        std::fprintf(stderr, "%d check(s) failed\n", failures);
        return 2;
    }
    std::printf("host sanitizer driver: ok\n");
    return 0;
}
