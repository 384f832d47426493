// Host-only check of the workspace planner (plan.h), built with the address
// and undefined-behaviour sanitizers by tests/test_plan_sanitized.py.  For a
// sweep of shapes it checks that head chunks cover every query head exactly
// once with the right key/value heads, that trunks cover the sequence, and
// that the carved workspace regions are 256-byte aligned, lie inside the
// total and do not overlap.
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "plan.h"

static int fails = 0;
#define CHECK(c, ...)                                             \
    do {                                                          \
        if (!(c)) {                                               \
            ++fails;                                              \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);  \
            fprintf(stderr, __VA_ARGS__);                         \
            fprintf(stderr, "\n");                                \
        }                                                         \
    } while (0)

struct Region { size_t off, bytes; };

static void check_plan(const hc::Plan& p) {
    // chunks: consecutive, ascending, covering [0, Hq)
    int next = 0;
    for (int c = 0; c < p.nchunks; ++c) {
        const hc::Chunk ch = p.chunk(c);
        CHECK(ch.h0 == next && ch.nh >= 1 && ch.nh <= p.hc, "chunk %d of Hq=%d hc=%d", c, p.Hq, p.hc);
        CHECK(ch.kv0 == ch.h0 / p.g && ch.kv0 + ch.nkv - 1 == (ch.h0 + ch.nh - 1) / p.g,
              "kv heads of chunk %d", c);
        CHECK(ch.nkv <= p.kvc, "kvc");
        next = ch.h0 + ch.nh;
    }
    CHECK(next == p.Hq, "chunks end at %d, Hq=%d", next, p.Hq);
    // trunks cover [0, S)
    int64_t rows = 0;
    for (int64_t t = 0; t < p.N; ++t) {
        CHECK(p.trunk_begin(t) == rows && p.trunk_rows(t) >= 1 && p.trunk_rows(t) <= p.T, "trunk %lld",
              (long long)t);
        rows += p.trunk_rows(t);
    }
    CHECK(rows == p.S, "trunks cover %lld of %lld", (long long)rows, (long long)p.S);
    // regions: sizes as the drivers use them
    const size_t E = (size_t)p.S * p.D * 2, Et = (size_t)p.T * p.D * 2;
    std::vector<Region> r;
    if (!p.bwd) {
        if (!p.trunked) {
            r = {{p.q_c, p.hc * E}, {p.k_c, p.kvc * E}, {p.v_c, p.kvc * E}};
        } else {
            r = {{p.q_c, p.hc * Et}, {p.o_run, p.hc * Et * 2}, {p.o_t, p.hc * Et * 2},
                 {p.l_run, (size_t)p.hc * p.T * 4}, {p.l_t, (size_t)p.hc * p.T * 4},
                 {p.st_l, (size_t)p.hc * p.T * 8}};
            for (int s = 0; s < 2; ++s) {
                r.push_back({p.ring_k[s], p.kvc * Et});
                r.push_back({p.ring_v[s], p.kvc * Et});
            }
        }
    } else {
        const size_t rows_b = p.trunked ? Et : E;
        r = {{p.q_c, p.hc * E}, {p.do_c, p.hc * E}, {p.delta_c, (size_t)p.hc * p.S * 4},
             {p.lse2_c, (size_t)p.hc * p.S * 4}};
        // per-head fp32 partials only in the per-head dK/dV schedule (S below
        // the group-loop threshold)
        CHECK(p.group_loop == (p.S >= hc::kGroupLoopMinS), "group loop at S=%lld", (long long)p.S);
        if (!p.group_loop) {
            r.push_back({p.part_k, p.hc * rows_b * 2});
            r.push_back({p.part_v, p.hc * rows_b * 2});
        }
        if (!p.trunked) {
            r.push_back({p.k_c, p.kvc * E});
            r.push_back({p.v_c, p.kvc * E});
        } else {
            r.push_back({p.dq_acc, p.hc * E * 2});
            for (int s = 0; s < 2; ++s) {
                r.push_back({p.ring_k[s], p.kvc * Et});
                r.push_back({p.ring_v[s], p.kvc * Et});
                r.push_back({p.stage_k[s], p.kvc * Et});
                r.push_back({p.stage_v[s], p.kvc * Et});
            }
        }
        // carries: fp32 [S][D]
        for (int s = 0; s < p.carry_slots; ++s) {
            r.push_back({p.carry_k[s], E * 2});
            r.push_back({p.carry_v[s], E * 2});
        }
    }
    std::sort(r.begin(), r.end(), [](const Region& a, const Region& b) { return a.off < b.off; });
    for (size_t i = 0; i < r.size(); ++i) {
        CHECK(r[i].off % hc::kAlign == 0, "region at %zu not aligned", r[i].off);
        CHECK(r[i].off + r[i].bytes <= p.total, "region [%zu, +%zu) past total %zu", r[i].off,
              r[i].bytes, p.total);
        if (i + 1 < r.size())
            CHECK(r[i].off + r[i].bytes <= r[i + 1].off, "regions at %zu and %zu overlap", r[i].off,
                  r[i + 1].off);
    }
}

int main() {
    const int64_t Ss[] = {1, 2, 63, 64, 255, 256, 257, 1000, 32768, 65535, 65536, 262144,
                          524288, 5242880, (int64_t)1 << 30};
    const int HqHkv[][2] = {{1, 1}, {2, 1}, {4, 2}, {8, 2}, {8, 1}, {32, 8}, {40, 8}, {4, 1}, {6, 3}};
    const int64_t Ts[] = {0, 256, 512, 65536, 262144};
    char err[256];
    long n = 0;
    for (int64_t S : Ss)
        for (auto& hh : HqHkv)
            for (int D : {64, 128})
                for (int hc = 0; hc <= hh[0]; ++hc)
                    for (int64_t T : Ts)
                        for (int bwd = 0; bwd < 2; ++bwd) {
                            hc::Plan p;
                            const int rc = hc::make_plan(bwd, S, hh[0], hh[1], D, 1, hc, T, &p, err,
                                                         sizeof err);
                            CHECK(rc == 0, "make_plan(S=%lld, %d/%d, D=%d, hc=%d, T=%lld): %s",
                                  (long long)S, hh[0], hh[1], D, hc, (long long)T, err);
                            if (rc == 0) check_plan(p);
                            ++n;
                        }
    // rejections: each returns an error and writes a message
    struct Bad { int64_t S; int Hq, Hkv, D, causal, hc; int64_t T; int rc; };
    const Bad bad[] = {{0, 4, 2, 128, 1, 0, 0, -1},      {100, 4, 3, 128, 1, 0, 0, -1},
                       {100, 4, 2, 96, 1, 0, 0, -2},     {100, 4, 2, 128, 2, 0, 0, -1},
                       {100, 4, 2, 128, 1, 5, 0, -1},    {1000, 4, 2, 128, 1, 0, 100, -1},
                       {((int64_t)1 << 30) + 1, 4, 2, 128, 1, 0, 0, -2},
                       {(int64_t)1 << 30, 1 << 30, 1, 128, 1, 0, 0, -2},
                       {(int64_t)1 << 30, 2147483647, 2147483647, 128, 1, 0, 0, -2}};
    for (const Bad& b : bad) {
        hc::Plan p;
        err[0] = 0;
        const int rc = hc::make_plan(true, b.S, b.Hq, b.Hkv, b.D, b.causal, b.hc, b.T, &p, err, sizeof err);
        CHECK(rc == b.rc && err[0] != 0, "bad case S=%lld Hq=%d Hkv=%d D=%d: rc=%d", (long long)b.S,
              b.Hq, b.Hkv, b.D, rc);
    }
    printf("plans checked: %ld, failures: %d\n", n, fails);
    return fails ? 1 : 0;
}
