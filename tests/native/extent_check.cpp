// Host-only check of every global-memory access the library's kernels and
// copies make, built with the address and undefined-behaviour sanitizers by
// tests/test_extent_check.py.
//
// The library's real host pipeline (hcattn.cpp: the C ABI, planner, chunk
// and trunk loops, ring and staging slots) is linked against a fake HIP
// runtime defined here.  "Device" buffers are host allocations registered
// with the fake runtime (pinned host ones likewise, pageable ones not), so
// attn_fwd / attn_bwd run their argument and pointer checks unchanged.
// Instead of launching kernels, the launch_* entry points below replay each
// kernel's addressing: a host replica of the index arithmetic of every load
// and store in fwd.hip, bwd.hip, aux.hip and gemm.hip (per workgroup, wave and lane,
// including the clamping of ragged tiles), and hipMemcpy2DAsync checks the
// rows it copies.  Each access must lie inside one checked region: a user
// tensor of exactly the size the ABI states, or one workspace region of the
// size the planner carves (so a read that runs from one region into the next,
// or past the workspace, is reported even though it stays in mapped memory).
//
// With --plant-dkdv-overread the dK/dV kernel's loads of K and V rows into
// registers are replayed without their clamp (lanes past the last key of a
// short last tile reading their own key row), which must be reported:
// evidence that the check sees reads.  With --plant-dkdv-fast-run its runs of
// steps whose Q / dO loads take the unchecked full-tile form lose their
// limit at the last full tile of a head, which must be reported too; with
// --plant-fwd-v-ring4 the forward's V ring loses its fifth slot, which must be
// reported as a slot loaded while a wave can still read it.
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "../../include/hcattn.h"
#include "kernels.h"
#include "plan.h"

static bool g_plant = false;
static bool g_plant_fast = false;
static bool g_plant_vring = false;
static int64_t g_gl_min_s = hc::kGroupLoopMinS;  // the library's group-loop threshold
static long g_fails = 0, g_checks = 0;
// failure injection: the copy / kernel launch with this index (counted from
// when it is armed) fails; -1 = none
static long g_copy_fail_at = -1, g_copy_calls = 0, g_launch_fail_at = -1, g_launch_calls = 0;
static bool inject_launch() { return g_launch_fail_at >= 0 && g_launch_calls++ == g_launch_fail_at; }
static std::string g_case;

// ------------------------------------------------------------ buffer model

struct Region {
    uintptr_t lo, hi;
    std::string name;
};
static std::vector<Region> g_regions;  // checked regions (user tensors, workspace regions)

struct Alloc {
    uintptr_t lo, hi;
    bool host;  // pinned host (device otherwise)
};
static std::vector<Alloc> g_allocs;  // what hipPointerGetAttributes knows

static void fail_msg(const char* fmt, const char* what, uintptr_t a, size_t n) {
    if (++g_fails <= 20) {
        fprintf(stderr, "FAIL [%s] %s: ", g_case.c_str(), what);
        fprintf(stderr, fmt, (unsigned long long)a, (unsigned long long)n);
        fprintf(stderr, "\n");
    }
}

// [p, p + bytes) must lie inside one region
static void touch(const void* p, int64_t bytes, const char* what) {
    ++g_checks;
    const uintptr_t a = (uintptr_t)p;
    for (const Region& r : g_regions) {
        if (a >= r.lo && a < r.hi) {
            if (bytes < 0 || a + (uintptr_t)bytes > r.hi)
                fail_msg("access at %#llx of %llu bytes runs past its region", what, a,
                         (size_t)bytes);
            return;
        }
    }
    fail_msg("access at %#llx (%llu bytes) is in no region", what, a, (size_t)bytes);
}

// element offset arithmetic on addresses (the replicas may compute addresses
// outside every buffer; that is what they look for)
template <class T>
static const void* at(const T* base, int64_t elems) {
    return (const void*)((uintptr_t)base + (uintptr_t)(elems * (int64_t)sizeof(T)));
}

// ------------------------------------------------------------ fake HIP

static uintptr_t g_handle = 0x1000;

extern "C" {
hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned int) {
    *s = reinterpret_cast<hipStream_t>(g_handle += 16);
    return hipSuccess;
}
hipError_t hipStreamDestroy(hipStream_t) { return hipSuccess; }
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
    *e = reinterpret_cast<hipEvent_t>(g_handle += 16);
    return hipSuccess;
}
hipError_t hipEventCreate(hipEvent_t* e) { return hipEventCreateWithFlags(e, 0); }
hipError_t hipEventDestroy(hipEvent_t) { return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t, unsigned int) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) { *ms = 0.f; return hipSuccess; }
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "(fake runtime)"; }
hipError_t hipPointerGetAttributes(hipPointerAttribute_t* a, const void* p) {
    const uintptr_t x = (uintptr_t)p;
    for (const Alloc& al : g_allocs) {
        if (x >= al.lo && x < al.hi) {
            memset(a, 0, sizeof(*a));
            a->type = al.host ? hipMemoryTypeHost : hipMemoryTypeDevice;
            return hipSuccess;
        }
    }
    return hipErrorInvalidValue;
}
hipError_t hipMemcpy2DAsync(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width,
                            size_t height, hipMemcpyKind, hipStream_t) {
    if (g_copy_fail_at >= 0 && g_copy_calls++ == g_copy_fail_at) return hipErrorInvalidValue;
    for (size_t r = 0; r < height; ++r) {
        touch((const void*)((uintptr_t)src + r * spitch), (int64_t)width, "copy source row");
        touch((const void*)((uintptr_t)dst + r * dpitch), (int64_t)width, "copy destination row");
    }
    return hipSuccess;
}
}  // extern "C"

// ------------------------------------------------------------ kernel replicas

// the built-in workspace of attn_fwd_noalloc: one registered buffer standing
// in for the device array, its regions added by the driver before each call
static std::vector<char> g_scratch;
static char* scratch_base() {
    if (g_scratch.empty()) g_scratch.resize(hc::kScratchBytes + 256);
    return g_scratch.data() + (256 - (uintptr_t)g_scratch.data() % 256) % 256;
}

namespace hc {

hipError_t scratch_address(void** out) {
    *out = scratch_base();
    return hipSuccess;
}

// Rows a 64-row tile load reads from `base` (stride rs elements): rows at or
// past nvalid re-read row nvalid - 1 (TileDma64 / direct_tile64).
static void tile64(const uint16_t* base, int64_t rs, int64_t nvalid, int HD, const char* what) {
    if (nvalid < 1) {
        fail_msg("tile load with nvalid < 1 (base %#llx, %llu)", what, (uintptr_t)base, 0);
        return;
    }
    const int64_t n = nvalid >= 64 ? 64 : nvalid;
    for (int64_t r = 0; r < n; ++r) touch(at(base, r * rs), (int64_t)HD * 2, what);
}
// 64 consecutive fp32 (direct_vec64): entries past nvalid repeat nvalid - 1
static void vec64(const float* src, int64_t nvalid, const char* what) {
    if (nvalid < 1) {
        fail_msg("vector load with nvalid < 1 (base %#llx, %llu)", what, (uintptr_t)src, 0);
        return;
    }
    touch(src, (nvalid >= 64 ? 64 : nvalid) * 4, what);
}

hipError_t launch_pack(const PackParams& p, hipStream_t) {
    if (inject_launch()) return hipErrorLaunchFailure;
    if (p.nh <= 0 || p.rows <= 0) return hipSuccess;
    for (int64_t h = 0; h < p.nh; ++h)
        for (int64_t row = 0; row < p.rows; ++row) {
            touch(at(p.src, h * p.s_hs + row * p.s_rs), (int64_t)p.D * 2, "pack read");
            touch(at(p.dst, h * p.d_hs + row * p.d_rs), (int64_t)p.D * 2, "pack write");
        }
    return hipSuccess;
}

hipError_t launch_merge(const MergeParams& p, hipStream_t) {
    if (inject_launch()) return hipErrorLaunchFailure;
    if (p.nh <= 0 || p.rows <= 0) return hipSuccess;
    for (int64_t h = 0; h < p.nh; ++h)
        for (int64_t row = 0; row < p.rows; ++row) {
            const int64_t hr = h * p.rows + row;
            touch(p.l_r + hr, 4, "merge l_r");
            touch(p.l_t + hr, 4, "merge l_t");
            touch(at(p.o_r, hr * p.D), (int64_t)p.D * 4, "merge o_r");
            touch(at(p.o_t, hr * p.D), (int64_t)p.D * 4, "merge o_t");
            if (p.final_out) {
                touch(at(p.out, h * p.out_hs + row * p.out_rs), (int64_t)p.D * 2, "merge out");
                if (p.lse_out) touch(p.lse_out + h * p.lse_hs + row, 4, "merge lse_out");
            }
        }
    return hipSuccess;
}

hipError_t launch_prep(const PrepParams& p, hipStream_t) {
    if (inject_launch()) return hipErrorLaunchFailure;
    if (p.nh <= 0 || p.rows <= 0) return hipSuccess;
    for (int64_t h = 0; h < p.nh; ++h)
        for (int64_t row = 0; row < p.rows; ++row) {
            touch(at(p.o, h * p.o_hs + row * p.o_rs), (int64_t)p.D * 2, "prep o");
            touch(at(p.dO, h * p.do_hs + row * p.do_rs), (int64_t)p.D * 2, "prep dO");
            touch(at(p.dO_c, h * p.c_hs + row * p.c_rs), (int64_t)p.D * 2, "prep dO_c");
            touch(p.ndelta + h * p.ndelta_hs + row, 4, "prep ndelta");
            touch(p.nlse2 + h * p.nlse2_hs + row, 4, "prep nlse2");
            touch(p.lse + h * p.lse_hs + row, 4, "prep lse");
        }
    return hipSuccess;
}

// fwd_kernel<HD, NW> as launched by launch_fwd
// The 8-wave forward's ring schedule over ntiles K / V tiles: between two
// barriers (tile pair j, j + 1) waves 0-3 read K and V of tiles j and j + 1;
// waves 4-7 read V of tile j - 1 (their deferred P V product), K of j and
// j + 1 and V of j; K and V of tiles j + 2 and j + 3 load into their slots
// meanwhile.  No slot may be loaded while a wave can still read another tile
// from it.
static void fwd_ring_check(int ntiles, int nvb) {
    const int nkb = 4;
    for (int j = 0; j < ntiles; j += 2) {
        std::vector<int> rk, rv;
        for (int t = j; t < j + 2 && t < ntiles; ++t) {
            rk.push_back(t);
            rv.push_back(t);
        }
        if (j >= 2) rv.push_back(j - 1);
        for (int t = j + 2; t < j + 4 && t < ntiles; ++t) {
            ++g_checks;
            for (int r : rk)
                if (r % nkb == t % nkb)
                    fail_msg("K tile %llu loaded into the slot of tile %llu still being read",
                             "fwd K ring", (uintptr_t)t, (size_t)r);
            for (int r : rv)
                if (r % nvb == t % nvb)
                    fail_msg("V tile %llu loaded into the slot of tile %llu still being read",
                             "fwd V ring", (uintptr_t)t, (size_t)r);
        }
    }
}

hipError_t launch_fwd(const FwdParams& p, int HD, hipStream_t) {
    if (inject_launch()) return hipErrorLaunchFailure;
    if (p.nq <= 0 || p.nh <= 0) return hipSuccess;
    const bool wide = (p.nq + 255) / 256 * p.nh >= kWideMinBlocks;
    const int NW = wide ? 8 : 4, WQ = 32, BM = NW * WQ, BN = 64;
    const int64_t nqt = (p.nq + BM - 1) / BM;
    const int64_t blocks = nqt * p.nh;
    for (int64_t b = 0; b < blocks; ++b) {
        const int head = (int)(b % p.nh);
        const int64_t qt = nqt - 1 - b / p.nh;
        const int64_t q0 = qt * BM;
        const int kvl = (p.h0 + head) / p.group - p.kv_base;
        const uint16_t* qh = p.q + (int64_t)head * p.q_hs;
        const uint16_t* kh = p.k + (int64_t)kvl * p.k_hs;
        const uint16_t* vh = p.v + (int64_t)kvl * p.v_hs;
        const int64_t wg_last = (q0 + BM - 1 < p.nq - 1) ? q0 + BM - 1 : p.nq - 1;
        int64_t kend = p.nk;
        if (p.causal) {
            const int64_t a = p.q_pos0 + wg_last - p.k_pos0 + 1;
            kend = a < kend ? a : kend;
        }
        const int ntiles = kend > 0 ? (int)((kend + BN - 1) / BN) : 0;
        if (wide) {
            // the schedule depends on ntiles alone: check each count once
            static std::vector<char> done;
            if ((size_t)ntiles >= done.size()) done.resize((size_t)ntiles + 1, 0);
            if (!done[ntiles]) {
                done[ntiles] = 1;
                fwd_ring_check(ntiles, g_plant_vring ? 4 : 5);
            }
        }
        for (int t = 0; t < ntiles; ++t) {
            const int64_t nb = (int64_t)t * BN;
            tile64(kh + nb * p.k_rs, p.k_rs, p.nk - nb, HD, "fwd K tile");
            tile64(vh + nb * p.v_rs, p.v_rs, p.nk - nb, HD, "fwd V tile");
        }
        for (int w = 0; w < NW; ++w) {
            const int64_t wq0 = q0 + w * WQ;
            const bool wave_live = wq0 < p.nq;
            for (int l = 0; l < 32; ++l) {
                const int64_t myq = wq0 + l;
                if (myq >= p.nq) continue;
                touch(at(qh, myq * p.q_rs), HD * 2, "fwd Q row");
                const int64_t sr = (int64_t)head * p.st_hs + myq;
                if (p.carry_in || p.carry_out) {
                    touch(p.st_m + sr, 4, "fwd carried m");
                    touch(p.st_l + 2 * sr, 8, "fwd carried row sums");
                    touch(at(p.st_o, (int64_t)head * p.st_o_hs + myq * HD), HD * 4, "fwd carried O");
                }
                if (!wave_live || p.carry_out) continue;
                if (p.mode == kFwdFinal) {
                    touch(at((const uint16_t*)p.o, (int64_t)head * p.o_hs + myq * p.o_rs), HD * 2,
                          "fwd O (bf16)");
                    if (p.lse) touch(p.lse + (int64_t)head * p.lse_hs + myq, 4, "fwd LSE");
                } else {
                    touch(at((const float*)p.o, (int64_t)head * p.o_hs + myq * p.o_rs), HD * 4,
                          "fwd O partial (fp32)");
                    touch(p.lse + (int64_t)head * p.lse_hs + myq, 4, "fwd LSE partial");
                }
            }
        }
    }
    return hipSuccess;
}

// dkdv_kernel<HD, RUNS, GLOOP> as launched by launch_dkdv
hipError_t launch_dkdv(const DkdvParams& p, int HD, hipStream_t) {
    if (inject_launch()) return hipErrorLaunchFailure;
    const int units = p.group_loop ? p.nkv : p.nh;
    if (p.nk <= 0 || units <= 0) return hipSuccess;
    const int BQ = 64, BNK = 128;
    const int64_t blocks = (p.nk + BNK - 1) / BNK * units;
    if ((p.nq + 63) / 64 * (p.group_loop ? p.group : 1) > 0x7fffffffLL) return hipErrorInvalidValue;
    const bool runs = units % 4 != 0;
    std::vector<char> seen((size_t)blocks, 0);
    for (int64_t b = 0; b < blocks; ++b) {
        int unit;
        int64_t kt;
        if (runs) {
            const unsigned RUN = 32, WIN = 8 * RUN;
            unsigned item = (unsigned)b;
            const unsigned w = item / WIN;
            if ((w + 1) * WIN <= (unsigned)blocks) {
                const unsigned x = item % 8, o = (item / 8) % RUN;
                item = w * WIN + ((w & 1) ? 7 - x : x) * RUN + o;
            }
            if ((int64_t)item >= blocks || seen[item]) {
                fail_msg("work item %#llx repeated or out of range (%llu)", "dkdv order", item,
                         (size_t)blocks);
                continue;
            }
            seen[item] = 1;
            unit = (int)(item % (unsigned)units);
            kt = (int64_t)(item / (unsigned)units);
        } else {
            unit = (int)(b % units);
            kt = b / units;
        }
        int kvl, hb, he;
        if (p.group_loop) {
            kvl = unit;
            const int gh0 = (p.kv_base + kvl) * p.group - p.h0;
            hb = gh0 < 0 ? 0 : gh0;
            he = gh0 + p.group > p.nh ? p.nh : gh0 + p.group;
            if (hb >= he) fail_msg("kv head %#llx of the chunk has no query head (%llu)",
                                   "dkdv group", (uintptr_t)kvl, (size_t)hb);
        } else {
            hb = unit;
            he = unit + 1;
            kvl = (p.h0 + unit) / p.group - p.kv_base;
        }
        if (kvl < 0 || kvl >= (p.group_loop ? p.nkv : 1 << 30))
            fail_msg("kv head %#llx out of range (%llu)", "dkdv kv head", (uintptr_t)kvl, 0);
        const int64_t j0 = kt * BNK;
        // each lane's key row of K and V (16-byte reads of its 8-column
        // slices), clamped to the last key
        for (int kw = 0; kw < 4; ++kw)
            for (int l = 0; l < 32; ++l) {
                const int64_t myk = j0 + kw * 32 + l;
                const int64_t kk = g_plant ? myk : (myk < p.nk ? myk : p.nk - 1);
                touch(p.k + (int64_t)kvl * p.k_hs + kk * p.k_rs, HD * 2, "dkdv K row");
                touch(p.v + (int64_t)kvl * p.v_hs + kk * p.v_rs, HD * 2, "dkdv V row");
            }
        const int64_t nqt = (p.nq + BQ - 1) / BQ;
        int64_t qt0 = 0;
        if (p.causal) {
            const int64_t first = p.k_pos0 + j0;
            qt0 = first >= p.nq ? nqt : first / BQ;
        }
        const int64_t nsteps = j0 < p.nk ? nqt - qt0 : 0;
        // each wave's step schedule: a run of unmasked steps issues the loads
        // of step n + 3 in the full-tile form, without a row check, so every
        // such step needs step n + 3 to exist and the issue cursor's tile
        // (head ih, step is; three steps ahead) to lie wholly inside nq
        {
            const int64_t total = nsteps * (he - hb);
            const int64_t nfull = (p.nq - qt0 * BQ) / BQ;
            const bool fast_rs = p.q_rs < ((int64_t)1 << 24) && p.do_rs < ((int64_t)1 << 24);
            for (int kw = 0; kw < 4; ++kw) {
                const int64_t wj0 = j0 + kw * 32, wkpos = p.k_pos0 + wj0;
                const bool edge_k = wj0 + 32 > p.nk;
                int64_t d_end = 0;
                if (p.causal) {
                    const int64_t t = (wkpos + 32 - 2 + BQ) / BQ - qt0;
                    d_end = t < 0 ? 0 : (t > nsteps ? nsteps : t);
                }
                const int64_t u_end = nsteps - (((qt0 + nsteps) * BQ > p.nq) ? 1 : 0);
                int64_t is = 0, n = 0;
                int ih = hb;
                auto cursor_next = [&]() {
                    if (++is == nsteps) {
                        is = 0;
                        ++ih;
                    }
                };
                for (int64_t i = 0; i < 3 && i < total; ++i) cursor_next();
                for (int h = hb; h < he; ++h) {
                    int64_t st = 0;
                    while (st < nsteps) {
                        int64_t nf = 0;
                        if (!edge_k && st >= d_end && st < u_end && fast_rs && is < nfull) {
                            nf = u_end - st;
                            if (total - 3 - n < nf) nf = total - 3 - n;
                            if (!g_plant_fast && nfull < nsteps && nfull - is < nf) nf = nfull - is;
                        }
                        if (nf <= 0) {
                            if (n + 3 < total) cursor_next();
                            ++st;
                            ++n;
                            continue;
                        }
                        for (const int64_t e = st + nf; st < e; ++st, ++n) {
                            ++g_checks;
                            if (n + 3 >= total || ih >= he)
                                fail_msg("step %#llx issues full-tile loads past the last step (%llu)",
                                         "dkdv fast run", (uintptr_t)n, (size_t)total);
                            else if (p.nq - (qt0 + is) * BQ < BQ)
                                fail_msg("full-tile loads of a partial tile at row %#llx (nq %llu)",
                                         "dkdv fast run", (uintptr_t)((qt0 + is) * BQ), (size_t)p.nq);
                            cursor_next();
                        }
                    }
                }
            }
        }
        for (int h = hb; h < he; ++h)
            for (int64_t n = 0; n < nsteps; ++n) {
                const int64_t i0 = (qt0 + n) * BQ;
                tile64(p.q + (int64_t)h * p.q_hs + i0 * p.q_rs, p.q_rs, p.nq - i0, HD, "dkdv Q tile");
                tile64(p.dO + (int64_t)h * p.do_hs + i0 * p.do_rs, p.do_rs, p.nq - i0, HD,
                       "dkdv dO tile");
                vec64(p.nlse2 + (int64_t)h * p.nlse2_hs + i0, p.nq - i0, "dkdv -LSE log2e");
                vec64(p.ndelta + (int64_t)h * p.ndelta_hs + i0, p.nq - i0, "dkdv -Delta");
            }
        for (int kw = 0; kw < 4; ++kw)
            for (int l = 0; l < 32; ++l) {
                const int64_t myk = j0 + kw * 32 + l;
                if (myk >= p.nk) continue;
                if (!p.group_loop) {
                    touch(at(p.part_k, ((int64_t)hb * p.nk + myk) * HD), HD * 4, "dkdv dK partial");
                    touch(at(p.part_v, ((int64_t)hb * p.nk + myk) * HD), HD * 4, "dkdv dV partial");
                    continue;
                }
                if (kvl == p.carry_kv_in) {
                    touch(at(p.carry_in_k, myk * HD), HD * 4, "dkdv carry in dK");
                    touch(at(p.carry_in_v, myk * HD), HD * 4, "dkdv carry in dV");
                }
                if (kvl == p.carry_kv_out) {
                    touch(at(p.carry_out_k, myk * HD), HD * 4, "dkdv carry out dK");
                    touch(at(p.carry_out_v, myk * HD), HD * 4, "dkdv carry out dV");
                }
                if (kvl != p.carry_kv_out) {
                    touch(at(p.dk, (int64_t)kvl * p.dk_hs + myk * p.dk_rs), HD * 2, "dkdv dK out");
                    touch(at(p.dv, (int64_t)kvl * p.dk_hs + myk * p.dk_rs), HD * 2, "dkdv dV out");
                }
            }
    }
    return hipSuccess;
}

hipError_t launch_dkdv_reduce(const DkdvReduceParams& p, hipStream_t) {
    if (inject_launch()) return hipErrorLaunchFailure;
    if (p.nk <= 0 || p.nkv <= 0) return hipSuccess;
    for (int kvl = 0; kvl < p.nkv; ++kvl) {
        const int kvg = p.kv_base + kvl;
        int hb = kvg * p.group - p.h0, he = (kvg + 1) * p.group - p.h0;
        hb = hb < 0 ? 0 : hb;
        he = he > p.nh ? p.nh : he;
        for (int64_t key = 0; key < p.nk; ++key) {
            if (kvl == p.carry_kv_in) {
                touch(at(p.carry_in_k, key * p.D), p.D * 4, "reduce carry in dK");
                touch(at(p.carry_in_v, key * p.D), p.D * 4, "reduce carry in dV");
            }
            for (int h = hb; h < he; ++h) {
                touch(at(p.part_k, ((int64_t)h * p.nk + key) * p.D), p.D * 4, "reduce dK partial");
                touch(at(p.part_v, ((int64_t)h * p.nk + key) * p.D), p.D * 4, "reduce dV partial");
            }
            if (kvl == p.carry_kv_out) {
                touch(at(p.carry_out_k, key * p.D), p.D * 4, "reduce carry out dK");
                touch(at(p.carry_out_v, key * p.D), p.D * 4, "reduce carry out dV");
            } else {
                touch(at(p.dk, (int64_t)kvl * p.dk_hs + key * p.dk_rs), p.D * 2, "reduce dK out");
                touch(at(p.dv, (int64_t)kvl * p.dk_hs + key * p.dk_rs), p.D * 2, "reduce dV out");
            }
        }
    }
    return hipSuccess;
}

// dq_kernel<HD, NW> as launched by launch_dq
hipError_t launch_dq(const DqParams& p, int HD, hipStream_t) {
    if (inject_launch()) return hipErrorLaunchFailure;
    if (p.nq <= p.q_begin || p.nh <= 0) return hipSuccess;
    const bool wide = ((p.nq + 255) / 256 - p.q_begin / 256) * p.nh >= kWideMinBlocks;
    const int bm = wide ? 256 : 128;
    if (p.q_begin % bm != 0) return hipErrorInvalidValue;
    const int NW = wide ? 8 : 4, WQ = 32, BM = NW * WQ, BN = 64;
    const int64_t qtb = p.q_begin / BM;
    const int64_t nqt = (p.nq + BM - 1) / BM - qtb;
    const int64_t blocks = nqt * p.nh;
    for (int64_t b = 0; b < blocks; ++b) {
        const int head = (int)(b % p.nh);
        const int64_t qt = qtb + nqt - 1 - b / p.nh;
        const int64_t q0 = qt * BM;
        const int kvl = (p.h0 + head) / p.group - p.kv_base;
        const uint16_t* kh = p.k + (int64_t)kvl * p.k_hs;
        const uint16_t* vh = p.v + (int64_t)kvl * p.v_hs;
        const int64_t wg_last = (q0 + BM - 1 < p.nq - 1) ? q0 + BM - 1 : p.nq - 1;
        int64_t kend = p.nk;
        if (p.causal) {
            const int64_t a = wg_last - p.k_pos0 + 1;
            kend = a < kend ? a : kend;
        }
        const int ntiles = kend > 0 ? (int)((kend + BN - 1) / BN) : 0;
        for (int t = 0; t < ntiles; ++t) {
            const int64_t nb = (int64_t)t * BN;
            tile64(kh + nb * p.k_rs, p.k_rs, p.nk - nb, HD, "dq K tile");
            tile64(vh + nb * p.v_rs, p.v_rs, p.nk - nb, HD, "dq V tile");
        }
        for (int w = 0; w < NW; ++w)
            for (int l = 0; l < 32; ++l) {
                const int64_t myq = q0 + w * WQ + l;
                if (myq >= p.nq) continue;
                touch(at(p.q, (int64_t)head * p.q_hs + myq * p.q_rs), HD * 2, "dq Q row");
                touch(at(p.dO, (int64_t)head * p.do_hs + myq * p.do_rs), HD * 2, "dq dO row");
                touch(p.nlse2 + (int64_t)head * p.nlse2_hs + myq, 4, "dq -LSE log2e");
                touch(p.ndelta + (int64_t)head * p.ndelta_hs + myq, 4, "dq -Delta");
                if (p.acc_in)
                    touch(at(p.acc_in, (int64_t)head * p.ain_hs + myq * p.ain_rs), HD * 4,
                          "dq fp32 carry in");
                if (myq < p.final_before || p.acc_out == nullptr)
                    touch(at(p.dq, (int64_t)head * p.dq_hs + myq * p.dq_rs), HD * 2, "dq out");
                else
                    touch(at(p.acc_out, (int64_t)head * p.aout_hs + myq * p.aout_rs), HD * 4,
                          "dq fp32 carry out");
            }
    }
    return hipSuccess;
}

// gemm_kernel<A_KC, B_KC> as launched by launch_gemm (every tile of C once,
// whatever the dispatch order): every 16-byte operand
// chunk a 128 x 64 tile load reads (the kernel's per-thread offset plus its
// per-step segment offset, which equals this formula while a k-contiguous
// segment is a multiple of 64), and every C row segment the epilogue (and
// the accumulating prologue) touches
static const int kGemmBK = 64;  // reduction indices per operand tile load
static void gemm_operand(const uint16_t* base, int64_t rs, int64_t seg, int64_t segs, bool kc,
                         int64_t r0, int64_t R, int64_t k0, int64_t K, const char* what) {
    for (int idx = 0; idx < 128 * kGemmBK / 8; ++idx) {
        int64_t row, k;
        if (kc) { row = r0 + idx / (kGemmBK / 8); k = k0 + (idx % (kGemmBK / 8)) * 8; }
        else { k = k0 + idx / 16; row = r0 + (idx % 16) * 8; }
        if (row >= R || k >= K) continue;
        const int64_t off = kc ? (k / seg) * segs + row * rs + k % seg
                               : (row / seg) * segs + k * rs + row % seg;
        touch(at(base, off), 16, what);
    }
}

hipError_t launch_gemm(const GemmParams& p, bool a_kc, bool b_kc, int splits, hipStream_t) {
    if (inject_launch()) return hipErrorLaunchFailure;
    if (p.M <= 0 || p.N <= 0) return hipSuccess;
    if ((a_kc || b_kc) && p.K % 8 != 0) return hipErrorInvalidValue;
    if ((a_kc && p.a_seg % kGemmBK != 0) || (b_kc && p.b_seg % kGemmBK != 0)) return hipErrorInvalidValue;
    if (p.k_parts > 1) {
        if (p.k_parts > kGemmMaxParts || p.k_split != 0 || splits != 1 || p.k_at[0] != 0 ||
            p.k_at[p.k_parts] != p.K)
            return hipErrorInvalidValue;
        for (int i = 0; i < p.k_parts; ++i)
            if (p.k_at[i + 1] <= p.k_at[i] || p.k_at[i + 1] % kGemmBK != 0 || !p.a_at[i] || !p.b_at[i])
                return hipErrorInvalidValue;
    }
    if (!a_kc && p.M % 8 != 0) return hipErrorInvalidValue;
    if (p.N % 8 != 0 || p.a_seg % 8 != 0 || p.b_seg % 8 != 0 || p.c_seg % 4 != 0 ||
        (p.k_split > 0 && p.k_split % kGemmBK != 0) || splits < 1 || splits > 65535)
        return hipErrorInvalidValue;
    const int64_t gx = (p.M + 127) / 128, gy = (p.N + 127) / 128;
    if (gx * gy > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    for (int z = 0; z < splits; ++z)
        for (int64_t bx = 0; bx < gx; ++bx)
            for (int64_t by = 0; by < gy; ++by) {
                const int64_t m0 = bx * 128, n0 = by * 128;
                const int64_t kb = p.k_split > 0 ? (int64_t)z * p.k_split : 0;
                int64_t ke = p.k_split > 0 ? kb + p.k_split : p.K;
                ke = ke < p.K ? ke : p.K;
                if (p.k_parts > 1) {
                    // part i: its own operands, k counted from the part's start
                    for (int i = 0; i < p.k_parts; ++i) {
                        const int64_t kl = p.k_at[i + 1] - p.k_at[i];
                        for (int64_t k0 = 0; k0 < kl; k0 += kGemmBK) {
                            gemm_operand(p.a_at[i], p.a_rs, p.a_seg, p.a_segs, a_kc, m0, p.M, k0, kl, "gemm A part");
                            gemm_operand(p.b_at[i], p.b_rs, p.b_seg, p.b_segs, b_kc, n0, p.N, k0, kl, "gemm B part");
                        }
                    }
                } else {
                    for (int64_t k0 = kb; k0 < ke; k0 += kGemmBK) {
                        gemm_operand(p.a, p.a_rs, p.a_seg, p.a_segs, a_kc, m0, p.M, k0, ke, "gemm A");
                        gemm_operand(p.b, p.b_rs, p.b_seg, p.b_segs, b_kc, n0, p.N, k0, ke, "gemm B");
                    }
                }
                const int esz = p.out_mode == kGemmBf16 ? 2 : 4;
                const char* cz = (const char*)p.c + (int64_t)z * p.c_zs * esz;
                for (int64_t m = m0; m < m0 + 128 && m < p.M; ++m)
                    for (int64_t n = n0; n < n0 + 128 && n < p.N; n += 4) {
                        const int64_t o = (n / p.c_seg) * p.c_segs + m * p.c_rs + n % p.c_seg;
                        touch(cz + o * esz, 4 * esz, "gemm C");
                    }
            }
    return hipSuccess;
}

hipError_t launch_gemm_reduce(const GemmReduceParams& p, hipStream_t) {
    if (inject_launch()) return hipErrorLaunchFailure;
    if (p.M <= 0 || p.N <= 0) return hipSuccess;
    if (p.N % 4 != 0 || p.splits < 1) return hipErrorInvalidValue;
    for (int64_t m = 0; m < p.M; ++m) {
        for (int z = 0; z < p.splits; ++z)
            touch(at(p.part, z * p.part_zs + m * p.N), p.N * 4, "gemm partial");
        touch(at(p.out, m * p.out_rs), p.N * 4, "gemm reduce out");
    }
    return hipSuccess;
}

}  // namespace hc

// ------------------------------------------------------------ driver

struct Buffer {
    std::vector<char> mem;
    void* p() { return mem.data(); }
};

static void add_region(const void* p, size_t bytes, const std::string& name) {
    g_regions.push_back({(uintptr_t)p, (uintptr_t)p + bytes, name});
}

// the workspace regions as the planner carves them (sizes restated here from
// the layout each kernel reads and writes)
static void add_workspace(char* ws, const hc::Plan& p) {
    const size_t E = (size_t)p.S * p.D * 2, Et = (size_t)p.T * p.D * 2;
    auto R = [&](size_t off, size_t bytes, const char* n) { add_region(ws + off, bytes, n); };
    if (!p.bwd) {
        if (!p.trunked) {
            R(p.q_c, p.hc * E, "ws Q_c");
            R(p.k_c, p.kvc * E, "ws K_c");
            R(p.v_c, p.kvc * E, "ws V_c");
        } else {
            R(p.q_c, p.hc * Et, "ws Q_m");
            R(p.o_run, p.hc * Et * 2, "ws O_run");
            R(p.o_t, p.hc * Et * 2, "ws O_t");
            R(p.l_run, (size_t)p.hc * p.T * 4, "ws L_run");
            R(p.l_t, (size_t)p.hc * p.T * 4, "ws L_t");
            R(p.st_l, (size_t)p.hc * p.T * 8, "ws row sums");
            for (int s = 0; s < 2; ++s) {
                R(p.ring_k[s], p.kvc * Et, "ws ring K");
                R(p.ring_v[s], p.kvc * Et, "ws ring V");
            }
        }
    } else {
        R(p.q_c, p.hc * E, "ws Q_c");
        R(p.do_c, p.hc * E, "ws dO_c");
        R(p.delta_c, (size_t)p.hc * p.S * 4, "ws -Delta");
        R(p.lse2_c, (size_t)p.hc * p.S * 4, "ws -LSE log2e");
        if (!p.group_loop) {
            const size_t rows = p.trunked ? Et : E;
            R(p.part_k, p.hc * rows * 2, "ws dK partials");
            R(p.part_v, p.hc * rows * 2, "ws dV partials");
        }
        if (!p.trunked) {
            R(p.k_c, p.kvc * E, "ws K_c");
            R(p.v_c, p.kvc * E, "ws V_c");
        } else {
            R(p.dq_acc, p.hc * E * 2, "ws dQ carry");
            for (int s = 0; s < 2; ++s) {
                R(p.ring_k[s], p.kvc * Et, "ws ring K");
                R(p.ring_v[s], p.kvc * Et, "ws ring V");
                R(p.stage_k[s], p.kvc * Et, "ws staging dK");
                R(p.stage_v[s], p.kvc * Et, "ws staging dV");
            }
        }
        for (int s = 0; s < p.carry_slots; ++s) {
            R(p.carry_k[s], E * 2, "ws dK carry");
            R(p.carry_v[s], E * 2, "ws dV carry");
        }
    }
}

// one attn_fwd + attn_bwd call pair on exactly sized buffers
// one armed failure: ABI call `call` (0 forward, 1 backward) sees the copy
// (copy) or kernel launch with index `at` of that call fail
struct Inject {
    int call = -1;
    bool copy = false;
    long at = 0;
};
static Inject g_inj;
static long g_inject_hits = 0;

// one ABI call.  With the failure armed for it, the call must return
// ATTN_EHIP naming the failing HIP call, and the same call unarmed must then
// succeed: an error leaves nothing half-done that breaks the next call.
template <class F>
static void checked_call(int which, const char* what, F&& f) {
    const bool armed = g_inj.call == which;
    if (armed) {
        g_copy_calls = g_launch_calls = 0;
        (g_inj.copy ? g_copy_fail_at : g_launch_fail_at) = g_inj.at;
    }
    int rc = f();
    const bool hit = armed && (g_inj.copy ? g_copy_calls : g_launch_calls) > g_inj.at;
    g_copy_fail_at = g_launch_fail_at = -1;
    if (!hit) {
        if (rc != ATTN_OK) fail_msg("call returned %llu (%llu)", what, (size_t)rc, 0);
        return;
    }
    const char* want = g_inj.copy ? "hipMemcpy2DAsync" : "launch_";
    if (rc != ATTN_EHIP || strstr(attn_last_error(), want) == nullptr) {
        fprintf(stderr, "  injected failure, message: %s\n", attn_last_error());
        fail_msg("an injected failure returned %llu (%llu), not ATTN_EHIP naming the call", what,
                 (size_t)rc, 0);
        return;
    }
    ++g_inject_hits;
    rc = f();
    if (rc != ATTN_OK) fail_msg("the call after an injected failure returned %llu (%llu)", what, (size_t)rc, 0);
}

static void run_case(int64_t S, int Hq, int Hkv, int D, int causal, int hc, int64_t T, bool host) {
    char name[160];
    snprintf(name, sizeof name, "S=%lld Hq=%d Hkv=%d D=%d causal=%d hc=%d T=%lld host=%d",
             (long long)S, Hq, Hkv, D, causal, hc, (long long)T, (int)host);
    g_case = name;
    const size_t qb = (size_t)S * Hq * D * 2, kb = (size_t)S * Hkv * D * 2, lb = (size_t)Hq * S * 4;
    Buffer q, k, v, o, lse, dout, dq, dk, dv, wsf, wsb;
    q.mem.resize(qb); o.mem.resize(qb); dout.mem.resize(qb); dq.mem.resize(qb);
    k.mem.resize(kb); v.mem.resize(kb); dk.mem.resize(kb); dv.mem.resize(kb);
    lse.mem.resize(lb);
    const size_t nf = attn_fwd_workspace_bytes(S, Hq, Hkv, D, causal, hc, T);
    const size_t nb = attn_bwd_workspace_bytes(S, Hq, Hkv, D, causal, hc, T);
    if (nf == 0 || nb == 0) {
        fail_msg("workspace query failed (%llu, %llu)", attn_last_error(), nf, nb);
        return;
    }
    // 256-byte aligned workspaces of exactly the queried size
    std::vector<char> fbuf(nf + 256), bbuf(nb + 256);
    char* wf = fbuf.data() + (256 - (uintptr_t)fbuf.data() % 256) % 256;
    char* wb = bbuf.data() + (256 - (uintptr_t)bbuf.data() % 256) % 256;
    g_regions.clear();
    g_allocs.clear();
    auto reg = [&](Buffer& b, const char* n, bool is_host) {
        add_region(b.p(), b.mem.size(), n);
        g_allocs.push_back({(uintptr_t)b.p(), (uintptr_t)b.p() + b.mem.size(), is_host});
    };
    reg(q, "q", false); reg(o, "o", false); reg(dout, "dout", false); reg(dq, "dq", false);
    reg(lse, "lse", false);
    reg(k, "k", host); reg(v, "v", host); reg(dk, "dk", host); reg(dv, "dv", host);
    g_allocs.push_back({(uintptr_t)wf, (uintptr_t)wf + nf, false});
    hc::Plan pf, pb;
    char msg[256];
    hc::make_plan(false, S, Hq, Hkv, D, causal, hc, T, &pf, msg, sizeof msg, g_gl_min_s);
    const size_t keep = g_regions.size();
    add_workspace(wf, pf);
    checked_call(0, "attn_fwd", [&]() {
        return attn_fwd(q.p(), k.p(), v.p(), o.p(), (float*)lse.p(), S, Hq, Hkv, D, causal, hc, T, wf,
                        nf, nullptr);
    });
    g_regions.resize(keep);
    g_allocs.pop_back();
    int rc;
    if (nf <= ATTN_NOALLOC_WORKSPACE_BYTES && g_inj.call < 0) {
        // the same forward on the built-in workspace
        char* sb = scratch_base();
        g_allocs.push_back({(uintptr_t)sb, (uintptr_t)sb + hc::kScratchBytes, false});
        add_workspace(sb, pf);
        rc = attn_fwd_noalloc(q.p(), k.p(), v.p(), o.p(), (float*)lse.p(), S, Hq, Hkv, D, causal,
                              hc, T, nullptr);
        if (rc != ATTN_OK)
            fail_msg("attn_fwd_noalloc returned %llu (%llu)", attn_last_error(), (size_t)rc, 0);
        g_regions.resize(keep);
        g_allocs.pop_back();
    }
    g_allocs.push_back({(uintptr_t)wb, (uintptr_t)wb + nb, false});
    hc::make_plan(true, S, Hq, Hkv, D, causal, hc, T, &pb, msg, sizeof msg, g_gl_min_s);
    add_workspace(wb, pb);
    checked_call(1, "attn_bwd", [&]() {
        return attn_bwd(q.p(), k.p(), v.p(), o.p(), dout.p(), (const float*)lse.p(), dq.p(), dk.p(),
                        dv.p(), S, Hq, Hkv, D, causal, hc, T, wb, nb, nullptr);
    });
}

// attn_layer_fwd and attn_layer_bwd, each without and with the kept
// attention output, on exactly sized buffers; the
// workspace regions restate the layer's carve: the attention plan's regions,
// then O_c (and for the backward LSE_c, dQ_c, dK_c, dV_c and the split-K
// partials of the weight gradients)
static void run_layer_case(int64_t S, int dm, int Hq, int Hkv, int D, int causal, int hc) {
    char name[160];
    snprintf(name, sizeof name, "layer S=%lld dm=%d Hq=%d Hkv=%d D=%d causal=%d hc=%d",
             (long long)S, dm, Hq, Hkv, D, causal, hc);
    g_case = name;
    Buffer x, wq, wk, wv, wo, y, lse, dy, dx, dwq, dwk, dwv, dwo, o;
    x.mem.resize((size_t)S * dm * 2); dy.mem.resize((size_t)S * dm * 2);
    o.mem.resize((size_t)Hq * S * D * 2);
    wq.mem.resize((size_t)Hq * D * dm * 2); wo.mem.resize((size_t)Hq * D * dm * 2);
    wk.mem.resize((size_t)Hkv * D * dm * 2); wv.mem.resize((size_t)Hkv * D * dm * 2);
    y.mem.resize((size_t)S * dm * 4); dx.mem.resize((size_t)S * dm * 4);
    lse.mem.resize((size_t)Hq * S * 4);
    dwq.mem.resize((size_t)Hq * D * dm * 4); dwo.mem.resize((size_t)Hq * D * dm * 4);
    dwk.mem.resize((size_t)Hkv * D * dm * 4); dwv.mem.resize((size_t)Hkv * D * dm * 4);
    const size_t nf = attn_layer_fwd_workspace_bytes(S, dm, Hq, Hkv, D, causal, hc);
    const size_t nb = attn_layer_bwd_workspace_bytes(S, dm, Hq, Hkv, D, causal, hc);
    if (nf == 0 || nb == 0) {
        fail_msg("layer workspace query failed (%llu, %llu)", attn_last_error(), nf, nb);
        return;
    }
    std::vector<char> fbuf(nf + 256), bbuf(nb + 256);
    char* wf = fbuf.data() + (256 - (uintptr_t)fbuf.data() % 256) % 256;
    char* wb = bbuf.data() + (256 - (uintptr_t)bbuf.data() % 256) % 256;
    g_regions.clear();
    g_allocs.clear();
    Buffer* bufs[] = {&x, &wq, &wk, &wv, &wo, &y, &lse, &dy, &dx, &dwq, &dwk, &dwv, &dwo, &o};
    const char* names[] = {"x", "wq", "wk", "wv", "wo", "y", "lse", "dy", "dx", "dwq", "dwk",
                           "dwv", "dwo", "o_keep"};
    for (int i = 0; i < 14; ++i) {
        add_region(bufs[i]->p(), bufs[i]->mem.size(), names[i]);
        g_allocs.push_back({(uintptr_t)bufs[i]->p(), (uintptr_t)bufs[i]->p() + bufs[i]->mem.size(),
                            false});
    }
    const size_t keep = g_regions.size();
    const size_t E = (size_t)S * D * 2;
    char msg[256];
    // forward, forward keeping O, backward recomputing O, backward reading it
    for (int it = 0; it < 4; ++it) {
        const int bwd = it >= 2;
        const bool kept = it & 1;
        hc::Plan p;
        hc::make_plan(bwd, S, Hq, Hkv, D, causal, hc, 0, &p, msg, sizeof msg, g_gl_min_s);
        char* ws = bwd ? wb : wf;
        add_workspace(ws, p);
        size_t off = p.total;
        auto R = [&](size_t bytes, const char* n) {
            add_region(ws + off, bytes, n);
            off = hc::align_up(off + bytes);
        };
        R(p.hc * E, "ws O_c");
        if (bwd) {
            R((size_t)p.hc * S * 4, "ws LSE_c");
            R(p.hc * E, "ws dQ_c");
            R(p.kvc * E, "ws dK_c");
            R(p.kvc * E, "ws dV_c");
            const int64_t ks = (S + 64 * 8 - 1) / (64 * 8) * 64;
            const int64_t splits = (S + ks - 1) / ks;
            R((size_t)splits * p.hc * D * dm * 4, "ws weight-gradient partials");
        }
        if (off != (bwd ? nb : nf))
            fail_msg("layer workspace carve %llu != queried %llu", "layer plan", off, bwd ? nb : nf);
        g_allocs.push_back({(uintptr_t)ws, (uintptr_t)ws + (bwd ? nb : nf), false});
        int rc;
        if (!bwd)
            rc = attn_layer_fwd(x.p(), wq.p(), wk.p(), wv.p(), wo.p(), (float*)y.p(), (float*)lse.p(),
                                kept ? o.p() : nullptr, S, dm, Hq, Hkv, D, causal, hc, wf, nf, nullptr);
        else
            rc = attn_layer_bwd(x.p(), wq.p(), wk.p(), wv.p(), wo.p(), dy.p(), kept ? o.p() : nullptr,
                                kept ? (const float*)lse.p() : nullptr, (float*)dx.p(),
                                (float*)dwq.p(), (float*)dwk.p(), (float*)dwv.p(), (float*)dwo.p(),
                                S, dm, Hq, Hkv, D, causal, hc, wb, nb, nullptr);
        if (rc != ATTN_OK)
            fail_msg("attn_layer returned %llu (%llu)", attn_last_error(), (size_t)rc, bwd);
        g_regions.resize(keep);
        g_allocs.pop_back();
    }
}

int main(int argc, char** argv) {
    bool inject = false;
    for (int i = 1; i < argc; ++i) {
        if (strcmp(argv[i], "--plant-dkdv-overread") == 0) g_plant = true;
        if (strcmp(argv[i], "--plant-dkdv-fast-run") == 0) g_plant_fast = true;
        if (strcmp(argv[i], "--plant-fwd-v-ring4") == 0) g_plant_vring = true;
        if (strcmp(argv[i], "--inject") == 0) inject = true;
    }
    if (inject) {
        // a failing trunk copy (pinned host K/V: forward and backward) or
        // kernel launch, early, in the middle and late in each call
        long cases = 0;
        for (int call = 0; call < 2; ++call)
            for (int copy = 0; copy < 2; ++copy)
                for (long at : {0L, 1L, 5L, 17L}) {
                    g_inj.call = call;
                    g_inj.copy = copy != 0;
                    g_inj.at = at;
                    run_case(1100, 8, 2, 128, 1, 4, 256, true);
                    run_case(700, 4, 2, 64, 1, 2, 0, false);
                    cases += 2;
                }
        g_inj = Inject{};
        printf("injection cases: %ld  failures injected: %ld  failures: %ld\n", cases, g_inject_hits,
               g_fails);
        return g_fails == 0 && g_inject_hits > 0 ? 0 : 1;
    }
    // sequence lengths at and around tile edges (64-row tiles, 128-key dK/dV
    // tiles, 128/256-row forward and dQ workgroups, 256-token trunks)
    const int64_t Ss[] = {1, 2, 33, 63, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256, 257,
                          300, 319, 320, 321, 383, 384, 385, 511, 512, 513, 600, 700, 777, 1100};
    struct Heads { int Hq, Hkv; };
    const Heads hs[] = {{1, 1}, {2, 1}, {4, 2}, {8, 2}, {8, 1}, {4, 4}, {6, 2}};
    long cases = 0;
    // the 8-wave forward's ring schedule for every tile count up to 64 (the
    // launches below are too small to take that shape)
    for (int nt = 0; nt <= 64; ++nt) hc::fwd_ring_check(nt, g_plant_vring ? 4 : 5);
    for (int pass = 0; pass < 2; ++pass) {
    // pass 1: the group-loop dK/dV schedule at every length
    g_gl_min_s = pass == 0 ? hc::kGroupLoopMinS : 1;
    attn_set_group_loop_min_s(g_gl_min_s);
    unsigned rng = 12345u;
    auto pick = [&](int n) { rng = rng * 1103515245u + 12345u; return (int)((rng >> 16) % (unsigned)n); };
    for (int64_t S : Ss)
        for (const Heads& h : hs)
            for (int D : {64, 128}) {
                // every head_chunk for one causal setting, a sampled one otherwise
                const int causal = pick(4) != 0;
                for (int hc = 1; hc <= h.Hq; ++hc) {
                    if (hc > 1 && hc < h.Hq && pick(2)) continue;
                    int64_t T = 0;
                    bool host = false;
                    const int tsel = S > 256 ? pick(3) : 0;
                    if (tsel && 256 * tsel < S) {  // a trunk at or past S is untrunked
                        T = 256 * tsel;
                        host = pick(2) != 0;
                    }
                    run_case(S, h.Hq, h.Hkv, D, causal, hc, T, host);
                    ++cases;
                }
            }
    // the workload shapes at a short length: 32/8 and 40/8 heads, one-group chunks
    for (int64_t S : {1000, 1024}) {
        run_case(S, 32, 8, 128, 1, 4, 0, false); ++cases;
        run_case(S, 40, 8, 128, 1, 5, 256, true); ++cases;
        run_case(S, 4, 1, 128, 1, 1, 512, false); ++cases;
    }
    // the attention layer: ragged S, groups split across chunks, D 64 / 128
    for (int64_t S : {1, 65, 300, 513})
        for (int hc : {1, 2, 3, 8}) {
            run_layer_case(S, 128, 8, 2, 64, 1, hc); ++cases;
        }
    run_layer_case(200, 192, 4, 1, 128, 0, 2); ++cases;
    run_layer_case(777, 256, 4, 2, 128, 1, 4); ++cases;
    }
    printf("cases: %ld  accesses checked: %ld  failures: %ld\n", cases, g_checks, g_fails);
    return g_fails == 0 ? 0 : 1;
}
