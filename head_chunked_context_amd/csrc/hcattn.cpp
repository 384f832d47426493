// hcattn.cpp - the C ABI (include/hcattn.h) and the host pipeline behind it.
//
// Forward, per head chunk (Road to 5 Million Tokens talk, U-Pipe paragraph:
// one group of heads at a time, partial result stored, buffers reused):
//   untrunked: pack the chunk's Q, K, V head-major -> flash kernel -> bf16 O, LSE
//   trunked  : for query trunk m: pack Q_m; for key trunk t = 0..m (causal) the
//              copy stream fills ring slot t%2 with K_t, V_t (pinned host or
//              device) while the previous trunk computes (FPDT summary,
//              "Technical Deep Dive": trunking, host offload, double buffer,
//              separate compute and offload streams).  The flash kernel
//              carries the query trunk's running softmax state (O, m, row
//              sums, fp32) from key trunk to key trunk and normalises after
//              the last one, which makes the result bitwise that of the
//              untrunked forward; attn_set_trunk_merge(1) selects the
//              partial-output schedule instead: each key trunk gives a
//              normalised partial with its LSE, merged into the running
//              output by log-sum-exp (same section, softmax statistics
//              updated until the trunk's final output).
// Backward, per head chunk: pack Q, dO (+ Delta), then per key range (the
// whole sequence, or key trunk t with the same ring) the dK/dV kernel and the
// dQ kernel; dQ is carried in fp32 across trunks, dK/dV in fp32 across chunks
// when a GQA group spans chunks.  Finished dK/dV of host-resident k/v leave
// through a staging slot and a device-to-host copy on the copy stream.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/hcattn.h"
#include "kernels.h"
#include "plan.h"

namespace {

thread_local char g_err[512];
std::atomic<int> g_single_stream{0};
std::atomic<int> g_trunk_merge{0};
std::atomic<int64_t> g_group_loop_min_s{hc::kGroupLoopMinS};

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

#define HIPCHK(expr)                                                                   \
    do {                                                                               \
        hipError_t e_ = (expr);                                                        \
        if (e_ != hipSuccess) {                                                        \
            return fail(ATTN_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));     \
        }                                                                              \
    } while (0)

// Events used by one call, per device.
enum Ev {
    EV_ENTRY,
    EV_LOADED0, EV_LOADED1,     // ring slot filled (copy stream)
    EV_FREE0, EV_FREE1,         // ring slot no longer read (compute stream)
    EV_STAGED0, EV_STAGED1,     // staging slot written (compute stream)
    EV_SFREE0, EV_SFREE1,       // staging slot copied out (copy stream)
    EV_EXIT,
    EV_COUNT
};

struct Device {
    std::mutex mu;
    bool ready = false;
    hipStream_t copy = nullptr;
    hipEvent_t ev[EV_COUNT] = {};
};
constexpr int kMaxDevices = 64;
Device g_dev[kMaxDevices];
std::mutex g_init;

int device_resources(Device** out) {
    int dev = 0;
    HIPCHK(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_EHIP, "device index %d out of range", dev);
    Device& d = g_dev[dev];
    std::lock_guard<std::mutex> lk(g_init);
    if (!d.ready) {
        // default priority on purpose: every stream here runs at one priority
        HIPCHK(hipStreamCreateWithFlags(&d.copy, hipStreamNonBlocking));
        for (int i = 0; i < EV_COUNT; ++i) {
            const hipError_t e = hipEventCreateWithFlags(&d.ev[i], hipEventDisableTiming);
            if (e != hipSuccess) {
                // undo, so that a later call starts over cleanly
                for (int k = 0; k < i; ++k) (void)hipEventDestroy(d.ev[k]);
                (void)hipStreamDestroy(d.copy);
                d.copy = nullptr;
                return fail(ATTN_EHIP, "hipEventCreateWithFlags failed: %s", hipGetErrorString(e));
            }
        }
        d.ready = true;
    }
    *out = &d;
    return ATTN_OK;
}

enum Loc { kLocDevice, kLocHost, kLocBad };

Loc where(const void* ptr) {
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, ptr) != hipSuccess) {
        (void)hipGetLastError();
        return kLocBad;
    }
    if (a.type == hipMemoryTypeDevice) return kLocDevice;
    if (a.type == hipMemoryTypeHost) return kLocHost;
    return kLocBad;
}


struct Common {
    hc::Plan pl;
    char* ws;
    hipStream_t st;    // caller's stream = compute stream
    hipStream_t cp;    // copy stream (== st in single-stream mode)
    Device* dev;
    float scale, scale_log2;
};

int plan_or_fail(bool bwd, int64_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t causal,
                 int32_t head_chunk, int64_t kv_trunk, hc::Plan* pl) {
    char msg[256];
    const int r = hc::make_plan(bwd, S, Hq, Hkv, D, causal, head_chunk, kv_trunk, pl, msg,
                                sizeof msg, g_group_loop_min_s.load());
    if (r == -1) return fail(ATTN_EINVAL, "%s", msg);
    if (r == -2) return fail(ATTN_EUNSUPPORTED, "%s", msg);
    return ATTN_OK;
}

int check_workspace(const hc::Plan& pl, void* ws, size_t bytes) {
    if (ws == nullptr) return fail(ATTN_EWORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(ws) % hc::kAlign != 0)
        return fail(ATTN_EWORKSPACE, "workspace must be %zu-byte aligned", hc::kAlign);
    if (bytes < pl.total)
        return fail(ATTN_EWORKSPACE, "workspace has %zu bytes, needs %zu", bytes, pl.total);
    return ATTN_OK;
}

// Copy rows [r0, r0 + rows) of heads [kv0, kv0 + nkv) of a token-major
// [S][H][D] bf16 tensor into a token-major [rows][nkv][D] slot (or back).
int copy_rows_in(void* dst, const void* src, int64_t r0, int64_t rows, int H, int kv0, int nkv,
                 int D, hipStream_t s) {
    const size_t row_b = (size_t)nkv * D * 2, pitch = (size_t)H * D * 2;
    const char* from = static_cast<const char*>(src) + ((size_t)r0 * H + kv0) * D * 2;
    HIPCHK(hipMemcpy2DAsync(dst, row_b, from, pitch, row_b, (size_t)rows, hipMemcpyDefault, s));
    return ATTN_OK;
}
int copy_rows_out(void* dst, const void* src, int64_t r0, int64_t rows, int H, int kv0, int nkv,
                  int src_nkv, int D, hipStream_t s) {
    const size_t row_b = (size_t)nkv * D * 2, pitch = (size_t)H * D * 2;
    char* to = static_cast<char*>(dst) + ((size_t)r0 * H + kv0) * D * 2;
    HIPCHK(hipMemcpy2DAsync(to, pitch, src, (size_t)src_nkv * D * 2, row_b, (size_t)rows,
                            hipMemcpyDefault, s));
    return ATTN_OK;
}

// Two-slot ring for key/value trunks: the copy stream fills slot n % 2 with
// the n-th trunk of the call while the compute stream reads slot (n-1) % 2.
struct Ring {
    Common* c;
    int uses[2] = {0, 0};
    int n = 0;
    // enqueue the copy of key trunk t (heads kv0..kv0+nkv) into the next slot
    int fill(const void* k, const void* v, int64_t t, int kv0, int nkv, int* slot) {
        const hc::Plan& p = c->pl;
        const int s = n & 1;
        Device* d = c->dev;
        HIPCHK(hipStreamWaitEvent(c->cp, d->ev[uses[s] == 0 ? EV_ENTRY : EV_FREE0 + s], 0));
        int r = copy_rows_in(c->ws + p.ring_k[s], k, p.trunk_begin(t), p.trunk_rows(t), p.Hkv, kv0,
                             nkv, p.D, c->cp);
        if (r) return r;
        r = copy_rows_in(c->ws + p.ring_v[s], v, p.trunk_begin(t), p.trunk_rows(t), p.Hkv, kv0, nkv,
                         p.D, c->cp);
        if (r) return r;
        HIPCHK(hipEventRecord(d->ev[EV_LOADED0 + s], c->cp));
        HIPCHK(hipStreamWaitEvent(c->st, d->ev[EV_LOADED0 + s], 0));
        ++uses[s];
        ++n;
        *slot = s;
        return ATTN_OK;
    }
    // the compute stream is done reading slot s
    int release(int s) {
        HIPCHK(hipEventRecord(c->dev->ev[EV_FREE0 + s], c->st));
        return ATTN_OK;
    }
};

// Called with the device's mutex held: orders the copy stream after all work
// the caller enqueued on st before this call.
int enter(Common& c, hipStream_t st) {
    c.st = st;
    c.cp = g_single_stream.load() ? st : c.dev->copy;
    HIPCHK(hipEventRecord(c.dev->ev[EV_ENTRY], st));
    return ATTN_OK;
}

int leave(Common& c) {
    HIPCHK(hipEventRecord(c.dev->ev[EV_EXIT], c.cp));
    HIPCHK(hipStreamWaitEvent(c.st, c.dev->ev[EV_EXIT], 0));
    return ATTN_OK;
}

// ------------------------------------------------------------ kernel timing

enum Kid { K_FWD, K_MERGE, K_PACK, K_PREP, K_DKDV, K_REDUCE, K_DQ, K_GEMM, K_COUNT };
const char* const kKernelNames[K_COUNT] = {"fwd", "merge", "pack", "prep", "dkdv", "reduce", "dq",
                                           "gemm"};

struct TimingRec {
    int kid;
    hipEvent_t a, b;
    double bytes;  // HBM bytes the launch reads and writes by its parameters (0: not a pass)
};
std::atomic<int> g_timing{0};
std::mutex g_tmu;
std::vector<TimingRec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t pool_event() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Launch through `launch` (returns hipError_t); when timing is on, bracket it
// with events on stream st.
template <class F>
hipError_t timed(int kid, hipStream_t st, double bytes, F&& launch) {
    if (!g_timing.load()) return launch();
    std::lock_guard<std::mutex> lk(g_tmu);
    TimingRec r{kid, pool_event(), pool_event(), bytes};
    if (r.a == nullptr || r.b == nullptr) return hipErrorOutOfMemory;
    hipError_t e = hipEventRecord(r.a, st);
    if (e != hipSuccess) return e;
    e = launch();
    if (e != hipSuccess) return e;
    e = hipEventRecord(r.b, st);
    if (e != hipSuccess) return e;
    g_recs.push_back(r);
    return hipSuccess;
}

#define KCHK(expr)                                                                         \
    do {                                                                                   \
        hipError_t e_ = (expr);                                                            \
        if (e_ != hipSuccess) return fail(ATTN_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)
#define LAUNCH(kid, call) KCHK(timed(kid, c.st, 0.0, [&]() { return (call); }))
// the streaming passes also record the bytes they move (read + write), which
// follow from their parameters alone
#define LAUNCH_PASS(kid, prm, call) KCHK(timed(kid, c.st, moved_bytes(prm), [&]() { return (call); }))

double moved_bytes(const hc::PackParams& p) {
    return 2.0 * p.nh * (double)p.rows * p.D * 2;  // bf16 in, bf16 out
}
double moved_bytes(const hc::PrepParams& p) {
    // O and dO in, packed dO out (bf16); LSE in, -Delta and -LSE log2(e) out (fp32)
    return (double)p.nh * p.rows * (3.0 * p.D * 2 + 12);
}
double moved_bytes(const hc::MergeParams& p) {
    // running and trunk O (fp32) and LSE in; running O / LSE or bf16 O / LSE out
    const double out = p.final_out ? p.D * 2.0 + 4 : p.D * 4.0 + 4;
    return (double)p.nh * p.rows * (2.0 * p.D * 4 + 8 + out);
}
double moved_bytes(const hc::DkdvReduceParams& p) {
    const double row = (double)p.nk * p.D;
    double b = p.nh * row * 8;                    // fp32 dK and dV partials of every head
    if (p.carry_kv_in >= 0) b += row * 8;         // fp32 carry in
    const int carry_out = p.carry_kv_out >= 0 ? 1 : 0;
    b += (p.nkv - carry_out) * row * 4;           // bf16 dK, dV
    b += carry_out * row * 8;                     // fp32 carry out
    return b;
}

// ------------------------------------------------------------------ forward

int fwd_untrunked(Common& c, const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                  float* lse) {
    const hc::Plan& p = c.pl;
    const int64_t S = p.S;
    const int D = p.D;
    uint16_t* Qc = reinterpret_cast<uint16_t*>(c.ws + p.q_c);
    uint16_t* Kc = reinterpret_cast<uint16_t*>(c.ws + p.k_c);
    uint16_t* Vc = reinterpret_cast<uint16_t*>(c.ws + p.v_c);
    for (int ci = 0; ci < p.nchunks; ++ci) {
        const hc::Chunk ch = p.chunk(ci);
        hc::PackParams pk{q + (size_t)ch.h0 * D, (int64_t)p.Hq * D, D, Qc, D, S * D, ch.nh, S, D};
        LAUNCH_PASS(K_PACK, pk, hc::launch_pack(pk, c.st));
        pk = {k + (size_t)ch.kv0 * D, (int64_t)p.Hkv * D, D, Kc, D, S * D, ch.nkv, S, D};
        LAUNCH_PASS(K_PACK, pk, hc::launch_pack(pk, c.st));
        pk = {v + (size_t)ch.kv0 * D, (int64_t)p.Hkv * D, D, Vc, D, S * D, ch.nkv, S, D};
        LAUNCH_PASS(K_PACK, pk, hc::launch_pack(pk, c.st));
        hc::FwdParams f{};
        f.q = Qc; f.q_rs = D; f.q_hs = S * D;
        f.k = Kc; f.k_rs = D; f.k_hs = S * D;
        f.v = Vc; f.v_rs = D; f.v_hs = S * D;
        f.o = o + (size_t)ch.h0 * D; f.o_rs = (int64_t)p.Hq * D; f.o_hs = D;
        f.lse = lse ? lse + (size_t)ch.h0 * S : nullptr; f.lse_hs = S;
        f.nh = ch.nh; f.group = p.g; f.h0 = ch.h0; f.kv_base = ch.kv0;
        f.nq = S; f.q_pos0 = 0; f.nk = S; f.k_pos0 = 0;
        f.causal = p.causal; f.mode = hc::kFwdFinal; f.scale_log2 = c.scale_log2;
        LAUNCH(K_FWD, hc::launch_fwd(f, D, c.st));
    }
    return ATTN_OK;
}

int fwd_trunked(Common& c, const uint16_t* q, const void* k, const void* v, uint16_t* o, float* lse) {
    const hc::Plan& p = c.pl;
    const int D = p.D;
    const int64_t T = p.T;
    const bool merge = g_trunk_merge.load() != 0;
    uint16_t* Qm = reinterpret_cast<uint16_t*>(c.ws + p.q_c);
    float* Orun = reinterpret_cast<float*>(c.ws + p.o_run);
    float* Ot = reinterpret_cast<float*>(c.ws + p.o_t);
    float* Lrun = reinterpret_cast<float*>(c.ws + p.l_run);
    float* Lt = reinterpret_cast<float*>(c.ws + p.l_t);
    float* Lpair = reinterpret_cast<float*>(c.ws + p.st_l);
    Ring ring{&c};
    for (int ci = 0; ci < p.nchunks; ++ci) {
        const hc::Chunk ch = p.chunk(ci);
        for (int64_t m = 0; m < p.N; ++m) {
            const int64_t qr0 = p.trunk_begin(m), nq = p.trunk_rows(m);
            hc::PackParams pk{q + ((size_t)qr0 * p.Hq + ch.h0) * D, (int64_t)p.Hq * D, D, Qm, D,
                              T * D, ch.nh, nq, D};
            LAUNCH_PASS(K_PACK, pk, hc::launch_pack(pk, c.st));
            float* lse_m = lse ? lse + (size_t)ch.h0 * p.S + qr0 : nullptr;
            uint16_t* o_m = o + ((size_t)qr0 * p.Hq + ch.h0) * D;
            const int64_t tlast = p.causal ? m : p.N - 1;
            for (int64_t t = 0; t <= tlast; ++t) {
                int slot = 0;
                int r = ring.fill(k, v, t, ch.kv0, ch.nkv, &slot);
                if (r) return r;
                hc::FwdParams f{};
                f.q = Qm; f.q_rs = D; f.q_hs = T * D;
                f.k = reinterpret_cast<const uint16_t*>(c.ws + p.ring_k[slot]);
                f.k_rs = (int64_t)ch.nkv * D; f.k_hs = D;
                f.v = reinterpret_cast<const uint16_t*>(c.ws + p.ring_v[slot]);
                f.v_rs = (int64_t)ch.nkv * D; f.v_hs = D;
                f.nh = ch.nh; f.group = p.g; f.h0 = ch.h0; f.kv_base = ch.kv0;
                f.nq = nq; f.q_pos0 = qr0; f.nk = p.trunk_rows(t); f.k_pos0 = p.trunk_begin(t);
                f.causal = p.causal; f.scale_log2 = c.scale_log2;
                const bool last = t == tlast;
                if (!merge) {
                    // the running softmax state goes from trunk to trunk through
                    // the workspace; the last trunk writes the normalised output
                    f.carry_in = t > 0;
                    f.carry_out = !last;
                    f.st_o = Orun; f.st_o_hs = nq * D;
                    f.st_m = Lrun; f.st_l = Lpair; f.st_hs = nq;
                    f.mode = hc::kFwdFinal;
                    f.o = o_m; f.o_rs = (int64_t)p.Hq * D; f.o_hs = D;
                    f.lse = lse_m; f.lse_hs = p.S;
                } else if (tlast == 0) {
                    f.mode = hc::kFwdFinal;
                    f.o = o_m; f.o_rs = (int64_t)p.Hq * D; f.o_hs = D;
                    f.lse = lse_m; f.lse_hs = p.S;
                } else {
                    f.mode = hc::kFwdPartial;
                    f.o = t == 0 ? Orun : Ot; f.o_rs = D; f.o_hs = nq * D;
                    f.lse = t == 0 ? Lrun : Lt; f.lse_hs = nq;
                }
                LAUNCH(K_FWD, hc::launch_fwd(f, D, c.st));
                r = ring.release(slot);
                if (r) return r;
                if (merge && t > 0) {
                    hc::MergeParams mg{};
                    mg.o_r = Orun; mg.l_r = Lrun; mg.o_t = Ot; mg.l_t = Lt;
                    mg.nh = ch.nh; mg.rows = nq; mg.D = D;
                    mg.final_out = last;
                    mg.out = o_m; mg.out_rs = (int64_t)p.Hq * D; mg.out_hs = D;
                    mg.lse_out = lse_m; mg.lse_hs = p.S;
                    LAUNCH_PASS(K_MERGE, mg, hc::launch_merge(mg, c.st));
                }
            }
        }
    }
    return ATTN_OK;
}

// ----------------------------------------------------------------- backward

struct BwdIO {
    const uint16_t *q, *o, *dout;
    const void *k, *v;
    const float* lse;
    uint16_t* dq;
    void *dk, *dv;
    bool kv_host;
};

// dK/dV partial kernel parameters for chunk ch over keys [kr0, kr0 + nk) held in (kk, vv)
hc::DkdvParams dkdv_params(const Common& c, const hc::Chunk& ch, const BwdIO& io,
                           const uint16_t* kk, const uint16_t* vv, int64_t k_rs, int64_t k_hs,
                           int64_t kr0, int64_t nk) {
    const hc::Plan& p = c.pl;
    const int D = p.D;
    hc::DkdvParams d{};
    d.q = reinterpret_cast<const uint16_t*>(c.ws + p.q_c); d.q_rs = D; d.q_hs = p.S * D;
    d.dO = reinterpret_cast<const uint16_t*>(c.ws + p.do_c); d.do_rs = D; d.do_hs = p.S * D;
    d.nlse2 = reinterpret_cast<const float*>(c.ws + p.lse2_c); d.nlse2_hs = p.S;
    d.ndelta = reinterpret_cast<const float*>(c.ws + p.delta_c); d.ndelta_hs = p.S;
    d.k = kk; d.v = vv; d.k_rs = d.v_rs = k_rs; d.k_hs = d.v_hs = k_hs;
    d.nh = ch.nh; d.group = p.g; d.h0 = ch.h0; d.kv_base = ch.kv0;
    d.nq = p.S; d.nk = nk; d.k_pos0 = kr0; d.causal = p.causal;
    d.scale_log2 = c.scale_log2;
    d.part_k = reinterpret_cast<float*>(c.ws + p.part_k);
    d.part_v = reinterpret_cast<float*>(c.ws + p.part_v);
    d.group_loop = p.group_loop ? 1 : 0;
    d.nkv = ch.nkv;
    d.carry_kv_in = -1;
    d.carry_kv_out = -1;
    d.scale = c.scale;
    return d;
}

// Ordered head sum of the partials, with the fp32 carries of groups that span
// chunks; final bf16 rows go to (dk, dv) with the given strides.
hc::DkdvReduceParams reduce_params(const Common& c, const hc::Chunk& ch, int ci, int64_t kr0,
                                   int64_t nk, uint16_t* dk, uint16_t* dv, int64_t rs, int64_t hs) {
    const hc::Plan& p = c.pl;
    const int D = p.D;
    hc::DkdvReduceParams r{};
    r.part_k = reinterpret_cast<const float*>(c.ws + p.part_k);
    r.part_v = reinterpret_cast<const float*>(c.ws + p.part_v);
    r.nh = ch.nh; r.group = p.g; r.h0 = ch.h0; r.kv_base = ch.kv0; r.nkv = ch.nkv;
    r.nk = nk; r.D = D;
    const int in_s = p.carry_in_slot(ci), out_s = p.carry_out_slot(ci);
    r.carry_kv_in = -1;
    r.carry_kv_out = -1;
    if (in_s >= 0) {
        r.carry_in_k = reinterpret_cast<const float*>(c.ws + p.carry_k[in_s]) + (size_t)kr0 * D;
        r.carry_in_v = reinterpret_cast<const float*>(c.ws + p.carry_v[in_s]) + (size_t)kr0 * D;
        r.carry_kv_in = 0;
    }
    if (out_s >= 0) {
        r.carry_out_k = reinterpret_cast<float*>(c.ws + p.carry_k[out_s]) + (size_t)kr0 * D;
        r.carry_out_v = reinterpret_cast<float*>(c.ws + p.carry_v[out_s]) + (size_t)kr0 * D;
        r.carry_kv_out = ch.nkv - 1;
    }
    r.dk = dk; r.dv = dv; r.dk_rs = rs; r.dk_hs = hs;
    r.scale = c.scale;
    return r;
}

// dK/dV of chunk ci over keys [kr0, kr0 + nk) held in (kk, vv): bf16 results
// of the kv heads whose group ends in this chunk go to (dk, dv) with strides
// (rs, hs); a group that continues leaves fp32 sums in a carry slot.
// Group-loop schedule: one launch writes both.  Per-head schedule: per-head
// partials, then the ordered reduce over the group's heads.
int dkdv_run(Common& c, const hc::Chunk& ch, int ci, const BwdIO& io, const uint16_t* kk,
             const uint16_t* vv, int64_t k_rs, int64_t k_hs, int64_t kr0, int64_t nk,
             uint16_t* dk, uint16_t* dv, int64_t rs, int64_t hs) {
    const hc::Plan& p = c.pl;
    const int D = p.D;
    hc::DkdvParams d = dkdv_params(c, ch, io, kk, vv, k_rs, k_hs, kr0, nk);
    if (!p.group_loop) {
        LAUNCH(K_DKDV, hc::launch_dkdv(d, D, c.st));
        hc::DkdvReduceParams rd = reduce_params(c, ch, ci, kr0, nk, dk, dv, rs, hs);
        LAUNCH_PASS(K_REDUCE, rd, hc::launch_dkdv_reduce(rd, c.st));
        return ATTN_OK;
    }
    // carries: [S][D] fp32 per slot, at this launch's first key
    const int in_s = p.carry_in_slot(ci), out_s = p.carry_out_slot(ci);
    if (in_s >= 0) {
        d.carry_in_k = reinterpret_cast<const float*>(c.ws + p.carry_k[in_s]) + (size_t)kr0 * D;
        d.carry_in_v = reinterpret_cast<const float*>(c.ws + p.carry_v[in_s]) + (size_t)kr0 * D;
        d.carry_kv_in = 0;
    }
    if (out_s >= 0) {
        d.carry_out_k = reinterpret_cast<float*>(c.ws + p.carry_k[out_s]) + (size_t)kr0 * D;
        d.carry_out_v = reinterpret_cast<float*>(c.ws + p.carry_v[out_s]) + (size_t)kr0 * D;
        d.carry_kv_out = ch.nkv - 1;
    }
    d.dk = dk; d.dv = dv; d.dk_rs = rs; d.dk_hs = hs;
    LAUNCH(K_DKDV, hc::launch_dkdv(d, D, c.st));
    return ATTN_OK;
}

int bwd_chunk_prep(Common& c, const hc::Chunk& ch, const BwdIO& io) {
    const hc::Plan& p = c.pl;
    const int D = p.D;
    const int64_t S = p.S;
    uint16_t* Qc = reinterpret_cast<uint16_t*>(c.ws + p.q_c);
    hc::PackParams pk{io.q + (size_t)ch.h0 * D, (int64_t)p.Hq * D, D, Qc, D, S * D, ch.nh, S, D};
    LAUNCH_PASS(K_PACK, pk, hc::launch_pack(pk, c.st));
    hc::PrepParams pr{};
    pr.o = io.o + (size_t)ch.h0 * D; pr.o_rs = (int64_t)p.Hq * D; pr.o_hs = D;
    pr.dO = io.dout + (size_t)ch.h0 * D; pr.do_rs = (int64_t)p.Hq * D; pr.do_hs = D;
    pr.lse = io.lse + (size_t)ch.h0 * S; pr.lse_hs = S;
    pr.dO_c = reinterpret_cast<uint16_t*>(c.ws + p.do_c); pr.c_rs = D; pr.c_hs = S * D;
    pr.ndelta = reinterpret_cast<float*>(c.ws + p.delta_c); pr.ndelta_hs = S;
    pr.nlse2 = reinterpret_cast<float*>(c.ws + p.lse2_c); pr.nlse2_hs = S;
    pr.nh = ch.nh; pr.rows = S; pr.D = D;
    LAUNCH_PASS(K_PREP, pr, hc::launch_prep(pr, c.st));
    return ATTN_OK;
}

hc::DqParams dq_params(const Common& c, const hc::Chunk& ch, const BwdIO& io, const uint16_t* kk,
                       const uint16_t* vv, int64_t k_rs, int64_t k_hs, int64_t kr0, int64_t nk) {
    const hc::Plan& p = c.pl;
    const int D = p.D;
    hc::DqParams d{};
    d.q = reinterpret_cast<const uint16_t*>(c.ws + p.q_c); d.q_rs = D; d.q_hs = p.S * D;
    d.dO = reinterpret_cast<const uint16_t*>(c.ws + p.do_c); d.do_rs = D; d.do_hs = p.S * D;
    d.nlse2 = reinterpret_cast<const float*>(c.ws + p.lse2_c); d.nlse2_hs = p.S;
    d.ndelta = reinterpret_cast<const float*>(c.ws + p.delta_c); d.ndelta_hs = p.S;
    d.k = kk; d.v = vv; d.k_rs = d.v_rs = k_rs; d.k_hs = d.v_hs = k_hs;
    d.nh = ch.nh; d.group = p.g; d.h0 = ch.h0; d.kv_base = ch.kv0;
    d.nq = p.S; d.nk = nk; d.k_pos0 = kr0; d.causal = p.causal;
    d.scale = c.scale; d.scale_log2 = c.scale_log2;
    d.dq = io.dq + (size_t)ch.h0 * D; d.dq_rs = (int64_t)p.Hq * D; d.dq_hs = D;
    d.q_begin = 0;
    d.final_before = p.S;
    return d;
}

int bwd_untrunked(Common& c, const BwdIO& io) {
    const hc::Plan& p = c.pl;
    const int D = p.D;
    const int64_t S = p.S;
    uint16_t* Kc = reinterpret_cast<uint16_t*>(c.ws + p.k_c);
    uint16_t* Vc = reinterpret_cast<uint16_t*>(c.ws + p.v_c);
    for (int ci = 0; ci < p.nchunks; ++ci) {
        const hc::Chunk ch = p.chunk(ci);
        int r = bwd_chunk_prep(c, ch, io);
        if (r) return r;
        const uint16_t* k = static_cast<const uint16_t*>(io.k);
        const uint16_t* v = static_cast<const uint16_t*>(io.v);
        hc::PackParams pk{k + (size_t)ch.kv0 * D, (int64_t)p.Hkv * D, D, Kc, D, S * D, ch.nkv, S, D};
        LAUNCH_PASS(K_PACK, pk, hc::launch_pack(pk, c.st));
        pk = {v + (size_t)ch.kv0 * D, (int64_t)p.Hkv * D, D, Vc, D, S * D, ch.nkv, S, D};
        LAUNCH_PASS(K_PACK, pk, hc::launch_pack(pk, c.st));
        r = dkdv_run(c, ch, ci, io, Kc, Vc, D, S * D, 0, S,
                     static_cast<uint16_t*>(io.dk) + (size_t)ch.kv0 * D,
                     static_cast<uint16_t*>(io.dv) + (size_t)ch.kv0 * D, (int64_t)p.Hkv * D, D);
        if (r) return r;
        hc::DqParams dq = dq_params(c, ch, io, Kc, Vc, D, S * D, 0, S);
        LAUNCH(K_DQ, hc::launch_dq(dq, D, c.st));
    }
    return ATTN_OK;
}

int bwd_trunked(Common& c, const BwdIO& io) {
    const hc::Plan& p = c.pl;
    const int D = p.D;
    const int64_t S = p.S;
    float* dQacc = reinterpret_cast<float*>(c.ws + p.dq_acc);
    Ring ring{&c};
    int stage_uses[2] = {0, 0}, nstage = 0;
    for (int ci = 0; ci < p.nchunks; ++ci) {
        const hc::Chunk ch = p.chunk(ci);
        int r = bwd_chunk_prep(c, ch, io);
        if (r) return r;
        const bool carry_out = p.carry_out_slot(ci) >= 0;
        const int nfin = ch.nkv - (carry_out ? 1 : 0);  // kv heads finished in this chunk
        for (int64_t t = 0; t < p.N; ++t) {
            const int64_t kr0 = p.trunk_begin(t), nk = p.trunk_rows(t);
            int slot = 0;
            r = ring.fill(io.k, io.v, t, ch.kv0, ch.nkv, &slot);
            if (r) return r;
            const uint16_t* kk = reinterpret_cast<const uint16_t*>(c.ws + p.ring_k[slot]);
            const uint16_t* vv = reinterpret_cast<const uint16_t*>(c.ws + p.ring_v[slot]);
            int ss = -1;
            if (io.kv_host) {
                ss = nstage & 1;
                Device* d = c.dev;
                if (stage_uses[ss] > 0) HIPCHK(hipStreamWaitEvent(c.st, d->ev[EV_SFREE0 + ss], 0));
                r = dkdv_run(c, ch, ci, io, kk, vv, (int64_t)ch.nkv * D, D, kr0, nk,
                             reinterpret_cast<uint16_t*>(c.ws + p.stage_k[ss]),
                             reinterpret_cast<uint16_t*>(c.ws + p.stage_v[ss]),
                             (int64_t)ch.nkv * D, D);
            } else {
                r = dkdv_run(c, ch, ci, io, kk, vv, (int64_t)ch.nkv * D, D, kr0, nk,
                             static_cast<uint16_t*>(io.dk) + ((size_t)kr0 * p.Hkv + ch.kv0) * D,
                             static_cast<uint16_t*>(io.dv) + ((size_t)kr0 * p.Hkv + ch.kv0) * D,
                             (int64_t)p.Hkv * D, D);
            }
            if (r) return r;
            // the finished dK/dV rows leave as soon as they are staged, so
            // their copy, and the next trunk's load queued behind it on the
            // copy stream, run while dQ of this trunk computes
            if (io.kv_host && nfin > 0) {
                Device* d = c.dev;
                HIPCHK(hipEventRecord(d->ev[EV_STAGED0 + ss], c.st));
                HIPCHK(hipStreamWaitEvent(c.cp, d->ev[EV_STAGED0 + ss], 0));
                r = copy_rows_out(io.dk, c.ws + p.stage_k[ss], kr0, nk, p.Hkv, ch.kv0, nfin, ch.nkv,
                                  D, c.cp);
                if (r) return r;
                r = copy_rows_out(io.dv, c.ws + p.stage_v[ss], kr0, nk, p.Hkv, ch.kv0, nfin, ch.nkv,
                                  D, c.cp);
                if (r) return r;
                HIPCHK(hipEventRecord(d->ev[EV_SFREE0 + ss], c.cp));
                ++stage_uses[ss];
                ++nstage;
            } else if (io.kv_host) {
                ++nstage;
            }
            hc::DqParams dq = dq_params(c, ch, io, kk, vv, (int64_t)ch.nkv * D, D, kr0, nk);
            dq.q_begin = p.causal ? kr0 : 0;
            dq.acc_in = t == 0 ? nullptr : dQacc;
            dq.ain_rs = D; dq.ain_hs = S * D;
            dq.acc_out = dQacc; dq.aout_rs = D; dq.aout_hs = S * D;
            dq.final_before = p.causal ? kr0 + nk : (t == p.N - 1 ? S : 0);
            LAUNCH(K_DQ, hc::launch_dq(dq, D, c.st));
            r = ring.release(slot);
            if (r) return r;
        }
    }
    return ATTN_OK;
}

// ------------------------------------------------------------ attention layer
//
// The layer around the attention, walked a head chunk at a time (Road to 5
// Million Tokens talk, the U-Pipe paragraph: the chunk's heads are
// recomputed, attended and their partial result stored, and the buffers are
// reused).  Weights in the [out][in] convention, y = x W^T:
//   x [S][dm] bf16; wq [Hq*D][dm], wk, wv [Hkv*D][dm], wo [dm][Hq*D] bf16;
//   y [S][dm] fp32 = sum over chunks of o_c wo[:, chunk columns]^T.
// Per chunk: Q_c, K_c, V_c = x W^T of the chunk's rows, written head-major
// straight by the matrix product; the flash kernel; y += O_c wo_c^T.  The
// backward recomputes the chunk's projections and attention output, then
// dO_c = dy wo_c, dWo_c = dy^T O_c, the attention backward, and per GQA group
// in ascending order dx += dQ_g Wq_g (+ dK Wk + dV Wv once the group's last
// head is done), dWq = dQ^T x, dWk = dK^T x, dWv = dV^T x.  Every fp32 sum
// into y and dx continues from the stored value in a fixed group order, so
// the results do not depend on head_chunk.

struct LayerPlan {
    hc::Plan at;                 // attention plan of the chunk loop (backward: its regions)
    int dm;
    size_t q_c = 0, k_c = 0, v_c = 0, o_c = 0;          // bf16 head-major chunk buffers
    size_t lse_c = 0, dq_c = 0, dk_c = 0, dv_c = 0;     // backward extras
    size_t wpart = 0;                                   // split-K partials of weight gradients
    int splits = 1;
    int64_t k_split = 0;
    size_t total = 0;
};

constexpr int kWgradSplits = 8;

int layer_plan(bool bwd, int64_t S, int dm, int Hq, int Hkv, int D, int causal, int head_chunk,
               LayerPlan* L) {
    int r = plan_or_fail(bwd, S, Hq, Hkv, D, causal, head_chunk, 0, &L->at);
    if (r) return r;
    if (dm < 64 || dm % 64 != 0) return fail(ATTN_EINVAL, "d_model must be a positive multiple of 64 (got %d)", dm);
    if ((double)S * dm * 16.0 > 0x1p62) return fail(ATTN_EUNSUPPORTED, "S x d_model too large");
    const hc::Plan& p = L->at;
    L->dm = dm;
    const size_t E = (size_t)S * D * 2;
    size_t off = p.total;
    auto take = [&](size_t bytes) { size_t o = off; off = hc::align_up(off + bytes); return o; };
    if (!bwd) {
        // the attention plan's own regions (Q_c, K_c, V_c) plus O_c
        L->q_c = p.q_c; L->k_c = p.k_c; L->v_c = p.v_c;
        L->o_c = take(p.hc * E);
    } else {
        L->q_c = p.q_c; L->k_c = p.k_c; L->v_c = p.v_c;
        L->o_c = take(p.hc * E);
        L->lse_c = take((size_t)p.hc * S * 4);
        L->dq_c = take(p.hc * E);
        L->dk_c = take(p.kvc * E);
        L->dv_c = take(p.kvc * E);
        // split-K of the weight gradients: a function of S only, so that every
        // weight row sums its terms the same way whatever the chunking
        L->k_split = (S + 64 * kWgradSplits - 1) / (64 * kWgradSplits) * 64;
        L->splits = (int)((S + L->k_split - 1) / L->k_split);
        L->wpart = take((size_t)L->splits * p.hc * D * dm * 4);
    }
    L->total = off;
    return ATTN_OK;
}

// C = x W^T for `rows` rows of W starting at w (row-major [*][dm]), written
// bf16 head-major [rows / D][S][D] at dst
hc::GemmParams proj_params(const uint16_t* x, const uint16_t* w, int rows, int64_t S, int dm,
                           int D, uint16_t* dst) {
    hc::GemmParams g{};
    g.a = x; g.a_rs = dm; g.a_seg = dm; g.a_segs = 0;
    g.b = w; g.b_rs = dm; g.b_seg = dm; g.b_segs = 0;
    g.M = S; g.N = rows; g.K = dm;
    g.c = dst; g.c_rs = D; g.c_seg = D; g.c_segs = S * D;
    g.out_mode = hc::kGemmBf16;
    return g;
}

#define LAUNCH_GEMM(prm, akc, bkc, splits) \
    KCHK(timed(K_GEMM, c.st, 0.0, [&]() { return hc::launch_gemm((prm), (akc), (bkc), (splits), c.st); }))

// the chunk's projections into the chunk buffers and, if Oc is given, its
// attention output into Oc (head-major [nh][S][D]) with the LSE
int layer_chunk_forward(Common& c, const LayerPlan& L, const hc::Chunk& ch, const uint16_t* x,
                        const uint16_t* wq, const uint16_t* wk, const uint16_t* wv, uint16_t* Oc,
                        float* lse, int64_t lse_hs) {
    const hc::Plan& p = L.at;
    const int64_t S = p.S;
    const int D = p.D, dm = L.dm;
    uint16_t* Qc = reinterpret_cast<uint16_t*>(c.ws + L.q_c);
    uint16_t* Kc = reinterpret_cast<uint16_t*>(c.ws + L.k_c);
    uint16_t* Vc = reinterpret_cast<uint16_t*>(c.ws + L.v_c);
    hc::GemmParams g = proj_params(x, wq + (size_t)ch.h0 * D * dm, ch.nh * D, S, dm, D, Qc);
    LAUNCH_GEMM(g, true, true, 1);
    g = proj_params(x, wk + (size_t)ch.kv0 * D * dm, ch.nkv * D, S, dm, D, Kc);
    LAUNCH_GEMM(g, true, true, 1);
    g = proj_params(x, wv + (size_t)ch.kv0 * D * dm, ch.nkv * D, S, dm, D, Vc);
    LAUNCH_GEMM(g, true, true, 1);
    if (Oc == nullptr) return ATTN_OK;
    hc::FwdParams f{};
    f.q = Qc; f.q_rs = D; f.q_hs = S * D;
    f.k = Kc; f.k_rs = D; f.k_hs = S * D;
    f.v = Vc; f.v_rs = D; f.v_hs = S * D;
    f.o = Oc; f.o_rs = D; f.o_hs = S * D;
    f.lse = lse; f.lse_hs = lse_hs;
    f.nh = ch.nh; f.group = p.g; f.h0 = ch.h0; f.kv_base = ch.kv0;
    f.nq = S; f.q_pos0 = 0; f.nk = S; f.k_pos0 = 0;
    f.causal = p.causal; f.mode = hc::kFwdFinal; f.scale_log2 = c.scale_log2;
    LAUNCH(K_FWD, hc::launch_fwd(f, D, c.st));
    return ATTN_OK;
}

int layer_fwd_run(Common& c, const LayerPlan& L, const uint16_t* x, const uint16_t* wq,
                  const uint16_t* wk, const uint16_t* wv, const uint16_t* wo, float* y, float* lse,
                  uint16_t* o_keep) {
    const hc::Plan& p = L.at;
    const int64_t S = p.S;
    const int D = p.D, dm = L.dm;
    for (int ci = 0; ci < p.nchunks; ++ci) {
        const hc::Chunk ch = p.chunk(ci);
        // the chunk's attention output: the reused chunk buffer, or its heads
        // of the caller's kept output
        uint16_t* Oc = o_keep ? o_keep + (size_t)ch.h0 * S * D : reinterpret_cast<uint16_t*>(c.ws + L.o_c);
        int r = layer_chunk_forward(c, L, ch, x, wq, wk, wv, Oc,
                                    lse ? lse + (size_t)ch.h0 * S : nullptr, S);
        if (r) return r;
        // y += O_c wo[:, h0 D .. (h0 + nh) D]^T
        hc::GemmParams g{};
        g.a = Oc; g.a_rs = D; g.a_seg = D; g.a_segs = S * D;
        g.b = wo + (size_t)ch.h0 * D; g.b_rs = (int64_t)p.Hq * D; g.b_seg = (int64_t)p.Hq * D; g.b_segs = 0;
        g.M = S; g.N = dm; g.K = (int64_t)ch.nh * D;
        g.c = y; g.c_rs = dm; g.c_seg = dm; g.c_segs = 0;
        g.out_mode = ci == 0 ? hc::kGemmF32 : hc::kGemmF32Add;
        LAUNCH_GEMM(g, true, true, 1);
    }
    return ATTN_OK;
}

// weight gradient rows: out[m][n] = sum_s A(m, s) B(n, s) over the whole
// sequence (A, B r-contiguous), split-K into the partial buffer and reduced
// in ascending split order
int wgrad(Common& c, const LayerPlan& L, hc::GemmParams g, float* out, int64_t out_rs) {
    float* part = reinterpret_cast<float*>(c.ws + L.wpart);
    g.c = part; g.c_rs = g.N; g.c_seg = g.N; g.c_segs = 0;
    g.out_mode = hc::kGemmF32;
    g.k_split = L.k_split; g.c_zs = g.M * g.N;
    LAUNCH_GEMM(g, false, false, L.splits);
    hc::GemmReduceParams rp{part, g.M * g.N, L.splits, g.M, g.N, out, out_rs, 0};
    KCHK(timed(K_GEMM, c.st, 0.0, [&]() { return hc::launch_gemm_reduce(rp, c.st); }));
    return ATTN_OK;
}

int layer_bwd_run(Common& c, const LayerPlan& L, const uint16_t* x, const uint16_t* wq,
                  const uint16_t* wk, const uint16_t* wv, const uint16_t* wo, const uint16_t* dy,
                  const uint16_t* o_kept, const float* lse_kept, float* dx, float* dwq, float* dwk,
                  float* dwv, float* dwo) {
    const hc::Plan& p = L.at;
    const int64_t S = p.S;
    const int D = p.D, dm = L.dm, Hq = p.Hq;
    uint16_t* Kc = reinterpret_cast<uint16_t*>(c.ws + L.k_c);
    uint16_t* Vc = reinterpret_cast<uint16_t*>(c.ws + L.v_c);
    uint16_t* Oc = reinterpret_cast<uint16_t*>(c.ws + L.o_c);
    uint16_t* dOc = reinterpret_cast<uint16_t*>(c.ws + p.do_c);
    uint16_t* dQc = reinterpret_cast<uint16_t*>(c.ws + L.dq_c);
    uint16_t* dKc = reinterpret_cast<uint16_t*>(c.ws + L.dk_c);
    uint16_t* dVc = reinterpret_cast<uint16_t*>(c.ws + L.dv_c);
    float* lse_c = reinterpret_cast<float*>(c.ws + L.lse_c);
    bool dx_started = false;
    // dx += sum over parts i of A_i(m = s, k) B_i(n, k), k < K_i, in part
    // order, in one product: A_i head-major [K_i / D][S][D] (k contiguous),
    // B_i = rows of a weight [*][dm] read n-contiguous
    auto dx_add = [&](int nparts, const uint16_t* const* a, const uint16_t* const* w,
                      const int64_t* kk) -> int {
        hc::GemmParams g{};
        g.a = a[0]; g.a_rs = D; g.a_seg = D; g.a_segs = S * D;
        g.b = w[0]; g.b_rs = dm; g.b_seg = dm; g.b_segs = 0;
        g.M = S; g.N = dm; g.K = 0;
        g.k_parts = nparts;
        for (int i = 0; i < nparts; ++i) {
            g.k_at[i] = g.K;
            g.a_at[i] = a[i];
            g.b_at[i] = w[i];
            g.K += kk[i];
        }
        g.k_at[nparts] = g.K;
        g.c = dx; g.c_rs = dm; g.c_seg = dm; g.c_segs = 0;
        g.out_mode = dx_started ? hc::kGemmF32Add : hc::kGemmF32;
        dx_started = true;
        LAUNCH_GEMM(g, true, false, 1);
        return ATTN_OK;
    };
    // rows [r0, r0 + K) of a weight gradient: out = A^T x with A head-major
    auto w_rows = [&](const uint16_t* a, int64_t rows, float* out) -> int {
        hc::GemmParams g{};
        g.a = a; g.a_rs = D; g.a_seg = D; g.a_segs = S * D;   // A(m, s) = a[m / D][s][m % D]
        g.b = x; g.b_rs = dm; g.b_seg = dm; g.b_segs = 0;      // B(n, s) = x[s][n]
        g.M = rows; g.N = dm; g.K = S;
        return wgrad(c, L, g, out, dm);
    };
    for (int ci = 0; ci < p.nchunks; ++ci) {
        const hc::Chunk ch = p.chunk(ci);
        // the chunk's projections, and its attention output and LSE unless the
        // forward kept them (the same kernels on the same inputs: same bits)
        int r = layer_chunk_forward(c, L, ch, x, wq, wk, wv, o_kept ? nullptr : Oc, lse_c, S);
        if (r) return r;
        const uint16_t* Ou = o_kept ? o_kept + (size_t)ch.h0 * S * D : Oc;
        const float* lse_u = o_kept ? lse_kept + (size_t)ch.h0 * S : lse_c;
        // dO_c = dy wo[:, chunk columns]  (bf16, head-major, where prep reads it)
        hc::GemmParams g{};
        g.a = dy; g.a_rs = dm; g.a_seg = dm; g.a_segs = 0;
        g.b = wo + (size_t)ch.h0 * D; g.b_rs = (int64_t)Hq * D; g.b_seg = (int64_t)Hq * D; g.b_segs = 0;
        g.M = S; g.N = (int64_t)ch.nh * D; g.K = dm;
        g.c = dOc; g.c_rs = D; g.c_seg = D; g.c_segs = S * D;
        g.out_mode = hc::kGemmBf16;
        LAUNCH_GEMM(g, true, false, 1);
        // dWo[:, chunk columns] = dy^T O_c
        g = hc::GemmParams{};
        g.a = dy; g.a_rs = dm; g.a_seg = dm; g.a_segs = 0;    // A(m, s) = dy[s][m]
        g.b = Ou; g.b_rs = D; g.b_seg = D; g.b_segs = S * D;  // B(n, s) = O_c[n / D][s][n % D]
        g.M = dm; g.N = (int64_t)ch.nh * D; g.K = S;
        if ((r = wgrad(c, L, g, dwo + (size_t)ch.h0 * D, (int64_t)Hq * D))) return r;
        // attention backward of the chunk (Delta from O_c, dO_c in place)
        hc::PrepParams pr{};
        pr.o = Ou; pr.o_rs = D; pr.o_hs = S * D;
        pr.dO = dOc; pr.do_rs = D; pr.do_hs = S * D;
        pr.lse = lse_u; pr.lse_hs = S;
        pr.dO_c = dOc; pr.c_rs = D; pr.c_hs = S * D;
        pr.ndelta = reinterpret_cast<float*>(c.ws + p.delta_c); pr.ndelta_hs = S;
        pr.nlse2 = reinterpret_cast<float*>(c.ws + p.lse2_c); pr.nlse2_hs = S;
        pr.nh = ch.nh; pr.rows = S; pr.D = D;
        LAUNCH_PASS(K_PREP, pr, hc::launch_prep(pr, c.st));
        BwdIO io{};
        io.dq = dQc;
        if ((r = dkdv_run(c, ch, ci, io, Kc, Vc, D, S * D, 0, S, dKc, dVc, D, S * D))) return r;
        hc::DqParams dq = dq_params(c, ch, io, Kc, Vc, D, S * D, 0, S);
        dq.dq = dQc; dq.dq_rs = D; dq.dq_hs = S * D;
        LAUNCH(K_DQ, hc::launch_dq(dq, D, c.st));
        // per GQA group, ascending: dx += dQ_g Wq_g, then dK Wk + dV Wv when the
        // group's last head is in this chunk (one product, parts in that
        // order); weight-gradient rows
        const int carry_out = p.carry_out_slot(ci) >= 0 ? 1 : 0;
        for (int kl = 0; kl < ch.nkv; ++kl) {
            const int kvg = ch.kv0 + kl;
            int hb = kvg * p.g, he = hb + p.g;
            hb = hb < ch.h0 ? ch.h0 : hb;
            he = he > ch.h0 + ch.nh ? ch.h0 + ch.nh : he;
            const bool done = !(carry_out && kl == ch.nkv - 1);
            const uint16_t* a[3] = {dQc + (size_t)(hb - ch.h0) * S * D, dKc + (size_t)kl * S * D,
                                    dVc + (size_t)kl * S * D};
            const uint16_t* w[3] = {wq + (size_t)hb * D * dm, wk + (size_t)kvg * D * dm,
                                    wv + (size_t)kvg * D * dm};
            const int64_t kk[3] = {(int64_t)(he - hb) * D, D, D};
            if ((r = dx_add(done ? 3 : 1, a, w, kk))) return r;
        }
        if ((r = w_rows(dQc, (int64_t)ch.nh * D, dwq + (size_t)ch.h0 * D * dm))) return r;
        const int nfin = ch.nkv - carry_out;
        if (nfin > 0) {
            if ((r = w_rows(dKc, (int64_t)nfin * D, dwk + (size_t)ch.kv0 * D * dm))) return r;
            if ((r = w_rows(dVc, (int64_t)nfin * D, dwv + (size_t)ch.kv0 * D * dm))) return r;
        }
    }
    return ATTN_OK;
}

int check_ptr(const void* p, const char* name, bool host_ok, bool* is_host) {
    if (p == nullptr) return fail(ATTN_EPOINTER, "%s is NULL", name);
    const Loc l = where(p);
    if (l == kLocDevice) {
        if (is_host) *is_host = false;
        return ATTN_OK;
    }
    if (l == kLocHost && host_ok) {
        if (is_host) *is_host = true;
        return ATTN_OK;
    }
    if (l == kLocHost)
        return fail(ATTN_EPOINTER, "%s is host memory; only k/v/dk/dv of the trunked path may be", name);
    return fail(ATTN_EPOINTER, "%s is neither device nor pinned host memory", name);
}

void init_common(Common& c, const hc::Plan& pl, void* ws) {
    c.pl = pl;
    c.ws = static_cast<char*>(ws);
    c.scale = (float)(1.0 / std::sqrt((double)pl.D));
    c.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)pl.D));
}

}  // namespace

extern "C" {

size_t attn_fwd_workspace_bytes(int64_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t causal,
                                int32_t head_chunk, int64_t kv_trunk) {
    hc::Plan pl;
    if (plan_or_fail(false, S, Hq, Hkv, D, causal, head_chunk, kv_trunk, &pl)) return 0;
    return pl.total;
}

size_t attn_bwd_workspace_bytes(int64_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t causal,
                                int32_t head_chunk, int64_t kv_trunk) {
    hc::Plan pl;
    if (plan_or_fail(true, S, Hq, Hkv, D, causal, head_chunk, kv_trunk, &pl)) return 0;
    return pl.total;
}

int attn_pick_kv_trunk(int64_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t causal,
                       int32_t head_chunk, int32_t kv_on_host, int32_t with_backward,
                       size_t budget_bytes, double link_bytes_per_s, double flops_per_s,
                       int32_t num_cus, int64_t* kv_trunk) {
    g_err[0] = 0;
    if (kv_trunk == nullptr) return fail(ATTN_EPOINTER, "kv_trunk is NULL");
    // defaults: the pinned-host-to-device copy rate and the forward kernel's
    // rate measured on one MI355X, and its compute-unit count
    const double link = link_bytes_per_s > 0.0 ? link_bytes_per_s : 57.0e9;
    const double flops = flops_per_s > 0.0 ? flops_per_s : 1.0e15;
    const int cus = num_cus > 0 ? num_cus : 256;
    char msg[256];
    int64_t t = 0;
    const int r = hc::pick_kv_trunk(S, Hq, Hkv, D, causal, head_chunk, kv_on_host != 0,
                                    with_backward != 0, budget_bytes, link, flops, cus, &t, msg,
                                    sizeof msg, g_group_loop_min_s.load());
    if (r == -1) return fail(ATTN_EINVAL, "%s", msg);
    if (r == -2) return fail(ATTN_EUNSUPPORTED, "%s", msg);
    if (r == -3) return fail(ATTN_EWORKSPACE, "%s", msg);
    *kv_trunk = t;
    return ATTN_OK;
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t S,
             int32_t Hq, int32_t Hkv, int32_t D, int32_t causal, int32_t head_chunk,
             int64_t kv_trunk, void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    hc::Plan pl;
    int r = plan_or_fail(false, S, Hq, Hkv, D, causal, head_chunk, kv_trunk, &pl);
    if (r) return r;
    if ((r = check_workspace(pl, workspace, workspace_bytes))) return r;
    bool kh = false, vh = false;
    if ((r = check_ptr(q, "q", false, nullptr)) || (r = check_ptr(k, "k", pl.trunked, &kh)) ||
        (r = check_ptr(v, "v", pl.trunked, &vh)) || (r = check_ptr(o, "o", false, nullptr)) ||
        (lse != nullptr && (r = check_ptr(lse, "lse", false, nullptr))) ||
        (r = check_ptr(workspace, "workspace", false, nullptr)))
        return r;
    Common c;
    init_common(c, pl, workspace);
    if ((r = device_resources(&c.dev))) return r;
    std::lock_guard<std::mutex> lk(c.dev->mu);
    if ((r = enter(c, static_cast<hipStream_t>(stream)))) return r;
    if (!pl.trunked)
        r = fwd_untrunked(c, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                          static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse);
    else
        r = fwd_trunked(c, static_cast<const uint16_t*>(q), k, v, static_cast<uint16_t*>(o), lse);
    const int r2 = leave(c);
    return r ? r : r2;
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int64_t S, int32_t Hq, int32_t Hkv,
             int32_t D, int32_t causal, int32_t head_chunk, int64_t kv_trunk, void* workspace,
             size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    hc::Plan pl;
    int r = plan_or_fail(true, S, Hq, Hkv, D, causal, head_chunk, kv_trunk, &pl);
    if (r) return r;
    if ((r = check_workspace(pl, workspace, workspace_bytes))) return r;
    bool kh = false, vh = false, dkh = false, dvh = false;
    if ((r = check_ptr(q, "q", false, nullptr)) || (r = check_ptr(k, "k", pl.trunked, &kh)) ||
        (r = check_ptr(v, "v", pl.trunked, &vh)) || (r = check_ptr(o, "o", false, nullptr)) ||
        (r = check_ptr(dout, "dout", false, nullptr)) ||
        (r = check_ptr(lse, "lse", false, nullptr)) || (r = check_ptr(dq, "dq", false, nullptr)) ||
        (r = check_ptr(dk, "dk", pl.trunked, &dkh)) || (r = check_ptr(dv, "dv", pl.trunked, &dvh)) ||
        (r = check_ptr(workspace, "workspace", false, nullptr)))
        return r;
    if (dkh != dvh)
        return fail(ATTN_EPOINTER, "dk and dv must both be device or both be pinned host memory");
    Common c;
    init_common(c, pl, workspace);
    if ((r = device_resources(&c.dev))) return r;
    std::lock_guard<std::mutex> lk(c.dev->mu);
    if ((r = enter(c, static_cast<hipStream_t>(stream)))) return r;
    BwdIO io{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(o),
             static_cast<const uint16_t*>(dout), k, v, lse, static_cast<uint16_t*>(dq), dk, dv, dkh};
    r = pl.trunked ? bwd_trunked(c, io) : bwd_untrunked(c, io);
    const int r2 = leave(c);
    return r ? r : r2;
}

int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int64_t S,
                     int32_t Hq, int32_t Hkv, int32_t D, int32_t causal, int32_t head_chunk,
                     int64_t kv_trunk, void* stream) {
    g_err[0] = 0;
    hc::Plan pl;
    int r = plan_or_fail(false, S, Hq, Hkv, D, causal, head_chunk, kv_trunk, &pl);
    if (r) return r;
    if (pl.total > hc::kScratchBytes)
        return fail(ATTN_EWORKSPACE,
                    "these arguments need %zu bytes of workspace; the built-in one holds %zu "
                    "(use a smaller head_chunk or kv_trunk, or attn_fwd with a workspace)",
                    pl.total, hc::kScratchBytes);
    void* ws = nullptr;
    HIPCHK(hc::scratch_address(&ws));
    return attn_fwd(q, k, v, o, lse, S, Hq, Hkv, D, causal, head_chunk, kv_trunk, ws,
                    hc::kScratchBytes, stream);
}

const char* attn_last_error(void) { return g_err; }

int attn_set_single_stream(int on) { return g_single_stream.exchange(on ? 1 : 0); }

int attn_set_trunk_merge(int on) { return g_trunk_merge.exchange(on ? 1 : 0); }

int64_t attn_set_group_loop_min_s(int64_t min_s) {
    return g_group_loop_min_s.exchange(min_s > 0 ? min_s : hc::kGroupLoopMinS);
}

size_t attn_layer_fwd_workspace_bytes(int64_t S, int32_t d_model, int32_t Hq, int32_t Hkv,
                                      int32_t D, int32_t causal, int32_t head_chunk) {
    LayerPlan L;
    if (layer_plan(false, S, d_model, Hq, Hkv, D, causal, head_chunk, &L)) return 0;
    return L.total;
}

size_t attn_layer_bwd_workspace_bytes(int64_t S, int32_t d_model, int32_t Hq, int32_t Hkv,
                                      int32_t D, int32_t causal, int32_t head_chunk) {
    LayerPlan L;
    if (layer_plan(true, S, d_model, Hq, Hkv, D, causal, head_chunk, &L)) return 0;
    return L.total;
}

int attn_layer_fwd(const void* x, const void* wq, const void* wk, const void* wv, const void* wo,
                   float* y, float* lse, void* o_keep, int64_t S, int32_t d_model, int32_t Hq,
                   int32_t Hkv, int32_t D, int32_t causal, int32_t head_chunk, void* workspace,
                   size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    LayerPlan L;
    int r = layer_plan(false, S, d_model, Hq, Hkv, D, causal, head_chunk, &L);
    if (r) return r;
    if (workspace == nullptr) return fail(ATTN_EWORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) % hc::kAlign != 0)
        return fail(ATTN_EWORKSPACE, "workspace must be %zu-byte aligned", hc::kAlign);
    if (workspace_bytes < L.total)
        return fail(ATTN_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
    const void* ins[] = {x, wq, wk, wv, wo, y, workspace};
    const char* names[] = {"x", "wq", "wk", "wv", "wo", "y", "workspace"};
    for (int i = 0; i < 7; ++i)
        if ((r = check_ptr(ins[i], names[i], false, nullptr))) return r;
    if (lse != nullptr && (r = check_ptr(lse, "lse", false, nullptr))) return r;
    if (o_keep != nullptr && (r = check_ptr(o_keep, "o_keep", false, nullptr))) return r;
    Common c;
    init_common(c, L.at, workspace);
    if ((r = device_resources(&c.dev))) return r;
    std::lock_guard<std::mutex> lk(c.dev->mu);
    if ((r = enter(c, static_cast<hipStream_t>(stream)))) return r;
    r = layer_fwd_run(c, L, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wq),
                      static_cast<const uint16_t*>(wk), static_cast<const uint16_t*>(wv),
                      static_cast<const uint16_t*>(wo), y, lse, static_cast<uint16_t*>(o_keep));
    const int r2 = leave(c);
    return r ? r : r2;
}

int attn_layer_bwd(const void* x, const void* wq, const void* wk, const void* wv, const void* wo,
                   const void* dy, const void* o_kept, const float* lse_kept, float* dx, float* dwq,
                   float* dwk, float* dwv, float* dwo, int64_t S, int32_t d_model, int32_t Hq,
                   int32_t Hkv, int32_t D, int32_t causal, int32_t head_chunk, void* workspace,
                   size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    LayerPlan L;
    int r = layer_plan(true, S, d_model, Hq, Hkv, D, causal, head_chunk, &L);
    if (r) return r;
    if (workspace == nullptr) return fail(ATTN_EWORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) % hc::kAlign != 0)
        return fail(ATTN_EWORKSPACE, "workspace must be %zu-byte aligned", hc::kAlign);
    if (workspace_bytes < L.total)
        return fail(ATTN_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
    const void* ins[] = {x, wq, wk, wv, wo, dy, dx, dwq, dwk, dwv, dwo, workspace};
    const char* names[] = {"x", "wq", "wk", "wv", "wo", "dy", "dx", "dwq", "dwk", "dwv", "dwo",
                           "workspace"};
    for (int i = 0; i < 12; ++i)
        if ((r = check_ptr(ins[i], names[i], false, nullptr))) return r;
    if ((o_kept == nullptr) != (lse_kept == nullptr))
        return fail(ATTN_EINVAL, "o_kept and lse_kept come together (both NULL: recompute)");
    if (o_kept != nullptr) {
        if ((r = check_ptr(o_kept, "o_kept", false, nullptr))) return r;
        if ((r = check_ptr(lse_kept, "lse_kept", false, nullptr))) return r;
    }
    Common c;
    init_common(c, L.at, workspace);
    if ((r = device_resources(&c.dev))) return r;
    std::lock_guard<std::mutex> lk(c.dev->mu);
    if ((r = enter(c, static_cast<hipStream_t>(stream)))) return r;
    r = layer_bwd_run(c, L, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wq),
                      static_cast<const uint16_t*>(wk), static_cast<const uint16_t*>(wv),
                      static_cast<const uint16_t*>(wo), static_cast<const uint16_t*>(dy),
                      static_cast<const uint16_t*>(o_kept), lse_kept, dx, dwq, dwk, dwv, dwo);
    const int r2 = leave(c);
    return r ? r : r2;
}

const char* attn_version(void) { return "0.3.0"; }

int attn_timing_enable(int on) { return g_timing.exchange(on ? 1 : 0); }

void attn_timing_reset(void) {
    std::lock_guard<std::mutex> lk(g_tmu);
    for (const TimingRec& r : g_recs) {
        (void)hipEventSynchronize(r.b);
        g_pool.push_back(r.a);
        g_pool.push_back(r.b);
    }
    g_recs.clear();
}

int attn_timing_read(const char* name, int64_t* launches, double* total_ms) {
    int kid = -1;
    for (int i = 0; i < K_COUNT; ++i)
        if (name && std::strcmp(name, kKernelNames[i]) == 0) kid = i;
    if (kid < 0) return fail(ATTN_EINVAL, "unknown kernel family '%s'", name ? name : "(null)");
    std::lock_guard<std::mutex> lk(g_tmu);
    int64_t n = 0;
    double ms = 0.0;
    for (const TimingRec& r : g_recs) {
        if (r.kid != kid) continue;
        HIPCHK(hipEventSynchronize(r.b));
        float t = 0.f;
        HIPCHK(hipEventElapsedTime(&t, r.a, r.b));
        ms += t;
        ++n;
    }
    if (launches) *launches = n;
    if (total_ms) *total_ms = ms;
    return ATTN_OK;
}

int attn_timing_bytes(const char* name, double* bytes) {
    int kid = -1;
    for (int i = 0; i < K_COUNT; ++i)
        if (name && std::strcmp(name, kKernelNames[i]) == 0) kid = i;
    if (kid < 0) return fail(ATTN_EINVAL, "unknown kernel family '%s'", name ? name : "(null)");
    if (bytes == nullptr) return fail(ATTN_EPOINTER, "bytes is NULL");
    std::lock_guard<std::mutex> lk(g_tmu);
    double b = 0.0;
    for (const TimingRec& r : g_recs)
        if (r.kid == kid) b += r.bytes;
    *bytes = b;
    return ATTN_OK;
}

}  // extern "C"
