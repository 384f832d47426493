// plan.h - host-side planning: argument checks, head chunks, key/value
// trunks and the workspace carve.  Pure integer arithmetic, no HIP calls.
//
// Head chunks: query heads [c*hc, min((c+1)*hc, Hq)), ascending, walked one
// after another through one workspace that every chunk reuses (Road to 5
// Million Tokens talk, U-Pipe paragraph: compute a group of heads, store the
// partial result, move on reusing the buffers).  The chunk's key/value heads
// are kv = h / g for its query heads.
// Trunks: sequence slices of T tokens, N = ceil(S / T) (FPDT summary, "Key
// Findings" item 1 and "Technical Deep Dive", the S/N trunk paragraph).
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <stdio.h>

namespace hc {

constexpr int64_t kTrunkGranule = 256;  // trunk length must be a multiple
constexpr size_t kAlign = 256;
// Sequences at least this long take the group-loop dK/dV schedule: one
// workgroup per (128-key tile, kv head) walks the chunk's heads of that
// group itself, keeping dK/dV in registers and writing bf16 dK/dV directly
// (no per-head fp32 partials, no reduce pass).  Shorter sequences have too
// few key tiles to spread that longer work over the compute units and keep
// one workgroup per (key tile, query head) with per-head partials.  The
// choice depends on S only, so every head_chunk and kv_trunk at one S runs
// the same arithmetic.
constexpr int64_t kGroupLoopMinS = 65536;

struct Chunk {
    int h0, nh;    // query heads [h0, h0 + nh)
    int kv0, nkv;  // key/value heads [kv0, kv0 + nkv)
};

struct Plan {
    bool bwd;
    int64_t S;
    int Hq, Hkv, D, causal, hc, g;
    int64_t T, N;  // trunk length (S when untrunked), number of trunks
    bool trunked;
    int nchunks, kvc;   // chunks, max kv heads in a chunk
    int carry_slots;    // fp32 dK/dV carries (bwd, group spanning chunks)
    bool group_loop;    // bwd: group-loop dK/dV schedule (S >= group_loop_min_s)

    // workspace regions, byte offsets
    size_t q_c = 0, k_c = 0, v_c = 0;                   // packed chunk buffers
    size_t o_run = 0, o_t = 0, l_run = 0, l_t = 0;      // fwd trunk partials / carried state
    size_t st_l = 0;                                    // fwd carried lane-pair row sums
    size_t ring_k[2] = {0, 0}, ring_v[2] = {0, 0};      // trunk ring slots
    size_t do_c = 0, delta_c = 0, lse2_c = 0, dq_acc = 0; // bwd chunk buffers
    size_t part_k = 0, part_v = 0;                      // bwd per-head fp32 dK/dV (not group_loop)
    size_t carry_k[2] = {0, 0}, carry_v[2] = {0, 0};    // bwd fp32 carries ([S][D])
    size_t stage_k[2] = {0, 0}, stage_v[2] = {0, 0};    // bwd dK/dV staging
    size_t total = 0;

    Chunk chunk(int c) const {
        Chunk ch;
        ch.h0 = c * hc;
        ch.nh = (ch.h0 + hc <= Hq) ? hc : Hq - ch.h0;
        ch.kv0 = ch.h0 / g;
        ch.nkv = (ch.h0 + ch.nh - 1) / g - ch.kv0 + 1;
        return ch;
    }
    int64_t trunk_begin(int64_t t) const { return t * T; }
    int64_t trunk_rows(int64_t t) const { return (t + 1) * T <= S ? T : S - t * T; }
    // carry slot a chunk reads its first kv head's fp32 dK/dV from, or -1
    int carry_in_slot(int c) const {
        if (carry_slots == 0) return -1;
        const Chunk ch = chunk(c);
        if (ch.h0 % g == 0) return -1;  // first kv head starts in this chunk
        return carry_slots == 1 ? 0 : (c - 1) & 1;
    }
    // carry slot a chunk writes its last kv head's fp32 dK/dV to, or -1
    int carry_out_slot(int c) const {
        if (carry_slots == 0) return -1;
        const Chunk ch = chunk(c);
        if ((ch.h0 + ch.nh) % g == 0) return -1;  // last kv head ends here
        return carry_slots == 1 ? 0 : c & 1;
    }
};

static inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Returns 0 and fills *pl, or -1 (invalid) / -2 (unsupported) with a message.
static inline int make_plan(bool bwd, int64_t S, int Hq, int Hkv, int D, int causal,
                            int head_chunk, int64_t kv_trunk, Plan* pl, char* err, size_t errlen,
                            int64_t group_loop_min_s = kGroupLoopMinS) {
    if (S < 1) { snprintf(err, errlen, "S must be >= 1 (got %lld)", (long long)S); return -1; }
    if (Hq < 1 || Hkv < 1) { snprintf(err, errlen, "Hq and Hkv must be >= 1"); return -1; }
    if (Hq % Hkv != 0) {
        snprintf(err, errlen, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
        return -1;
    }
    if (causal != 0 && causal != 1) { snprintf(err, errlen, "causal must be 0 or 1"); return -1; }
    if (head_chunk < 0 || head_chunk > Hq) {
        snprintf(err, errlen, "head_chunk must be in [0, Hq=%d] (got %d)", Hq, head_chunk);
        return -1;
    }
    if (kv_trunk < 0) { snprintf(err, errlen, "kv_trunk must be >= 0"); return -1; }
    if (D != 64 && D != 128) {
        snprintf(err, errlen, "head dimension %d not supported (64 or 128)", D);
        return -2;
    }
    // row and key offsets inside the kernels are 32-bit (with up to a tile of
    // headroom), so sequences are limited to 2^30 tokens
    if (S > (int64_t(1) << 30)) {
        snprintf(err, errlen, "S = %lld exceeds 2^30 tokens", (long long)S);
        return -2;
    }
    // every workspace region is at most a few dozen bytes per (head, token,
    // channel); refuse shapes whose byte counts could wrap a 64-bit size
    if ((double)S * ((double)Hq + (double)Hkv) * (double)D * 64.0 > 0x1p62) {
        snprintf(err, errlen, "S = %lld with %d + %d heads is too large to address",
                 (long long)S, Hq, Hkv);
        return -2;
    }
    Plan p;
    p.bwd = bwd;
    p.S = S; p.Hq = Hq; p.Hkv = Hkv; p.D = D; p.causal = causal;
    p.hc = head_chunk == 0 ? Hq : head_chunk;
    p.g = Hq / Hkv;
    p.trunked = kv_trunk > 0 && kv_trunk < S;
    if (p.trunked && kv_trunk % kTrunkGranule != 0) {
        snprintf(err, errlen, "kv_trunk (%lld) must be a multiple of %lld", (long long)kv_trunk,
                 (long long)kTrunkGranule);
        return -1;
    }
    p.T = p.trunked ? kv_trunk : S;
    p.N = (S + p.T - 1) / p.T;
    p.nchunks = (Hq + p.hc - 1) / p.hc;
    p.kvc = 0;
    for (int c = 0; c < p.nchunks; ++c) {
        const Chunk ch = p.chunk(c);
        if (ch.nkv > p.kvc) p.kvc = ch.nkv;
    }
    p.carry_slots = 0;
    if (bwd && p.hc % p.g != 0) p.carry_slots = (p.g % p.hc == 0) ? 1 : 2;
    p.group_loop = bwd && S >= group_loop_min_s;

    const size_t E = (size_t)S * D * 2;         // one bf16 head slice
    const size_t Et = (size_t)p.T * D * 2;      // one bf16 trunk slice
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
    if (!bwd) {
        if (!p.trunked) {
            p.q_c = take(p.hc * E);
            p.k_c = take(p.kvc * E);
            p.v_c = take(p.kvc * E);
        } else {
            p.q_c = take(p.hc * Et);                          // query trunk
            p.o_run = take(p.hc * Et * 2);                    // fp32 running O
            p.o_t = take(p.hc * Et * 2);                      // fp32 trunk partial
            p.l_run = take((size_t)p.hc * p.T * 4);
            p.l_t = take((size_t)p.hc * p.T * 4);
            p.st_l = take((size_t)p.hc * p.T * 8);            // carried row sums, 2 per row
            for (int s = 0; s < 2; ++s) {
                p.ring_k[s] = take(p.kvc * Et);
                p.ring_v[s] = take(p.kvc * Et);
            }
        }
    } else {
        p.q_c = take(p.hc * E);
        p.do_c = take(p.hc * E);
        p.delta_c = take((size_t)p.hc * S * 4);           // -Delta, fp32 [hc][S]
        p.lse2_c = take((size_t)p.hc * S * 4);            // -LSE * log2(e), fp32 [hc][S]
        if (!p.group_loop) {
            const size_t rows = p.trunked ? Et : E;       // keys per dK/dV launch, bf16 bytes
            p.part_k = take(p.hc * rows * 2);             // fp32 [hc][rows][D]
            p.part_v = take(p.hc * rows * 2);
        }
        if (!p.trunked) {
            p.k_c = take(p.kvc * E);
            p.v_c = take(p.kvc * E);
        } else {
            p.dq_acc = take(p.hc * E * 2);                    // fp32 dQ carried over trunks
            for (int s = 0; s < 2; ++s) {
                p.ring_k[s] = take(p.kvc * Et);
                p.ring_v[s] = take(p.kvc * Et);
                p.stage_k[s] = take(p.kvc * Et);
                p.stage_v[s] = take(p.kvc * Et);
            }
        }
        for (int s = 0; s < p.carry_slots; ++s) {
            p.carry_k[s] = take(E * 2);                       // fp32 [S][D]
            p.carry_v[s] = take(E * 2);
        }
    }
    p.total = off;
    *pl = p;
    return 0;
}

// Key/value trunk length for a memory budget (FPDT summary, "Technical Deep
// Dive": the trunk is sized so that fetching the next trunk takes about as
// long as computing on the current one; past that point a longer trunk only
// costs device memory).  Candidates are T = 256 * 2^k < S.  T qualifies when
//   fits:     the workspace of attn_fwd (and of attn_bwd, if with_bwd) at T is
//             within the budget (budget 0 = no limit);
//   balanced: with K/V in host memory, copying one trunk of the chunk's K and
//             V heads (4 T kvc D bytes) takes no longer than one full
//             query-trunk x key-trunk block of the forward (4 T^2 D hc FLOP):
//             T >= kvc * flops / (hc * link);
//   fills:    one forward launch has at least four rounds of workgroups
//             (128 query rows at two per compute unit, or 256 at one), so
//             a last partial round costs little: ceil(T / 128) * hc >=
//             8 * num_cus.
// The smallest qualifying T wins.  Device-resident K/V whose untrunked
// workspaces fit take T = 0 (no trunks).  When no T qualifies, the longest
// one that fits is taken.  Returns 0, -1 (bad arguments or host K/V with
// S <= 256, which cannot be trunked) or -3 (nothing fits the budget).
static inline int pick_kv_trunk(int64_t S, int Hq, int Hkv, int D, int causal, int head_chunk,
                                bool kv_on_host, bool with_bwd, size_t budget, double link,
                                double flops, int num_cus, int64_t* out, char* err, size_t errlen,
                                int64_t group_loop_min_s = kGroupLoopMinS) {
    Plan p;
    int r = make_plan(false, S, Hq, Hkv, D, causal, head_chunk, 0, &p, err, errlen);
    if (r) return r;
    if (!(link > 0.0) || !(flops > 0.0) || num_cus < 1) {
        snprintf(err, errlen, "link rate, FLOP rate and compute-unit count must be positive");
        return -1;
    }
    auto need = [&](int64_t T, size_t* bytes) -> int {
        Plan f, b;
        int rr = make_plan(false, S, Hq, Hkv, D, causal, head_chunk, T, &f, err, errlen);
        if (rr) return rr;
        size_t n = f.total;
        if (with_bwd) {
            rr = make_plan(true, S, Hq, Hkv, D, causal, head_chunk, T, &b, err, errlen,
                           group_loop_min_s);
            if (rr) return rr;
            if (b.total > n) n = b.total;
        }
        *bytes = n;
        return 0;
    };
    auto fits = [&](size_t bytes) { return budget == 0 || bytes <= budget; };
    size_t bytes = 0;
    if (!kv_on_host) {
        if ((r = need(0, &bytes))) return r;
        if (fits(bytes)) { *out = 0; return 0; }
    }
    int64_t best_fit = -1, pick = -1;
    for (int64_t T = kTrunkGranule; T < S; T *= 2) {
        if ((r = need(T, &bytes))) return r;
        if (!fits(bytes)) break;  // the workspaces grow with T
        best_fit = T;
        const bool balanced =
            !kv_on_host || (double)T >= (double)p.kvc * flops / ((double)p.hc * link);
        const bool fills = (T + 127) / 128 * p.hc >= 8 * (int64_t)num_cus;
        if (balanced && fills) { pick = T; break; }
    }
    if (pick < 0) pick = best_fit;
    if (pick < 0) {
        if (kv_on_host && S <= kTrunkGranule) {
            snprintf(err, errlen, "S = %lld is too short to trunk (host K/V need S > %lld)",
                     (long long)S, (long long)kTrunkGranule);
            return -1;
        }
        snprintf(err, errlen, "no key/value trunk fits a workspace budget of %zu bytes", budget);
        return -3;
    }
    *out = pick;
    return 0;
}

}  // namespace hc
