// fwd.hip - forward flash attention kernel for gfx950 (bf16 MFMA, fp32 softmax).
//
// Exact softmax attention computed one key tile at a time with running
// statistics (row maximum and row sum), the blockwise scheme the FPDT talk
// summary likens trunk processing to ("Technical Deep Dive", the paragraph on
// online softmax and FlashAttention).  Causal visibility: a query sees keys at
// or before its own position (same section, auto-regressive paragraph).
//
// Workgroup = NW waves x 32 query rows of one head; the key loop walks 64-key
// tiles of K and V loaded straight from global memory into LDS (global_load_
// lds) through a ring of slots.  Large launches take NW = 8 (256 rows, one
// workgroup per compute unit, waves 0-3 load K and waves 4-7 load V): each
// tile then serves twice the rows, and a 4-slot K ring (5 for V) lets the
// workgroup work on two tiles per barrier while the next two load (measured
// 8% and then another 5% faster than NW = 4 with one barrier per tile, at
// S = 32768).  Wave w + 4 runs one phase behind wave w, which shares its
// SIMD, so that one's softmax overlaps the other's products.
// Smaller launches take NW = 4 (128 rows, two workgroups per compute unit,
// double-buffered, one barrier per tile) so more compute units get work.  Per wave and tile, in the transposed form that keeps one query row
// per lane pair:
//   S^T[key][q] = K Q^T          A = K tile (LDS, 16-byte reads), B = Q (regs)
//   online softmax on S^T        lane l and l^32 share query l % 32
//   O^T[d][q]  += V^T P^T        A = V tile (LDS transposed reads), B = P (regs)
// so the row statistics never leave the lane pair and O rescaling is per lane.
// Tiles past a wave's last visible key are skipped; only tiles that cross the
// causal diagonal or the end of the keys are masked.  Workgroups are issued
// heaviest first (last query tile first) to even out the causal triangle.
#include "device_common.h"
#include "kernels.h"

namespace hc {

// Online-softmax update of one 64-key tile for this lane's query row.  The
// raw scores s (S^T blocks, lane = query) stay unscaled: the row maximum is
// taken on them and the scale (softmax scale * log2 e) is folded into the
// exponent, p = 2^(s * c - m) with m a running reference in log2 units.  MASK
// adds the causal / ragged test with keys relative to the tile.
template <bool MASK>
__device__ __forceinline__ void fwd_softmax(f32x16 (&s)[2], float c, int hi, int qrel, int klim,
                                            float& m, float& lpart, float& alpha,
                                            bf16x8 (&pb)[2][2]) {
    if constexpr (MASK) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                // key (relative to the tile) visible iff key <= query and key < klim
                const int key = b * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
                s[b][r] = (key <= qrel && key < klim) ? s[b][r] : -INFINITY;
            }
        }
    }
    float rmax = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int r = 0; r < 16; ++r) rmax = fmaxf(rmax, s[b][r]);
    }
    rmax = pair_max(rmax) * c;
    // lazy reference: m moves (to the tile's maximum) only when that maximum
    // exceeds it by more than 8 in log2 units, so every p = 2^(s c - m) stays
    // <= 2^8, well inside fp32 and bf16 range, and O is rescaled only on such
    // jumps; the softmax itself does not depend on the choice of m
    const float mnew = (rmax > m + 8.0f) ? rmax : m;
    const float msafe = mnew == -INFINITY ? 0.f : mnew;
    alpha = fast_exp2(m - msafe);
    m = mnew;
    float psum = 0.f;

#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float p0 = fast_exp2(__builtin_fmaf(s[b][h2 * 8 + e], c, -msafe));
                const float p1 = fast_exp2(__builtin_fmaf(s[b][h2 * 8 + e + 1], c, -msafe));
                psum += p0;
                psum += p1;
                const bf16x2 pk = to_bf16x2(p0, p1);
                pb[b][h2][e] = pk[0];
                pb[b][h2][e + 1] = pk[1];
            }
        }
    }
    lpart = lpart * alpha + psum;
}

template <int HD, int NW>
__global__ __launch_bounds__(NW * 64, 8 / NW) void fwd_kernel(FwdParams p) {
    constexpr int BN = 64, WQ = 32, BM = NW * WQ;
    constexpr int NS = HD / 16;  // reduction steps of K Q^T
    constexpr int NDB = HD / 32; // 32-wide d blocks of O
    constexpr int TILE = BN * HD * 2;
    // K/V ring slots: 8 waves work on two tiles per barrier while the next
    // two load; 4 waves double-buffer single tiles
    constexpr int NBUF = NW == 8 ? 4 : 2;
    // one V slot more with 8 waves, for the deferred P V products below
    constexpr int NVB = NW == 8 ? NBUF + 1 : NBUF;
    __shared__ __attribute__((aligned(1024))) char ksm[NBUF][TILE];
    __shared__ __attribute__((aligned(1024))) char vsm[NVB][TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps per-wave values scalar
    const int hi = lane >> 5, l32 = lane & 31;

    const int64_t nqt = (p.nq + BM - 1) / BM;
    const int head = blockIdx.x % p.nh;
    const int64_t qt = nqt - 1 - (int64_t)(blockIdx.x / p.nh);
    const int64_t q0 = qt * BM;
    const int kvl = (p.h0 + head) / p.group - p.kv_base;

    const uint16_t* qh = p.q + (int64_t)head * p.q_hs;
    const uint16_t* kh = p.k + (int64_t)kvl * p.k_hs;
    const uint16_t* vh = p.v + (int64_t)kvl * p.v_hs;

    const int64_t wq0 = q0 + wave * WQ;       // first row of this wave
    const int64_t myq = wq0 + l32;            // this lane's query row
    const bool wave_live = wq0 < p.nq;

    // query fragments (B operand of K Q^T): lane holds Q[myq][s*16 + hi*8 .. +8]
    bf16x8 qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        if (myq < p.nq)
            qf[s] = *reinterpret_cast<const bf16x8*>(qh + myq * p.q_rs + s * 16 + hi * 8);
        else
            qf[s] = bf16x8{};
    }

    // key ranges: keys [0, kend) for the workgroup, [0, kend_w) for this wave
    const int64_t wg_last = (q0 + BM - 1 < p.nq - 1) ? q0 + BM - 1 : p.nq - 1;
    const int64_t w_last = (wq0 + WQ - 1 < p.nq - 1) ? wq0 + WQ - 1 : p.nq - 1;
    int64_t kend = p.nk, kend_w = wave_live ? p.nk : 0;
    if (p.causal) {
        const int64_t a = p.q_pos0 + wg_last - p.k_pos0 + 1;
        const int64_t b = p.q_pos0 + w_last - p.k_pos0 + 1;
        kend = a < kend ? a : kend;
        kend_w = b < kend_w ? b : kend_w;
    }
    const int ntiles = kend > 0 ? (int)((kend + BN - 1) / BN) : 0;
    const int ntiles_w = kend_w > 0 ? (int)((kend_w + BN - 1) / BN) : 0;

    float m = -INFINITY, lpart = 0.f;
    f32x16 o[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) o[i] = f32x16{};
    // continue the state a previous key range left for this row
    if (p.carry_in && myq < p.nq) {
        const int64_t sr = (int64_t)head * p.st_hs + myq;
        m = p.st_m[sr];
        lpart = p.st_l[2 * sr + hi];
        const float* so = p.st_o + (int64_t)head * p.st_o_hs + myq * HD;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(so + db * 32 + g4 * 8 + hi * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) o[db][g4 * 4 + e] = x[e];
            }
        }
        settle(m);
        settle(lpart);
#pragma unroll
        for (int db = 0; db < NDB; ++db) settle(o[db]);
    }

    const int kv_sel = wave >> 2;
    const uint16_t* kvh = kv_sel == 0 ? kh : vh;
    const int64_t kv_rs = kv_sel == 0 ? p.k_rs : p.v_rs;
    // per-lane parts of the tile-load addresses (8 waves: K or V; 4 waves: both)
    const TileDma64<HD, true> dkv(NW == 8 ? kv_rs : p.k_rs, wave & 3, lane);
    const TileDma64<HD, true> dv2(p.v_rs, wave & 3, lane);
    auto issue = [&](int t) {
        const int64_t nb = (int64_t)t * BN;
        if constexpr (NW == 8) {
            dkv.load(kv_sel == 0 ? ksm[t % NBUF] : vsm[t % NVB], kvh + nb * kv_rs, kv_rs, p.nk - nb, wave & 3, lane);
        } else {
            dkv.load(ksm[t % NBUF], kh + nb * p.k_rs, p.k_rs, p.nk - nb, wave, lane);
            dv2.load(vsm[t % NVB], vh + nb * p.v_rs, p.v_rs, p.nk - nb, wave, lane);
        }
    };
    // registers loaded above settle first; then tiles 0 .. NBUF-2 go in flight
    wait_vm_loads();
#pragma unroll
    for (int s = 0; s < NS; ++s) settle(qf[s]);
    // 8 waves: tiles go in pairs (one barrier per pair), 0 and 1 first;
    // 4 waves: tile 0 first, one barrier per tile
    const int pre = ntiles < NBUF / 2 ? ntiles : NBUF / 2;
    for (int t = 0; t < pre; ++t) issue(t);
    wait_vm_loads();
    __syncthreads();

    // per-lane offsets of the K (row-major) and V (transposed) operand reads
    const OperandOffsets<HD> off(lane);
    // this lane's query position relative to the key positions of tile 0
    const int64_t qrel_base = p.q_pos0 + myq - p.k_pos0;
    // front part of tile j: S^T, the online-softmax update and the O
    // rescale, leaving the tile's P^T operands in pb; false when the wave
    // sees no key of the tile
    auto front = [&](int j, bf16x8 (&pb)[2][2]) __attribute__((always_inline)) -> bool {
        if (j >= ntiles_w) return false;
        {
            const char* Ks = ksm[j % NBUF];
            // S^T = K Q^T for two 32-key blocks (first step starts from zero):
            // MFMA j covers block j % 2 over d 16 (j / 2) .., its K operand
            // read 3 MFMAs ahead.  Both product phases run at a raised wave
            // priority: the SIMD's other wave, on its softmax, yields the
            // issue slots to them, so the two waves drift apart in phase and
            // one's vector work runs under the other's products.
            f32x16 s[2];
            __builtin_amdgcn_s_setprio(1);
            {
                constexpr int NJ = 2 * NS, DIST = 3;
                auto rdk = [&](int j) __attribute__((always_inline)) {
                    return lds_read_b128(Ks, off.row[j >> 1] + (j & 1) * 32 * HD * 2);
                };
                bf16x8 ring[DIST];
#pragma unroll
                for (int j = 0; j < DIST; ++j) ring[j] = rdk(j);
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const bf16x8 a = ring[j % DIST];
                    if (j + DIST < NJ) ring[j % DIST] = rdk(j + DIST);
                    const int b = j & 1, st = j >> 1;
                    s[b] = mfma32(a, qf[st], st == 0 ? f32x16{} : s[b]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            const int64_t kb = (int64_t)j * BN;
            const bool need_mask = (kb + BN > p.nk) ||
                                   (p.causal && p.k_pos0 + kb + BN - 1 > p.q_pos0 + wq0);
            float alpha;
            __builtin_amdgcn_s_setprio(0);
            if (need_mask) {
                const int64_t qr = p.causal ? qrel_base - kb : (int64_t)BN;
                fwd_softmax<true>(s, p.scale_log2, hi, (int)qr, (int)(p.nk - kb), m, lpart,
                                  alpha, pb);
            } else {
                fwd_softmax<false>(s, p.scale_log2, hi, 0, 0, m, lpart, alpha, pb);
            }
            // rescale O only when some row of the wave saw a new maximum
            // (alpha is exactly 1 otherwise, so skipping changes no bits)
            if (__any(alpha != 1.f)) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) o[db] *= alpha;
            }
        }
        return true;
    };
    // O^T += V^T P^T for the tile in V slot vs
    auto pv = [&](int vs, const bf16x8 (&pb)[2][2]) __attribute__((always_inline)) {
        {
            const char* Vs = vsm[vs];
            // O^T += V^T P^T: reduction over the tile's 64 keys in 4 steps of 16;
            // MFMA j covers d block j / 4, keys 16 (j % 4) .., its transposed V
            // operand read 3 MFMAs ahead
            __builtin_amdgcn_s_setprio(1);
            {
                constexpr int NJ = 4 * NDB, DIST = 3;
                auto rdv = [&](int j) __attribute__((always_inline)) {
                    return lds_read_tr_at<HD>(Vs, off, ((j >> 1) & 1) * 32 + (j & 1) * 16, j >> 2);
                };
                bf16x8 ring[DIST];
#pragma unroll
                for (int j = 0; j < DIST; ++j) ring[j] = rdv(j);
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const bf16x8 a = ring[j % DIST];
                    if (j + DIST < NJ) ring[j % DIST] = rdv(j + DIST);
                    o[j >> 2] = mfma32(a, pb[(j >> 1) & 1][j & 1], o[j >> 2]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __builtin_amdgcn_s_setprio(0);
        }
    };
    auto tile = [&](int j, int vs) __attribute__((always_inline)) {
        bf16x8 pb[2][2];
        if (front(j, pb)) pv(vs, pb);
    };
    if constexpr (NW == 8) {
        // wave w + 4 shares a SIMD with wave w and runs one phase behind it:
        // its P V product of each pair's second tile moves past the barrier,
        // to the start of the next pair, so that while one wave of the SIMD
        // is on its softmax the other is on its products (4% faster than
        // the same code without the shift).  Every wave reads all of a V
        // tile but loads only a quarter of one, so the ring has a fifth V
        // slot: the tile of a deferred product is not reloaded before every
        // wave has used it.  Each wave adds into O in the same order as
        // without the shift.
        const bool lag = kv_sel != 0;
        bf16x8 pbd[2][2];
        int pend = -1;   // tile whose P V product is deferred
        int vs0 = 0;     // V slot of tile j (j mod NVB)
        for (int j = 0; j < ntiles; j += 2) {
            const int vs1 = vs0 + 1 == NVB ? 0 : vs0 + 1;
            if (pend >= 0) pv(pend, pbd);
            pend = -1;
            // slots of tiles j - 2 and j - 1 (K) and j - 3 and j - 2 (V) are free
            if (j + 2 < ntiles) issue(j + 2);
            if (j + 3 < ntiles) issue(j + 3);
            tile(j, vs0);
            if (j + 1 < ntiles && front(j + 1, pbd)) {
                if (lag) pend = vs1;
                else pv(vs1, pbd);
            }
            vs0 = vs1 + 1 == NVB ? 0 : vs1 + 1;
            wait_vm_loads();  // tiles j + 2 and j + 3
            __syncthreads();
        }
        if (pend >= 0) pv(pend, pbd);
    } else {
        for (int j = 0; j < ntiles; ++j) {
            if (j + 1 < ntiles) issue(j + 1);
            tile(j, j % NBUF);
            wait_vm_loads();
            __syncthreads();
        }
    }

    if (!wave_live || myq >= p.nq) return;
    if (p.carry_out) {
        // hand the unnormalised state to the next key range, bit for bit
        const int64_t sr = (int64_t)head * p.st_hs + myq;
        if (hi == 0) p.st_m[sr] = m;
        p.st_l[2 * sr + hi] = lpart;
        float* so = p.st_o + (int64_t)head * p.st_o_hs + myq * HD;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = o[db][g4 * 4 + e];
                *reinterpret_cast<f32x4*>(so + db * 32 + g4 * 8 + hi * 4) = x;
            }
        }
        return;
    }
    const float ltot = pair_sum(lpart);
    if (p.mode == kFwdFinal) {
        const float inv = 1.0f / ltot;
        uint16_t* orow = reinterpret_cast<uint16_t*>(p.o) + (int64_t)head * p.o_hs + myq * p.o_rs;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                bf16x2 lo = to_bf16x2(o[db][g4 * 4 + 0] * inv, o[db][g4 * 4 + 1] * inv);
                bf16x2 hi2 = to_bf16x2(o[db][g4 * 4 + 2] * inv, o[db][g4 * 4 + 3] * inv);
                bf16x4 w = {lo[0], lo[1], hi2[0], hi2[1]};
                *reinterpret_cast<bf16x4*>(orow + db * 32 + g4 * 8 + hi * 4) = w;
            }
        }
        if (hi == 0 && p.lse != nullptr)
            p.lse[(int64_t)head * p.lse_hs + myq] = (m + __builtin_log2f(ltot)) * kLn2;
    } else {
        const bool empty = !(ltot > 0.f);
        const float inv = empty ? 0.f : 1.0f / ltot;
        float* orow = reinterpret_cast<float*>(p.o) + (int64_t)head * p.o_hs + myq * p.o_rs;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 w = {o[db][g4 * 4 + 0] * inv, o[db][g4 * 4 + 1] * inv,
                           o[db][g4 * 4 + 2] * inv, o[db][g4 * 4 + 3] * inv};
                *reinterpret_cast<f32x4*>(orow + db * 32 + g4 * 8 + hi * 4) = w;
            }
        }
        if (hi == 0)
            p.lse[(int64_t)head * p.lse_hs + myq] =
                empty ? -INFINITY : (m + __builtin_log2f(ltot)) * kLn2;
    }
}

hipError_t launch_fwd(const FwdParams& p, int D, hipStream_t st) {
    if (p.nq <= 0 || p.nh <= 0) return hipSuccess;
    if (D != 128 && D != 64) return hipErrorInvalidValue;
    // 256-row workgroups when they fill the chip; 128-row ones otherwise
    const bool wide = (p.nq + 255) / 256 * p.nh >= kWideMinBlocks;
    const int bm = wide ? 256 : 128;
    const int64_t blocks = (p.nq + bm - 1) / bm * p.nh;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks), block(wide ? 512 : 256);
    if (D == 128) {
        if (wide) hipLaunchKernelGGL((fwd_kernel<128, 8>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((fwd_kernel<128, 4>), grid, block, 0, st, p);
    } else {
        if (wide) hipLaunchKernelGGL((fwd_kernel<64, 8>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((fwd_kernel<64, 4>), grid, block, 0, st, p);
    }
    return hipGetLastError();
}

}  // namespace hc
