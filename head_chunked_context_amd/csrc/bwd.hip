// bwd.hip - backward kernels for gfx950: dK/dV per key tile and dQ per query tile.
//
// The backward of exact attention needs Q, K, V, O and the incoming gradient
// (FPDT talk summary, "Background", on the backward's memory).  P is not
// stored: it is recomputed from the forward's LSE, P = exp(s - LSE).  With
// Delta_i = rowsum(dO_i * O_i) (prep kernel):
//     dP = dO V^T,  dS = P * (dP - Delta),
//     dV = P^T dO,  dK = scale * dS^T Q,  dQ = scale * dS K.
// No atomics: dK/dV and dQ are produced by separate kernels, each owning its
// output tile, with fixed accumulation orders (dK/dV: the group's query heads
// ascending, then query tiles ascending; dQ: key tiles ascending).
//
// The preprocessing pass stores the two row statistics in the form the loops
// use: -Delta, which both kernels take as the starting value of the dP
// accumulator (the MFMAs then yield dP - Delta), and -LSE * log2(e), the
// addend of the exponent's fused multiply-add.
//
// dkdv_kernel: workgroup = 8 waves on 128 keys of one query head's kv head;
// K and V of the 128 keys sit in LDS for the whole kernel.  Each step loads a
// 64-row query tile of Q and dO (plus the rows' statistics) straight into LDS,
// double-buffered.  Waves w and w + 4 share keys 32 (w % 4) .. +31 and take
// the lower / upper 32 rows of every tile:
//   S[q][key]   = Q K^T        A = Q rows (LDS),   B = K (LDS)
//   dP[q][key]  = dO V^T       A = dO rows (LDS),  B = V (LDS)
//   dV^T[d][key] += dO^T P     A = dO rows, transposed LDS reads
//   dK^T[d][key] += Q^T dS     A = Q rows, transposed LDS reads
// so each lane owns one key (lanes l and l^32 split the wave's rows).  Two
// waves per SIMD let one wave's softmax-side VALU work run under the other's
// MFMAs.  At the end the upper-half wave hands its dK/dV partial to its
// partner through LDS, which adds it after its own (fixed order).
//
// dq_kernel: workgroup = NW waves x 32 query rows of one head (NW = 8 with a
// 4-slot K/V ring and two tiles per barrier for large launches, NW = 4
// double-buffered otherwise, as in the forward); Q and dO stay in registers;
// 64-key tiles of K and V are loaded straight into LDS:
//   S^T = K Q^T,  dP^T = V dO^T,  dQ^T[d][q] += K^T dS^T (transposed K reads)
#include "device_common.h"
#include "kernels.h"

namespace hc {


// P and dS of one 64-row query tile against this lane's key, as bf16 MFMA
// operands.  MASK adds the causal / ragged-edge test; the common interior
// tiles skip it entirely.
template <int NQB, bool MASK>
__device__ __forceinline__ void dkdv_p_ds(const f32x16 (&sacc)[NQB], const f32x16 (&dpacc)[NQB],
                                          const float* s_nlse2, int hi, float scale_log2,
                                          int qrel0, int krel, int qlim, bf16x8 (&pb)[NQB][2],
                                          bf16x8 (&dsb)[NQB][2]) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int qr = qb * 32 + g4 * 8 + hi * 4;  // tile rows qr..qr+3
            const f32x4 L = *reinterpret_cast<const f32x4*>(s_nlse2 + qr);
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
                const int r = g4 * 4 + e;
                float pv[2], dsv[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    float x = fast_exp2(__builtin_fmaf(sacc[qb][r + u], scale_log2, L[e + u]));
                    if constexpr (MASK) {
                        // qrel/krel: row and key relative to the key tile start;
                        // visible iff key <= row (causal) and row < qlim
                        const int qrel = qrel0 + qr + e + u;
                        x = (krel <= qrel && qrel < qlim) ? x : 0.f;
                    }
                    pv[u] = x;
                    dsv[u] = x * dpacc[qb][r + u];
                }
                const bf16x2 pk = to_bf16x2(pv[0], pv[1]);
                const bf16x2 dk2 = to_bf16x2(dsv[0], dsv[1]);
                pb[qb][r >> 3][r & 7] = pk[0];
                pb[qb][r >> 3][(r & 7) + 1] = pk[1];
                dsb[qb][r >> 3][r & 7] = dk2[0];
                dsb[qb][r >> 3][(r & 7) + 1] = dk2[1];
            }
        }
    }
}

template <int HD, bool RUNS, bool GLOOP>
__global__ __launch_bounds__(512, 1) void dkdv_kernel(DkdvParams p) {
    constexpr int BQ = 64, WQ = 32, WK = 32, BNK = 128;
    constexpr int NS = HD / 16, NDB = HD / 32;
    constexpr int TILE = BQ * HD * 2;
    __shared__ __attribute__((aligned(1024))) char smem[2][2][TILE];  // [buf][Q / dO]
    __shared__ __attribute__((aligned(1024))) char skv[2][2 * TILE];  // this tile's K, V
    __shared__ __attribute__((aligned(16))) float s_nlse2[2][BQ];   // -LSE * log2(e)
    __shared__ __attribute__((aligned(16))) float s_ndelta[2][BQ];  // -Delta

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps per-wave values scalar
    const int hi = lane >> 5, l32 = lane & 31;
    const int kw = wave & 3;   // key block of the wave (32 keys)
    const int rh = wave >> 2;  // half of every 64-row query tile the wave takes

    // work item = key tile * units + unit, key tiles ascending: heaviest
    // first (key tile 0 sees every query tile when causal).  A unit is a
    // query head of the chunk (per-head schedule) or a kv head of the chunk
    // (group loop).
    // Workgroup b runs on die b % 8, and each die's L2 serves its resident
    // workgroups' Q/dO rows.  When the unit count is a multiple of 4, plain
    // order already gives each die one or two units at key tiles 2 or 1
    // apart; otherwise (1, 2, 5 ... units: RUNS) each die takes runs of 32
    // consecutive items per window of 8 x 32, in a snake order across
    // windows (a last partial window keeps plain order), so that a die's
    // workgroups stream neighbouring key tiles of few heads.  Measured at
    // S = 262144 (per-head schedule): dK/dV 5% faster with 1 head, 3.6% with
    // 2, 4% with 5 (of 40 / 8 kv heads); 4 and 8 heads are 4% faster in
    // plain order.
    const int units = GLOOP ? p.nkv : p.nh;
    int unit;
    int64_t kt;
    if constexpr (RUNS) {
        constexpr unsigned RUN = 32, WIN = 8 * RUN;
        unsigned item = blockIdx.x;
        const unsigned w = item / WIN;
        if ((w + 1) * WIN <= gridDim.x) {
            const unsigned x = item % 8, o = (item / 8) % RUN;
            item = w * WIN + ((w & 1) ? 7 - x : x) * RUN + o;
        }
        unit = (int)(item % (unsigned)units);
        kt = (int64_t)(item / (unsigned)units);
    } else {
        unit = blockIdx.x % units;
        kt = (int64_t)(blockIdx.x / units);
    }
    // the unit's kv head (local) and its query heads [hb, he) (local to the chunk)
    int kvl, hb, he;
    if constexpr (GLOOP) {
        kvl = unit;
        const int gh0 = (p.kv_base + kvl) * p.group - p.h0;
        hb = gh0 < 0 ? 0 : gh0;
        he = gh0 + p.group > p.nh ? p.nh : gh0 + p.group;
    } else {
        hb = unit;
        he = unit + 1;
        kvl = (p.h0 + unit) / p.group - p.kv_base;
    }
    const int64_t j0 = kt * BNK;                  // first key of the workgroup
    const int64_t wj0 = j0 + kw * WK;             // first key of this wave
    const int64_t myk = wj0 + l32;                // this lane's key

    // the workgroup's 128 keys of K (waves 0-3) and V (waves 4-7) go to LDS
    // (rows past nk repeat the last key; their P is masked to zero).  When
    // the tile holds 64 keys or fewer, every row of the second half repeats
    // key nk - 1, so no lane reads past the last key.
    if (j0 < p.nk) {
        const int64_t nv = p.nk - j0;
        const int64_t rs = rh == 0 ? p.k_rs : p.v_rs;
        const uint16_t* src = rh == 0 ? p.k + (int64_t)kvl * p.k_hs + j0 * p.k_rs
                                      : p.v + (int64_t)kvl * p.v_hs + j0 * p.v_rs;
        direct_tile64<HD>(skv[rh], src, rs, nv, kw, lane);
        if (nv > 64)
            direct_tile64<HD>(skv[rh] + TILE, src + 64 * rs, rs, nv - 64, kw, lane);
        else
            direct_tile64<HD>(skv[rh] + TILE, src + (nv - 1) * rs, rs, 1, kw, lane);
    }
    f32x16 dk[NDB], dv[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
    }
    // a group continued from the previous chunk resumes from its row half's sums
    if (GLOOP && kvl == p.carry_kv_in && myk < p.nk) {
        const float* ck = p.carry_in_k + rh * p.carry_hs + myk * HD;
        const float* cv = p.carry_in_v + rh * p.carry_hs + myk * HD;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(ck + db * 32 + g4 * 8 + hi * 4);
                const f32x4 y = *reinterpret_cast<const f32x4*>(cv + db * 32 + g4 * 8 + hi * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dk[db][g4 * 4 + e] = x[e];
                    dv[db][g4 * 4 + e] = y[e];
                }
            }
        }
    }

    // query tiles: causal rows start at the workgroup's first key position
    const int64_t nqt = (p.nq + BQ - 1) / BQ;
    int64_t qt0 = 0;
    if (p.causal) {
        const int64_t first = p.k_pos0 + j0;
        qt0 = first >= p.nq ? nqt : first / BQ;
    }
    // steps: heads hb..he-1 ascending, each over query tiles qt0..nqt-1 ascending
    const int64_t nsteps = j0 < p.nk ? nqt - qt0 : 0;
    const int64_t total = nsteps * (he - hb);

    // one step = Q (waves 0-3) and dO (waves 4-7) rows [i0, i0 + 64) of head
    // h plus their LSE (wave 0) and Delta (wave 4), straight into LDS buffer b
    // each wave loads one contiguous run of the tile's rows: with the
    // interleaved order this kernel ran 7-12% slower at S = 262144 with 32
    // heads per launch (the forward and dQ kernels showed no difference)
    const TileDma64<HD, false> dqo(rh == 0 ? p.q_rs : p.do_rs, kw, lane);
    auto issue_step = [&](int h, int64_t s, int b) {
        const int64_t i0 = (qt0 + s) * BQ;
        if (rh == 0)
            dqo.load(smem[b][0], p.q + (int64_t)h * p.q_hs + i0 * p.q_rs, p.q_rs, p.nq - i0, kw, lane);
        else
            dqo.load(smem[b][1], p.dO + (int64_t)h * p.do_hs + i0 * p.do_rs, p.do_rs, p.nq - i0, kw,
                     lane);
        if (wave == 0) direct_vec64(s_nlse2[b], p.nlse2 + (int64_t)h * p.nlse2_hs + i0, p.nq - i0, lane);
        if (wave == 4) direct_vec64(s_ndelta[b], p.ndelta + (int64_t)h * p.ndelta_hs + i0, p.nq - i0, lane);
    };
    if (total > 0) issue_step(hb, 0, 0);
    wait_vm_loads();
    __syncthreads();

    const OperandOffsets<HD> off(lane);  // K / V / Q / dO operand reads
    // positions relative to this wave's first key, in 32-bit
    const int64_t wkpos = p.k_pos0 + wj0;
    const int krel = l32;
    // cursor (head, query step) of step n, and of step n + 1
    int h_cur = hb;
    int64_t s_cur = 0;
    for (int64_t n = 0; n < total; ++n) {
        const int buf = (int)(n & 1);
        int h_nxt = h_cur;
        int64_t s_nxt = s_cur + 1;
        if (s_nxt == nsteps) {
            s_nxt = 0;
            ++h_nxt;
        }
        if (n + 1 < total) issue_step(h_nxt, s_nxt, buf ^ 1);
        const int64_t r0 = (qt0 + s_cur) * BQ + rh * WQ;  // first row of this wave
        // a wave works on the tile only if some of its rows sees one of its keys
        const bool live = wj0 < p.nk && r0 < p.nq && (!p.causal || r0 + WQ - 1 >= wkpos);
        if (live) {
            const char* Qs = smem[buf][0];
            const char* Os = smem[buf][1];
            const float* sl = s_nlse2[buf] + rh * WQ;
            // dP accumulates onto -Delta of each register's row, so it comes out
            // as dP - Delta (register r holds row (r / 4) * 8 + hi * 4 + r % 4)
            f32x16 sacc[1], dpacc[1];
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 nd = *reinterpret_cast<const f32x4*>(s_ndelta[buf] + rh * WQ + g4 * 8 + hi * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) dpacc[0][g4 * 4 + e] = nd[e];
            }
            // MFMA j: S (even j) or dP (odd j) over d 16 (j / 2) ..; both of
            // its operands are read DIST MFMAs ahead
            {
                constexpr int NJ = 2 * NS, DIST = 2;
                auto rd = [&](int j, bf16x8& x, bf16x8& y) {
                    const int st = j >> 1;
                    const int ko = off.row[st] + kw * 32 * HD * 2;
                    const int qo = off.row[st] + rh * 32 * HD * 2;
                    x = lds_read_b128((j & 1) ? Os : Qs, qo);
                    y = lds_read_b128(skv[j & 1], ko);
                };
                bf16x8 ra[DIST], rb[DIST];
#pragma unroll
                for (int j = 0; j < DIST; ++j) rd(j, ra[j], rb[j]);
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const bf16x8 a = ra[j % DIST], b = rb[j % DIST];
                    if (j + DIST < NJ) rd(j + DIST, ra[j % DIST], rb[j % DIST]);
                    const int st = j >> 1;
                    if (j & 1) dpacc[0] = mfma32(a, b, dpacc[0]);
                    else sacc[0] = mfma32(a, b, st == 0 ? f32x16{} : sacc[0]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            bf16x8 pb[1][2], dsb[1][2];
            const bool edge_k = wj0 + WK > p.nk;
            const bool edge_q = r0 + WQ > p.nq;
            const bool diag = p.causal && r0 < wkpos + WK - 1;
            if (edge_k || edge_q || diag) {
                // rows relative to the wave's first key; keys past nk and rows
                // past nq are invisible; non-causal sees every row
                const int qrel0 = (int)(p.causal ? r0 - wkpos : WK + r0);
                const int qlim = (int)(p.causal ? p.nq - wkpos : WK + p.nq);
                const int kr = (myk < p.nk) ? krel : (1 << 30);
                dkdv_p_ds<1, true>(sacc, dpacc, sl, hi, p.scale_log2, qrel0, kr, qlim, pb, dsb);
            } else {
                dkdv_p_ds<1, false>(sacc, dpacc, sl, hi, p.scale_log2, 0, 0, 0, pb, dsb);
            }
            // dV^T += dO^T P and dK^T += Q^T dS, reduction over the wave's 32 rows
            {
                // MFMA j: dV (even j) or dK (odd j) of d block j / 4, rows
                // 16 ((j / 2) % 2) ..; its A operand is read 2 MFMAs ahead
                constexpr int NJ = 4 * NDB, DIST = 3;
                auto rd = [&](int j) {
                    return lds_read_tr_at<HD>((j & 1) ? Qs : Os, off, rh * 32 + ((j >> 1) & 1) * 16, j >> 2);
                };
                bf16x8 ring[DIST];
#pragma unroll
                for (int j = 0; j < DIST; ++j) ring[j] = rd(j);
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const bf16x8 a = ring[j % DIST];
                    if (j + DIST < NJ) ring[j % DIST] = rd(j + DIST);
                    const int db = j >> 2, h2 = (j >> 1) & 1;
                    if (j & 1) dk[db] = mfma32(a, dsb[0][h2], dk[db]);
                    else dv[db] = mfma32(a, pb[0][h2], dv[db]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        h_cur = h_nxt;
        s_cur = s_nxt;
        wait_vm_loads();
        __syncthreads();
    }

    // group continuing in the next chunk: each row half leaves its own sums
    if (GLOOP && kvl == p.carry_kv_out) {
        if (myk >= p.nk) return;
        float* ck = p.carry_out_k + rh * p.carry_hs + myk * HD;
        float* cv = p.carry_out_v + rh * p.carry_hs + myk * HD;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 x, y;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] = dk[db][g4 * 4 + e];
                    y[e] = dv[db][g4 * 4 + e];
                }
                *reinterpret_cast<f32x4*>(ck + db * 32 + g4 * 8 + hi * 4) = x;
                *reinterpret_cast<f32x4*>(cv + db * 32 + g4 * 8 + hi * 4) = y;
            }
        }
        return;
    }

    // the two waves of a key block hold partial sums over the two row halves:
    // waves 4-7 hand theirs over through LDS (free after the last barrier) and
    // waves 0-3 add them, lower half first
    f32x4* xk = reinterpret_cast<f32x4*>(&smem[0][0][0]) + kw * (NDB * 4 * 64);
    f32x4* xv = reinterpret_cast<f32x4*>(&skv[0][0]) + kw * (NDB * 4 * 64);
    if (rh == 1) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 x, y;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] = dk[db][g4 * 4 + e];
                    y[e] = dv[db][g4 * 4 + e];
                }
                xk[(db * 4 + g4) * 64 + lane] = x;
                xv[(db * 4 + g4) * 64 + lane] = y;
            }
        }
    }
    __syncthreads();
    if (rh == 1 || myk >= p.nk) return;
    if constexpr (GLOOP) {
        // the group is complete: bf16(scale * dK), bf16(dV)
        uint16_t* ok = p.dk + (int64_t)kvl * p.dk_hs + myk * p.dk_rs;
        uint16_t* ov = p.dv + (int64_t)kvl * p.dk_hs + myk * p.dk_rs;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 uk = xk[(db * 4 + g4) * 64 + lane];
                const f32x4 uv = xv[(db * 4 + g4) * 64 + lane];
                f32x4 x, y;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] = dk[db][g4 * 4 + e] + uk[e];
                    y[e] = dv[db][g4 * 4 + e] + uv[e];
                }
                const bf16x2 k0 = to_bf16x2(x[0] * p.scale, x[1] * p.scale);
                const bf16x2 k1 = to_bf16x2(x[2] * p.scale, x[3] * p.scale);
                const bf16x2 v0 = to_bf16x2(y[0], y[1]), v1 = to_bf16x2(y[2], y[3]);
                *reinterpret_cast<bf16x4*>(ok + db * 32 + g4 * 8 + hi * 4) = bf16x4{k0[0], k0[1], k1[0], k1[1]};
                *reinterpret_cast<bf16x4*>(ov + db * 32 + g4 * 8 + hi * 4) = bf16x4{v0[0], v0[1], v1[0], v1[1]};
            }
        }
    } else {
        float* ak = p.part_k + ((int64_t)hb * p.nk + myk) * HD;
        float* av = p.part_v + ((int64_t)hb * p.nk + myk) * HD;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 ok = xk[(db * 4 + g4) * 64 + lane];
                const f32x4 ov = xv[(db * 4 + g4) * 64 + lane];
                f32x4 x, y;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] = dk[db][g4 * 4 + e] + ok[e];
                    y[e] = dv[db][g4 * 4 + e] + ov[e];
                }
                *reinterpret_cast<f32x4*>(ak + db * 32 + g4 * 8 + hi * 4) = x;
                *reinterpret_cast<f32x4*>(av + db * 32 + g4 * 8 + hi * 4) = y;
            }
        }
    }
}

// One thread per 4 consecutive fp32 of a (kv head, key) row.
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(DkdvReduceParams p) {
    const int cpr = p.D / 4;
    const int64_t total = (int64_t)p.nkv * p.nk * cpr;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(idx % cpr);
        const int64_t kr = idx / cpr;
        const int64_t key = kr % p.nk;
        const int kvl = (int)(kr / p.nk);
        const int kvg = p.kv_base + kvl;
        int hb = kvg * p.group - p.h0, he = (kvg + 1) * p.group - p.h0;
        hb = hb < 0 ? 0 : hb;
        he = he > p.nh ? p.nh : he;
        f32x4 ak = {0.f, 0.f, 0.f, 0.f}, av = {0.f, 0.f, 0.f, 0.f};
        if (kvl == p.carry_kv_in) {
            ak = *reinterpret_cast<const f32x4*>(p.carry_in_k + key * p.D + c * 4);
            av = *reinterpret_cast<const f32x4*>(p.carry_in_v + key * p.D + c * 4);
        }
        for (int h = hb; h < he; ++h) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(p.part_k + ((int64_t)h * p.nk + key) * p.D + c * 4);
            const f32x4 y = *reinterpret_cast<const f32x4*>(p.part_v + ((int64_t)h * p.nk + key) * p.D + c * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ak[e] = ak[e] + x[e];
                av[e] = av[e] + y[e];
            }
        }
        if (kvl == p.carry_kv_out) {
            *reinterpret_cast<f32x4*>(p.carry_out_k + key * p.D + c * 4) = ak;
            *reinterpret_cast<f32x4*>(p.carry_out_v + key * p.D + c * 4) = av;
        } else {
            const bf16x2 k0 = to_bf16x2(ak[0] * p.scale, ak[1] * p.scale);
            const bf16x2 k1 = to_bf16x2(ak[2] * p.scale, ak[3] * p.scale);
            const bf16x2 v0 = to_bf16x2(av[0], av[1]), v1 = to_bf16x2(av[2], av[3]);
            const int64_t o = (int64_t)kvl * p.dk_hs + key * p.dk_rs + c * 4;
            *reinterpret_cast<bf16x4*>(p.dk + o) = bf16x4{k0[0], k0[1], k1[0], k1[1]};
            *reinterpret_cast<bf16x4*>(p.dv + o) = bf16x4{v0[0], v0[1], v1[0], v1[1]};
        }
    }
}

// dS^T of NB 32-key blocks for this lane's query row as bf16 MFMA operands.
// MASK adds the causal / ragged test with keys relative to the first block.
template <int NB, bool MASK>
__device__ __forceinline__ void dq_ds(const f32x16 (&s)[NB], const f32x16 (&dp)[NB], float scale_log2,
                                      float nlse2, int hi, int qrel, int klim,
                                      bf16x8 (&dsb)[NB][2]) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            float dsv[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                float x = fast_exp2(__builtin_fmaf(s[b][r + u], scale_log2, nlse2));
                if constexpr (MASK) {
                    const int key = b * 32 + ((r + u) >> 2) * 8 + hi * 4 + ((r + u) & 3);
                    x = (key <= qrel && key < klim) ? x : 0.f;
                }
                dsv[u] = x * dp[b][r + u];
            }
            const bf16x2 d2 = to_bf16x2(dsv[0], dsv[1]);
            dsb[b][r >> 3][r & 7] = d2[0];
            dsb[b][r >> 3][(r & 7) + 1] = d2[1];
        }
    }
}

template <int HD, int NW>
__global__ __launch_bounds__(NW * 64, 8 / NW) void dq_kernel(DqParams p) {
    constexpr int BN = 64, WQ = 32, BM = NW * WQ;
    constexpr int NS = HD / 16, NDB = HD / 32;
    constexpr int TILE = BN * HD * 2;
    // K/V ring slots: 8 waves work on two tiles per barrier while the next
    // two load; 4 waves double-buffer single tiles
    constexpr int NBUF = NW == 8 ? 4 : 2;
    __shared__ __attribute__((aligned(1024))) char smem[NBUF][2][TILE];  // [slot][K / V]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps per-wave values scalar
    const int hi = lane >> 5, l32 = lane & 31;

    const int64_t qtb = p.q_begin / BM;
    const int64_t nqt = (p.nq + BM - 1) / BM - qtb;
    const int head = blockIdx.x % p.nh;
    const int64_t qt = qtb + nqt - 1 - (int64_t)(blockIdx.x / p.nh);
    const int64_t q0 = qt * BM;
    const int kvl = (p.h0 + head) / p.group - p.kv_base;
    const uint16_t* kh = p.k + (int64_t)kvl * p.k_hs;
    const uint16_t* vh = p.v + (int64_t)kvl * p.v_hs;

    const int64_t wq0 = q0 + wave * WQ;
    const int64_t myq = wq0 + l32;
    const bool wave_live = wq0 < p.nq;
    const bool row_ok = myq < p.nq;

    bf16x8 qf[NS], df[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        if (row_ok) {
            qf[s] = *reinterpret_cast<const bf16x8*>(p.q + (int64_t)head * p.q_hs + myq * p.q_rs + s * 16 + hi * 8);
            df[s] = *reinterpret_cast<const bf16x8*>(p.dO + (int64_t)head * p.do_hs + myq * p.do_rs + s * 16 + hi * 8);
        } else {
            qf[s] = bf16x8{};
            df[s] = bf16x8{};
        }
    }
    const float nlse2 = row_ok ? p.nlse2[(int64_t)head * p.nlse2_hs + myq] : -INFINITY;
    const float ndlt = row_ok ? p.ndelta[(int64_t)head * p.ndelta_hs + myq] : 0.f;

    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        acc[db] = f32x16{};
        if (p.acc_in != nullptr && row_ok) {
            const float* a = p.acc_in + (int64_t)head * p.ain_hs + myq * p.ain_rs;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(a + db * 32 + g4 * 8 + hi * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[db][g4 * 4 + e] = x[e];
            }
        }
    }

    const int64_t wg_last = (q0 + BM - 1 < p.nq - 1) ? q0 + BM - 1 : p.nq - 1;
    const int64_t w_last = (wq0 + WQ - 1 < p.nq - 1) ? wq0 + WQ - 1 : p.nq - 1;
    int64_t kend = p.nk, kend_w = wave_live ? p.nk : 0;
    if (p.causal) {
        const int64_t a = wg_last - p.k_pos0 + 1, b = w_last - p.k_pos0 + 1;
        kend = a < kend ? a : kend;
        kend_w = b < kend_w ? b : kend_w;
    }
    const int ntiles = kend > 0 ? (int)((kend + BN - 1) / BN) : 0;
    const int ntiles_w = kend_w > 0 ? (int)((kend_w + BN - 1) / BN) : 0;

    // 8 waves: K tiles by waves 0-3, V tiles by waves 4-7; 4 waves: both
    const int kv_sel = wave >> 2;
    const uint16_t* kvh = kv_sel == 0 ? kh : vh;
    const int64_t kv_rs = kv_sel == 0 ? p.k_rs : p.v_rs;
    // per-lane parts of the tile-load addresses (8 waves: K or V; 4 waves: both)
    const TileDma64<HD, true> dkv(NW == 8 ? kv_rs : p.k_rs, wave & 3, lane);
    const TileDma64<HD, true> dv2(p.v_rs, wave & 3, lane);
    auto issue = [&](int t) {
        const int64_t nb = (int64_t)t * BN;
        if constexpr (NW == 8) {
            dkv.load(smem[t % NBUF][kv_sel], kvh + nb * kv_rs, kv_rs, p.nk - nb, wave & 3, lane);
        } else {
            dkv.load(smem[t % NBUF][0], kh + nb * p.k_rs, p.k_rs, p.nk - nb, wave, lane);
            dv2.load(smem[t % NBUF][1], vh + nb * p.v_rs, p.v_rs, p.nk - nb, wave, lane);
        }
    };
    wait_vm_loads();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        settle(qf[s]);
        settle(df[s]);
    }
    settle(nlse2);
    settle(ndlt);
    // every register of the lane's dP accumulator starts at -Delta of its
    // row, so the MFMAs yield dP - Delta
    f32x16 ndsplat;
#pragma unroll
    for (int r = 0; r < 16; ++r) ndsplat[r] = ndlt;
#pragma unroll
    for (int db = 0; db < NDB; ++db) settle(acc[db]);
    const int pre = ntiles < NBUF / 2 ? ntiles : NBUF / 2;
    for (int t = 0; t < pre; ++t) issue(t);
    wait_vm_loads();
    __syncthreads();

    const OperandOffsets<HD> off(lane);         // K / V operand reads
    const int64_t qrel_base = myq - p.k_pos0;  // query position relative to key 0
    auto tile = [&](int j, int buf) {
        if (j < ntiles_w) {
            const char* Ks = smem[buf][0];
            const char* Vs = smem[buf][1];
            const int64_t kb = (int64_t)j * BN;
            const bool need_mask = (kb + BN > p.nk) || (p.causal && p.k_pos0 + kb + BN - 1 > wq0);
            // the tile's two 32-key halves one after the other (half the score
            // registers live at a time)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                f32x16 s[1], dp[1];
                // MFMA j: S^T (even j) or dP^T (odd j) over d 16 (j / 2) ..;
                // its A operand (K or V rows) is read DIST MFMAs ahead
                constexpr int NJ = 2 * NS, DIST = 2;
                auto read_a = [&](int j) {
                    return lds_read_b128((j & 1) ? Vs : Ks, off.row[j >> 1] + b * 32 * HD * 2);
                };
                bf16x8 ring[DIST];
#pragma unroll
                for (int j = 0; j < DIST; ++j) ring[j] = read_a(j);
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const bf16x8 a = ring[j % DIST];
                    if (j + DIST < NJ) ring[j % DIST] = read_a(j + DIST);
                    const int st = j >> 1;
                    if (j & 1) dp[0] = mfma32(a, df[st], st == 0 ? ndsplat : dp[0]);
                    else s[0] = mfma32(a, qf[st], st == 0 ? f32x16{} : s[0]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                bf16x8 dsb[1][2];
                if (need_mask) {
                    const int64_t qr = p.causal ? qrel_base - kb - b * 32 : (int64_t)BN;
                    const int kl = (int)(p.nk - kb - b * 32);
                    dq_ds<1, true>(s, dp, p.scale_log2, nlse2, hi, (int)qr, kl, dsb);
                } else {
                    dq_ds<1, false>(s, dp, p.scale_log2, nlse2, hi, 0, 0, dsb);
                }
                // dQ^T += K^T dS^T over the half's 32 keys; MFMA j (d block
                // j / 2, keys 16 (j % 2) ..) has its K^T operand read DIST ahead
                {
                    constexpr int NJ = 2 * NDB, DIST = 3;
                    auto rdt = [&](int j) { return lds_read_tr_at<HD>(Ks, off, b * 32 + (j & 1) * 16, j >> 1); };
                    bf16x8 ring[DIST];
#pragma unroll
                    for (int j = 0; j < DIST; ++j) ring[j] = rdt(j);
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        const bf16x8 ak = ring[j % DIST];
                        if (j + DIST < NJ) ring[j % DIST] = rdt(j + DIST);
                        acc[j >> 1] = mfma32(ak, dsb[0][j & 1], acc[j >> 1]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        }
    };
    if constexpr (NW == 8) {
        for (int j = 0; j < ntiles; j += 2) {
            // slots of tiles j - 2 and j - 1 were released by the last barrier
            if (j + 2 < ntiles) issue(j + 2);
            if (j + 3 < ntiles) issue(j + 3);
            tile(j, j % NBUF);
            if (j + 1 < ntiles) tile(j + 1, (j + 1) % NBUF);
            wait_vm_loads();  // tiles j + 2 and j + 3
            __syncthreads();
        }
    } else {
        for (int j = 0; j < ntiles; ++j) {
            if (j + 1 < ntiles) issue(j + 1);
            tile(j, j % NBUF);
            wait_vm_loads();
            __syncthreads();
        }
    }

    if (!row_ok) return;
    if (myq < p.final_before || p.acc_out == nullptr) {
        uint16_t* out = p.dq + (int64_t)head * p.dq_hs + myq * p.dq_rs;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const bf16x2 a0 = to_bf16x2(acc[db][g4 * 4 + 0] * p.scale, acc[db][g4 * 4 + 1] * p.scale);
                const bf16x2 a1 = to_bf16x2(acc[db][g4 * 4 + 2] * p.scale, acc[db][g4 * 4 + 3] * p.scale);
                *reinterpret_cast<bf16x4*>(out + db * 32 + g4 * 8 + hi * 4) = bf16x4{a0[0], a0[1], a1[0], a1[1]};
            }
        }
    } else {
        float* out = p.acc_out + (int64_t)head * p.aout_hs + myq * p.aout_rs;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = acc[db][g4 * 4 + e];
                *reinterpret_cast<f32x4*>(out + db * 32 + g4 * 8 + hi * 4) = x;
            }
        }
    }
}

hipError_t launch_dkdv(const DkdvParams& p, int D, hipStream_t st) {
    const int units = p.group_loop ? p.nkv : p.nh;
    if (p.nk <= 0 || units <= 0) return hipSuccess;
    const int64_t blocks = (p.nk + kDkdvBlockN - 1) / kDkdvBlockN * units;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // die-aware runs of work items unless the unit count is a multiple of 4
    const bool runs = units % 4 != 0;
    const dim3 grid((unsigned)blocks), block(512);
#define HC_DKDV(HD, R, G) hipLaunchKernelGGL((dkdv_kernel<HD, R, G>), grid, block, 0, st, p)
    if (D != 128 && D != 64) return hipErrorInvalidValue;
    if (p.group_loop) {
        if (D == 128) { if (runs) HC_DKDV(128, true, true); else HC_DKDV(128, false, true); }
        else { if (runs) HC_DKDV(64, true, true); else HC_DKDV(64, false, true); }
    } else {
        if (D == 128) { if (runs) HC_DKDV(128, true, false); else HC_DKDV(128, false, false); }
        else { if (runs) HC_DKDV(64, true, false); else HC_DKDV(64, false, false); }
    }
#undef HC_DKDV
    return hipGetLastError();
}

hipError_t launch_dkdv_reduce(const DkdvReduceParams& p, hipStream_t st) {
    if (p.nk <= 0 || p.nkv <= 0) return hipSuccess;
    int64_t b = ((int64_t)p.nkv * p.nk * (p.D / 4) + 255) / 256;
    b = b > 65536 ? 65536 : b;
    hipLaunchKernelGGL(dkdv_reduce_kernel, dim3((unsigned)b), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_dq(const DqParams& p, int D, hipStream_t st) {
    if (p.nq <= p.q_begin || p.nh <= 0) return hipSuccess;
    if (D != 128 && D != 64) return hipErrorInvalidValue;
    // 256-row workgroups when they fill the chip; 128-row ones otherwise (the
    // first row must start a workgroup: trunk starts are multiples of 256)
    const bool wide = ((p.nq + 255) / 256 - p.q_begin / 256) * p.nh >= kWideMinBlocks;
    const int bm = wide ? 256 : 128;
    if (p.q_begin % bm != 0) return hipErrorInvalidValue;
    const int64_t blocks = ((p.nq + bm - 1) / bm - p.q_begin / bm) * p.nh;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks), block(wide ? 512 : 256);
    if (D == 128) {
        if (wide) hipLaunchKernelGGL((dq_kernel<128, 8>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((dq_kernel<128, 4>), grid, block, 0, st, p);
    } else {
        if (wide) hipLaunchKernelGGL((dq_kernel<64, 8>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((dq_kernel<64, 4>), grid, block, 0, st, p);
    }
    return hipGetLastError();
}

}  // namespace hc
