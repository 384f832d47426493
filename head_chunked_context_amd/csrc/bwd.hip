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
// dkdv_kernel: workgroup = 4 waves x 32 keys (128 keys) of one kv head.  K and
// V stay in registers as MFMA operands; each step stages a 64-row query tile
// of Q and dO (plus LSE and Delta) through LDS, double-buffered:
//   S[q][key]   = Q K^T        A = Q tile (LDS),   B = K (regs)
//   dP[q][key]  = dO V^T       A = dO tile (LDS),  B = V (regs)
//   dV^T[d][key] += dO^T P     A = dO tile, transposed LDS reads
//   dK^T[d][key] += Q^T dS     A = Q tile, transposed LDS reads
// so each lane owns one key (lanes l and l^32 split the 64 query rows).
//
// dq_kernel: workgroup = 4 waves x 32 query rows of one head; Q and dO stay in
// registers; 64-key tiles of K and V go through LDS like the forward:
//   S^T = K Q^T,  dP^T = V dO^T,  dQ^T[d][q] += K^T dS^T (transposed K reads)
#include "device_common.h"
#include "kernels.h"

namespace hc {

constexpr float kLog2e = 1.4426950408889634f;

template <int HD>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(DkdvParams p) {
    constexpr int BQ = 64, WK = 32, BNK = 128;
    constexpr int NS = HD / 16, NDB = HD / 32;
    constexpr int TILE = BQ * HD * 2;
    __shared__ __attribute__((aligned(16))) char smem[2][2][TILE];  // [buf][Q / dO]
    __shared__ __attribute__((aligned(16))) float s_lse[2][BQ];
    __shared__ __attribute__((aligned(16))) float s_delta[2][BQ];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hi = lane >> 5, l32 = lane & 31;

    const int64_t nkt = (p.nk + BNK - 1) / BNK;
    const int kvl = blockIdx.x % p.nkv;
    const int64_t kt = nkt - 1 - (int64_t)(blockIdx.x / p.nkv);  // (any order works)
    const int64_t j0 = kt * BNK;                  // first key of the workgroup
    const int64_t wj0 = j0 + wave * WK;           // first key of this wave
    const int64_t myk = wj0 + l32;                // this lane's key
    const int64_t mykpos = p.k_pos0 + myk;
    const int kvg = p.kv_base + kvl;              // global kv head

    // query heads of this chunk that read kv head kvg, ascending
    int hb = kvg * p.group - p.h0, he = (kvg + 1) * p.group - p.h0;
    hb = hb < 0 ? 0 : hb;
    he = he > p.nh ? p.nh : he;

    // K and V of this lane's key as B operands (rows past nk are zero)
    const uint16_t* kh = p.k + (int64_t)kvl * p.k_hs;
    const uint16_t* vh = p.v + (int64_t)kvl * p.v_hs;
    bf16x8 kf[NS], vf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        if (myk < p.nk) {
            kf[s] = *reinterpret_cast<const bf16x8*>(kh + myk * p.k_rs + s * 16 + hi * 8);
            vf[s] = *reinterpret_cast<const bf16x8*>(vh + myk * p.v_rs + s * 16 + hi * 8);
        } else {
            kf[s] = bf16x8{};
            vf[s] = bf16x8{};
        }
    }

    f32x16 dk[NDB], dv[NDB];
    const bool carry_in = kvl == p.carry_kv_in && p.acc_in_k != nullptr;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
        if (carry_in && myk < p.nk) {
            const float* ak = p.acc_in_k + (int64_t)kvl * p.ain_hs + myk * p.ain_rs;
            const float* av = p.acc_in_v + (int64_t)kvl * p.ain_hs + myk * p.ain_rs;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(ak + db * 32 + g4 * 8 + hi * 4);
                const f32x4 y = *reinterpret_cast<const f32x4*>(av + db * 32 + g4 * 8 + hi * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dk[db][g4 * 4 + e] = x[e];
                    dv[db][g4 * 4 + e] = y[e];
                }
            }
        }
    }

    // query tiles: causal rows >= first key position of the workgroup
    const int64_t nqt = (p.nq + BQ - 1) / BQ;
    int64_t qt0 = 0;
    if (p.causal) {
        const int64_t first = p.k_pos0 + j0;
        qt0 = first >= p.nq ? nqt : first / BQ;
    }
    const int64_t nqi = nqt - qt0;
    const int64_t nsteps = (he > hb && j0 < p.nk) ? (int64_t)(he - hb) * nqi : 0;

    Tile64<HD> tq, tdo;
    float lse_r = 0.f, dl_r = 0.f;
    auto load_step = [&](int64_t n) {
        const int hl = hb + (int)(n / nqi);
        const int64_t i0 = (qt0 + n % nqi) * BQ;
        const uint16_t* qb = p.q + (int64_t)hl * p.q_hs + i0 * p.q_rs;
        const uint16_t* ob = p.dO + (int64_t)hl * p.do_hs + i0 * p.do_rs;
        tq.load(qb, p.q_rs, p.nq - i0, tid);
        tdo.load(ob, p.do_rs, p.nq - i0, tid);
        if (tid < BQ) {
            const int64_t row = i0 + tid;
            lse_r = row < p.nq ? p.lse[(int64_t)(p.h0 + hl) * p.lse_hs + row] * kLog2e : INFINITY;
            dl_r = row < p.nq ? p.delta[(int64_t)hl * p.delta_hs + row] : 0.f;
        }
    };
    auto store_step = [&](int buf) {
        tq.store(smem[buf][0], tid);
        tdo.store(smem[buf][1], tid);
        if (tid < BQ) {
            s_lse[buf][tid] = lse_r;
            s_delta[buf][tid] = dl_r;
        }
    };
    if (nsteps > 0) {
        load_step(0);
        store_step(0);
    }
    __syncthreads();

    for (int64_t n = 0; n < nsteps; ++n) {
        const int buf = (int)(n & 1);
        const bool more = n + 1 < nsteps;
        if (more) load_step(n + 1);
        const int64_t i0 = (qt0 + n % nqi) * BQ;
        // a wave works on the tile only if some row sees one of its keys
        const bool live = wj0 < p.nk && (!p.causal || i0 + BQ - 1 >= p.k_pos0 + wj0);
        if (live) {
            const char* Qs = smem[buf][0];
            const char* Os = smem[buf][1];
            f32x16 sacc[2] = {f32x16{}, f32x16{}}, dpacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int st = 0; st < NS; ++st) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    bf16x8 aq = lds_read_b128(Qs, lds_off<HD>(qb * 32 + l32, st * 16 + hi * 8));
                    sacc[qb] = mfma32(aq, kf[st], sacc[qb]);
                    bf16x8 ao = lds_read_b128(Os, lds_off<HD>(qb * 32 + l32, st * 16 + hi * 8));
                    dpacc[qb] = mfma32(ao, vf[st], dpacc[qb]);
                }
            }
            const bool need_mask = (wj0 + WK > p.nk) || (i0 + BQ > p.nq) ||
                                   (p.causal && i0 < p.k_pos0 + wj0 + WK - 1);
            bf16x8 pb[2][2], dsb[2][2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int qr = qb * 32 + g4 * 8 + hi * 4;  // rows qr..qr+3
                    const f32x4 L = *reinterpret_cast<const f32x4*>(&s_lse[buf][qr]);
                    const f32x4 Dl = *reinterpret_cast<const f32x4*>(&s_delta[buf][qr]);
#pragma unroll
                    for (int e = 0; e < 4; e += 2) {
                        const int r = g4 * 4 + e;
                        float pv[2], dsv[2];
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            float x = fast_exp2(sacc[qb][r + u] * p.scale_log2 - L[e + u]);
                            if (need_mask) {
                                const int64_t qrow = i0 + qr + e + u;
                                const bool ok = myk < p.nk && qrow < p.nq &&
                                                (!p.causal || mykpos <= qrow);
                                x = ok ? x : 0.f;
                            }
                            pv[u] = x;
                            dsv[u] = x * (dpacc[qb][r + u] - Dl[e + u]);
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
            // dV^T += dO^T P and dK^T += Q^T dS, reduction over the 64 query rows
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        bf16x8 ao = lds_read_tr_operand<HD>(Os, qb * 32 + h2 * 16, db * 32, lane);
                        dv[db] = mfma32(ao, pb[qb][h2], dv[db]);
                        bf16x8 aq = lds_read_tr_operand<HD>(Qs, qb * 32 + h2 * 16, db * 32, lane);
                        dk[db] = mfma32(aq, dsb[qb][h2], dk[db]);
                    }
                }
            }
        }
        if (more) store_step(buf ^ 1);
        __syncthreads();
    }

    if (myk >= p.nk) return;
    if (kvl == p.carry_kv_out && p.acc_out_k != nullptr) {
        float* ak = p.acc_out_k + (int64_t)kvl * p.aout_hs + myk * p.aout_rs;
        float* av = p.acc_out_v + (int64_t)kvl * p.aout_hs + myk * p.aout_rs;
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
                *reinterpret_cast<f32x4*>(ak + db * 32 + g4 * 8 + hi * 4) = x;
                *reinterpret_cast<f32x4*>(av + db * 32 + g4 * 8 + hi * 4) = y;
            }
        }
        return;
    }
    uint16_t* okp = p.dk + (int64_t)kvl * p.dk_hs + myk * p.dk_rs;
    uint16_t* ovp = p.dv + (int64_t)kvl * p.dk_hs + myk * p.dk_rs;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const bf16x2 a0 = to_bf16x2(dk[db][g4 * 4 + 0] * p.scale, dk[db][g4 * 4 + 1] * p.scale);
            const bf16x2 a1 = to_bf16x2(dk[db][g4 * 4 + 2] * p.scale, dk[db][g4 * 4 + 3] * p.scale);
            const bf16x2 b0 = to_bf16x2(dv[db][g4 * 4 + 0], dv[db][g4 * 4 + 1]);
            const bf16x2 b1 = to_bf16x2(dv[db][g4 * 4 + 2], dv[db][g4 * 4 + 3]);
            *reinterpret_cast<bf16x4*>(okp + db * 32 + g4 * 8 + hi * 4) = bf16x4{a0[0], a0[1], a1[0], a1[1]};
            *reinterpret_cast<bf16x4*>(ovp + db * 32 + g4 * 8 + hi * 4) = bf16x4{b0[0], b0[1], b1[0], b1[1]};
        }
    }
}

template <int HD>
__global__ __launch_bounds__(256, 1) void dq_kernel(DqParams p) {
    constexpr int BN = 64, WQ = 32, BM = 128;
    constexpr int NS = HD / 16, NDB = HD / 32;
    constexpr int TILE = BN * HD * 2;
    __shared__ __attribute__((aligned(16))) char smem[2][2][TILE];  // [buf][K / V]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
    const float lse2 = row_ok ? p.lse[(int64_t)(p.h0 + head) * p.lse_hs + myq] * kLog2e : INFINITY;
    const float dlt = row_ok ? p.delta[(int64_t)head * p.delta_hs + myq] : 0.f;

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

    Tile64<HD> tk, tv;
    if (ntiles > 0) {
        tk.load(kh, p.k_rs, p.nk, tid);
        tv.load(vh, p.v_rs, p.nk, tid);
        tk.store(smem[0][0], tid);
        tv.store(smem[0][1], tid);
    }
    __syncthreads();

    for (int j = 0; j < ntiles; ++j) {
        const int buf = j & 1;
        const bool more = j + 1 < ntiles;
        if (more) {
            const int64_t nb = (int64_t)(j + 1) * BN;
            tk.load(kh + nb * p.k_rs, p.k_rs, p.nk - nb, tid);
            tv.load(vh + nb * p.v_rs, p.v_rs, p.nk - nb, tid);
        }
        if (j < ntiles_w) {
            const char* Ks = smem[buf][0];
            const char* Vs = smem[buf][1];
            f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int st = 0; st < NS; ++st) {
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    bf16x8 ak = lds_read_b128(Ks, lds_off<HD>(b * 32 + l32, st * 16 + hi * 8));
                    s[b] = mfma32(ak, qf[st], s[b]);
                    bf16x8 av = lds_read_b128(Vs, lds_off<HD>(b * 32 + l32, st * 16 + hi * 8));
                    dp[b] = mfma32(av, df[st], dp[b]);
                }
            }
            const int64_t kb = (int64_t)j * BN;
            const bool need_mask = (kb + BN > p.nk) || (p.causal && p.k_pos0 + kb + BN - 1 > wq0);
            bf16x8 dsb[2][2];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    float dsv[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        float x = fast_exp2(s[b][r + u] * p.scale_log2 - lse2);
                        if (need_mask) {
                            const int64_t key = kb + b * 32 + ((r + u) >> 2) * 8 + hi * 4 + ((r + u) & 3);
                            const bool ok = key < p.nk && (!p.causal || p.k_pos0 + key <= myq);
                            x = ok ? x : 0.f;
                        }
                        dsv[u] = x * (dp[b][r + u] - dlt);
                    }
                    const bf16x2 d2 = to_bf16x2(dsv[0], dsv[1]);
                    dsb[b][r >> 3][r & 7] = d2[0];
                    dsb[b][r >> 3][(r & 7) + 1] = d2[1];
                }
            }
            // dQ^T += K^T dS^T over the tile's 64 keys
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int b = 0; b < 2; ++b) {
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        bf16x8 ak = lds_read_tr_operand<HD>(Ks, b * 32 + h2 * 16, db * 32, lane);
                        acc[db] = mfma32(ak, dsb[b][h2], acc[db]);
                    }
                }
            }
        }
        if (more) {
            tk.store(smem[buf ^ 1][0], tid);
            tv.store(smem[buf ^ 1][1], tid);
        }
        __syncthreads();
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
    if (p.nk <= 0 || p.nkv <= 0) return hipSuccess;
    const int64_t blocks = (p.nk + kDkdvBlockN - 1) / kDkdvBlockN * p.nkv;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (D == 128)
        hipLaunchKernelGGL(dkdv_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, st, p);
    else if (D == 64)
        hipLaunchKernelGGL(dkdv_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, st, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_dq(const DqParams& p, int D, hipStream_t st) {
    if (p.nq <= p.q_begin || p.nh <= 0) return hipSuccess;
    const int64_t qtb = p.q_begin / kDqBlockM;
    const int64_t blocks = ((p.nq + kDqBlockM - 1) / kDqBlockM - qtb) * p.nh;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (D == 128)
        hipLaunchKernelGGL(dq_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, st, p);
    else if (D == 64)
        hipLaunchKernelGGL(dq_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, st, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace hc
