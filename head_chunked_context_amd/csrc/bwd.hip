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
// dkdv_kernel: workgroup = 4 waves (one per SIMD) on 128 keys of one kv head;
// wave w owns keys 32 w .. 32 w + 31 for the whole kernel, with their K and V
// rows as MFMA operands in registers and their fp32 dK/dV sums in the
// accumulation registers.  Each step covers a 64-row query tile (two 32-row
// blocks b), whose Q and dO rows (plus the rows' statistics) are loaded
// straight into a 4-slot LDS ring three steps ahead:
//   S_b[q][key]   = Q_b K^T       A = Q rows (LDS),   B = K (registers)
//   dP_b[q][key]  = dO_b V^T      A = dO rows (LDS),  B = V (registers)
//   dV^T[d][key] += dO_b^T P_b    A = dO rows, transposed LDS reads
//   dK^T[d][key] += Q_b^T dS_b    A = Q rows, transposed LDS reads
// so each lane owns one key (lanes l and l^32 split the rows).  With one wave
// per SIMD nothing hides one wave's vector work under another's MFMAs, so
// each step is a fixed sequence of 64 MFMA groups (S/dP of block 0, S/dP of
// block 1, dV/dK of block 0, dV/dK of block 1) with the exponentials and
// products of one block spread over the MFMAs of the next phase, every
// operand read four MFMAs ahead, and the next step's loads and first operand
// reads in the last phase.  Per MFMA this reads 1 KB from LDS (2 KB for the
// S/dP MFMAs of the two-waves-per-SIMD layout with K/V in LDS).
//
// dq_kernel: workgroup = NW waves x 32 query rows of one head (NW = 8 with a
// 4-slot K/V ring and two tiles per barrier for large launches, NW = 4
// double-buffered otherwise, as in the forward); Q and dO stay in registers;
// 64-key tiles of K and V are loaded straight into LDS:
//   S^T = K Q^T,  dP^T = V dO^T,  dQ^T[d][q] += K^T dS^T (transposed K reads)
#include "device_common.h"
#include "kernels.h"

namespace hc {


// dK / dV accumulation with the accumulator held in the accumulation
// registers (AGPRs) for the whole kernel, while the score MFMAs keep theirs in
// ordinary VGPRs (the compiler, left to itself, shuttles the dK / dV sums
// between the two files around every MFMA).  The compiler does not know this
// instruction is an MFMA, so it supplies no wait states around it: the step
// loop that uses it has no other access to the accumulators, and
// agpr_settle() waits before anything after that loop reads or moves them.
__device__ __forceinline__ void mfma32_agpr(f32x16& c, bf16x8 a, bf16x8 b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// the same with its own wait states: two before it (for a vector write of an
// operand just before) and sixteen after it (for a read of the result, or a
// write of the accumulator, just after); for code in which the compiler may
// move the accumulators between registers around it
__device__ __forceinline__ void mfma32_agpr_padded(f32x16& c, bf16x8 a, bf16x8 b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(c) : "v"(a), "v"(b));
}
// 24 wait states after the last mfma32_agpr, ordered before any later use of
// the accumulators (each passes through an asm statement here)
template <int N>
__device__ __forceinline__ void agpr_settle(f32x16 (&x)[N], f32x16 (&y)[N]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(x[0]), "+a"(y[0]));
#pragma unroll
    for (int i = 1; i < N; ++i) asm volatile("" : "+a"(x[i]), "+a"(y[i]));
}

// LDS reads a dK/dV step issues per MFMA group x (PH MFMAs per phase, NG
// groups, operands read DIST groups ahead, P/dS pairs every GPP groups), in
// the order the group issues them: the operand of group x + DIST (one 16-byte
// read in the S / dP phases, two transposed reads in the dV / dK phases), the
// -Delta starting values (groups 0 and 1), -LSE log2(e) of a row quad, and
// at the end of the step the first operands of the next one.
template <int PH, int NG, int DIST, int GPP>
struct DkdvLdsOps {
    static constexpr int rd(int x) { return x + DIST < NG ? ((x + DIST) / PH < 2 ? 1 : 2) : 0; }
    static constexpr int init(int x) { return x < 2 ? 4 : 0; }
    static constexpr int lrd(int x) {
        int c = 0;
        for (int b = 0; b < 2; ++b)
            for (int g4 = 0; g4 < 4; ++g4) c += x == (b + 1) * PH + 2 * g4 * GPP - 4;
        return c;
    }
    static constexpr int nxt(int x) { return x + DIST >= NG ? 1 : 0; }
    static constexpr int all(int x) { return rd(x) + init(x) + lrd(x) + nxt(x); }
    // reads still allowed in flight at the top of group g once the operands
    // of MFMAs g and g + 1 have arrived: those issued after the operand of
    // g + 1 (read in group g + 1 - DIST, or last in that group of the step
    // before)
    static constexpr int pair_wait(int g) {
        const int src = g + 1 - DIST;
        int k = 0;
        if (src >= 0) {
            k = init(src) + lrd(src) + nxt(src);
            for (int x = src + 1; x < g; ++x) k += all(x);
        } else {
            for (int x = NG + src + 1; x < NG; ++x) k += all(x);
            for (int x = 0; x < g; ++x) k += all(x);
        }
        return k > 15 ? 15 : k;
    }
};

template <int HD, bool RUNS, bool GLOOP>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(DkdvParams p) {
    constexpr int BQ = 64, WK = 32, BNK = 128, NBUF = 4;
    constexpr int NS = HD / 16, NDB = HD / 32;
    constexpr int TILE = BQ * HD * 2;
    constexpr int NI = TileDma64<HD, false>::NI;  // tile loads per wave
    constexpr int PH = 2 * NS;        // MFMAs per phase
    constexpr int GPP = PH / 8;       // groups per pair of score elements
    constexpr int NG = 4 * PH;        // MFMA groups per step
    constexpr int DIST = 4;           // operand reads ahead (divides NG)
    // the step's barrier, and after it the loads of the step three ahead,
    // sit 3/8 of the way into the last phase (group 54 of 64 at D = 128):
    // late enough that the slowest wave rarely holds the others there, early
    // enough for the loads to be issued and the barrier to have published
    // the next step's tiles before its first operand reads
    constexpr int BAR_G = 3 * PH + 6 * PH / 16;
    static_assert(BAR_G + 2 * NI < NG && BAR_G <= NG - DIST, "barrier placement");
    __shared__ __attribute__((aligned(1024))) char smem[NBUF][2][TILE];  // [slot][Q / dO]
    __shared__ __attribute__((aligned(16))) float s_nlse2[NBUF][BQ];
    __shared__ __attribute__((aligned(16))) float s_ndelta[NBUF][BQ];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hi = lane >> 5, l32 = lane & 31;

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
    const int64_t j0 = kt * BNK;
    const int64_t wj0 = j0 + wave * WK;
    const int64_t myk = wj0 + l32;

    // K and V of this lane's key (the last key for lanes past it) as B operands
    bf16x8 kf[NS], vf[NS];
    {
        const int64_t kk = myk < p.nk ? myk : p.nk - 1;
        const uint16_t* kr = p.k + (int64_t)kvl * p.k_hs + kk * p.k_rs + hi * 8;
        const uint16_t* vr = p.v + (int64_t)kvl * p.v_hs + kk * p.v_rs + hi * 8;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            kf[st] = *reinterpret_cast<const bf16x8*>(kr + st * 16);
            vf[st] = *reinterpret_cast<const bf16x8*>(vr + st * 16);
        }
    }
    f32x16 dk[NDB], dv[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
    }
    if (GLOOP && kvl == p.carry_kv_in && myk < p.nk) {
        const float* ck = p.carry_in_k + myk * HD;
        const float* cv = p.carry_in_v + myk * HD;
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
    wait_vm_loads();
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        settle(kf[st]);
        settle(vf[st]);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        settle(dk[db]);
        settle(dv[db]);
    }

    const int64_t nqt = (p.nq + BQ - 1) / BQ;
    int64_t qt0 = 0;
    if (p.causal) {
        const int64_t first = p.k_pos0 + j0;
        qt0 = first >= p.nq ? nqt : first / BQ;
    }
    const int nsteps = j0 < p.nk ? (int)(nqt - qt0) : 0;
    const int total = nsteps * (he - hb);

    // Loads run three steps ahead into a 4-slot ring.  The issue cursor
    // (head ih, step is) keeps scalar pointers to the rows it loads next.
    const TileDma64<HD, false> dmq(p.q_rs, wave, lane), dmo(p.do_rs, wave, lane);
    int ih = hb;
    int is = 0;
    const uint16_t* iq = nullptr;
    const uint16_t* io = nullptr;
    const float* ist = nullptr;
    auto cursor_set = [&]() {
        const int64_t i0 = qt0 * BQ;
        iq = p.q + (int64_t)ih * p.q_hs + i0 * p.q_rs;
        io = p.dO + (int64_t)ih * p.do_hs + i0 * p.do_rs;
        ist = ((wave & 1) ? p.ndelta + (int64_t)ih * p.ndelta_hs : p.nlse2 + (int64_t)ih * p.nlse2_hs) + i0;
    };
    const int64_t q_step = BQ * p.q_rs, do_step = BQ * p.do_rs;
    auto cursor_next = [&]() {
        iq += q_step;
        io += do_step;
        ist += BQ;
        if (++is == nsteps) {
            is = 0;
            if (++ih < he) cursor_set();
        }
    };
    // LDS byte addresses of ring slot 0's tiles and statistics (wave-uniform)
    const uint32_t lds_t0 = __builtin_amdgcn_readfirstlane(lds_addr(&smem[0][0][0]));
    const uint32_t lds_l0 = __builtin_amdgcn_readfirstlane(lds_addr((wave & 1) ? &s_ndelta[0][0] : &s_nlse2[0][0]));
    const bool fast_rs = p.q_rs < TileDma64<HD, false>::kMaxRs && p.do_rs < TileDma64<HD, false>::kMaxRs;
    // query tiles (from qt0) with all 64 rows inside nq: the cursor's tile is
    // full while is < nfull
    const int nfull = (int)((p.nq - qt0 * BQ) / BQ);
    auto cursor_rows = [&]() { return p.nq - (qt0 + is) * BQ; };
    // load k of the cursor's step into ring slot b: k < NI: block k of the
    // wave's quarter of the Q tile; k < 2 NI: the same of the dO tile;
    // k = 2 NI: -LSE log2(e) (waves 0, 2) or -Delta (waves 1, 3; each vector
    // is written twice with the same values, so that every wave issues the
    // same number of loads).  A tile with fewer than 64 valid rows goes by
    // direct_tile64 (the same number of loads).
    auto issue_one = [&](auto kc, int b) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        if constexpr (k < 2 * NI) {
            constexpr int t = k / NI, i = k % NI;
            const uint16_t* src = t == 0 ? iq : io;
            if (is < nfull && fast_rs) {
                const uint32_t lds = lds_t0 + (uint32_t)b * (2 * TILE) + t * TILE + wave * (NI * 1024) + i * 1024;
                dma16(src, (t == 0 ? dmq : dmo).voff[i], lds);
            } else if constexpr (i == 0) {
                direct_tile64<HD>(smem[b][t], src, t == 0 ? p.q_rs : p.do_rs, cursor_rows(), wave, lane);
            }
        } else {
            if (is < nfull) dma4(ist, (uint32_t)lane * 4u, lds_l0 + (uint32_t)b * (BQ * 4));
            else direct_vec64((wave & 1) ? s_ndelta[b] : s_nlse2[b], ist, cursor_rows(), lane);
        }
    };
    // loads per wave and step
    constexpr int LT = 2 * TileDma64<HD, false>::NI + 1;
    // until the loads of one step have landed, with those of the step after
    // it still in flight when `more`
    auto wait_step = [&](bool more) {
        if (!more) wait_vm_le<0>();
        else wait_vm_le<LT>();
    };
    auto barrier = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    cursor_set();
    for (int i = 0; i < 3; ++i) {
        if (i < total) {
            static_for<2 * NI + 1>([&](auto kc) __attribute__((always_inline)) { issue_one(kc, i); });
            cursor_next();
        }
    }
    if (total > 2) {
        wait_vm_le<2 * LT>();
    } else {
        wait_step(total > 1);
    }
    barrier();

    const OperandOffsets<HD> off(lane);
    const int64_t wkpos = p.k_pos0 + wj0;
    const int krel = l32;
    const bool edge_k = wj0 + WK > p.nk;
    // query steps of each head that need the causal / ragged mask for this
    // wave: the first d_end (tiles starting before the wave's last key) and
    // the last one when its tile runs past nq; a wave with keys past nk masks
    // every step.  The steps in between see all of the wave's keys in all rows.
    int d_end = 0;
    if (p.causal) {
        const int64_t t = (wkpos + WK - 2 + BQ) / BQ - qt0;
        d_end = t < 0 ? 0 : (t > nsteps ? nsteps : (int)t);
    }
    const int u_end = nsteps - (((qt0 + nsteps) * BQ > p.nq) ? 1 : 0);

    // operand A of MFMA g of a step in ring slot `slot`: Q / dO rows of block
    // g / PH (S, dP phases) or their transposed 16-row slices (dV, dK phases)
    auto rd = [&](auto gc, int slot) __attribute__((always_inline)) -> bf16x8 {
        constexpr int g = decltype(gc)::value, ph = g / PH, idx = g % PH;
        const char* Qs = smem[slot][0];
        const char* Os = smem[slot][1];
        if constexpr (ph < 2)
            return lds_read_b128(idx < NS ? Qs : Os, off.row[idx % NS] + ph * 32 * HD * 2);
        else
            return lds_read_tr_at<HD>((idx & 1) ? Qs : Os, off, (ph - 2) * 32 + ((idx >> 1) & 1) * 16, idx >> 2);
    };
    bf16x8 ring[DIST];
    static_for<DIST>([&](auto gc) __attribute__((always_inline)) { ring[decltype(gc)::value] = rd(gc, 0); });

    // one step (ring slot n % 4): the MFMAs of the S and dP phases and of the
    // first dV / dK block with the vector work interleaved; then a barrier
    // (after waiting for the next step's loads), the second dV / dK block with
    // the loads of step n + 3 and the first operand reads of step n + 1
    // FAST: the loads of step n + 3 are due and take the fast form (a full
    // tile, row strides in range), so the step issues them unconditionally
    auto step = [&](auto mask_tag, auto fast_tag, int n, int s) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        constexpr bool FAST = decltype(fast_tag)::value;
        const int slot = (int)(n & (NBUF - 1));
        const int nslot = (slot + 1) & (NBUF - 1);
        const int lslot = (slot + 3) & (NBUF - 1);
        const bool load = n + 3 < total;
        // LDS addresses of the wave's part of the load slot's tiles and of
        // its statistics vector
        const uint32_t lds_lt = lds_t0 + (uint32_t)lslot * (2 * TILE) + wave * (NI * 1024);
        const uint32_t lds_ls = lds_l0 + (uint32_t)lslot * (BQ * 4);
        const int64_t i0 = (qt0 + s) * BQ;
        bool live = true;
        if constexpr (MASK) live = wj0 < p.nk && i0 < p.nq && (!p.causal || i0 + BQ - 1 >= wkpos);
        const float* sl = s_nlse2[slot];
        const float* sd = s_ndelta[slot];
        // rows relative to the wave's first key; keys past nk and rows past
        // nq are invisible; non-causal sees every row
        const int qrel0 = (int)(p.causal ? i0 - wkpos : WK + i0);
        const int qlim = (int)(p.causal ? p.nq - wkpos : WK + p.nq);
        const int kr = (myk < p.nk) ? krel : (1 << 30);
        f32x16 sacc[2], dpacc[2];
        bf16x8 pb[2][2], dsb[2][2];
        f32x4 L[2][4];
        float px[2][2];
        auto group = [&](auto gc) __attribute__((always_inline)) {
            constexpr int g = decltype(gc)::value, ph = g / PH, idx = g % PH;
            // one wait for the operands of two MFMAs (the compiler adds none
            // before the second)
            if constexpr (FAST && g % 2 == 0) {
                __builtin_amdgcn_s_waitcnt(0xC07F | (DkdvLdsOps<PH, NG, DIST, GPP>::pair_wait(g) << 8));
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (g == BAR_G) {
                if constexpr (FAST) wait_vm_le<LT>();
                else wait_step(n + 2 < total);
                barrier();
            }
            {
                const bf16x8 a = ring[g % DIST];
                if constexpr (g + DIST < NG) ring[g % DIST] = rd(std::integral_constant<int, g + DIST>{}, slot);
                // dP accumulators start at -Delta of their rows
                if constexpr (g < 2) {
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const f32x4 nd = *reinterpret_cast<const f32x4*>(sd + g * 32 + g4 * 8 + hi * 4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) dpacc[g][g4 * 4 + e] = nd[e];
                    }
                }
                // -LSE log2(e) of the rows of element quad g4, four groups
                // before the first exponential that needs it (so that the
                // paired operand waits cover it)
                static_for<2>([&](auto bc) __attribute__((always_inline)) {
                    constexpr int b = decltype(bc)::value, base = (b + 1) * PH;
                    static_for<4>([&](auto qc) __attribute__((always_inline)) {
                        constexpr int g4 = decltype(qc)::value;
                        if constexpr (g == base + 2 * g4 * GPP - 4)
                            L[b][g4] = *reinterpret_cast<const f32x4*>(sl + b * 32 + g4 * 8 + hi * 4);
                    });
                });
                if constexpr (ph < 2) {
                    constexpr int st = idx % NS;
                    if constexpr (idx < NS) sacc[ph] = mfma32(a, kf[st], st == 0 ? f32x16{} : sacc[ph]);
                    else dpacc[ph] = mfma32(a, vf[st], dpacc[ph]);
                } else {
                    constexpr int qb = ph - 2, db = idx >> 2, h2 = (idx >> 1) & 1;
                    if constexpr (MASK) {
                        if constexpr (idx & 1) mfma32_agpr_padded(dk[db], a, dsb[qb][h2]);
                        else mfma32_agpr_padded(dv[db], a, pb[qb][h2]);
                    } else {
                        if constexpr (idx & 1) mfma32_agpr(dk[db], a, dsb[qb][h2]);
                        else mfma32_agpr(dv[db], a, pb[qb][h2]);
                    }
                }
                // P and dS of score element pairs: pair j of block b takes its
                // exponentials at group base + j GPP and its products and
                // bf16 conversions one group later, so that no group waits on
                // a result of its own vector work.  Block b starts right after
                // its last dP MFMA, so its last conversion lands two groups or
                // more before the dV/dK MFMA that reads it (an inline MFMA
                // gets no wait states after a vector write of its operand)
                static_for<2>([&](auto bc) __attribute__((always_inline)) {
                    constexpr int b = decltype(bc)::value, base = (b + 1) * PH;
                    static_for<8>([&](auto jc) __attribute__((always_inline)) {
                        constexpr int j = decltype(jc)::value, r = 2 * j, g4 = r >> 2, e = r & 3;
                        if constexpr (g == base + j * GPP) {
                            float x0 = fast_exp2(__builtin_fmaf(sacc[b][r], p.scale_log2, L[b][g4][e]));
                            float x1 = fast_exp2(__builtin_fmaf(sacc[b][r + 1], p.scale_log2, L[b][g4][e + 1]));
                            if constexpr (MASK) {
                                const int qrel = qrel0 + b * 32 + g4 * 8 + hi * 4 + e;
                                x0 = (kr <= qrel && qrel < qlim) ? x0 : 0.f;
                                x1 = (kr <= qrel + 1 && qrel + 1 < qlim) ? x1 : 0.f;
                            }
                            px[j & 1][0] = x0;
                            px[j & 1][1] = x1;
                        }
                        if constexpr (g == base + j * GPP + 1) {
                            const float x0 = px[j & 1][0], x1 = px[j & 1][1];
                            const bf16x2 pk = to_bf16x2(x0, x1);
                            const bf16x2 d2 = to_bf16x2(x0 * dpacc[b][r], x1 * dpacc[b][r + 1]);
                            pb[b][r >> 3][r & 7] = pk[0];
                            pb[b][r >> 3][(r & 7) + 1] = pk[1];
                            dsb[b][r >> 3][r & 7] = d2[0];
                            dsb[b][r >> 3][(r & 7) + 1] = d2[1];
                        }
                    });
                });
            }
            // the loads of step n + 3, one per group from the barrier on
            if constexpr (g >= BAR_G && g <= BAR_G + 2 * NI) {
                constexpr int k = g - BAR_G;
                if constexpr (FAST) {
                    if constexpr (k < 2 * NI) {
                        constexpr int t = k / NI, i = k % NI;
                        dma16(t == 0 ? iq : io, (t == 0 ? dmq : dmo).voff[i], lds_lt + t * TILE + i * 1024);
                    } else {
                        dma4(ist, (uint32_t)lane * 4u, lds_ls);
                    }
                } else if (load) {
                    issue_one(std::integral_constant<int, k>{}, lslot);
                }
            }
            if constexpr (g == BAR_G + 2 * NI) {
                if (FAST || load) cursor_next();
            }
            // the first operands of step n + 1
            if constexpr (g + DIST >= NG) ring[g % DIST] = rd(std::integral_constant<int, g + DIST - NG>{}, nslot);
            __builtin_amdgcn_sched_barrier(0);
        };
        if constexpr (!MASK) {
            static_for<NG>(group);
        } else if (live) {
            static_for<NG>(group);
            agpr_settle(dk, dv);
        } else {
            // no row of the tile sees the wave's keys: only the barrier, the
            // loads of step n + 3 and the first operand reads of step n + 1
            wait_step(n + 2 < total);
            barrier();
            if (load) {
                static_for<2 * NI + 1>([&](auto kc) __attribute__((always_inline)) { issue_one(kc, lslot); });
                cursor_next();
            }
            static_for<DIST>([&](auto gc) __attribute__((always_inline)) {
                ring[decltype(gc)::value] = rd(gc, nslot);
            });
        }
    };

    int n = 0;
    for (int h = hb; h < he; ++h) {
        int s = 0;
        while (s < nsteps) {
            // a run of unmasked steps whose loads take the fast form: steps
            // that need no mask, while step n + 3 exists and the cursor's
            // tile is full (every tile of a head is when nfull == nsteps);
            // any other step goes by the masked body, which also handles the
            // general loads (its mask keeps every element of an unmasked step)
            int nf = 0;
            if (!edge_k && s >= d_end && s < u_end && fast_rs && is < nfull) {
                nf = u_end - s;
                if (total - 3 - n < nf) nf = total - 3 - n;
                if (nfull < nsteps && nfull - is < nf) nf = nfull - is;
            }
            if (nf <= 0) {
                step(std::integral_constant<bool, true>{}, std::integral_constant<bool, false>{}, n, s);
                ++s;
                ++n;
            } else {
                for (const int e = s + nf; s < e; ++s, ++n)
                    step(std::integral_constant<bool, false>{}, std::integral_constant<bool, true>{}, n, s);
                agpr_settle(dk, dv);
            }
        }
    }

    if (myk >= p.nk) return;
    if (GLOOP && kvl == p.carry_kv_out) {
        float* ck = p.carry_out_k + myk * HD;
        float* cv = p.carry_out_v + myk * HD;
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
    if constexpr (GLOOP) {
        uint16_t* ok = p.dk + (int64_t)kvl * p.dk_hs + myk * p.dk_rs;
        uint16_t* ov = p.dv + (int64_t)kvl * p.dk_hs + myk * p.dk_rs;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 x = {dk[db][g4 * 4], dk[db][g4 * 4 + 1], dk[db][g4 * 4 + 2], dk[db][g4 * 4 + 3]};
                const f32x4 y = {dv[db][g4 * 4], dv[db][g4 * 4 + 1], dv[db][g4 * 4 + 2], dv[db][g4 * 4 + 3]};
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
                // the S / dP products at a raised wave priority: the SIMD's
                // other wave, on its dS vector work or its dQ products, then
                // yields the issue slots to them, so the two waves drift apart
                // in phase instead of reaching their vector work together
                __builtin_amdgcn_s_setprio(1);
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
                __builtin_amdgcn_s_setprio(0);
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
    // a workgroup counts its steps (query tiles x heads of its group) in 32 bits
    if ((p.nq + 63) / 64 * (p.group_loop ? p.group : 1) > 0x7fffffffLL) return hipErrorInvalidValue;
    // die-aware runs of work items unless the unit count is a multiple of 4
    const bool runs = units % 4 != 0;
    const dim3 grid((unsigned)blocks), block(256);
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
