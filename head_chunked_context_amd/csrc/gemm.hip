// gemm.hip - bf16 MFMA matrix products of the attention layer around the
// attention: the Q/K/V projections a head chunk recomputes, the chunk's
// share of the output projection, and their gradients (Road to 5 Million
// Tokens talk, the U-Pipe paragraph: a group of heads is recomputed, attended
// and its partial result stored, then the buffers are reused).
//
//   C[m][n] = sum_k A(m, k) B(n, k)        m < M, n < N, k < K, fp32 accumulate
//
// Operands are bf16 in "segmented" strided layouts, so one kernel reads the
// token-major activations ([S][dm]), the [out][in] weights and the head-major
// chunk buffers ([h][S][D], whose columns h * D + d jump by S * D at every D):
//   A_KC (k contiguous):  A(m, k) = a[(k / a_seg) a_segs + m a_rs + k % a_seg]
//   else (m contiguous):  A(m, k) = a[(m / a_seg) a_segs + k a_rs + m % a_seg]
// and the same for B with n in place of m.  Segments are multiples of 8, and
// of 64 for a k-contiguous operand.
//
// Workgroup = 4 waves on a 128 x 128 tile of C (2 x 2 waves of 64 x 64) or 8
// waves on a 256 x 256 one (2 x 4 waves of 128 x 64); K in steps of 64 staged
// through LDS (global -> registers -> LDS, double-buffered, one barrier per
// step).  A
// k-contiguous operand tile is [128][64] with rows padded by 8 bytes
// (conflict-free 8-byte reads); an m- or n-contiguous one
// is [64][128] with the XOR-swizzled rows of the attention kernels, read
// transposed by ds_read_b64_tr_b16.  Both reads deliver the 16 reduction
// indices of an MFMA step in the same order (k0 + 4c + 0..3, k0 + 8 + 4c +
// 0..3 for lane half c), so any pair of layouts multiplies consistently.
// Each wave computes C^T blocks (MFMA rows = n, columns = m): a lane then
// holds one row m of C with runs of 4 consecutive n, written as 8- or
// 16-byte stores.
//
// Outputs: bf16 (head-major scatter through the segmented C layout), fp32, or
// fp32 accumulated into C: the accumulators then start from C's values, so a
// reduction split over several launches (one head chunk each) adds its terms
// in the same order as a single launch, bit for bit.
// Split-K: blockIdx.z takes k in [z * k_split, (z + 1) * k_split) (k_split a
// multiple of 64) and writes
// fp32 partials at c + z * c_zs; gemm_reduce adds the slices in ascending z.
#include "device_common.h"
#include "kernels.h"

namespace hc {

namespace {

constexpr int GBK = 64;

// Tile configurations: a BM x BN tile of C per workgroup of WM x WN waves,
// each wave 32 MB x 32 NB.  The small one (4 waves, 64 x 64 per wave) serves
// narrow products; the large one (8 waves, 128 x 64 per wave) halves the
// operand traffic per product term where both dimensions allow it.
template <int BM_, int BN_, int WM_, int WN_>
struct GemmCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int THREADS = WM * WN * 64;
    static constexpr int MB = BM / WM / 32, NB = BN / WN / 32;
};
using GemmSmall = GemmCfg<128, 128, 2, 2>;
using GemmLarge = GemmCfg<256, 256, 2, 4>;
// bf16 per padded row of a k-contiguous tile: 136 bytes, so that the 32 rows
// one 8-byte read pass touches start 34 words apart, on 32 distinct even banks
// of the 64 (a 16-byte pad repeats the banks every 16 rows: 2-way conflicts)
constexpr int KC_PITCH = GBK + 4;

// 16 reduction indices of one MFMA step from a k-contiguous [rows][KC_PITCH]
// tile, row `row`, in the transposed-read order
__device__ __forceinline__ bf16x8 kc_frag(const char* tile, int row, int k0, int c) {
    const char* p = tile + row * (KC_PITCH * 2) + (k0 + 4 * c) * 2;
    const s16x4 a = *reinterpret_cast<const s16x4*>(p);
    const s16x4 b = *reinterpret_cast<const s16x4*>(p + 16);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ROWS x 64 operand tile (ROWS a multiple of 128) loaded by THREADS threads;
// an r-contiguous one sits in LDS as ROWS / 128 sub-tiles [64][128]
template <bool KC, int ROWS, int THREADS>
struct OperandTile {
    static constexpr int NCH = ROWS * GBK / 8 / THREADS;  // 16-byte chunks per thread
    static constexpr int KCH = GBK / 8;  // chunks per k-contiguous row
    static constexpr int RCH = ROWS / 8;  // chunks per r-contiguous row
    uint4 r[NCH];
    int64_t off[NCH];  // element offset of the thread's chunk i at the tile's first k
    int kk[NCH];       // its reduction index relative to the tile's first k
    bool row_ok[NCH];

    // The per-thread part of every address is worked out once: a thread's
    // chunks keep their rows, and a 64-wide k step never leaves a segment
    // (k-contiguous segments are multiples of 64), so a step only moves the
    // offsets by a wave-uniform amount.
    __device__ __forceinline__ void init(int64_t rs, int64_t seg, int64_t segs, int64_t r0,
                                         int64_t R, int tid) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int idx = tid + i * THREADS;
            if constexpr (KC) {
                const int64_t row = r0 + idx / KCH;
                kk[i] = (idx % KCH) * 8;
                row_ok[i] = row < R;
                off[i] = row * rs + kk[i];
            } else {
                const int64_t row = r0 + (idx % RCH) * 8;
                kk[i] = idx / RCH;
                row_ok[i] = row < R;
                off[i] = (row / seg) * segs + row % seg + kk[i] * rs;
            }
        }
    }
    // wave-uniform state: the current part's operand and where that part
    // ends, the offset of the current tile's first k in it, and
    // (k-contiguous) that k's position in its segment
    const uint16_t* base;
    int64_t k0, cur, kr, kend;
    int part;
    __device__ __forceinline__ void begin(const uint16_t* x, int64_t rs, int64_t seg, int64_t segs,
                                          int64_t k, int64_t part_end) {
        base = x;
        part = 0;
        kend = part_end;
        k0 = k;
        kr = KC ? k % seg : 0;
        cur = KC ? (k / seg) * segs + kr : k * rs;
    }
    __device__ __forceinline__ void advance(const GemmParams& p, bool is_a, int64_t rs,
                                            int64_t seg, int64_t segs) {
        k0 += GBK;
        if (k0 == kend && part + 1 < p.k_parts) {  // into the next part
            ++part;
            base = is_a ? p.a_at[part] : p.b_at[part];
            kend = p.k_at[part + 1];
            kr = 0;
            cur = 0;
            return;
        }
        if constexpr (KC) {
            kr += GBK;
            cur += GBK;
            if (kr == seg) {  // into the next segment
                kr = 0;
                cur += segs - seg;
            }
        } else {
            cur += GBK * rs;
        }
    }
    // the current tile into registers; zero outside [0, R) x [k0, K)
    __device__ __forceinline__ void load(int64_t K) {
        const uint16_t* b = base + cur;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            if (row_ok[i] && k0 + kk[i] < K) r[i] = *reinterpret_cast<const uint4*>(b + off[i]);
            else r[i] = make_uint4(0, 0, 0, 0);
        }
    }
    __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int idx = tid + i * THREADS;
            if constexpr (KC) {
                // 8-byte aligned rows: the chunk goes in two 8-byte halves
                const int o = (idx / KCH) * (KC_PITCH * 2) + (idx % KCH) * 16;
                const uint4 v = r[i];
                *reinterpret_cast<uint2*>(lds + o) = make_uint2(v.x, v.y);
                *reinterpret_cast<uint2*>(lds + o + 8) = make_uint2(v.z, v.w);
            } else {
                const int k = idx / RCH, row = (idx % RCH) * 8;
                *reinterpret_cast<uint4*>(lds + (row / 128) * (GBK * 128 * 2) + lds_off<128>(k, row % 128)) =
                    r[i];
            }
        }
    }
};

template <bool KC>
__device__ __forceinline__ bf16x8 frag(const char* tile, const OperandOffsets<128>& off,
                                       int blk32, int k0, int lane) {
    if constexpr (KC) return kc_frag(tile, blk32 * 32 + (lane & 31), k0, lane >> 5);
    else return lds_read_tr_at<128>(tile + (blk32 / 4) * (GBK * 128 * 2), off, k0, blk32 % 4);
}

}  // namespace

template <bool A_KC, bool B_KC, class CFG>
__global__ __launch_bounds__(CFG::THREADS) void gemm_kernel(GemmParams p) {
    constexpr int GBM = CFG::BM, GBN = CFG::BN, MB = CFG::MB, NB = CFG::NB, NT = CFG::THREADS;
    constexpr int TA = A_KC ? GBM * KC_PITCH * 2 : GBK * GBM * 2;
    constexpr int TB = B_KC ? GBN * KC_PITCH * 2 : GBK * GBN * 2;
    __shared__ __attribute__((aligned(1024))) char sa[2][TA];
    __shared__ __attribute__((aligned(1024))) char sb[2][TB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / CFG::WN, wn = wave % CFG::WN, hi = lane >> 5;
    // tile order: the workgroups of a row of C tiles (one m tile, every n
    // tile) are consecutive and, with workgroup b running on die b % 8, on one
    // die, so they share that die's L2 copy of their A tile
    const int64_t gy = (p.N + GBN - 1) / GBN, ntiles = (int64_t)gridDim.x;
    int64_t t = blockIdx.x;
    if (t < ntiles / 8 * 8) t = (t % 8) * (ntiles / 8) + t / 8;
    const int64_t m0 = (t / gy) * GBM, n0 = (t % gy) * GBN;
    const int64_t kb = p.k_split > 0 ? (int64_t)blockIdx.z * p.k_split : 0;
    int64_t ke = p.k_split > 0 ? kb + p.k_split : p.K;
    ke = ke < p.K ? ke : p.K;
    const int nkt = ke > kb ? (int)((ke - kb + GBK - 1) / GBK) : 0;

    OperandTile<A_KC, GBM, NT> ta;
    OperandTile<B_KC, GBN, NT> tb;
    // lane: row m of C; register group g4 of block nb: columns n .. n + 3
    char* cz = static_cast<char*>(p.c) +
               (int64_t)blockIdx.z * p.c_zs * (p.out_mode == kGemmBf16 ? 2 : 4);
    auto c_off = [&](int mb, int nb, int g4, int64_t* m, int64_t* n) {
        *m = m0 + wm * (32 * MB) + mb * 32 + (lane & 31);
        *n = n0 + wn * (32 * NB) + nb * 32 + g4 * 8 + hi * 4;
        return (*n / p.c_seg) * p.c_segs + *m * p.c_rs + *n % p.c_seg;
    };
    // accumulating products start from C itself, so a product whose reduction
    // is split over several launches adds in the same order as one launch
    f32x16 acc[NB][MB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            acc[nb][mb] = f32x16{};
            if (p.out_mode == kGemmF32Add) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    int64_t m, n;
                    const int64_t o = c_off(mb, nb, g4, &m, &n);
                    if (m < p.M && n < p.N) {
                        const f32x4 x = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(cz) + o);
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[nb][mb][g4 * 4 + e] = x[e];
                    }
                }
            }
        }

    const OperandOffsets<128> off(lane);
    ta.init(p.a_rs, p.a_seg, p.a_segs, m0, p.M, tid);
    tb.init(p.b_rs, p.b_seg, p.b_segs, n0, p.N, tid);
    if (p.k_parts > 1) {  // (no split: kb = 0)
        ta.begin(p.a_at[0], p.a_rs, p.a_seg, p.a_segs, 0, p.k_at[1]);
        tb.begin(p.b_at[0], p.b_rs, p.b_seg, p.b_segs, 0, p.k_at[1]);
    } else {
        ta.begin(p.a, p.a_rs, p.a_seg, p.a_segs, kb, ke);
        tb.begin(p.b, p.b_rs, p.b_seg, p.b_segs, kb, ke);
    }
    // k tiles: tile j is multiplied from LDS buffer j % 2 while tile j + 1
    // loads into registers, which go to the other buffer at the end of the step
    auto multiply = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < GBK / 16; ++ks) {
            bf16x8 bf[NB], af[MB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) bf[nb] = frag<B_KC>(sb[buf], off, wn * NB + nb, ks * 16, lane);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) af[mb] = frag<A_KC>(sa[buf], off, wm * MB + mb, ks * 16, lane);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = mfma32(bf[nb], af[mb], acc[nb][mb]);
        }
    };
    if (nkt > 0) {
        ta.load(ke);
        tb.load(ke);
        ta.store(sa[0], tid);
        tb.store(sb[0], tid);
    }
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nkt) {
            ta.advance(p, true, p.a_rs, p.a_seg, p.a_segs);
            tb.advance(p, false, p.b_rs, p.b_seg, p.b_segs);
            ta.load(ke);
            tb.load(ke);
        }
        multiply(buf);
        if (kt + 1 < nkt) {
            ta.store(sa[buf ^ 1], tid);
            tb.store(sb[buf ^ 1], tid);
        }
        __syncthreads();
    }

#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                int64_t m, n;
                const int64_t o = c_off(mb, nb, g4, &m, &n);
                if (m >= p.M || n >= p.N) continue;
                const f32x16& a = acc[nb][mb];
                if (p.out_mode == kGemmBf16) {
                    const bf16x2 lo = to_bf16x2(a[g4 * 4 + 0], a[g4 * 4 + 1]);
                    const bf16x2 hi2 = to_bf16x2(a[g4 * 4 + 2], a[g4 * 4 + 3]);
                    *reinterpret_cast<bf16x4*>(reinterpret_cast<uint16_t*>(cz) + o) =
                        bf16x4{lo[0], lo[1], hi2[0], hi2[1]};
                } else {
                    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(cz) + o) =
                        f32x4{a[g4 * 4 + 0], a[g4 * 4 + 1], a[g4 * 4 + 2], a[g4 * 4 + 3]};
                }
            }
        }
    }
}

// out[m][n] (+)= sum_{z ascending} part[z][m][n], 4 fp32 per thread
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmReduceParams p) {
    const int64_t cpr = p.N / 4;
    const int64_t total = p.M * cpr;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = idx / cpr, n = (idx % cpr) * 4;
        f32x4 s = *reinterpret_cast<const f32x4*>(p.part + m * p.N + n);
        for (int z = 1; z < p.splits; ++z) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(p.part + z * p.part_zs + m * p.N + n);
            s = f32x4{s[0] + x[0], s[1] + x[1], s[2] + x[2], s[3] + x[3]};
        }
        f32x4* dst = reinterpret_cast<f32x4*>(p.out + m * p.out_rs + n);
        if (p.add) {
            const f32x4 old = *dst;
            s = f32x4{old[0] + s[0], old[1] + s[1], old[2] + s[2], old[3] + s[3]};
        }
        *dst = s;
    }
}

hipError_t launch_gemm(const GemmParams& p, bool a_kc, bool b_kc, int splits, hipStream_t st) {
    if (p.M <= 0 || p.N <= 0) return hipSuccess;
    // 16-byte operand chunks never straddle a segment, the end of a k-contiguous
    // row or the end of an r-contiguous one
    if ((a_kc || b_kc) && p.K % 8 != 0) return hipErrorInvalidValue;
    // a 64-wide k step of a k-contiguous operand stays inside one segment
    if ((a_kc && p.a_seg % GBK != 0) || (b_kc && p.b_seg % GBK != 0)) return hipErrorInvalidValue;
    // reduction parts: ascending multiples of 64 from 0 to K, no split-K
    if (p.k_parts > 1) {
        if (p.k_parts > kGemmMaxParts || p.k_split != 0 || splits != 1 || p.k_at[0] != 0 ||
            p.k_at[p.k_parts] != p.K)
            return hipErrorInvalidValue;
        for (int i = 0; i < p.k_parts; ++i)
            if (p.k_at[i + 1] <= p.k_at[i] || p.k_at[i + 1] % GBK != 0 || !p.a_at[i] || !p.b_at[i])
                return hipErrorInvalidValue;
    }
    if (!a_kc && p.M % 8 != 0) return hipErrorInvalidValue;
    if (p.N % 8 != 0 || p.a_seg % 8 != 0 || p.b_seg % 8 != 0 || p.c_seg % 4 != 0 ||
        (p.k_split > 0 && p.k_split % GBK != 0) || splits < 1 || splits > 65535)
        return hipErrorInvalidValue;
    // the large tiles where both dimensions fill them
    const bool large = p.M >= GemmLarge::BM && p.N >= GemmLarge::BN;
    const int64_t bm = large ? GemmLarge::BM : GemmSmall::BM, bn = large ? GemmLarge::BN : GemmSmall::BN;
    const int64_t gx = (p.M + bm - 1) / bm, gy = (p.N + bn - 1) / bn;
    if (gx * gy > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)(gx * gy), 1, (unsigned)splits);
#define HC_GEMM(AK, BK, CFG) \
    hipLaunchKernelGGL((gemm_kernel<AK, BK, CFG>), grid, dim3(CFG::THREADS), 0, st, p)
    if (large) {
        if (a_kc && b_kc) HC_GEMM(true, true, GemmLarge);
        else if (a_kc) HC_GEMM(true, false, GemmLarge);
        else if (b_kc) HC_GEMM(false, true, GemmLarge);
        else HC_GEMM(false, false, GemmLarge);
    } else {
        if (a_kc && b_kc) HC_GEMM(true, true, GemmSmall);
        else if (a_kc) HC_GEMM(true, false, GemmSmall);
        else if (b_kc) HC_GEMM(false, true, GemmSmall);
        else HC_GEMM(false, false, GemmSmall);
    }
#undef HC_GEMM
    return hipGetLastError();
}

hipError_t launch_gemm_reduce(const GemmReduceParams& p, hipStream_t st) {
    if (p.M <= 0 || p.N <= 0) return hipSuccess;
    if (p.N % 4 != 0 || p.splits < 1) return hipErrorInvalidValue;
    int64_t b = (p.M * (p.N / 4) + 255) / 256;
    b = b > 65536 ? 65536 : b;
    hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)b), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace hc
