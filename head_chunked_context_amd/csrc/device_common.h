// device_common.h - gfx950 building blocks shared by the attention kernels.
//
// MFMA v_mfma_f32_32x32x16_bf16 (one wave64):
//   A operand, lane l: A[m = l % 32][k = (l / 32) * 8 + 0..7]  (8 bf16)
//   B operand, lane l: B[k = (l / 32) * 8 + 0..7][n = l % 32]  (8 bf16)
//   C/D, lane l, register r: C[m = (r / 4) * 8 + (l / 32) * 4 + r % 4][n = l % 32]
// ds_read_b64_tr_b16, within each group of 16 lanes: lane j points at 4
// consecutive bf16 X[j][0..3]; lane i receives X[4t + i / 4][i % 4], t = 0..3.
// Pointing lane j at tile[row0 + j / 4][col0 + 4 * (j % 4)] therefore gives
// lane i the column tile[row0 + 0..3][col0 + i]: a transposed operand read
// straight from a row-major tile.
//
// LDS tiles are row-major [rows][HD] bf16 with the 16-byte chunks of each row
// XOR-swizzled.  For HD = 128 (16 chunks per row) swz(row) = 4 * (row % 4) +
// (row / 4) % 4: 16 consecutive rows read at one chunk column land in 16
// different chunk slots (16-byte reads), and the 4 rows x 64 bytes that 32
// lanes touch in a transposed read land in 16 different slots; row-major
// 16-byte writes of whole rows are conflict-free too.  (Checked with the
// SQ_LDS_BANK_CONFLICT counter on gfx950: zero conflicts for all three
// patterns, where a row % 8 XOR conflicts on the transposed reads.)  HD = 64
// (8 chunks per row) uses 4 * (row % 2) + (row / 2) % 4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace hc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((address_space(3))) void lds_void;

template <int HD>
__device__ __forceinline__ int swz(int row) {
    if constexpr (HD == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return ((row & 1) << 2) | ((row >> 1) & 3);
}

// byte offset of element (row, col) in a swizzled [rows][HD] bf16 LDS tile
template <int HD>
__device__ __forceinline__ int lds_off(int row, int col) {
    return row * (HD * 2) + ((((col >> 3) ^ swz<HD>(row))) << 4) + ((col & 7) << 1);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const char* base, int off) {
    return *reinterpret_cast<const bf16x8*>(base + off);
}

__device__ __forceinline__ s16x4 lds_read_tr(const char* p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// Per-lane byte offsets of the MFMA operand reads in a [rows][HD] tile,
// computed once per kernel: row-major 16-byte reads of row (lane % 32) at
// reduction step st, and the two halves (rows +0..7 and +8..15) of the
// transposed read of d block db.  The swizzle depends on row % 16 only, so
// reads 16 * n rows further down are the same offsets plus n * 16 rows of
// bytes (an immediate), and the loops need no address arithmetic per tile.
template <int HD>
struct OperandOffsets {
    int row[HD / 16];
    int tr[HD / 32][2];
    __device__ __forceinline__ explicit OperandOffsets(int lane) {
        const int hi = lane >> 5, l32 = lane & 31;
#pragma unroll
        for (int st = 0; st < HD / 16; ++st) row[st] = lds_off<HD>(l32, st * 16 + hi * 8);
        const int j = lane & 15;
        const int r = ((lane >> 5) << 2) + (j >> 2);
        const int c = (((lane >> 4) & 1) << 4) + ((j & 3) << 2);
#pragma unroll
        for (int db = 0; db < HD / 32; ++db) {
            tr[db][0] = lds_off<HD>(r, db * 32 + c);
            tr[db][1] = lds_off<HD>(r + 8, db * 32 + c);
        }
    }
};

// Transposed A/B operand for the 16 reduction indices k0 + {c*4 + 0..3,
// 8 + c*4 + 0..3} (c = lane / 32, k0 a multiple of 16) of the 32 columns
// db*32 .. db*32+31 of a row-major tile (reduction index = tile row): lane l
// receives column db*32 + l % 32.
template <int HD>
__device__ __forceinline__ bf16x8 lds_read_tr_at(const char* tile, const OperandOffsets<HD>& off,
                                                 int k0, int db) {
    const s16x4 a = lds_read_tr(tile + off.tr[db][0] + k0 * HD * 2);
    const s16x4 b = lds_read_tr(tile + off.tr[db][1] + k0 * HD * 2);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// max / sum of x over lanes l and l ^ 32; the same bits land in both lanes
// (the sum always adds the lower lane's value first).
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x2 to_bf16x2(float a, float b) {
    f32x2 f = {a, b};
    return __builtin_convertvector(f, bf16x2);
}

// Wait until every vector-memory load of this wave has landed (including the
// direct global -> LDS loads below, which do not pass through registers).
__device__ __forceinline__ void wait_vm_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Direct global -> LDS loads (global_load_lds_dword[x4]): lane l's 4 / 16 bytes
// from `src` land at LDS byte lds_addr + 4 l / 16 l (M0 holds the wave-uniform
// base).  Issued as inline assembly on purpose: the compiler then does not
// treat them as pending LDS writes, and adds no vmcnt wait before the reads of
// the other buffer while the prefetch is in flight; the kernels order them
// with wait_vm_loads() and a barrier before the buffer is read.  M0 is written
// by these loads only (no other code in the kernels uses it).
// An empty use of registers loaded from global memory: the compiler places
// the wait for those loads here (before a loop) rather than at their first use
// inside the loop, where it would also wait for prefetches in flight.
// (The host pass of hipcc parses this too; the operand is a GPU register only
// in the device pass.)
template <class T>
__device__ __forceinline__ void settle(const T& x) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" :: "v"(x));
#else
    (void)x;
#endif
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)((const lds_void*)p);
}
// (lds_base must be the same in all lanes; readfirstlane makes it a scalar.)
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(m0) : "memory");
}
__device__ __forceinline__ void lds_dma4(const void* src, uint32_t lds_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :: "v"(src), "s"(m0) : "memory");
}

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N-1: fully unrolled, with i a
// compile-time constant in every call
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Wait until at most N vector-memory loads of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm_le() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Direct global -> LDS loads with a wave-uniform 64-bit global base, a
// per-lane byte offset and a wave-uniform LDS byte address: lane l writes its
// 16 / 4 bytes at lds + 16 l / 4 l.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(gbase), "s"(lds) : "memory");
}
__device__ __forceinline__ void dma4(const void* gbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :: "v"(voff), "s"(gbase), "s"(lds) : "memory");
}

// 64-row x HD-column bf16 tile loaded straight from global memory into the
// swizzled LDS layout with global_load_lds_dwordx4: lane l of a wave writes
// LDS bytes base + 16 l, so each lane fetches the global chunk that the
// swizzle maps there.  4 waves share the tile (16 rows each).  Rows at or past
// nvalid (>= 1) re-read row nvalid - 1: finite values that the kernels mask.
template <int HD>
__device__ __forceinline__ void direct_tile64(char* lds_tile, const uint16_t* base, int64_t rs,
                                              int64_t nvalid, int wave, int lane) {
    constexpr int ROWB = HD * 2;          // bytes per row
    constexpr int CPR = ROWB / 16;        // chunks per row
    constexpr int RPI = 1024 / ROWB;      // rows per wave instruction
    constexpr int NI = 64 / (4 * RPI);    // instructions per wave
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int blk = wave * NI + i;
        const int row = blk * RPI + lane / CPR;
        const int lc = (lane % CPR) ^ swz<HD>(row);
        const int64_t srow = row < nvalid ? row : nvalid - 1;
        lds_dma16(base + srow * rs + lc * 8, lds_addr(lds_tile + blk * 1024));
    }
}

// The same loads in the scalar-base form: a wave-uniform 64-bit global
// address in an SGPR pair plus a 32-bit per-lane byte offset (below 2^31
// here), so a load needs no per-lane 64-bit address arithmetic.  The base
// must be the same in every lane: readfirstlane keeps the first active
// lane's value.
__device__ __forceinline__ uint64_t uniform_addr(const void* p) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ void lds_dma16_sv(const void* sbase, uint32_t voff, uint32_t lds_base) {
    const uint64_t sb = uniform_addr(sbase);
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(sb), "s"(m0) : "memory");
}
__device__ __forceinline__ void lds_dma4_sv(const void* sbase, uint32_t voff, uint32_t lds_base) {
    const uint64_t sb = uniform_addr(sbase);
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :: "v"(voff), "s"(sb), "s"(m0) : "memory");
}

// 64-row tile loads with the per-lane part of the address worked out once.
// INTERLEAVED: wave w (of the 4 sharing a tile) issues its instruction i for
// the 1 KB block 4 i + w; with that assignment the swizzled chunk a lane
// fetches is the same for every i (for both HD = 128 and HD = 64), so one
// per-lane byte offset serves all i and instruction i only moves the
// wave-uniform base by 4 i blocks of rows.  Otherwise wave w takes the
// consecutive blocks NI w + i (each wave one contiguous run of rows, the order
// of direct_tile64) with one offset per instruction.  The LDS image is the one
// direct_tile64 writes.  Tiles with fewer than 64 valid rows, or strides too
// long for a 32-bit offset, take direct_tile64.
template <int HD, bool INTERLEAVED>
struct TileDma64 {
    static constexpr int ROWB = HD * 2, CPR = ROWB / 16, RPI = 1024 / ROWB, NI = 64 / (4 * RPI);
    static constexpr int NOFF = INTERLEAVED ? 1 : NI;
    static constexpr int64_t kMaxRs = (int64_t)1 << 24;  // 64 rows x rs x 2 B < 2^31
    uint32_t voff[NOFF];
    __device__ __forceinline__ TileDma64(int64_t rs, int wave, int lane) {
#pragma unroll
        for (int i = 0; i < NOFF; ++i) {
            const int blk = INTERLEAVED ? wave : wave * NI + i;
            const int row = blk * RPI + lane / CPR;
            const int lc = (lane % CPR) ^ swz<HD>(row);
            voff[i] = rs < kMaxRs ? (uint32_t)((row * rs + lc * 8) * 2) : 0u;
        }
    }
    __device__ __forceinline__ void load(char* lds_tile, const uint16_t* base, int64_t rs,
                                         int64_t nvalid, int wave, int lane) const {
        if (nvalid >= 64 && rs < kMaxRs) {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                if constexpr (INTERLEAVED)
                    lds_dma16_sv(base + (int64_t)i * 4 * RPI * rs, voff[0],
                                 lds_addr(lds_tile + (i * 4 + wave) * 1024));
                else
                    lds_dma16_sv(base, voff[i], lds_addr(lds_tile + (wave * NI + i) * 1024));
            }
        } else {
            direct_tile64<HD>(lds_tile, base, rs, nvalid, wave, lane);
        }
    }
};

// 64 consecutive fp32 (one per lane of one wave) straight into LDS; entries at
// or past nvalid (>= 1) repeat entry nvalid - 1.
__device__ __forceinline__ void direct_vec64(float* lds_vec, const float* src, int64_t nvalid, int lane) {
    if (nvalid >= 64) {
        lds_dma4_sv(src, (uint32_t)lane * 4u, lds_addr(lds_vec));
    } else {
        const int64_t i = lane < nvalid ? lane : nvalid - 1;
        lds_dma4(src + i, lds_addr(lds_vec));
    }
}

// 64-row x HD-column bf16 tile: global -> registers -> swizzled LDS, 256 threads.
template <int HD>
struct Tile64 {
    static constexpr int CPR = HD / 8;       // 16-byte chunks per row
    static constexpr int RPI = 256 / CPR;    // rows per pass
    static constexpr int NI = 64 / RPI;      // passes
    uint4 r[NI];

    // rows at or beyond nvalid read as zero
    __device__ __forceinline__ void load(const uint16_t* base, int64_t rs, int64_t nvalid, int tid) {
        const int c = tid % CPR, r0 = tid / CPR;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int row = r0 + i * RPI;
            if (row < nvalid)
                r[i] = *reinterpret_cast<const uint4*>(base + (int64_t)row * rs + c * 8);
            else
                r[i] = make_uint4(0, 0, 0, 0);
        }
    }
    __device__ __forceinline__ void store(char* lds, int tid) const {
        const int c = tid % CPR, r0 = tid / CPR;
#pragma unroll
        for (int i = 0; i < NI; ++i)
            *reinterpret_cast<uint4*>(lds + lds_off<HD>(r0 + i * RPI, c * 8)) = r[i];
    }
};

}  // namespace hc
