// aux.hip - the HBM-bound passes around the flash kernels.
//
//  pack   : gathers a chunk's heads from the token-major user tensors into the
//           head-major chunk buffers (the one-device stand-in for the
//           per-chunk all-to-all that moves a chunk of heads; Road to 5
//           Million Tokens talk, U-Pipe paragraph; FPDT summary, "Technical
//           Deep Dive", the Ulysses all-to-all description).
//  merge  : folds a key-trunk partial into the running output by log-sum-exp,
//           the softmax-statistics update of the FPDT summary, "Technical
//           Deep Dive" (trunk paragraph).
//  prep   : backward preprocessing Delta = rowsum(dO * O) plus the packed dO.
// All are plain streaming kernels: 16-byte vector loads/stores, grid-stride
// loops over 64-bit indices.
#include "device_common.h"
#include "kernels.h"

namespace hc {

__global__ __launch_bounds__(256) void pack_kernel(PackParams p) {
    const int cpr = p.D / 8;
    const int64_t total = (int64_t)p.nh * p.rows * cpr;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(idx % cpr);
        const int64_t rh = idx / cpr;
        const int64_t row = rh % p.rows;
        const int64_t h = rh / p.rows;
        const uint4 x = *reinterpret_cast<const uint4*>(p.src + h * p.s_hs + row * p.s_rs + c * 8);
        *reinterpret_cast<uint4*>(p.dst + h * p.d_hs + row * p.d_rs + c * 8) = x;
    }
}

// One thread per 4 consecutive fp32 of a row.
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
    const int cpr = p.D / 4;
    const int64_t total = (int64_t)p.nh * p.rows * cpr;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(idx % cpr);
        const int64_t hr = idx / cpr;  // h * rows + row
        const int64_t row = hr % p.rows, h = hr / p.rows;
        const float a = p.l_r[hr], b = p.l_t[hr];
        const float mx = fmaxf(a, b);
        float wa, wb, L;
        if (mx == -INFINITY) {
            wa = 0.f; wb = 0.f; L = -INFINITY;
        } else {
            // natural log-sum-exp of the two partial statistics
            const float ea = expf(a - mx), eb = expf(b - mx);
            L = mx + logf(ea + eb);
            wa = expf(a - L);
            wb = expf(b - L);
        }
        const f32x4 x = *reinterpret_cast<const f32x4*>(p.o_r + hr * p.D + c * 4);
        const f32x4 y = *reinterpret_cast<const f32x4*>(p.o_t + hr * p.D + c * 4);
        const f32x4 z = {wa * x[0] + wb * y[0], wa * x[1] + wb * y[1], wa * x[2] + wb * y[2],
                         wa * x[3] + wb * y[3]};
        if (p.final_out) {
            bf16x2 lo = to_bf16x2(z[0], z[1]), hi = to_bf16x2(z[2], z[3]);
            bf16x4 w = {lo[0], lo[1], hi[0], hi[1]};
            *reinterpret_cast<bf16x4*>(p.out + h * p.out_hs + row * p.out_rs + c * 4) = w;
            if (c == 0 && p.lse_out != nullptr) p.lse_out[h * p.lse_hs + row] = L;
        } else {
            *reinterpret_cast<f32x4*>(p.o_r + hr * p.D + c * 4) = z;
        }
    }
    // The running statistics l_r are rewritten by merge_stats_kernel, launched
    // after this one, so every thread here reads the old value.
}

__global__ __launch_bounds__(256) void merge_stats_kernel(MergeParams p) {
    const int64_t total = (int64_t)p.nh * p.rows;
    for (int64_t hr = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; hr < total;
         hr += (int64_t)gridDim.x * blockDim.x) {
        const float a = p.l_r[hr], b = p.l_t[hr];
        const float mx = fmaxf(a, b);
        p.l_r[hr] = mx == -INFINITY ? -INFINITY : mx + logf(expf(a - mx) + expf(b - mx));
    }
}

// 16 lanes per row of D = 128 (8 lanes for D = 64): each lane multiplies 8
// pairs in order, then a fixed xor-butterfly adds the lane partials, so Delta
// has one summation order whatever the launch shape.
// Grid: x over row blocks, y = head; D / 8 lanes per row, a fixed
// shuffle-tree row sum.
__global__ __launch_bounds__(256) void prep_kernel(PrepParams p) {
    const int lg = p.D == 128 ? 4 : 3;  // log2 of the lanes per row
    const int lpr = 1 << lg;
    const int sub = threadIdx.x & (lpr - 1);
    const int rpb = 256 >> lg;          // rows per block and pass
    const int64_t h = blockIdx.y;
    for (int64_t row = (int64_t)blockIdx.x * rpb + (threadIdx.x >> lg); row < p.rows;
         row += (int64_t)gridDim.x * rpb) {
        const uint4 ov = *reinterpret_cast<const uint4*>(p.o + h * p.o_hs + row * p.o_rs + sub * 8);
        const uint4 dv = *reinterpret_cast<const uint4*>(p.dO + h * p.do_hs + row * p.do_rs + sub * 8);
        *reinterpret_cast<uint4*>(p.dO_c + h * p.c_hs + row * p.c_rs + sub * 8) = dv;
        const bf16x8 ob = __builtin_bit_cast(bf16x8, ov);
        const bf16x8 db = __builtin_bit_cast(bf16x8, dv);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)db[e], (float)ob[e], acc);
        for (int off = lpr / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, lpr);
        if (sub == 0) {
            p.ndelta[h * p.ndelta_hs + row] = -acc;
            p.nlse2[h * p.nlse2_hs + row] = -(p.lse[h * p.lse_hs + row] * kLog2e);
        }
    }
}

static unsigned grid_for(int64_t work, int per_block) {
    int64_t b = (work + per_block - 1) / per_block;
    if (b > 65536) b = 65536;
    if (b < 1) b = 1;
    return (unsigned)b;
}

hipError_t launch_pack(const PackParams& p, hipStream_t st) {
    if (p.nh <= 0 || p.rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(pack_kernel, dim3(grid_for((int64_t)p.nh * p.rows * (p.D / 8), 256)),
                       dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, hipStream_t st) {
    if (p.nh <= 0 || p.rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(merge_kernel, dim3(grid_for((int64_t)p.nh * p.rows * (p.D / 4), 256)),
                       dim3(256), 0, st, p);
    if (!p.final_out)
        hipLaunchKernelGGL(merge_stats_kernel, dim3(grid_for((int64_t)p.nh * p.rows, 256)),
                           dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_prep(const PrepParams& p, hipStream_t st) {
    if (p.nh <= 0 || p.rows <= 0) return hipSuccess;
    if (p.nh > 65535 || (p.D != 128 && p.D != 64)) return hipErrorInvalidValue;
    const int64_t rpb = 256 / (p.D / 8);
    int64_t bx = (p.rows + rpb - 1) / rpb;
    const int64_t cap = (4096 + p.nh - 1) / p.nh;
    bx = bx > cap ? cap : bx;
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)bx, (unsigned)p.nh), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace hc
