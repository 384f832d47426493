// kernels.h - launch parameters and host-side launchers of the gfx950 kernels.
//
// Every tensor is addressed as base + head * head_stride + row * row_stride +
// column, in elements, so one kernel reads the token-major user layout
// ([S][H][D]: row_stride = H*D, head_stride = D), the head-major chunk
// buffers ([H][S][D]: row_stride = D, head_stride = S*D) and trunk ring slots
// alike.  bf16 values travel as uint16_t bit patterns on the host side.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace hc {

// Forward flash kernel output modes.
enum FwdMode : int {
    kFwdFinal = 0,    // bf16 O (strided) + natural-log LSE, normalised
    kFwdPartial = 1,  // fp32 O normalised over this key range + LSE (-inf if empty)
};

struct FwdParams {
    const uint16_t* q;  int64_t q_rs, q_hs;   // nh query heads, nq rows
    const uint16_t* k;  int64_t k_rs, k_hs;   // key heads, nk rows
    const uint16_t* v;  int64_t v_rs, v_hs;
    void* o;            int64_t o_rs, o_hs;   // bf16 (final) or fp32 (partial)
    float* lse;         int64_t lse_hs;       // lse[head * lse_hs + row]
    int nh;             // query heads in this launch
    int group;          // query heads per key/value head
    int h0;             // global index of query head 0 of this launch
    int kv_base;        // global index of key/value head 0 of k/v
    int64_t nq, q_pos0; // query rows and the sequence position of row 0
    int64_t nk, k_pos0; // keys and the sequence position of key 0
    int causal;
    int mode;
    float scale_log2;   // softmax scale * log2(e)
    // Running state of the online softmax carried across key ranges (trunks):
    // with carry_in the kernel starts from the state in st_*, with carry_out
    // it stores its state there instead of an output (mode is then unused).
    // State per (head, row): unnormalised O [D] fp32 at st_o + head * st_o_hs
    // + row * D, the reference m (log2 units) at st_m[head * st_hs + row] and
    // the two lanes' partial sums at st_l[2 * (head * st_hs + row) + 0 / 1].
    int carry_in, carry_out;
    float* st_o; int64_t st_o_hs;
    float* st_m; float* st_l; int64_t st_hs;
};

// Copy nh heads x rows x D bf16 between strided layouts (16-byte vectors).
struct PackParams {
    const uint16_t* src; int64_t s_rs, s_hs;
    uint16_t* dst;       int64_t d_rs, d_hs;
    int nh;
    int64_t rows;
    int D;
};

// Log-sum-exp merge of a trunk partial (o_t, l_t) into the running (o_r, l_r).
// final != 0 writes bf16 O into out (strided) and natural LSE into lse_out.
struct MergeParams {
    float* o_r; float* l_r;              // [nh][rows][D], [nh][rows]
    const float* o_t; const float* l_t;  // same shapes
    int nh;
    int64_t rows;
    int D;
    int final_out;
    uint16_t* out; int64_t out_rs, out_hs;
    float* lse_out; int64_t lse_hs;
};

// Backward preprocessing: Delta[h][i] = sum_d dO[i,h,d] * O[i,h,d] (fp32,
// fixed order) and the packed copy of dO.
// Backward preprocessing of a chunk: packs dO head-major and writes, per
// (head, row), the two row statistics the backward kernels read, in the form
// they use them: ndelta = -rowsum(dO * O) and nlse2 = -LSE * log2(e).
struct PrepParams {
    const uint16_t* o;  int64_t o_rs, o_hs;
    const uint16_t* dO; int64_t do_rs, do_hs;
    const float* lse;   int64_t lse_hs;      // the chunk's heads, natural log
    uint16_t* dO_c;     int64_t c_rs, c_hs;
    float* ndelta;      int64_t ndelta_hs;
    float* nlse2;       int64_t nlse2_hs;
    int nh;
    int64_t rows;
    int D;
};

// dK/dV of one chunk over a key range, in one of two schedules:
//  * per head (group_loop = 0): one workgroup per (key tile of 128 keys,
//    query head of the chunk).  Each head's contribution over its query
//    tiles (ascending) is written in fp32, unscaled, to part_k/part_v
//    [nh][nk][D]; dkdv_reduce then adds the heads of each group in ascending
//    order.  Rows of part_* are keys of this launch (0..nk).
//  * group loop (group_loop = 1): one workgroup per (key tile, kv head of the
//    chunk) walks the chunk's heads of that group, ascending, each over its
//    query tiles, ascending, into the same fp32 registers.  A group that
//    continues in the next chunk leaves its fp32 sums in carry_out ([nk][D])
//    and resumes from carry_in; a finished group writes bf16(scale * dK) to
//    dk and bf16(dV) to dv (strides dk_rs, dk_hs), with no reduce pass.
struct DkdvParams {
    const uint16_t* q;  int64_t q_rs, q_hs;    // chunk query heads (local 0..nh)
    const uint16_t* dO; int64_t do_rs, do_hs;
    const float* nlse2;  int64_t nlse2_hs;     // -LSE * log2(e), [local head][row]
    const float* ndelta; int64_t ndelta_hs;    // -Delta, [local head][row]
    const uint16_t* k;  int64_t k_rs, k_hs;    // kv heads (local 0..nkv)
    const uint16_t* v;  int64_t v_rs, v_hs;
    int nh, group, h0, kv_base;
    int64_t nq;                                // query rows (positions 0..nq)
    int64_t nk, k_pos0;                        // keys of this launch, position of key 0
    int causal;
    float scale_log2;
    float* part_k; float* part_v;              // [nh][nk][D] fp32 (per-head schedule)
    // group-loop schedule
    int group_loop;
    int nkv;                                   // kv heads of the chunk
    const float* carry_in_k; const float* carry_in_v; int carry_kv_in;  // local kv head or -1
    float* carry_out_k; float* carry_out_v; int carry_kv_out;
    uint16_t* dk; uint16_t* dv; int64_t dk_rs, dk_hs;
    float scale;
};

// Ordered sum over a group's heads: for each kv head of the chunk and key,
//   acc = (carry_in or 0) + part[h_first] + part[h_first+1] + ...  (ascending)
// then either acc -> carry_out (fp32, group continues in the next chunk) or
// bf16(acc * scale) -> dk and bf16(acc) -> dv.  Carries are [nk][D] fp32 of
// one kv head: carry_kv_in / carry_kv_out name the local kv head (-1 none).
struct DkdvReduceParams {
    const float* part_k; const float* part_v;
    int nh, group, h0, kv_base, nkv;
    int64_t nk;
    int D;
    const float* carry_in_k; const float* carry_in_v; int carry_kv_in;
    float* carry_out_k; float* carry_out_v; int carry_kv_out;
    uint16_t* dk; uint16_t* dv; int64_t dk_rs, dk_hs;
    float scale;
};

// dQ of one chunk over a key range: one workgroup per (query tile, head).
struct DqParams {
    const uint16_t* q;  int64_t q_rs, q_hs;
    const uint16_t* dO; int64_t do_rs, do_hs;
    const float* nlse2;  int64_t nlse2_hs;     // -LSE * log2(e), [local head][row]
    const float* ndelta; int64_t ndelta_hs;    // -Delta, [local head][row]
    const uint16_t* k;  int64_t k_rs, k_hs;
    const uint16_t* v;  int64_t v_rs, v_hs;
    int nh, group, h0, kv_base;
    int64_t nq;                  // query rows (positions 0..nq)
    int64_t nk, k_pos0;          // keys of this launch
    int causal;
    float scale, scale_log2;
    const float* acc_in;  int64_t ain_rs, ain_hs;   // fp32 dQ carry in (null = 0)
    float* acc_out;       int64_t aout_rs, aout_hs; // fp32 carry out (null = final)
    uint16_t* dq;         int64_t dq_rs, dq_hs;     // final bf16 output
    int64_t q_begin;      // first query row processed (earlier rows untouched)
    int64_t final_before; // rows < final_before write bf16 dq, the rest fp32 acc_out
};

// Matrix product of the attention layer (gemm.hip):
//   C[m][n] = sum_k A(m, k) B(n, k),  fp32 accumulate over bf16 operands.
// A k-contiguous operand X(r, k) (r = m for A, n for B) sits at
//   x[(k / x_seg) * x_segs + r * x_rs + k % x_seg],
// an r-contiguous one at x[(r / x_seg) * x_segs + k * x_rs + r % x_seg]
// (which form is a launch argument); C(m, n) at
//   c[(n / c_seg) * c_segs + m * c_rs + n % c_seg]  (+ z * c_zs for split-K).
enum GemmOut : int {
    kGemmBf16 = 0,    // C = bf16(A B)
    kGemmF32 = 1,     // C = A B in fp32
    kGemmF32Add = 2,  // C = C + A B in fp32 (accumulators start from C)
};
// The reduction may also run over up to kGemmMaxParts parts (k_parts > 1,
// no split-K): part i covers k in [k_at[i], k_at[i + 1]) (boundaries
// multiples of 64, k_at[0] = 0, k_at[k_parts] = K) and reads A from a_at[i]
// and B from b_at[i] with the strides above, k counted from k_at[i]; one
// product then adds several operand pairs in order, as the same products
// launched one after another into an accumulating C would, bit for bit.
constexpr int kGemmMaxParts = 3;
struct GemmParams {
    const uint16_t* a; int64_t a_rs, a_seg, a_segs;
    const uint16_t* b; int64_t b_rs, b_seg, b_segs;
    int64_t M, N, K;
    void* c;           int64_t c_rs, c_seg, c_segs;
    int out_mode;
    int64_t k_split;   // reduction indices per split (multiple of 64); 0 = no split
    int64_t c_zs;      // elements between the splits' fp32 partial outputs
    int k_parts;       // 0 or 1: one part (a, b)
    int64_t k_at[kGemmMaxParts + 1];
    const uint16_t* a_at[kGemmMaxParts];
    const uint16_t* b_at[kGemmMaxParts];
};
// out[m][n] (+ out[m][n] if add) = sum over z ascending of part[z * part_zs + m * N + n]
struct GemmReduceParams {
    const float* part; int64_t part_zs;
    int splits;
    int64_t M, N;
    float* out; int64_t out_rs;
    int add;
};

hipError_t launch_fwd(const FwdParams& p, int D, hipStream_t st);
hipError_t launch_pack(const PackParams& p, hipStream_t st);
hipError_t launch_merge(const MergeParams& p, hipStream_t st);
hipError_t launch_prep(const PrepParams& p, hipStream_t st);
hipError_t launch_dkdv(const DkdvParams& p, int D, hipStream_t st);
hipError_t launch_dkdv_reduce(const DkdvReduceParams& p, hipStream_t st);
hipError_t launch_dq(const DqParams& p, int D, hipStream_t st);
hipError_t launch_gemm(const GemmParams& p, bool a_kc, bool b_kc, int splits, hipStream_t st);
hipError_t launch_gemm_reduce(const GemmReduceParams& p, hipStream_t st);

// Launch shapes.  The forward and dQ kernels take 256-row workgroups (8
// waves, one per compute unit) once a launch has at least kWideMinBlocks of
// them, else 128-row workgroups (4 waves, two per compute unit); the rows of
// each query are computed the same way in both, bit for bit.  dK/dV
// workgroups take 128 keys (4 waves, one per compute unit).
constexpr int kWideMinBlocks = 256;
constexpr int kDkdvBlockN = 128;

// The built-in workspace of attn_fwd_noalloc (scratch.hip): 64 MiB per device.
constexpr size_t kScratchBytes = (size_t)64 << 20;
// Device address of the current device's built-in workspace (looked up once
// per device with hipGetSymbolAddress, then cached).
hipError_t scratch_address(void** out);

}  // namespace hc
