/*
 * hcattn.h - C ABI of libhcattn.so: exact causal grouped-query attention,
 * forward and backward, on one AMD MI355X (gfx950), scheduled in query-head
 * chunks that reuse one workspace and, optionally, over key/value trunks that
 * can stream from pinned host memory and are merged by log-sum-exp.
 *
 * What is computed (per query head h, key/value head kv = h / (Hq / Hkv),
 * scale c = 1 / sqrt(D), query row i, visible keys J(i) = {0..i} when causal,
 * {0..S-1} otherwise):
 *     s_ij = c <q_i, k_j>,  LSE_i = log sum_{J(i)} exp(s_ij),
 *     O_i = sum_{J(i)} exp(s_ij - LSE_i) v_j
 * and the gradients of sum(O * dO) with respect to q, k, v.
 *   - A query attends to the keys that precede it or sit at its position:
 *     FPDT talk summary (MLSys 2025), "Technical Deep Dive", paragraph on the
 *     auto-regressive nature of LLMs.
 *   - Exact softmax attention computed block by block with running softmax
 *     statistics (the maximum logit and the sum): same section, the paragraph
 *     comparing trunk processing with online softmax and FlashAttention.
 *   - Query heads processed a group ("chunk") at a time through buffers that
 *     every chunk reuses: Road to 5 Million Tokens talk, the U-Pipe paragraph;
 *     the UPipe abstract (arXiv 2602.21196) for head-level chunking.
 *   - Key/value trunks, their host-memory offload and double-buffered
 *     prefetch on a separate copy stream: FPDT summary, "Key Findings" items
 *     1-3 and "Technical Deep Dive" (trunking, offloading, double buffer,
 *     three streams).
 *
 * Common arguments
 *   q, o, dout, dq : bf16 [S][Hq][D], token-major, contiguous, device memory.
 *   k, v, dk, dv   : bf16 [S][Hkv][D], token-major, contiguous.  Device
 *                    memory, or pinned host memory (hipHostMalloc / torch
 *                    pin_memory) when kv_trunk selects the trunked path.
 *   lse            : fp32 [Hq][S], device memory; natural-log LSE of the
 *                    scaled scores (output of attn_fwd, input of attn_bwd).
 *                    attn_fwd accepts NULL (forward-only use: no LSE kept).
 *   1 <= S <= 2^30 (longer: ATTN_EUNSUPPORTED); Hq, Hkv >= 1 with
 *   Hq % Hkv == 0; D == 64 or 128; S * (Hq + Hkv) * D * 64 <= 2^62 (larger
 *   shapes could wrap the 64-bit workspace sizes: ATTN_EUNSUPPORTED);
 *   causal 0 or 1 (1 is the measured case; 0 runs the same kernels).
 *   head_chunk     : query heads per chunk, 0 means Hq; 1..Hq.  Chunks are
 *                    consecutive ascending head ranges; the last may be short.
 *   kv_trunk       : 0, or >= S, for the untrunked path; otherwise the trunk
 *                    length in tokens, a positive multiple of 256.
 *   workspace      : device memory of at least attn_*_workspace_bytes(...)
 *                    bytes, 256-byte aligned; owned by the caller, fully
 *                    overwritten; its contents are undefined afterwards.
 *   stream         : a hipStream_t (NULL = the default stream).  All work is
 *                    ordered after prior work on it; later work on it sees the
 *                    outputs.  The call never synchronises the host.
 *
 * Ownership and concurrency
 *   The caller owns every buffer.  The library allocates no device memory; it
 *   creates one copy stream and a few events per device on first use and keeps
 *   them until unload.  No pointer is kept after a call returns.  Outputs must
 *   not alias inputs or the workspace.  Calls from several host threads on one
 *   device are serialised while they enqueue work.
 *
 * Graph capture
 *   attn_fwd and attn_bwd may be captured into a HIP graph on `stream`: the
 *   library's copy stream forks from and joins `stream` through events, and
 *   nothing else is enqueued (no memset nodes).  Make one ordinary call on the
 *   device first (it creates the copy stream and events), keep kernel timing
 *   off while capturing, and pass buffers that stay valid for every replay.
 *
 * Errors
 *   Every entry point returns ATTN_OK (0) or a negative status.  Argument
 *   checks run before anything is enqueued; on failure nothing is enqueued.
 *   ATTN_EHIP means a HIP call failed mid-call: outputs are undefined, the
 *   library stays usable.  attn_last_error() returns this thread's text for
 *   the last non-zero status.
 *
 * Determinism
 *   Results are bitwise reproducible run to run and bitwise identical for
 *   every head_chunk value (no atomics; fixed accumulation orders).  The
 *   backward result is also bitwise identical with and without kv_trunk for
 *   the same o and lse, and so is the forward (the softmax state is carried
 *   from trunk to trunk exactly); with attn_set_trunk_merge(1) the trunked
 *   forward agrees with the untrunked one to rounding (the log-sum-exp merge
 *   rounds).
 */
#ifndef HCATTN_H
#define HCATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_status {
    ATTN_OK = 0,
    ATTN_EINVAL = -1,       /* bad shape, flag or size                      */
    ATTN_EUNSUPPORTED = -2, /* valid but not built (e.g. D not 64/128)      */
    ATTN_EWORKSPACE = -3,   /* workspace NULL, misaligned or too small      */
    ATTN_EPOINTER = -4,     /* NULL, unregistered host or misplaced pointer */
    ATTN_EHIP = -5          /* a HIP runtime call failed                    */
};

/*
 * Bytes of device workspace attn_fwd needs for these arguments.  It grows
 * with head_chunk (the chunk's packed Q/K/V, or with kv_trunk the chunk's
 * query trunk, fp32 partials and the two-slot K/V ring), not with Hq.
 * Returns 0 when the arguments are invalid (attn_last_error says why).
 */
size_t attn_fwd_workspace_bytes(int64_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t causal,
                                int32_t head_chunk, int64_t kv_trunk);

/* Same for attn_bwd (chunk's packed Q, dO, K, V, the rows' Delta and scaled
 * LSE, fp32 dQ/dK/dV carries, and with kv_trunk the K/V ring and dK/dV
 * staging). 0 on invalid arguments. */
size_t attn_bwd_workspace_bytes(int64_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t causal,
                                int32_t head_chunk, int64_t kv_trunk);

/*
 * Picks kv_trunk for a device-memory budget, the way the FPDT summary sizes
 * trunks ("Technical Deep Dive" and the trunk-size Q&A: the copy of the next
 * trunk should take about as long as computing on the current one; longer
 * trunks then only cost memory).  Candidates are 256 * 2^k < S.  A candidate
 * qualifies when (a) the workspace of attn_fwd, and of attn_bwd if
 * with_backward, fits budget_bytes (0 = no limit); (b) if kv_on_host, copying
 * one trunk of the chunk's K and V heads over a link of link_bytes_per_s is
 * no slower than the forward's FLOPs on one query-trunk x key-trunk block at
 * flops_per_s; (c) one forward launch has at least four rounds of
 * workgroups on num_cus compute units.  The smallest qualifying candidate is written to
 * *kv_trunk; device-resident K/V whose untrunked workspaces fit get 0; if
 * none qualifies, the longest candidate that fits.  Rates and counts <= 0
 * take the values measured on one MI355X: 57e9 B/s pinned-host copies, 1e15
 * FLOP/s forward, 256 compute units.  Host-only arithmetic (no HIP call).
 * Returns ATTN_OK; ATTN_EINVAL / ATTN_EUNSUPPORTED for shapes attn_fwd would
 * reject (and host K/V with S <= 256); ATTN_EWORKSPACE when no candidate fits
 * the budget; ATTN_EPOINTER when kv_trunk is NULL.
 */
int attn_pick_kv_trunk(int64_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t causal,
                       int32_t head_chunk, int32_t kv_on_host, int32_t with_backward,
                       size_t budget_bytes, double link_bytes_per_s, double flops_per_s,
                       int32_t num_cus, int64_t* kv_trunk);

/*
 * Forward: writes o (bf16, round-to-nearest-even from fp32) and lse (unless
 * lse is NULL).  For each chunk the chunk's query heads and the key/value
 * heads they read are packed head-major into the workspace (the one-device
 * stand-in for the per-chunk all-to-all), then the flash kernel runs on them.
 * With kv_trunk, query trunk m attends to key/value trunks 0..m (0..N-1
 * non-causal), each copied into a ring slot on the copy stream while the
 * previous trunk computes; the query trunk's running softmax state (O, the
 * running maximum, row sums; fp32) passes from trunk to trunk through the
 * workspace, or, after attn_set_trunk_merge(1), each trunk's normalised
 * partial output is merged into the running one by log-sum-exp.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t S,
             int32_t Hq, int32_t Hkv, int32_t D, int32_t causal, int32_t head_chunk,
             int64_t kv_trunk, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward: given q, k, v, the forward's o and lse, and dout, writes dq, dk,
 * dv (bf16).  Delta = rowsum(dout * o) is computed first from the bf16 o; P is
 * recomputed from lse.  dK/dV of a key/value head accumulate over the heads of
 * its group in ascending order, then over query tiles in ascending order, in
 * fp32 (carried exactly in fp32 across chunks when a group spans chunks);
 * dQ accumulates over key tiles in ascending order (carried in fp32 across
 * trunks).  With kv_trunk the key/value trunks are the outer loop.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int64_t S, int32_t Hq, int32_t Hkv,
             int32_t D, int32_t causal, int32_t head_chunk, int64_t kv_trunk, void* workspace,
             size_t workspace_bytes, void* stream);

/*
 * attn_fwd without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  It allocates nothing (no hipMalloc, no library
 * allocation); the workspace is the library's built-in device array of
 * ATTN_NOALLOC_WORKSPACE_BYTES per GPU, held from the first use on a device
 * until the process ends.  Arguments, outputs and results are attn_fwd's, bit
 * for bit.  Returns ATTN_EWORKSPACE, before any work, when
 * attn_fwd_workspace_bytes(...) exceeds that size (a smaller head_chunk or a
 * kv_trunk brings any shape under it: the trunked forward's workspace does not
 * grow with S).  Every call on one GPU uses that GPU's one array: calls that
 * overlap on a device (several streams or host threads at once) race; order
 * them.
 */
#define ATTN_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int64_t S,
                     int32_t Hq, int32_t Hkv, int32_t D, int32_t causal, int32_t head_chunk,
                     int64_t kv_trunk, void* stream);

/*
 * The attention layer around the attention, walked a head chunk at a time the
 * way the U-Pipe paragraph of the Road to 5 Million Tokens talk describes it:
 * for each group of query heads the group's Q/K/V projections are
 * (re)computed into the reused chunk buffers, attention runs on them, and the
 * group's share of the output projection is added into the layer output.
 * Peak intermediate memory (the workspace) grows with head_chunk, not Hq.
 *   x        : bf16 [S][d_model], device memory.
 *   wq       : bf16 [Hq*D][d_model]; wk, wv: bf16 [Hkv*D][d_model];
 *   wo       : bf16 [d_model][Hq*D]  (weights as [out][in]: y = x W^T).
 *   y        : fp32 [S][d_model] = attention(x wq^T, x wk^T, x wv^T) wo^T,
 *              accumulated over chunks in fp32 (written, not added to).
 *   lse      : fp32 [Hq][S] or NULL, as attn_fwd.
 *   o_keep   : bf16 [Hq][S][D] (head-major) or NULL.  When given, receives
 *              the attention output before the output projection, for an
 *              attn_layer_bwd that then skips recomputing it (pass lse too).
 *              The caller owns it; it is an activation kept from forward to
 *              backward, outside the workspace.
 *   d_model a positive multiple of 64; other shape rules as attn_fwd; no
 *   key/value trunks; no bias or rotary embedding.
 * The chunk's projections are written head-major by the library's matrix
 * kernels and rounded to bf16 (so is the attention output before the output
 * projection).  Results are bitwise identical for every head_chunk: each fp32
 * sum into y continues from the stored partial in a fixed order.
 */
size_t attn_layer_fwd_workspace_bytes(int64_t S, int32_t d_model, int32_t Hq, int32_t Hkv,
                                      int32_t D, int32_t causal, int32_t head_chunk);
int attn_layer_fwd(const void* x, const void* wq, const void* wk, const void* wv, const void* wo,
                   float* y, float* lse, void* o_keep, int64_t S, int32_t d_model, int32_t Hq,
                   int32_t Hkv, int32_t D, int32_t causal, int32_t head_chunk, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * Backward of attn_layer_fwd for L = sum(y * dy): dy bf16 [S][d_model]; writes
 * fp32 dx [S][d_model], dwq [Hq*D][d_model], dwk, dwv [Hkv*D][d_model], dwo
 * [d_model][Hq*D].  Per chunk it recomputes the chunk's projections and
 * attention output (nothing of the forward is kept but x and the weights),
 * then dO_c = dy wo_c, dWo_c = dy^T O_c, the attention backward (attn_bwd's
 * kernels and accumulation orders), and per GQA group, ascending,
 * dx += dQ_g wq_g (+ dK wk + dV wv once the group's last head is done),
 * dwq = dQ^T x, dwk = dK^T x, dwv = dV^T x.  Bitwise identical for every
 * head_chunk.
 *   o_kept, lse_kept : both NULL (recompute), or the o_keep and lse a forward
 *              on the same x and weights (any head_chunk) wrote: the chunk's
 *              attention output is then read from them instead of being
 *              recomputed (the projections still are).  Results are bitwise
 *              identical either way.  One given without the other is
 *              ATTN_EINVAL.  The workspace is the same in both modes.
 */
size_t attn_layer_bwd_workspace_bytes(int64_t S, int32_t d_model, int32_t Hq, int32_t Hkv,
                                      int32_t D, int32_t causal, int32_t head_chunk);
int attn_layer_bwd(const void* x, const void* wq, const void* wk, const void* wv, const void* wo,
                   const void* dy, const void* o_kept, const float* lse_kept, float* dx, float* dwq,
                   float* dwk, float* dwv, float* dwo, int64_t S, int32_t d_model, int32_t Hq,
                   int32_t Hkv, int32_t D, int32_t causal, int32_t head_chunk, void* workspace,
                   size_t workspace_bytes, void* stream);

/* This thread's message for the last non-zero status ("" if none). */
const char* attn_last_error(void);

/*
 * Debug switch: on != 0 makes the copy stream the caller's stream, so trunk
 * copies and kernels run strictly in order (a race check: results must be
 * bitwise equal to the overlapped run).  Returns the previous setting.
 */
int attn_set_single_stream(int on);

/*
 * Schedule of the trunked forward.  on == 0 (the default): the flash kernel
 * carries the running softmax state across key/value trunks (result bitwise
 * equal to the untrunked forward; no merge pass).  on != 0: every trunk
 * yields a normalised fp32 partial output and its LSE, folded into the
 * running output by a log-sum-exp merge pass after each trunk, the order the
 * FPDT talk summary describes ("Technical Deep Dive": the softmax statistics
 * of a query trunk are updated until its final output).  Both need the same
 * workspace.  Process-wide; returns the previous setting.
 */
int attn_set_trunk_merge(int on);

/*
 * Schedule of the dK/dV pass.  Sequences of at least min_s tokens (default
 * 65536) take the group-loop schedule: one workgroup per (128-key tile, kv
 * head) walks the chunk's heads of that group and writes bf16 dK/dV itself
 * (no per-head fp32 partials in the workspace, no reduce pass; a group that
 * spans chunks carries its fp32 sums).  Shorter sequences
 * keep one workgroup per (key tile, query head) with per-head partials and
 * an ordered reduce, which spreads the causal triangle over more
 * workgroups.  Both are deterministic and bitwise identical across
 * head_chunk and kv_trunk at one S; they round differently from each other.
 * Affects attn_bwd, attn_layer_bwd and their workspace queries: change it
 * before querying sizes.  min_s <= 0 restores the default.  Process-wide;
 * returns the previous threshold.
 */
int64_t attn_set_group_loop_min_s(int64_t min_s);

/*
 * Kernel timing for measurement tools.  While enabled, every kernel the
 * library launches is bracketed by two HIP timing events recorded on the
 * stream it runs on (the caller's stream); attn_timing_read waits for those
 * events and returns, for the kernel family `name` ("fwd", "merge", "pack",
 * "prep", "dkdv", "reduce", "dq", "gemm"), the number of launches and their summed
 * duration in milliseconds since the last reset.  Events come from a pool the library
 * keeps until unload.  attn_timing_enable returns the previous setting;
 * attn_timing_read returns ATTN_OK or ATTN_EINVAL (unknown name) or ATTN_EHIP.
 */
int attn_timing_enable(int on);
int attn_timing_read(const char* name, int64_t* launches, double* total_ms);
void attn_timing_reset(void);

/*
 * Bytes moved (read + written) by the timed launches of one streaming-pass
 * family ("pack", "prep", "merge", "reduce") since the last reset, as their
 * parameters fix them: the algorithmic traffic, against which the timed
 * duration gives GB/s.  The MFMA families report 0.  Returns ATTN_OK,
 * ATTN_EINVAL (unknown name) or ATTN_EPOINTER (bytes NULL).
 */
int attn_timing_bytes(const char* name, double* bytes);

/* Library version, "major.minor.patch". */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* HCATTN_H */
