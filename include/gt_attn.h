/* gt_attn.h — C ABI of the biased full-graph attention library (libgt_attn.so), gfx950.
 *
 * Method (MegaGraph pages, abstract: every Graph-Transformer layer forms an
 * attention score matrix together with a topology-aware bias matrix; Fig. 4
 * caption: the bias is processed column-block by column-block, each slice
 * matched to the key/value block it is used with). Read here as
 *
 *     B[h,i,j] = table[h, code(i,j)]            code = clipped hop distance (gt_spd_build)
 *     S[h,i,j] = <q[i,h,:], k[j,h,:]> / sqrt(D) + B[h,i,j]
 *     out[i,h,:] = sum_j softmax_j(S[h,i,:]) v[j,h,:],   lse[i,h] = log sum_j exp S[h,i,j]
 *
 * over all N x N node pairs (no mask; unreachable pairs use their own bucket).
 * Neither S nor B is ever stored: kernels rebuild each bias tile from the
 * uint8 code tile and a copy of the table held on chip.
 *
 * Conventions shared by every entry point
 *   - Layouts (row-major, node-major):
 *       q, k, v, out, dout, dq, dk, dv   [N, H, D]   (= [N, H*D], hidden index h*D + d)
 *       lse                              [N, H]      float32, natural log
 *       spd                              [N, N]      uint8, row = query node i, column = key node j
 *       table, dtable                    [H, NB]     float32
 *   - dtype selects the storage type of the inputs q, k, v and dout: GT_F32
 *     (float) or GT_BF16 (bfloat16 bits). Every output (out, lse, dq, dk, dv,
 *     dtable) is float32, so a bfloat16 caller loses nothing to output
 *     rounding; table is float32. Accumulation is float32 everywhere.
 *   - Operand precision. GT_F32 inputs, and shapes without a matrix-core
 *     kernel, compute every product in float32. The matrix-core paths (GT_BF16
 *     with H = 8 and D in {8, 32}) differ in two ways:
 *       * q, k, v and dout are converted to IEEE half precision for the
 *         backward's score products and for P.V (exact for bfloat16 values
 *         with 2^-14 <= |x| < 65504; smaller values become half subnormals,
 *         absolute error <= 2^-25, and 0 below 2^-25);
 *       * the softmax probabilities P and the score gradients
 *         dS = P * (dO.V - delta) enter the contractions over nodes (P.V,
 *         P^T dO, dS^T Q, dS K) as half (relative error 2^-11).
 *     Input range on those paths: |q|, |k|, |v|, |dout| < 65504, and
 *     |dS| < 65504, which |dout| * |v| * 2 * D < 65504 guarantees (|P| <= 1,
 *     |delta| <= max_j |dout_i . v_j|). Outside it the half values overflow
 *     to infinity and the affected outputs are not finite (never silently
 *     finite and wrong). A caller whose data may exceed these limits passes
 *     float32 inputs, which take the float32 kernels.
 *   - Pointers marked "device" are device memory owned by the caller; the
 *     library never allocates or frees device memory, and keeps no state
 *     between calls. Every base pointer must be 16-byte aligned.
 *   - Graph capture: every device entry point except gt_spd_build_device only
 *     enqueues kernels on `stream` (no allocation, memset, copy or
 *     synchronisation), so calls may be captured into a HIP graph and replayed;
 *     every kernel is deterministic, so a replay reproduces the eager call bit
 *     for bit. gt_spd_build_device copies host arrays and waits for the copies.
 *   - A code >= NB in spd is a caller error; kernels clamp it to NB-1.
 *   - Device calls are asynchronous on `stream` (a hipStream_t; NULL = the
 *     null stream) and return once the kernels are enqueued. Device faults
 *     surface at the caller's next synchronisation.
 *   - Return value: GT_OK, or a negative gt_status. Argument errors are
 *     reported before anything is enqueued. gt_last_error() then returns a
 *     message for the calling thread.
 *   - No exception crosses this interface. All calls are re-entrant.
 *   - Supported shapes: 1 <= N < 2^31, 1 <= H <= 64, D in {8, 16, 32, 64},
 *     H*D <= 512, 2 <= NB <= 64, H*NB <= 4096. Other sizes return
 *     GT_EUNSUPPORTED (the bucket-gradient partial sums are kept per thread in
 *     on-chip memory, which bounds NB).
 */
#ifndef GT_ATTN_H
#define GT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GT_F32 = 0, GT_BF16 = 1 } gt_dtype;

typedef enum {
  GT_OK = 0,
  GT_EINVAL = -1,        /* null or misaligned pointer, size out of range, workspace too small */
  GT_EUNSUPPORTED = -2,  /* valid arguments the library has no kernel for (D, H*D, dtype) */
  GT_EHIP = -3           /* the HIP runtime refused a launch */
} gt_status;

/* Forward of one biased attention layer (abstract and Fig. 4 of the MegaGraph pages).
 *   q, k, v  device [N,H,D] dtype        spd    device [N,N] uint8
 *   table    device [H,NB] float32       out    device [N,H,D] float32 (overwritten)
 *   lse      device [N,H] float32 (overwritten; the backward needs it)            */
int gt_attn_fwd(const void* q, const void* k, const void* v, const uint8_t* spd,
                const float* table, float* out, float* lse, int64_t N, int32_t H,
                int32_t D, int32_t NB, int32_t dtype, void* stream);

/* Bytes of device workspace gt_attn_fwd_ws needs for these sizes (0 on invalid sizes, and
 * 0 when the call needs none). Graphs too small to fill the GPU by query rows alone
 * are split along the keys; the workspace holds the partial results, which a second
 * kernel merges by their log-sum-exp.                                              */
size_t gt_attn_fwd_workspace_bytes(int64_t N, int32_t H, int32_t D, int32_t NB, int32_t dtype);

/* gt_attn_fwd with a workspace, which lets small graphs split the key loop (same
 * results up to float32 rounding order). workspace: device, >= gt_attn_fwd_workspace_bytes
 * bytes, 256-byte aligned, contents ignored on entry (NULL allowed when that size is
 * 0); calls that share one workspace must be ordered on one stream.                */
int gt_attn_fwd_ws(const void* q, const void* k, const void* v, const uint8_t* spd,
                   const float* table, float* out, float* lse, void* workspace, size_t workspace_bytes,
                   int64_t N, int32_t H, int32_t D, int32_t NB, int32_t dtype, void* stream);

/* Bytes of device workspace gt_attn_bwd needs for these sizes (0 on invalid sizes). For
 * graphs too small to fill the GPU by nodes alone it includes room for partial
 * gradients of a backward split along its inner loop, summed in a fixed order.      */
size_t gt_attn_bwd_workspace_bytes(int64_t N, int32_t H, int32_t D, int32_t NB, int32_t dtype);

/* Backward of gt_attn_fwd for the loss sum(dout * out): recomputes the scores and the
 * softmax from q, k, spd, table and lse (the forward's outputs out and lse are inputs).
 *   spd_t                  device [N,N] uint8, the transpose of spd (the key-outer pass
 *                          walks code columns as rows). For an undirected graph spd is
 *                          symmetric and the caller passes spd itself.
 *   out                    device [N,H,D] float32, as written by gt_attn_fwd
 *   dout                   device [N,H,D] dtype
 *   dq, dk, dv             device [N,H,D] float32 (overwritten)
 *   dtable                 device [H,NB]  float32 (overwritten, not accumulated):
 *                          dtable[h,b] = sum over pairs (i,j) with code b of dS[h,i,j]
 *   workspace              device, >= gt_attn_bwd_workspace_bytes(...) bytes, 256-byte
 *                          aligned, contents ignored on entry; calls that share one
 *                          workspace must be ordered on one stream.
 * Results are bitwise reproducible run to run (no floating-point atomics).           */
int gt_attn_bwd(const void* q, const void* k, const void* v, const uint8_t* spd,
                const uint8_t* spd_t, const float* table, const float* out, const float* lse, const void* dout,
                float* dq, float* dk, float* dv, float* dtable, void* workspace,
                size_t workspace_bytes, int64_t N, int32_t H, int32_t D, int32_t NB,
                int32_t dtype, void* stream);

/* gt_attn_bwd without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, kernels and results as gt_attn_bwd, bit for bit; the
 * scratch memory is a fixed array of GT_BWD_STATIC_SCRATCH_BYTES in the library's
 * device image, one per GPU, held from the first call on that GPU until the process
 * ends. The call itself allocates nothing. The first call on each device looks up the
 * array's address (make it outside graph capture); later calls reuse it.
 *   Errors: as gt_attn_bwd; GT_EINVAL when the sizes need more scratch than the array
 *   holds (gt_attn_bwd_workspace_bytes > GT_BWD_STATIC_SCRATCH_BYTES: 128 MiB covers
 *   N = 32768 at H = 8 with D = 8 or 32), GT_EHIP when the address lookup fails.
 *   Every call on one GPU shares that GPU's array and leaves its contents behind
 *   (nothing in it needs clearing: the kernels write before they read). Calls that
 *   overlap on one GPU, on different streams or from different threads, race on it:
 *   order them on one stream.                                                      */
#define GT_BWD_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
int gt_attn_bwd_static(const void* q, const void* k, const void* v, const uint8_t* spd,
                       const uint8_t* spd_t, const float* table, const float* out, const float* lse,
                       const void* dout, float* dq, float* dk, float* dv, float* dtable, int64_t N,
                       int32_t H, int32_t D, int32_t NB, int32_t dtype, void* stream);

/* ---- Key-block steps (MegaGraph pages, Fig. 4 and its caption: under graph-aware
 * context parallelism each device keeps its query rows while key/value blocks travel
 * around a ring, and each arriving block is paired with the matching column slice of
 * the bias). One call covers one device's work for one arriving block; running the
 * blocks of a key partition in turn and merging reproduces gt_attn_fwd/gt_attn_bwd.
 * For a key block [c0, c1) of a graph with N nodes and query rows [r0, r1):
 *     q = q_all + r0*H*D, k = k_all + c0*H*D, v = v_all + c0*H*D,
 *     spd = spd_all + r0*N + c0, ld = N          (column slice, rows stay N apart)
 *     spd_t = spd_t_all + c0*N + r0, ld_t = N    (row slice of the transpose)
 * Code pointers may have any alignment (16-byte aligned rows with ld a multiple of 16
 * take whole-row vector loads). Other conventions as above, with Nq queries and Nk keys.
 * ------------------------------------------------------------------------------- */

/* Bytes of device workspace gt_attn_fwd_block needs (0 on invalid sizes). */
size_t gt_attn_fwd_block_workspace_bytes(int64_t Nq, int64_t Nk, int32_t H, int32_t D, int32_t NB,
                                         int32_t dtype);

/* Partial forward of Nq queries against Nk keys:
 *   q          device [Nq,H,D] dtype          k, v   device [Nk,H,D] dtype
 *   spd        device uint8, code of (query i, key j) at spd[i*ld + j], ld >= Nk
 *   out        device [Nq,H,D] float32        lse    device [Nq,H] float32:
 *              accumulate = 0: overwritten with attention restricted to these keys and
 *              its log-sum-exp; accumulate = 1: on entry the result over other keys,
 *              merged with this block's (as gt_attn_merge does, without a separate call).
 *   workspace  device, >= gt_attn_fwd_block_workspace_bytes(...) bytes, 256-byte
 *              aligned, contents ignored on entry.
 * Sizes: 1 <= Nq, Nk < 2^31; H, D, NB, dtype as for gt_attn_fwd.                     */
int gt_attn_fwd_block(const void* q, const void* k, const void* v, const uint8_t* spd, int64_t ld,
                      const float* table, float* out, float* lse, void* workspace, size_t workspace_bytes,
                      int64_t Nq, int64_t Nk, int32_t H, int32_t D, int32_t NB, int32_t dtype,
                      int32_t accumulate, void* stream);

/* Merge of two partial results over disjoint key sets (log-sum-exp rescaling):
 *   lse = log(exp(lse_a) + exp(lse_b)),
 *   out = exp(lse_a - lse) * out_a + exp(lse_b - lse) * out_b
 * out_*: device [Nq,H,D] float32, lse_*: device [Nq,H] float32. out/lse may be the same
 * buffers as out_a/lse_a (or out_b/lse_b), which makes it a running merge. A side with
 * lse = -inf contributes nothing. D in {8,16,32,64}, 1 <= H <= 64.                   */
int gt_attn_merge(const float* out_a, const float* lse_a, const float* out_b, const float* lse_b,
                  float* out, float* lse, int64_t Nq, int32_t H, int32_t D, void* stream);

/* Bytes of device workspace gt_attn_bwd_block needs (0 on invalid sizes). */
size_t gt_attn_bwd_block_workspace_bytes(int64_t Nq, int64_t Nk, int32_t H, int32_t D, int32_t NB,
                                         int32_t dtype);

/* Backward of one key block for the loss sum(dout * out), where out and lse are the
 * MERGED results over all keys (so the block's probabilities are the full softmax's):
 *   spd, ld        as in gt_attn_fwd_block; spd_t: code of (query i, key j) at
 *                  spd_t[j*ld_t + i], ld_t >= Nq
 *   out, lse       device [Nq,H,D], [Nq,H] float32: merged forward results
 *   dout           device [Nq,H,D] dtype
 *   dq             device [Nq,H,D] float32: this block's share of dQ
 *   dk, dv         device [Nk,H,D] float32: the block's keys' gradients from these queries
 *   dtable         device [H,NB] float32: this block's share of the bucket gradient
 *   accumulate     GT_ACC_* bits: a set bit adds that output into what the buffer
 *                  holds (summing blocks), a clear bit overwrites it. In a ring, dq
 *                  stays with its rank (add from the second block on) while dk, dv
 *                  travel with their block (add from the second rank on).
 *   workspace      device, >= gt_attn_bwd_block_workspace_bytes(Nq, Nk, ...), as for
 *                  gt_attn_bwd.                                                       */
enum { GT_ACC_DQ = 1, GT_ACC_DKV = 2, GT_ACC_DTABLE = 4, GT_ACC_ALL = 7 };
int gt_attn_bwd_block(const void* q, const void* k, const void* v, const uint8_t* spd, int64_t ld,
                      const uint8_t* spd_t, int64_t ld_t, const float* table, const float* out,
                      const float* lse, const void* dout, float* dq, float* dk, float* dv, float* dtable,
                      void* workspace, size_t workspace_bytes, int64_t Nq, int64_t Nk, int32_t H,
                      int32_t D, int32_t NB, int32_t dtype, int32_t accumulate, void* stream);

/* Clipped hop-distance codes on the host (the topology that "topology-aware" refers to).
 *   indptr   host int64 [N+1], indices host int32 [indptr[N]]: an undirected graph in
 *            CSR form (both directions stored; neighbour order is free).
 *   spd      host uint8 [N,N] (overwritten): spd[i,j] = min(dist(i,j), C-1) if j is
 *            reachable from i (dist(i,i) = 0), else C.
 *   nthreads host threads to use (<= 0: all hardware threads).
 * Synchronous. Errors: GT_EINVAL for C outside [1,254], a malformed CSR, or an
 * adjacency that is not symmetric.                                                    */
int gt_spd_build(const int64_t* indptr, const int32_t* indices, int64_t N, int32_t C,
                 uint8_t* spd, int32_t nthreads);

/* Bytes of device workspace gt_spd_build_device needs for a graph of N nodes and nnz
 * stored adjacency entries (0 on invalid sizes). */
size_t gt_spd_build_device_workspace_bytes(int64_t N, int64_t nnz, int32_t C);

/* The codes of gt_spd_build, computed on the GPU (same values, byte for byte).
 *   indptr, indices  host CSR as for gt_spd_build (validated on the host, then copied
 *                    into the workspace; the call waits for those copies, so the host
 *                    arrays may be reused on return)
 *   spd              device uint8 [N,N] (overwritten; any alignment)
 *   workspace        device, >= gt_spd_build_device_workspace_bytes(N, indptr[N], C)
 *                    bytes, 256-byte aligned, contents ignored on entry.
 * Breadth-first search from all sources at once, 64 per bitmask, one launch per level
 * (MegaGraph pages, abstract: the bias matrix is topology-aware, i.e. it comes from the
 * graph's structure; the distance reading is stated with gt_spd_build). Component labels for
 * the codes C-1 / C come from a union-find on the host. The search kernels are
 * enqueued on `stream` and run asynchronously. Errors: as gt_spd_build, plus GT_EHIP. */
int gt_spd_build_device(const int64_t* indptr, const int32_t* indices, int64_t N, int32_t C,
                        uint8_t* spd, void* workspace, size_t workspace_bytes, void* stream);

/* ---- Stacked layers (MegaGraph pages, Fig. 8 caption: the evaluated Graph
 * Transformer has 16 layers, 8 heads and hidden size 64). Only the attention layers
 * and their Q/K/V projections are modelled, with no residual, normalisation or
 * feed-forward block. Per layer l, with hid = H*D and store() the rounding of a
 * float32 value to the storage dtype (bfloat16: nearest even; float32: none):
 *     [Q|K|V]_l = store(X_l W_{l,t}), t = q, k, v          (gt_qkv_fwd)
 *     X_{l+1}   = store(attention_l(Q_l, K_l, V_l))         (gt_attn_fwd, own table)
 * ------------------------------------------------------------------------------- */

/* Q/K/V projection of one layer, float32 accumulation, result stored in dtype.
 *   x        device [N, hid] dtype
 *   w        device [3, hid, hid] dtype: w[t][a][b] multiplies x[:, a] into column b of q, k, v
 *   q, k, v  device [N, hid] dtype (overwritten); as attention inputs they are [N, H, D]
 * Sizes: 1 <= N < 2^31, hid a multiple of 8 in [8, 512]. Errors: GT_EINVAL.        */
int gt_qkv_fwd(const void* x, const void* w, void* q, void* k, void* v, int64_t N, int32_t hid,
               int32_t dtype, void* stream);

/* Bytes of device workspace gt_qkv_bwd needs (0 on invalid sizes). */
size_t gt_qkv_bwd_workspace_bytes(int64_t N, int32_t hid);

/* Backward of gt_qkv_fwd for float32 output gradients dq, dk, dv:
 *   dx = dq w_q^T + dk w_k^T + dv w_v^T     device [N, hid] float32 (overwritten)
 *   dw[t] = x^T d_t                         device [3, hid, hid] float32 (overwritten)
 * dw is summed over fixed 256-node chunks, then over the chunks in order, so it is
 * bitwise reproducible. workspace: device, >= gt_qkv_bwd_workspace_bytes, 256-byte
 * aligned, contents ignored on entry.                                              */
int gt_qkv_bwd(const void* x, const void* w, const float* dq, const float* dk, const float* dv,
               float* dx, float* dw, void* workspace, size_t workspace_bytes, int64_t N,
               int32_t hid, int32_t dtype, void* stream);

/* dst[i] = store(src[i]) for i < n: float32 -> dtype (bfloat16: round to nearest even,
 * inputs finite; float32: a copy). src and dst device, 16-byte aligned; n = 0 is a no-op. */
int gt_store(const float* src, void* dst, int64_t n, int32_t dtype, void* stream);

/* Bytes of device workspace gt_stack_fwd_bwd needs (0 on invalid sizes). It holds
 * every layer's Q, K, V, attention output and lse for the backward. */
size_t gt_stack_workspace_bytes(int64_t N, int32_t L, int32_t H, int32_t D, int32_t NB,
                                int32_t dtype);

/* Forward and backward of L stacked layers for the loss sum(dout * X_L):
 *   x0       device [N, hid] dtype                 w       device [L, 3, hid, hid] dtype
 *   tables   device [L, H, NB] float32             spd, spd_t as in gt_attn_bwd
 *   dout     device [N, hid] dtype (the gradient of X_L)
 *   x_last   device [N, hid] dtype (overwritten with X_L)
 *   dx0      device [N, hid] float32 (overwritten with the gradient of x0)
 *   dw       device [L, 3, hid, hid] float32, dtable device [L, H, NB] float32 (overwritten)
 * In the backward, layer l's attention takes store(dX_{l+1}) as its dout; dq, dk, dv,
 * dX and dW stay float32. workspace: device, >= gt_stack_workspace_bytes, 256-byte
 * aligned. Shapes as for gt_attn_fwd, 1 <= L <= 1024.                               */
int gt_stack_fwd_bwd(const void* x0, const void* w, const float* tables, const uint8_t* spd,
                     const uint8_t* spd_t, const void* dout, void* x_last, float* dx0, float* dw,
                     float* dtable, void* workspace, size_t workspace_bytes, int64_t N, int32_t L,
                     int32_t H, int32_t D, int32_t NB, int32_t dtype, void* stream);

/* ---- The full Graph-Transformer model (MegaGraph pages, Fig. 8 caption: 16 layers,
 * 8 heads, hidden and feed-forward dimension 64; abstract: attention with a
 * topology-aware bias plus a feed-forward block per layer). The pages do not give the
 * layer's wiring; it is read as the pre-norm Transformer layer:
 *     A  = LN(X; g1, b1)                 Q, K, V = store(A Wq), store(A Wk), store(A Wv)
 *     O  = attention(Q, K, V)            (gt_attn_fwd, the layer's own bias table)
 *     X1 = X + O Wo                      B = LN(X1; g2, b2)
 *     X2 = X1 + gelu(B W1 + c1) W2 + c2
 * LN over the hidden dimension (biased variance, eps 1e-5), gelu(x) = x Phi(x). The
 * residual stream X, the attention output and all parameters are float32; store() is
 * the attention's input type (dtype), which also carries the attention's output
 * gradient in the backward.
 * One layer's parameters are one float32 vector: g1[64], b1[64], Wq, Wk, Wv, Wo
 * [64][64], g2[64], b2[64], W1 [64][64], c1[64], W2 [64][64], c2[64], where W[a][b]
 * multiplies input column a into output column b.
 * ------------------------------------------------------------------------------- */

/* Floats in one layer's parameter vector for hidden size hid and feed-forward size ffn
 * (24960 for 64 and 64; 0 for sizes without kernels). */
int32_t gt_model_param_count(int32_t hid, int32_t ffn);

/* Bytes of device workspace gt_model_fwd_bwd needs (0 on invalid sizes). */
size_t gt_model_workspace_bytes(int64_t N, int32_t L, int32_t H, int32_t D, int32_t NB, int32_t dtype);

/* Forward of L layers and the backward of the loss sum(dout * X_L):
 *   x0       device [N, 64] float32          params  device [L, P] float32 (P above)
 *   tables   device [L, H, NB] float32       spd, spd_t as in gt_attn_bwd
 *   dout     device [N, 64] float32 (the gradient of X_L)
 *   x_last   device [N, 64] float32 (overwritten with X_L)
 *   dx0      device [N, 64] float32 (overwritten with the gradient of x0)
 *   dparams  device [L, P] float32, dtables device [L, H, NB] float32 (overwritten)
 *   workspace device, >= gt_model_workspace_bytes, 256-byte aligned; it holds each
 *            layer's saved forward values.
 * Shapes: H*D = 64 (8 heads of 8, or any H, D with H*D = 64), NB, N and dtype as for
 * gt_attn_fwd; 1 <= L <= 1024. Errors: GT_EINVAL, GT_EUNSUPPORTED (H*D != 64).
 * Weight gradients are summed over fixed 256-node chunks, then over the chunks in
 * order, so results are reproducible run to run.                                   */
int gt_model_fwd_bwd(const float* x0, const float* params, const float* tables, const uint8_t* spd,
                     const uint8_t* spd_t, const float* dout, float* x_last, float* dx0, float* dparams,
                     float* dtables, void* workspace, size_t workspace_bytes, int64_t N, int32_t L,
                     int32_t H, int32_t D, int32_t NB, int32_t dtype, void* stream);

/* Message describing the last failed call on this thread ("" if none). */
const char* gt_last_error(void);

/* Library version string. */
const char* gt_version(void);

/* Kernel timing for benchmarks and profiling. While tracing is on for the calling
 * thread, every kernel the library enqueues from that thread is bracketed by a pair
 * of HIP events recorded on the kernel's own stream. gt_trace_collect waits for
 * those events, writes per-kernel launch counts and total milliseconds into
 * counts[id] / total_ms[id] for id < n (ids below; n >= GT_KERNEL_COUNT covers
 * all), and clears the record. Tracing adds two event records per launch.
 * gt_trace_enable returns GT_OK; gt_trace_collect returns GT_OK, or GT_EHIP if
 * an event could not be created or read.                                          */
enum {
  GT_KERNEL_FWD = 0,        /* forward (scores, bias, online softmax, PV)          */
  GT_KERNEL_BWD_DELTA = 1,  /* backward: delta = rowsum(dout * out)                */
  GT_KERNEL_BWD_KV = 2,     /* backward: key-outer dK, dV and bucket partial sums  */
  GT_KERNEL_BWD_Q = 3,      /* backward: query-outer dQ                            */
  GT_KERNEL_BWD_DTABLE = 4, /* backward: reduction of bucket partials to dtable    */
  GT_KERNEL_QKV_FWD = 5,    /* gt_qkv_fwd                                          */
  GT_KERNEL_QKV_BWD_DX = 6, /* gt_qkv_bwd: dX                                      */
  GT_KERNEL_QKV_BWD_DW = 7, /* gt_qkv_bwd: dW partial sums and their reduction     */
  GT_KERNEL_STORE = 8,      /* gt_store                                            */
  GT_KERNEL_MERGE = 9,      /* gt_attn_merge                                       */
  GT_KERNEL_FWD_MERGE = 10,  /* forward: merge of split or running partial results */
  GT_KERNEL_BWD_FINISH = 11, /* backward after a split: partial sums and dtable     */
  GT_KERNEL_SPD = 12,        /* gt_spd_build_device: all of its kernels together    */
  GT_KERNEL_LAYER_FWD = 13,  /* gt_model_fwd_bwd: norm, projections, FFN forward    */
  GT_KERNEL_LAYER_BWD = 14,  /* gt_model_fwd_bwd: their backward (node gradients)   */
  GT_KERNEL_LAYER_WGRAD = 15,/* gt_model_fwd_bwd: parameter gradients              */
  GT_KERNEL_BWD_FUSED = 16, /* backward in one pass: dK, dV, dQ partials, buckets  */
  GT_KERNEL_COUNT = 17
};
int gt_trace_enable(int32_t on);
int gt_trace_collect(int32_t* counts, double* total_ms, int32_t n);
const char* gt_kernel_name(int32_t id);

/* Unit-throughput probe, used to state the measured peaks the attention kernels are
 * held against (the exp-throughput bound in particular). Launches `blocks` workgroups
 * of 256 threads on `stream`; each thread runs `iters` steps of 8 independent chains.
 *   kind 0: v_exp_f32 (hardware exp2)            ops = blocks*256*iters*8
 *   kind 1: fp32 fused multiply-add               ops = blocks*256*iters*8
 *   kind 2: one exp2 + four fma per chain step    ops = blocks*256*iters*8 exps
 *   kind 3: bf16 MFMA 32x32x8                     flops = blocks*4*iters*4*16384
 *   kind 4: bf16 MFMA 32x32x16                    flops = blocks*4*iters*4*32768
 * sink: device float [blocks*256] (overwritten with values that keep the work live).
 * The caller times the launch. Errors: GT_EINVAL for kind outside [0,4], blocks
 * outside [1, 1<<20], iters < 1 or a null sink.                                      */
int gt_probe_peak(int32_t kind, int32_t blocks, int32_t iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GT_ATTN_H */
