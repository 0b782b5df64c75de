/*
 * fm_attn.h — C ABI of libfmattn: exact scaled-dot-product attention under
 * structural masks in column-sparse form, forward and backward, on one
 * AMD Instinct MI355X (gfx950).
 *
 * Source of the operation. "FlashMask-3: ядро внимания с масками для GPU
 * Hopper и распределённого обучения" (iitog.ru):
 *   - predecessor paragraph: the mask is held column-sparse, as four bound
 *     vectors on the query axis per key column (O(n) memory, not O(n^2));
 *   - contributions paragraph and "Key facts": a rank holding several
 *     fragments of the context localizes the mask by clip / shift / max on
 *     the bound vectors, with no communication, and the result feeds the
 *     single-GPU kernel unchanged.
 * "FlashAttention-2 ... GPU work partitioning" (iplexlaw.co.kr), section
 * "Block processing keeps the global normalization": the tiled computation
 * is exact attention (only the floating-point order differs); section
 * "Three ways to raise GPU utilization": work is split over batch, heads and
 * sequence, and Q rows are split among the waves of a workgroup while K/V are
 * shared.
 *
 * The pages give no interface, no vector names and no formula; the reading
 * used throughout is:
 *   query row i is MASKED for key column j  iff
 *       lts[j] <= i < lte[j]   ("lower" interval)   or
 *       uts[j] <= i < ute[j]   ("upper" interval).
 *   Intervals are half open; start >= end is empty. Any int32 value is
 *   accepted (bounds are never validated: the predicate is defined for all).
 *   O_i = sum_j softmax_j(scale * q_i . k_j over unmasked j) v_j;
 *   LSE_i = ln sum_{j unmasked} exp(scale * q_i . k_j)  (natural log);
 *   a row with no unmasked key has O_i = 0, LSE_i = -inf and zero gradients.
 *
 * Conventions for every entry point
 *   - Pointers marked "device" are device memory on the current HIP device;
 *     "host" pointers are read before the call returns. The caller owns every
 *     buffer. The library never allocates device memory.
 *   - Every kernel is launched asynchronously on `stream` (NULL = the null
 *     stream); no call synchronises the host, except the three that say so
 *     (fm_bwd_workspace_size_ds, fm_bwd_dq_path, fm_profile_end).
 *   - A status other than FM_OK means nothing was launched, except
 *     FM_ERR_HIP, which reports a HIP error raised by a launch. The message
 *     of the last failure on the calling thread is fm_last_error().
 *   - Tensor layout: Q, O, dO, dQ are [B, Sq, H, D] and K, V, dK, dV are
 *     [B, Sk, H_kv, D], addressed by (b, s, h) element strides with the head
 *     dimension D contiguous. LSE is [B, H, Sq] float32, contiguous.
 *   - Grouped-query attention ("Современное состояние Flash Attention на
 *     ROCm", kripta.biz, ranking paragraph, names GQA as a feature of the
 *     FA2 Triton backend; the usual reading is taken): H_kv divides H, query
 *     head h uses K/V head h / (H / H_kv), and dK, dV of a K/V head are the
 *     sums over the query heads of its group. H_kv = H is plain multi-head
 *     attention, H_kv = 1 multi-query attention.
 *   - Mask vectors are int32 [Bm, Hm, Sk] with the key axis contiguous and
 *     element strides (stride_b, stride_h); Bm in {1, B}, Hm in {1, H}; a
 *     size of 1 broadcasts over batch / heads.
 */
#ifndef FM_ATTN_H
#define FM_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FM_OK = 0,
  FM_ERR_INVALID_ARGUMENT = 1,  /* null pointer, bad size, stride, alignment, chunk list */
  FM_ERR_UNSUPPORTED = 2,       /* valid but not implemented (e.g. head_dim 96) */
  FM_ERR_WORKSPACE = 3,         /* workspace pointer missing or too small */
  FM_ERR_HIP = 4                /* a kernel launch reported a HIP error */
} fm_status;

typedef enum {
  FM_BF16 = 0,   /* bfloat16 inputs and outputs */
  FM_FP32 = 1,   /* float32 inputs and outputs; rounded to bf16 on load for the
                    matrix products (fp32 accumulation, fp32 softmax state) */
  FM_FP8_E4M3 = 2 /* forward only (fm_attn_fwd_fp8): q, k, v as OCP E4M3 codes,
                    one byte each, with one descale factor per tensor; o is
                    bfloat16 */
} fm_dtype;

/* Tile classes of the classification pre-pass. */
typedef enum {
  FM_TILE_SKIP = 0,     /* every (row, key) pair of the tile is masked      */
  FM_TILE_PARTIAL = 1,  /* may hold masked and unmasked pairs: apply mask    */
  FM_TILE_FULL = 2      /* no pair of the tile is masked                     */
} fm_tile_class;

/* Column-sparse mask: four device int32 vectors [Bm][Hm][Sk].
 * The lower pair (lts, lte) may be both NULL: the lower interval is then
 * empty for every column. Likewise the upper pair (uts, ute). Exactly one
 * NULL pointer in a pair is an error. */
typedef struct {
  const int32_t* lts;
  const int32_t* lte;
  const int32_t* uts;
  const int32_t* ute;
  int32_t batch;      /* Bm: 1 or B */
  int32_t heads;      /* Hm: 1 or H */
  int64_t stride_b;   /* element stride between batch rows of each vector */
  int64_t stride_h;   /* element stride between head rows of each vector  */
} fm_mask;

/* Problem description. Strides are in elements (bytes for FP8 codes), ordered (b, s, h); the head
 * dimension is contiguous. dO, dQ share the strides of O, Q; dK, dV share
 * those of K, V. Every tensor base pointer must be 16-byte aligned and every
 * (b, s, h) row must start 16-byte aligned. */
typedef struct {
  int32_t batch;         /* B  >= 1 */
  int32_t heads;         /* H  >= 1 */
  int32_t seqlen_q;      /* Sq >= 1 */
  int32_t seqlen_k;      /* Sk >= 1 */
  int32_t head_dim;      /* D in {64, 128} */
  fm_dtype dtype;
  float softmax_scale;   /* > 0 and finite, e.g. 1/sqrt(D) */
  int64_t q_stride[3];
  int64_t k_stride[3];   /* of K and dK, whose head axis has H_kv entries */
  int64_t v_stride[3];   /* of V and dV */
  int64_t o_stride[3];
  int32_t heads_kv;      /* H_kv: 0 (meaning H) or a divisor of H */
} fm_problem;

/* Tile sizes (rows of Q, columns of K) used by the forward (bwd = 0) or the
 * backward (bwd = 1) kernel for a head dimension. Unsupported head_dim
 * yields 0, 0. */
void fm_kernel_tile(int32_t head_dim, int32_t bwd, int32_t* block_q, int32_t* block_k);

/* Bytes of device workspace fm_attn_fwd (with_bwd = 0) or fm_attn_bwd
 * (with_bwd = 1) needs at least: tile summaries and class maps; for a forward
 * launch with few query tiles and long key ranges, float32 partial O and LSE
 * of the parts its key-tile lists are cut into; for the backward the per-row
 * terms LSE * log2(e) and D = rowsum(dO * O), the stored-dS plan counters
 * and, for grouped-query attention with a mask shared by all heads, float32
 * dK / dV partials per query head (8 * B * H * Sk * D bytes). With this much,
 * fm_attn_bwd recomputes S and dP a second time for dQ. */
fm_status fm_workspace_size(const fm_problem* problem, const fm_mask* mask,
                            int32_t with_bwd, size_t* bytes);

/* Bytes of workspace with which fm_attn_bwd keeps dS instead of recomputing
 * it: the dK/dV kernel writes the bf16 dS tiles it forms anyway, and dQ is the
 * product scale * dS K over the stored tiles. That is fm_workspace_size(.., 1)
 * plus one slot index per tile of the dK/dV tiling, one count per 64 of its
 * tiles, and 2 bytes per (query row, key) pair of every non-SKIP tile, for
 * every (b, h) (rows and keys padded to the tile). The count depends on the mask contents, so the call classifies
 * the mask on `stream` using `workspace` (device, at least
 * fm_workspace_size(.., 1) bytes, 256-byte aligned; contents overwritten) and
 * waits for the stream. */
fm_status fm_bwd_workspace_size_ds(const fm_problem* problem, const fm_mask* mask,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream,
                                   size_t* bytes);

/* Tile classification pre-pass (reading adopted; the pages do not describe
 * one). For key tile kt (columns [kt*block_k, min((kt+1)*block_k, Sk)))
 * the summary holds, as 8 int32, min and max of lts, lte, uts, ute over the
 * tile's columns (missing pairs count as the empty intervals [Sq, Sq) and
 * [0, 0)), in the order
 *   min lts, max lts, min lte, max lte, min uts, max uts, min ute, max ute.
 * The class of the pair (qt, kt), rows [r0, r1) = [qt*block_q,
 * min((qt+1)*block_q, Sq)), is
 *   SKIP    if for lower or upper: max(start) <= r0 and min(end) >= r1;
 *   FULL    else if for both: max(end) <= r0 or min(start) >= r1;
 *   PARTIAL otherwise.
 * Outputs (device):
 *   summary  int32 [Bm][Hm][Tk][8]
 *   classes  uint8 [Bm][Hm][Tq][Tk] (transposed = 0) or [Bm][Hm][Tk][Tq]
 *            (transposed = 1), Tq = ceil(Sq/block_q), Tk = ceil(Sk/block_k).
 * block_q and block_k must be in [1, 1024]. */
fm_status fm_tile_classify(const fm_mask* mask, int32_t seqlen_q, int32_t seqlen_k,
                           int32_t block_q, int32_t block_k, int32_t transposed,
                           int32_t* summary, uint8_t* classes, hipStream_t stream);

/* Forward. Inputs q [B,Sq,H,D], k, v [B,Sk,H,D] (device, problem dtype).
 * Outputs o [B,Sq,H,D] (device, problem dtype) and lse [B,H,Sq] (device,
 * float32). Fully masked (SKIP) tiles are never touched; the mask is
 * evaluated only on PARTIAL tiles. workspace: device, at least
 * fm_workspace_size(.., 0) bytes, 256-byte aligned. Tiles are launched
 * longest first (by their number of non-SKIP partner tiles), here and in the
 * backward; the order does not change any result. When the launch has few
 * query tiles and long key ranges, each query tile's list is cut into parts
 * whose normalised partial results a second kernel merges (exact up to
 * rounding order; deterministic). */
fm_status fm_attn_fwd(const fm_problem* problem, const void* q, const void* k, const void* v,
                      const fm_mask* mask, void* o, float* lse,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The forward (fm_attn_fwd), allocating nothing and taking no workspace:
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). Inputs,
 * outputs, layout, results and errors are those of fm_attn_fwd (bf16 or
 * float32 problems). Its tile classes, launch order and split partials go to
 * a scratch array of 64 MiB that the library holds on each GPU it runs on
 * until the process ends; a problem whose forward workspace cannot fit there
 * (even with its key-tile lists left whole) fails with FM_ERR_WORKSPACE.
 * Every byte of scratch a kernel reads was written earlier in the same call,
 * so nothing has to start at zero. All calls on one GPU share its scratch:
 * calls that may overlap on one GPU (other streams, other threads) race and
 * must be serialised by the caller. `stream` must belong to the current
 * device. */
fm_status fm_attn_fwd_noalloc(const fm_problem* problem, const void* q, const void* k, const void* v,
                              const fm_mask* mask, void* o, float* lse, hipStream_t stream);

/* Forward on 8-bit floating-point inputs ("Современное состояние Flash
 * Attention на ROCm", kripta.biz, paragraphs on the attention variants and
 * their ranking: the fastest variant is the FP8 forward; the page names no
 * format or scaling, the readings here are this library's).
 * problem->dtype must be FM_FP8_E4M3 (head_dim 64 or 128). q [B,Sq,H,D],
 * k, v [B,Sk,H_kv,D]: device, OCP E4M3 codes (1 sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; no infinities; the NaN codes 0x7F and 0xFF give
 * NaN results), strides in bytes, rows 16-byte aligned. descale: host array
 * of 3 floats (q, k, v), each positive and finite; the operand is code value
 * times descale. Computes the masked attention of these operands, as
 * fm_attn_fwd does, with both products on the FP8 matrix cores (fp32
 * accumulation) and the probabilities rounded to E4M3 for the second product
 * (they are at most 2^8 there); softmax state, row sums and LSE in fp32.
 * Outputs: o [B,Sq,H,D] bfloat16 (o_stride in elements), lse [B,H,Sq]
 * float32. workspace: device, at least fm_workspace_size(.., 0) bytes for
 * this problem (it includes a V^T copy of B * H_kv * ceil(Sk/64) * 64 * D
 * bytes), 256-byte aligned. Errors as fm_attn_fwd. fm_attn_bwd and fm_workspace_size(.., 1) reject FP8 problems
 * with FM_ERR_UNSUPPORTED. */
fm_status fm_attn_fwd_fp8(const fm_problem* problem, const void* q, const void* k, const void* v,
                          const float* descale, const fm_mask* mask, void* o, float* lse,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward. Inputs q, k, v, o (the forward output), lse (the forward LSE),
 * dout (gradient of o), all device. Outputs dq, dk, dv (device, problem
 * dtype, shapes of q, k, v). workspace: device, at least
 * fm_workspace_size(.., 1) bytes, 256-byte aligned. dK/dV come from a
 * key-stationary kernel that recomputes the probabilities from lse. dQ comes
 * from stored dS tiles (dQ = scale * dS K) when the workspace is at least
 * fm_bwd_workspace_size_ds bytes, which is decided on the device from the
 * classified mask, else from a query-stationary kernel that recomputes S and
 * dP. No atomics; results are deterministic for a given workspace size. */
fm_status fm_attn_bwd(const fm_problem* problem, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dout, const fm_mask* mask,
                      void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Which dQ path the last fm_attn_bwd call with this problem, mask and
 * workspace took (pages silent; a query of this library's own choice
 * between the two exact dQ kernels above). *stored_ds receives 1 when dQ
 * came from the stored dS tiles and 0 when it was recomputed. A workspace
 * smaller than the slot map always gives 0 without touching the device;
 * otherwise the flag the plan kernel wrote into the workspace is copied to
 * the host after waiting for `stream`. Call it after fm_attn_bwd on the same
 * stream, before the workspace is reused. */
fm_status fm_bwd_dq_path(const fm_problem* problem, const fm_mask* mask, const void* workspace,
                         size_t workspace_bytes, hipStream_t stream, int32_t* stored_ds);

/* Mask localization for one context-parallel rank (FlashMask-3 page,
 * contributions paragraph: clip, shift, max on the bound vectors, no
 * communication). The rank holds num_chunks fragments of the global query
 * axis, chunk c covering global rows [chunk_start[c], chunk_start[c] +
 * chunk_len[c]); its local rows are these rows in the listed order.
 * Chunks (host arrays) must be listed in ascending order, must not overlap,
 * must have chunk_len >= 1 and must lie in [0, seqlen_q_global];
 * 1 <= num_chunks <= 64. Each global bound x becomes
 *   x' = max(0, max_c min(clamp(x, 0, Sq_glob) - start_c + off_c,
 *                         off_c + len_c)),   off_c = sum of len before c,
 * i.e. the number of local rows whose global index is below x, so that local
 * row r is masked for key j exactly when its global row is.
 * out[0..3] (device, int32 [Bm][Hm][seqlen_k] contiguous) receive the
 * localized lts, lte, uts, ute. A pair that is NULL in `global` is skipped
 * (its out pointers are ignored and may be NULL). Keys are not localized. */
fm_status fm_mask_localize(const fm_mask* global, int32_t seqlen_k, int32_t seqlen_q_global,
                           const int32_t* chunk_start, const int32_t* chunk_len,
                           int32_t num_chunks, int32_t* const out[4], hipStream_t stream);

/* Mask-pruned K/V transfer set of one context-parallel rank (FlashMask-3
 * page, contributions paragraph and "Key facts": the overlap of computation
 * with communication drops the transfers that the mask makes useless; the
 * pages give no rule or granularity, the reading is stated here). `mask`
 * holds the rank's own bound vectors (e.g. from fm_mask_localize) for its
 * seqlen_q local rows. Key tile kt, keys [kt*block_k, min((kt+1)*block_k,
 * seqlen_k)), is needed exactly when some row in [0, seqlen_q) is unmasked for
 * some key of the tile; the test is exact for any bound values (it does not
 * go through the tile classes, which are exact on the structural mask
 * families and conservative otherwise). 1 <= block_k <= 2^30.
 * Outputs (device): need uint8 [Bm][Hm][Tk], Tk = ceil(seqlen_k / block_k),
 * 1 = needed, 0 = not; count int32 [Bm][Hm], the number of needed tiles per
 * mask row (may be NULL). */
fm_status fm_kv_transfer_set(const fm_mask* mask, int32_t seqlen_q, int32_t seqlen_k, int32_t block_k,
                             uint8_t* need, int32_t* count, hipStream_t stream);

/* Work per chunk of the global query axis, for a sparsity-aware chunk ->
 * rank assignment (FlashMask-3 page, contributions paragraph and "Key facts"
 * name the HCC-IPO load balancer and nothing more; the work measure is this
 * library's reading): work[mr][c] = the number of open (row, key) pairs of
 * mask row mr (= bm * Hm + hm) whose row lies in chunk c = [chunk_start[c],
 * chunk_start[c] + chunk_len[c]), exact for any bound values (int64).
 * Chunks (host arrays) as for fm_mask_localize: ascending, not overlapping,
 * chunk_len >= 1, inside [0, seqlen_q_global], 1 <= num_chunks <= 64.
 * work: device int64 [Bm*Hm][num_chunks], 8-byte aligned. */
fm_status fm_chunk_work(const fm_mask* global, int32_t seqlen_k, int32_t seqlen_q_global,
                        const int32_t* chunk_start, const int32_t* chunk_len, int32_t num_chunks, int64_t* work,
                        hipStream_t stream);

/* Chunk -> rank plan (host only; no device memory, no stream). Gives each of
 * num_ranks ranks exactly num_chunks / num_ranks chunks so that the largest
 * rank load (sum of chunk_work over its chunks; host array, >= 0) is small:
 * with two chunks per rank, sorted pairing (largest with smallest), which is
 * optimal; otherwise longest first into the least loaded rank with room; in
 * both cases and from the snake order (the dual-chunk assignment for two per
 * rank), single-chunk exchanges with the most loaded rank while they lower
 * it. The better plan is returned (never worse than the snake order).
 * rank_of_chunk: host int32 [num_chunks]; max_load (may be NULL) receives the
 * largest rank load. num_chunks must be a multiple of num_ranks, <= 4096. */
fm_status fm_cp_plan(const int64_t* chunk_work, int32_t num_chunks, int32_t num_ranks, int32_t* rank_of_chunk,
                     int64_t* max_load);

/* Per-kernel timing. Between fm_profile_begin and fm_profile_end the library
 * records a HIP event pair on the launch stream around each of its kernel
 * launches (at most max_launches pairs; later launches are not recorded).
 * fm_profile_end waits for those events and writes, per stage, the summed
 * duration in milliseconds and the number of recorded launches (arrays of
 * FM_NUM_STAGES entries). Not thread safe; profiling state is per process. */
typedef enum {
  FM_STAGE_CLASSIFY_SUMMARY = 0,
  FM_STAGE_CLASSIFY_MAP = 1,
  FM_STAGE_FWD = 2,
  FM_STAGE_BWD_PRE = 3,     /* backward: D = rowsum(dO * O), with the stored-dS slot map */
  FM_STAGE_BWD = 4,         /* dK / dV kernel */
  FM_STAGE_BWD_DQ = 5,      /* dQ kernel */
  FM_STAGE_LOCALIZE = 6,
  FM_STAGE_BWD_PLAN = 7,    /* not recorded: the stored-dS plan runs in the ORDER and BWD_PRE launches */
  FM_STAGE_BWD_DQ_DS = 8,   /* dQ from stored dS */
  FM_STAGE_ORDER = 9,       /* launch orders, longest tiles first (backward: with the stored-dS offsets) */
  FM_STAGE_TRANSFER = 10,   /* mask-pruned K/V transfer set */
  FM_STAGE_CHUNK_WORK = 11, /* open pairs per chunk of the query axis */
  FM_STAGE_VT = 12,         /* FP8 forward: V^T tile pre-pass */
  FM_NUM_STAGES = 13
} fm_stage;

fm_status fm_profile_begin(int32_t max_launches);
fm_status fm_profile_end(float* total_ms, int32_t* launches);

/* Message describing the last non-OK status returned on this thread. */
const char* fm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FM_ATTN_H */
