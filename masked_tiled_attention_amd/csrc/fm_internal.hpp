// Internal interfaces between the C-ABI layer (api.cpp) and the kernel
// translation units. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fm_attn.h"

namespace fm {

// Tile shapes of the attention kernels (rows of Q x columns of K).
constexpr int kFwdBlockQ = 128;
constexpr int kFwdBlockK = 64;
constexpr int kBwdBlockQ = 64;    // dK/dV kernel: query rows per inner tile
constexpr int kBwdBlockK = 128;   // dK/dV kernel: keys per workgroup
constexpr int kBwdListCap = 1024;  // dK/dV kernel: query tiles compacted per list pass
constexpr int kDqBlockPairs = 16;  // stored-dS dQ launch order: query-tile pairs per block
constexpr int kDqBlockQ = 128;    // dQ kernel: query rows per workgroup
constexpr int kDqBlockK = 32;     // dQ kernel: keys per inner tile

// Mask vectors as seen by the kernels. A missing pair is flagged and its
// pointers are not dereferenced.
struct MaskArgs {
  const int32_t* lts;
  const int32_t* lte;
  const int32_t* uts;
  const int32_t* ute;
  int64_t stride_b, stride_h;
  int32_t bm, hm;          // broadcast extents (1 or B / H)
  int32_t has_lower, has_upper;
};

struct ClassifyArgs {
  MaskArgs mask;
  int32_t seq_q, seq_k, block_q, block_k, tq, tk;
  int32_t* summary;        // [bm][hm][tk][8]
  uint8_t* classes;        // [bm][hm][tq][tk] or [bm][hm][tk][tq]
  int32_t transposed;
  int32_t* counts;         // nullptr, or [bm][hm][lines] non-SKIP entries per map line
  int32_t* chunk_pre;      // nullptr, or [bm][hm][lines][ceil(len / 64)] non-SKIP entries before each 64-entry chunk
  int32_t* first;          // nullptr, or (transposed maps) [bm][hm][lines]: the first entry of the dK/dV
                           // kernel's list for the line, -1 when the line has none (see map_line)
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int32_t batch, heads, seq_q, seq_k;
  float scale;             // softmax scale
  float scale_log2;        // scale * log2(e)
  MaskArgs mask;
  const uint8_t* classes;  // [bm][hm][tq][tk]
  int32_t tq, tk;
  // Launch order: workgroup p takes class-map row order[p / rep] (mask row *
  // tq + query tile), longest first, and (b, h) pair p % rep of that mask row.
  const int32_t* order;
  int32_t rep;             // (b, h) pairs per mask row
  int32_t group;           // query heads per K/V head: K/V head = h / group
  // FP8 forward only: V^T tiles from the pre-pass ([B][H_kv][tk][64 * D bytes]),
  // K/V heads, and the factor applied to O at the end (the V descale).
  const uint8_t* vt;
  int32_t heads_kv;
  float o_scale;
  // Split lists (bf16 / float32 forward): with ksplit > 1 each query tile's
  // compacted key-tile list is cut into ksplit contiguous parts, one workgroup
  // each, which write float32 partial O (normalised over their part) to
  // opart [ksplit][B][H][Sq][D] and their LSE to lpart [ksplit][B][H][Sq];
  // a second kernel merges them into O and LSE.
  int32_t ksplit;
  float* opart;
  float* lpart;
};

// V^T pre-pass of the FP8 forward: V [B][Sk][H_kv][D] E4M3 codes (strides
// in bytes) to 64-key tiles of four [128 channel][16 key] planes.
struct VtArgs {
  const uint8_t* v;
  int64_t v_sb, v_ss, v_sh;
  int32_t batch, heads_kv, seq_k, tk;
  uint8_t* vt;
};

// Lines ordered by their non-SKIP count, descending. Line r counts `group`
// class-map lines of up to `len` entries each, whose counts (from the class
// map pass) are counts[(r / inner) * outer_stride + (r % inner) +
// gi * group_stride] for gi < group.
struct OrderArgs {
  const int32_t* counts;
  int32_t rows, len, inner;
  int64_t outer_stride;
  int32_t group;
  int64_t group_stride;
  int32_t* order;          // [rows] line indices, longest first
  int32_t mark_empty;      // set: lines with no non-SKIP entry carry kEmptyLine and go last
  int32_t* live;           // with mark_empty, optional: the number of lines before the empty ones
  const int32_t* first_in;   // optional, per line: a value carried into first_out at the line's position
  int32_t* first_out;
};
constexpr uint32_t kEmptyLine = 0x80000000u;   // order entry flag: the line has no work

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* lse2;             // [B][H][Sp] float32: LSE * log2(e); +inf for rows that see no key or lie past Sq
  float* drow;             // [B][H][Sp] float32: D = rowsum(dO * O); 0 past Sq
  int32_t seq_pad;         // Sp: Sq rounded up to a multiple of 128
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int32_t batch, heads, seq_q, seq_k;
  int32_t heads_kv, group;   // K/V heads; query heads per K/V head
  float scale;
  float scale_log2;
  MaskArgs mask;
  const uint8_t* classes_t;  // [bm][hm][tk][tq] with the dK/dV kernel's tiles
  int32_t tq, tk;
  const uint8_t* classes_q;  // [bm][hm][tq_q][tk_q] with the dQ kernel's tiles
  int32_t tq_q, tk_q;
  // Stored dS (dQ from dS K), with the dK/dV tiling; plan == nullptr when the
  // workspace cannot hold the slot map at all.
  int32_t* row_cnt;          // [bm*hm][tk] non-SKIP tiles per key-tile row
  int32_t* row_off;          // [bm*hm][tk] exclusive prefix sums of row_cnt
  int32_t* chunk_pre;        // [bm*hm][tk][ceil(tq / 64)] non-SKIP tiles of the row before each 64-tile chunk
  int32_t* plan;             // [0] total non-SKIP tiles, [1] 1 if the dS store is in use
  int32_t* slots_q;          // [bm*hm][tq][tk] slot of each non-SKIP tile, query-major, -1 for SKIP tiles
  uint16_t* ds;              // [rep][total][kBwdBlockK keys][kBwdBlockQ rows] bf16
  int64_t ds_capacity;       // bytes available at ds
  int32_t rep;               // (b, h) pairs per mask row
  // The dK/dV kernel works per (b, K/V head, key tile) over the `group` query
  // heads of the K/V head; its lines are K/V mask rows (bm * hkm + hk with
  // hkm = heads_kv when the mask has a row per head, else 1) times key
  // tiles, and rep_kv (b, K/V head) pairs share one.
  int32_t rep_kv;
  // Launch orders, longest first (see FwdArgs::order): key tiles of the dK/dV
  // tiling and the recompute dQ kernel's query tiles (may be nullptr).
  const int32_t* order_k;   // key-tile lines longest first; empty lines flagged with kEmptyLine, last
  const int32_t* order_live;   // the number of order_k lines before the empty ones
  const int32_t* first_k;   // nullptr, or per order_k position: the query tile its line's list starts with
  const int32_t* order_qq;
  // Stored-dS dQ launch order (mask shared by all rows; else nullptr): blocks
  // of kDqBlockPairs query-tile pairs, counted from the last pair, longest
  // list first; counts_q = the dQ map's line counts, written by the map pass.
  const int32_t* counts_q;
  int32_t* dq_blocks;
  // Grouped-query attention with a mask shared by all heads: one dK/dV
  // workgroup per query head, float32 partials [2][B][H][Sk][D] (dK, then dV)
  // summed per K/V head afterwards; nullptr: a workgroup runs all the query
  // heads of its K/V head.
  float* part;
  // Stored-dS dQ with split lists: with dq_split > 1 each query-tile pair's
  // key-tile list is cut into dq_split parts, one workgroup each, writing
  // float32 partial dQ [dq_split][B][H][Sq][D] that a second kernel sums.
  int32_t dq_split;
  float* dqpart;
};

// (b, h) of workgroup p given the mask row it serves (see FwdArgs::order).
__device__ __forceinline__ void ordered_bh(int mr, int j, const MaskArgs& m, int heads, int* b, int* h) {
  *b = m.bm > 1 ? mr / m.hm : j / (m.hm > 1 ? 1 : heads);
  *h = m.hm > 1 ? mr % m.hm : j % heads;
}

hipError_t launch_bwd_dq_ds(const BwdArgs& a, int head_dim, bool f32, hipStream_t stream);

constexpr int kMaxChunks = 64;

struct LocalizeArgs {
  MaskArgs mask;
  int32_t seq_k, seq_q_global, num_chunks;
  int32_t chunk_start[kMaxChunks];
  int32_t chunk_len[kMaxChunks];
  int32_t chunk_off[kMaxChunks];
  int32_t* out[4];
};

struct TransferArgs {
  MaskArgs mask;
  int32_t seq_q, seq_k, block_k, tk;
  uint8_t* need;           // [bm][hm][tk]
  int32_t* count;          // [bm][hm] or null
};

struct ChunkWorkArgs {
  MaskArgs mask;
  int32_t seq_k, num_chunks;
  int32_t chunk_start[kMaxChunks];
  int32_t chunk_len[kMaxChunks];
  int64_t* work;           // [bm * hm][num_chunks]
};

// Launchers: enqueue on `stream`, return hipGetLastError() of the launch.
hipError_t launch_classify_summary(const ClassifyArgs& a, hipStream_t stream);
hipError_t launch_classify_map(const ClassifyArgs& a, hipStream_t stream);
hipError_t launch_order(const OrderArgs& a, hipStream_t stream);
// Backward pre-passes, fused into four launches:
//   summaries   the summaries of both tilings;
//   maps        both class maps with the line counts (row_cnt for the dK/dV
//               tiling, the dQ tiling's into cq.counts) and, with
//               ct.chunk_pre set, the chunk prefixes of the dK/dV rows;
//   orders      the launch orders ok and (oq.order set) oq, and, with
//               a.plan set, the slot offsets and the plan;
//   rows        the query-major slot map (`slots`, stored dS) and the row
//               pass D, LSE * log2(e) (`rows`; needs o, dout, lse).
hipError_t launch_bwd_summaries(const ClassifyArgs& ct, const ClassifyArgs& cq, hipStream_t stream);
hipError_t launch_bwd_maps(const ClassifyArgs& ct, const ClassifyArgs& cq, hipStream_t stream);
hipError_t launch_bwd_orders(const OrderArgs& ok, const OrderArgs& oq, const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_rows(const BwdArgs& a, bool slots, bool rows, int head_dim, bool f32, hipStream_t stream);
hipError_t launch_fwd(const FwdArgs& a, int head_dim, bool f32, hipStream_t stream);
hipError_t launch_fwd_fp8(const FwdArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_vt(const VtArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, bool f32, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, bool f32, hipStream_t stream);
hipError_t launch_localize(const LocalizeArgs& a, hipStream_t stream);
hipError_t launch_transfer_set(const TransferArgs& a, hipStream_t stream);
hipError_t launch_chunk_work(const ChunkWorkArgs& a, hipStream_t stream);
// Host: chunk -> rank plan (plan.cpp); returns the largest rank load.
int64_t plan_chunks(const int64_t* work, int num_chunks, int num_ranks, int32_t* rank_of_chunk);

}  // namespace fm
