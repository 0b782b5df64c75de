// C ABI of libfmattn (declared in include/fm_attn.h): argument validation,
// workspace layout, launch sequencing and per-launch event timing.
// Nothing here allocates device memory; every launch goes on the caller's
// stream and no call synchronises the host (fm_profile_end,
// fm_bwd_workspace_size_ds and fm_bwd_dq_path excepted).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "fm_attn.h"
#include "fm_internal.hpp"

namespace {

thread_local std::string g_err;

fm_status fail(fm_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

constexpr int64_t kMaxSeq = int64_t(1) << 24;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- profiling
struct Profiler {
  bool enabled = false;
  int cap = 0;
  int used = 0;
  std::vector<hipEvent_t> ev;     // 2 per record
  std::vector<int> stage;
};
Profiler g_prof;

template <class F>
hipError_t run_stage(fm_stage st, hipStream_t s, F&& launch) {
  bool rec = g_prof.enabled && g_prof.used < g_prof.cap;
  if (rec) rec = hipEventRecord(g_prof.ev[2 * g_prof.used], s) == hipSuccess;
  hipError_t e = launch();
  if (rec && hipEventRecord(g_prof.ev[2 * g_prof.used + 1], s) == hipSuccess) {
    g_prof.stage[g_prof.used] = (int)st;
    ++g_prof.used;
  }
  return e;
}

fm_status hip_fail(hipError_t e, const char* what) {
  return fail(FM_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

// ---------------------------------------------------------------- scratch
// Device memory of the allocation-free forward (fm_attn_fwd_noalloc): a
// file-scope device array, one copy per GPU the library runs on, held until
// the process ends. In host code `scratch` names a host-side stand-in, never
// the device memory: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is used.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The scratch array's device address on the current device, which must be
// the device of `stream` (a NULL stream is the current device's).
fm_status scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FM_ERR_UNSUPPORTED, "device %d out of range", dev);
  if (stream) {
    hipDevice_t sdev = -1;
    if ((e = hipStreamGetDevice(stream, &sdev)) != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
    if (sdev != dev)
      return fail(FM_ERR_INVALID_ARGUMENT, "stream belongs to device %d, the current device is %d", (int)sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || reinterpret_cast<uintptr_t>(ptr) % 256)
      return fail(FM_ERR_HIP, "scratch address %p is NULL or not 256-byte aligned", ptr);
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return FM_OK;
}

// ---------------------------------------------------------------- validation
fm_status check_mask(const fm_mask* m, int64_t B, int64_t H, fm::MaskArgs* out) {
  if (!m) return fail(FM_ERR_INVALID_ARGUMENT, "mask is NULL");
  const bool lo0 = m->lts == nullptr, lo1 = m->lte == nullptr;
  const bool up0 = m->uts == nullptr, up1 = m->ute == nullptr;
  if (lo0 != lo1) return fail(FM_ERR_INVALID_ARGUMENT, "mask: exactly one of lts/lte is NULL");
  if (up0 != up1) return fail(FM_ERR_INVALID_ARGUMENT, "mask: exactly one of uts/ute is NULL");
  if (!(m->batch == 1 || m->batch == B))
    return fail(FM_ERR_INVALID_ARGUMENT, "mask batch %d must be 1 or %lld", m->batch, (long long)B);
  if (!(m->heads == 1 || m->heads == H))
    return fail(FM_ERR_INVALID_ARGUMENT, "mask heads %d must be 1 or %lld", m->heads, (long long)H);
  if (m->stride_b < 0 || m->stride_h < 0) return fail(FM_ERR_INVALID_ARGUMENT, "mask strides must be >= 0");
  const int32_t* ptrs[4] = {m->lts, m->lte, m->uts, m->ute};
  for (int i = 0; i < 4; ++i)
    if (ptrs[i] && (reinterpret_cast<uintptr_t>(ptrs[i]) % 4))
      return fail(FM_ERR_INVALID_ARGUMENT, "mask vector %d is not 4-byte aligned", i);
  out->lts = m->lts;
  out->lte = m->lte;
  out->uts = m->uts;
  out->ute = m->ute;
  out->stride_b = m->stride_b;
  out->stride_h = m->stride_h;
  out->bm = m->batch;
  out->hm = m->heads;
  out->has_lower = !lo0;
  out->has_upper = !up0;
  return FM_OK;
}

fm_status check_problem(const fm_problem* p) {
  if (!p) return fail(FM_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (p->batch < 1 || p->heads < 1 || p->seqlen_q < 1 || p->seqlen_k < 1)
    return fail(FM_ERR_INVALID_ARGUMENT, "batch, heads, seqlen_q, seqlen_k must be >= 1");
  if (p->seqlen_q > kMaxSeq || p->seqlen_k > kMaxSeq)
    return fail(FM_ERR_INVALID_ARGUMENT, "sequence lengths must be <= %lld", (long long)kMaxSeq);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(FM_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", p->head_dim);
  if (p->dtype != FM_BF16 && p->dtype != FM_FP32 && p->dtype != FM_FP8_E4M3)
    return fail(FM_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)p->dtype);
  if (!(p->softmax_scale > 0.f) || !std::isfinite(p->softmax_scale))
    return fail(FM_ERR_INVALID_ARGUMENT, "softmax_scale must be positive and finite");
  if (p->heads_kv < 0 || (p->heads_kv > 0 && p->heads % p->heads_kv))
    return fail(FM_ERR_INVALID_ARGUMENT, "heads_kv %d must be 0 or divide heads %d", p->heads_kv, p->heads);
  // element bytes: inputs and output share the dtype, except that FP8
  // inputs give a bf16 output
  const int64_t es_in = p->dtype == FM_BF16 ? 2 : p->dtype == FM_FP32 ? 4 : 1;
  const int64_t es_out = p->dtype == FM_FP32 ? 4 : 2;
  const int64_t* st[4] = {p->q_stride, p->k_stride, p->v_stride, p->o_stride};
  const char* nm[4] = {"q", "k", "v", "o"};
  for (int t = 0; t < 4; ++t)
    for (int i = 0; i < 3; ++i) {
      const int64_t es = t == 3 ? es_out : es_in;
      if (st[t][i] < 0) return fail(FM_ERR_INVALID_ARGUMENT, "%s stride %d is negative", nm[t], i);
      if ((st[t][i] * es) % 16)
        return fail(FM_ERR_INVALID_ARGUMENT, "%s stride %d (%lld elements) breaks 16-byte row alignment",
                    nm[t], i, (long long)st[t][i]);
    }
  // kernels address one tile (at most 256 rows) with 32-bit byte offsets
  for (int t = 0; t < 4; ++t)
    if (st[t][1] * (t == 3 ? es_out : es_in) * 256 > INT32_MAX)
      return fail(FM_ERR_UNSUPPORTED, "%s sequence stride %lld elements is too large", nm[t], (long long)st[t][1]);
  const int64_t tq = ceil_div(p->seqlen_q, fm::kFwdBlockQ);
  if (tq * p->batch * p->heads > INT32_MAX)
    return fail(FM_ERR_INVALID_ARGUMENT, "problem too large for one launch");
  return FM_OK;
}

fm_status check_ptr(const void* ptr, const char* name) {
  if (!ptr) return fail(FM_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(ptr) % 16)
    return fail(FM_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  return FM_OK;
}

// Workspace: per tiling one summary [Bm][Hm][Tk][8] int32 and one class map
// [Bm][Hm][Tq][Tk] uint8 (forward: the forward tiles; backward: the dK/dV
// tiles, transposed, and the dQ tiles), plus for the backward the per-row
// LSE * log2(e) and D [B][H][Sp] float32 (Sp = Sq rounded up to 128, the
// padding rows neutral) and the stored-dS plan counters. total is the
// minimum. Beyond it, the backward may place the chunk prefixes of the dK/dV
// class rows [Bm*Hm][Tk][ceil(Tq / 64)] int32 at `chunk_pre`, the query-major
// stored-dS slot map [Bm*Hm][Tq][Tk] int32 at `slots_q` and the dS tiles from
// `ds` on.
// 256-byte aligned sections.
struct Layout {
  size_t summary = 0, map = 0, summary_q = 0, map_q = 0, lse2 = 0, drow = 0;
  size_t row_cnt = 0, row_off = 0, plan = 0, total = 0, chunk_pre = 0, slots_q = 0, ds = 0;
  size_t counts = 0, order = 0;   // forward launch order
  size_t vt = 0;                   // FP8 forward: V^T tiles [B][H_kv][Tk][8 KiB]
  size_t order_k = 0, order_qq = 0;   // backward launch orders (dQ: its counts, then the order)
  size_t first_k = 0;                 // dK/dV kernel: the first list entry per key-tile line
  size_t dq_blocks = 0;               // stored-dS dQ kernel: launch order of its pair blocks
  size_t part = 0;                     // split-head dK/dV partials (0: not used)
  size_t opart = 0, lpart = 0;         // split-list forward partials (0: not used)
  int32_t ksplit = 1;
  size_t dqpart = 0;                   // split-list stored-dS dQ partials (0: not used)
  int32_t dq_split = 1;
};

int64_t padded_rows(int64_t sq) { return ceil_div(sq, 128) * 128; }

int32_t kv_heads(const fm_problem* p) { return p->heads_kv > 0 ? p->heads_kv : p->heads; }

// Grouped-query attention whose mask is shared by all heads runs one dK/dV
// workgroup per query head (float32 partials summed afterwards): a workgroup
// that ran a whole group of heads over one key tile would be the longest one.
// Its partials take 8 * B * H * Sk * D bytes of workspace; beyond 4 GiB the
// workgroups run their K/V head's query heads in turn instead.
bool split_heads(const fm_problem* p, const fm_mask* m) {
  const uint64_t bytes = (uint64_t)p->batch * p->heads * p->seqlen_k * p->head_dim * 8;
  return kv_heads(p) < p->heads && m->heads == 1 && bytes <= (uint64_t(4) << 30);
}

// Parts per query-tile pair's key-tile list in the stored-dS dQ kernel (two
// workgroups per CU). A launch with few pairs and long lists is bound by its
// longest lists, so the count doubles (up to 8) while the split launch stays
// within 1024 workgroups and each part keeps at least 32 key tiles of 128
// keys. The host cannot see the list lengths; cutting short ones costs more
// than it saves.
int32_t dq_split(const fm_problem* p) {
  const int64_t nwg = ceil_div(ceil_div(p->seqlen_q, fm::kBwdBlockQ), 2) * p->batch * p->heads;
  const int64_t tk = ceil_div(p->seqlen_k, fm::kBwdBlockK);
  int32_t ks = 1;
  while (ks < 8 && nwg * 2 * ks <= 1024 && tk >= 64 * ks) ks *= 2;
  return ks;
}

// The same for the query tiles of the bf16 / float32 forward (two workgroups
// per CU, 512 at once): as many parts (up to 8) as keep the split launch
// within about three rounds of the 512, 1536 workgroups, and each part at
// least 64 key tiles of 64 keys. Each round costs every workgroup its fixed
// start and end, and each part a float32 partial row to write and merge, so
// three rounds measured better than four on the context-parallel rank share.
int32_t fwd_split(const fm_problem* p) {
  if (p->dtype == FM_FP8_E4M3) return 1;
  const int64_t nwg = ceil_div(p->seqlen_q, fm::kFwdBlockQ) * p->batch * p->heads;
  const int64_t tk = ceil_div(p->seqlen_k, fm::kFwdBlockK);
  return (int32_t)std::max<int64_t>(1, std::min<int64_t>({8, 1536 / nwg, tk / 64}));
}

// max_split caps the forward's list parts (1: no split partials).
Layout workspace_layout(const fm_problem* p, const fm_mask* m, bool bwd, int32_t max_split = 8) {
  Layout L;
  const int64_t bh = (int64_t)m->batch * m->heads;
  size_t off = 0;
  auto add_tiling = [&](int64_t bq, int64_t bk, size_t* summary, size_t* map) {
    const int64_t tq = ceil_div(p->seqlen_q, bq), tk = ceil_div(p->seqlen_k, bk);
    *summary = off;
    off = align256(off + (size_t)(bh * tk * 8 * 4));
    *map = off;
    off = align256(off + (size_t)(bh * tq * tk));
  };
  if (bwd) {
    add_tiling(fm::kBwdBlockQ, fm::kBwdBlockK, &L.summary, &L.map);
    add_tiling(fm::kDqBlockQ, fm::kDqBlockK, &L.summary_q, &L.map_q);
    const size_t rows = (size_t)p->batch * p->heads * padded_rows(p->seqlen_q) * 4;
    L.lse2 = off;
    off = align256(off + rows);
    L.drow = off;
    off = align256(off + rows);
    const int64_t mrows = (int64_t)m->batch * m->heads;
    const int64_t tq = ceil_div(p->seqlen_q, fm::kBwdBlockQ), tk = ceil_div(p->seqlen_k, fm::kBwdBlockK);
    L.row_cnt = off;
    off = align256(off + (size_t)(mrows * tk * 4));
    L.row_off = off;
    off = align256(off + (size_t)(mrows * tk * 4));
    L.plan = off;
    off = align256(off + 16);
    const int64_t tq_q = ceil_div(p->seqlen_q, fm::kDqBlockQ);
    L.order_k = off;   // the counts are row_cnt; then the number of lines with work
    off = align256(off + (size_t)(mrows * tk * 4) + 4);
    L.first_k = off;   // the first list entry of each key-tile line, then by order position
    off = align256(off + (size_t)(mrows * tk * 4) * 2);
    L.dq_blocks = off;
    off = align256(off + (size_t)(ceil_div(tq_q, fm::kDqBlockPairs) * 4));
    L.order_qq = off;
    off = align256(off + (size_t)(mrows * tq_q * 8));
    L.dq_split = dq_split(p);
    if (L.dq_split > 1) {   // float32 dQ partials of the split lists
      L.dqpart = off;
      off = align256(off + (size_t)L.dq_split * p->batch * p->heads * p->seqlen_q * p->head_dim * 4);
    }
    if (split_heads(p, m)) {   // float32 dK, dV partials per query head
      L.part = off;
      off = align256(off + (size_t)p->batch * p->heads * p->seqlen_k * p->head_dim * 4 * 2);
    }
    L.chunk_pre = off;
    L.slots_q = align256(L.chunk_pre + (size_t)(mrows * tk * ceil_div(tq, 64) * 4));
    L.ds = align256(L.slots_q + (size_t)(mrows * tq * tk * 4));
  } else {
    add_tiling(fm::kFwdBlockQ, fm::kFwdBlockK, &L.summary, &L.map);
    const size_t rows = (size_t)(bh * ceil_div(p->seqlen_q, fm::kFwdBlockQ)) * 4;
    L.counts = off;
    off = align256(off + rows);
    L.order = off;
    off = align256(off + rows);
    L.ksplit = std::min(fwd_split(p), std::max(max_split, 1));
    if (L.ksplit > 1) {
      const size_t rows_all = (size_t)L.ksplit * p->batch * p->heads * p->seqlen_q;
      L.opart = off;
      off = align256(off + rows_all * p->head_dim * 4);
      L.lpart = off;
      off = align256(off + rows_all * 4);
    }
    if (p->dtype == FM_FP8_E4M3) {
      L.vt = off;
      off = align256(off + (size_t)((int64_t)p->batch * kv_heads(p) * ceil_div(p->seqlen_k, fm::kFwdBlockK) *
                                    fm::kFwdBlockK * p->head_dim));
    }
  }
  L.total = off;
  return L;
}

fm::ClassifyArgs classify_args(const fm::MaskArgs& mk, int32_t sq, int32_t sk, int32_t bq, int32_t bk,
                               int32_t transposed, int32_t* summary, uint8_t* classes, int32_t* counts = nullptr) {
  fm::ClassifyArgs c{};
  c.mask = mk;
  c.seq_q = sq;
  c.seq_k = sk;
  c.block_q = bq;
  c.block_k = bk;
  c.tq = (int32_t)ceil_div(sq, bq);
  c.tk = (int32_t)ceil_div(sk, bk);
  c.summary = summary;
  c.classes = classes;
  c.transposed = transposed;
  c.counts = counts;
  return c;
}

// Summary and class map (with the line counts when `counts` is set).
fm_status classify_into(const fm::MaskArgs& mk, int32_t sq, int32_t sk, int32_t bq, int32_t bk,
                        int32_t transposed, int32_t* summary, uint8_t* classes, hipStream_t s,
                        int32_t* counts = nullptr) {
  const fm::ClassifyArgs c = classify_args(mk, sq, sk, bq, bk, transposed, summary, classes, counts);
  hipError_t e = run_stage(FM_STAGE_CLASSIFY_SUMMARY, s, [&] { return fm::launch_classify_summary(c, s); });
  if (e != hipSuccess) return hip_fail(e, "classify summary launch");
  e = run_stage(FM_STAGE_CLASSIFY_MAP, s, [&] { return fm::launch_classify_map(c, s); });
  if (e != hipSuccess) return hip_fail(e, "classify map launch");
  return FM_OK;
}

// Validation, the pre-passes and the arguments shared by fm_attn_bwd and
// fm_bwd_workspace_size_ds; the caller sets the tensor pointers beforehand.
// `rows`: run the row pass too (needs o, dout, lse). `size_query`: only the
// tile count is wanted (the plan scan runs whatever the workspace holds).
// Four launches: summaries, class maps with line counts, launch orders (+
// slot offsets), and the slot map (stored dS) with the row pass.
fm_status bwd_setup(const fm_problem* p, const fm_mask* mask, void* ws, size_t ws_bytes, hipStream_t stream,
                    bool rows, bool size_query, fm::BwdArgs* out, Layout* lay) {
  fm_status st = check_problem(p);
  if (st != FM_OK) return st;
  if (p->dtype == FM_FP8_E4M3) return fail(FM_ERR_UNSUPPORTED, "the backward takes bf16 or float32 inputs");
  fm::MaskArgs mk;
  st = check_mask(mask, p->batch, p->heads, &mk);
  if (st != FM_OK) return st;
  const Layout L = workspace_layout(p, mask, true);
  if (!ws || reinterpret_cast<uintptr_t>(ws) % 256)
    return fail(FM_ERR_WORKSPACE, "workspace is NULL or not 256-byte aligned");
  if (ws_bytes < L.total)
    return fail(FM_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L.total);
  const int32_t tq = (int32_t)ceil_div(p->seqlen_q, fm::kBwdBlockQ);
  const int32_t tk = (int32_t)ceil_div(p->seqlen_k, fm::kBwdBlockK);
  const int32_t tq_q = (int32_t)ceil_div(p->seqlen_q, fm::kDqBlockQ);
  const int32_t tk_q = (int32_t)ceil_div(p->seqlen_k, fm::kDqBlockK);
  if (tk > 65535 || tq_q > 65535) return fail(FM_ERR_INVALID_ARGUMENT, "sequence too long");
  char* w = static_cast<char*>(ws);
  uint8_t* classes_t = reinterpret_cast<uint8_t*>(w + L.map);
  uint8_t* classes_q = reinterpret_cast<uint8_t*>(w + L.map_q);
  const int64_t mrows = (int64_t)mk.bm * mk.hm;

  fm::BwdArgs& a = *out;
  a.lse2 = reinterpret_cast<float*>(w + L.lse2);
  a.drow = reinterpret_cast<float*>(w + L.drow);
  a.seq_pad = (int32_t)padded_rows(p->seqlen_q);
  a.q_sb = p->q_stride[0]; a.q_ss = p->q_stride[1]; a.q_sh = p->q_stride[2];
  a.k_sb = p->k_stride[0]; a.k_ss = p->k_stride[1]; a.k_sh = p->k_stride[2];
  a.v_sb = p->v_stride[0]; a.v_ss = p->v_stride[1]; a.v_sh = p->v_stride[2];
  a.o_sb = p->o_stride[0]; a.o_ss = p->o_stride[1]; a.o_sh = p->o_stride[2];
  a.batch = p->batch;
  a.heads = p->heads;
  a.heads_kv = kv_heads(p);
  a.group = p->heads / a.heads_kv;
  a.seq_q = p->seqlen_q;
  a.seq_k = p->seqlen_k;
  a.scale = p->softmax_scale;
  a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  a.mask = mk;
  a.classes_t = classes_t;
  a.tq = tq;
  a.tk = tk;
  a.classes_q = classes_q;
  a.tq_q = tq_q;
  a.tk_q = tk_q;
  a.row_cnt = reinterpret_cast<int32_t*>(w + L.row_cnt);
  a.row_off = reinterpret_cast<int32_t*>(w + L.row_off);
  a.rep = (mk.bm > 1 ? 1 : p->batch) * (mk.hm > 1 ? 1 : p->heads);
  a.rep_kv = (mk.bm > 1 ? 1 : p->batch) * (mk.hm > 1 ? 1 : a.heads_kv);
  a.part = L.part ? reinterpret_cast<float*>(w + L.part) : nullptr;
  a.dq_split = L.dq_split;
  a.dqpart = L.dqpart ? reinterpret_cast<float*>(w + L.dqpart) : nullptr;
  // Stored dS when the workspace can hold at least the slot map; whether it
  // holds every dS tile is decided on the device by the plan.
  const bool maybe_ds = !size_query && ws_bytes >= L.ds;
  a.plan = (maybe_ds || size_query) ? reinterpret_cast<int32_t*>(w + L.plan) : nullptr;
  if (maybe_ds) {
    a.chunk_pre = reinterpret_cast<int32_t*>(w + L.chunk_pre);
    a.slots_q = reinterpret_cast<int32_t*>(w + L.slots_q);
    a.ds = reinterpret_cast<uint16_t*>(w + L.ds);
    a.ds_capacity = (int64_t)(ws_bytes - L.ds);
  }
  const bool f32 = p->dtype == FM_FP32;
  int32_t* counts_q = reinterpret_cast<int32_t*>(w + L.order_qq);
  fm::ClassifyArgs ct = classify_args(mk, p->seqlen_q, p->seqlen_k, fm::kBwdBlockQ, fm::kBwdBlockK, 1,
                                      reinterpret_cast<int32_t*>(w + L.summary), classes_t, a.row_cnt);
  ct.chunk_pre = a.chunk_pre;
  ct.first = reinterpret_cast<int32_t*>(w + L.first_k);
  a.first_k = ct.first + mrows * tk;   // filled by the order sort
  if (maybe_ds && mrows == 1) {   // the stored-dS dQ kernel's block order (one mask row)
    a.counts_q = counts_q;
    a.dq_blocks = reinterpret_cast<int32_t*>(w + L.dq_blocks);
  }
  const fm::ClassifyArgs cq = classify_args(mk, p->seqlen_q, p->seqlen_k, fm::kDqBlockQ, fm::kDqBlockK, 0,
                                            reinterpret_cast<int32_t*>(w + L.summary_q), classes_q, counts_q);
  hipError_t e = run_stage(FM_STAGE_CLASSIFY_SUMMARY, stream, [&] { return fm::launch_bwd_summaries(ct, cq, stream); });
  if (e != hipSuccess) return hip_fail(e, "backward summary launch");
  e = run_stage(FM_STAGE_CLASSIFY_MAP, stream, [&] { return fm::launch_bwd_maps(ct, cq, stream); });
  if (e != hipSuccess) return hip_fail(e, "backward class map launch");

  // Launch orders: key-tile lines of the dK/dV map (one per K/V mask row and
  // key tile, counting the class rows of the K/V head's query heads when the
  // mask has a row per head) and, when its path is certain (the workspace
  // cannot hold the stored-dS slot map), the recompute dQ kernel's query-tile
  // lines; else that kernel keeps the default order.
  const int32_t kv_group = mk.hm > 1 ? a.group : 1;   // class rows per K/V mask row
  fm::OrderArgs ok{};
  ok.counts = a.row_cnt;
  ok.rows = (int32_t)((int64_t)mk.bm * (mk.hm > 1 ? a.heads_kv : 1) * tk);
  ok.len = tq;
  ok.inner = tk;
  ok.outer_stride = (int64_t)kv_group * tk;
  ok.group = kv_group;
  ok.group_stride = tk;
  ok.order = reinterpret_cast<int32_t*>(w + L.order_k);
  ok.mark_empty = 1;
  ok.live = ok.order + ok.rows;
  ok.first_in = ct.first;
  ok.first_out = const_cast<int32_t*>(a.first_k);
  fm::OrderArgs oq{};
  if (!size_query && ws_bytes < L.ds) {
    oq.counts = counts_q;
    oq.rows = (int32_t)(mrows * tq_q);
    oq.len = tk_q;
    oq.inner = oq.rows;
    oq.group = 1;
    oq.order = counts_q + oq.rows;
  }
  e = run_stage(FM_STAGE_ORDER, stream, [&] { return fm::launch_bwd_orders(ok, oq, a, stream); });
  if (e != hipSuccess) return hip_fail(e, "backward order launch");
  a.order_k = ok.order;
  a.order_live = ok.live;
  a.order_qq = oq.order;
  if (maybe_ds || rows) {
    e = run_stage(FM_STAGE_BWD_PRE, stream,
                  [&] { return fm::launch_bwd_rows(a, maybe_ds, rows, p->head_dim, f32, stream); });
    if (e != hipSuccess) return hip_fail(e, "backward row pass launch");
  }
  *lay = L;
  return FM_OK;
}

}  // namespace

extern "C" {

const char* fm_last_error(void) { return g_err.c_str(); }

void fm_kernel_tile(int32_t head_dim, int32_t bwd, int32_t* block_q, int32_t* block_k) {
  int32_t q = 0, k = 0;
  if (head_dim == 64 || head_dim == 128) {
    q = bwd ? fm::kBwdBlockQ : fm::kFwdBlockQ;
    k = bwd ? fm::kBwdBlockK : fm::kFwdBlockK;
  }
  if (block_q) *block_q = q;
  if (block_k) *block_k = k;
}

fm_status fm_workspace_size(const fm_problem* problem, const fm_mask* mask, int32_t with_bwd, size_t* bytes) {
  fm_status st = check_problem(problem);
  if (st != FM_OK) return st;
  fm::MaskArgs mk;
  st = check_mask(mask, problem->batch, problem->heads, &mk);
  if (st != FM_OK) return st;
  if (!bytes) return fail(FM_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (with_bwd && problem->dtype == FM_FP8_E4M3)
    return fail(FM_ERR_UNSUPPORTED, "the backward takes bf16 or float32 inputs");
  *bytes = workspace_layout(problem, mask, with_bwd != 0).total;
  return FM_OK;
}

fm_status fm_tile_classify(const fm_mask* mask, int32_t seqlen_q, int32_t seqlen_k, int32_t block_q,
                           int32_t block_k, int32_t transposed, int32_t* summary, uint8_t* classes,
                           hipStream_t stream) {
  fm::MaskArgs mk;
  if (!mask) return fail(FM_ERR_INVALID_ARGUMENT, "mask is NULL");
  fm_status st = check_mask(mask, mask->batch, mask->heads, &mk);
  if (st != FM_OK) return st;
  if (mask->batch < 1 || mask->heads < 1) return fail(FM_ERR_INVALID_ARGUMENT, "mask batch/heads must be >= 1");
  if (seqlen_q < 1 || seqlen_k < 1 || seqlen_q > kMaxSeq || seqlen_k > kMaxSeq)
    return fail(FM_ERR_INVALID_ARGUMENT, "sequence lengths must be in [1, %lld]", (long long)kMaxSeq);
  if (block_q < 1 || block_q > 1024 || block_k < 1 || block_k > 1024)
    return fail(FM_ERR_INVALID_ARGUMENT, "block sizes must be in [1, 1024]");
  const int64_t tq = ceil_div(seqlen_q, block_q), tk = ceil_div(seqlen_k, block_k);
  if ((transposed ? tk : tq) > 65535 || (int64_t)mask->batch * mask->heads > 65535)
    return fail(FM_ERR_INVALID_ARGUMENT, "too many tiles for one launch (reduce tiles or use larger blocks)");
  if (!summary || !classes) return fail(FM_ERR_INVALID_ARGUMENT, "summary/classes is NULL");
  if (reinterpret_cast<uintptr_t>(summary) % 4) return fail(FM_ERR_INVALID_ARGUMENT, "summary not 4-byte aligned");
  return classify_into(mk, seqlen_q, seqlen_k, block_q, block_k, transposed ? 1 : 0, summary, classes, stream);
}

}  // extern "C"

namespace {

// Both forwards: validation, classification, launch order, then (FP8) the
// V^T pre-pass and the FP8 kernel or the bf16/float32 kernel.
fm_status fwd_common(const fm_problem* p, const void* q, const void* k, const void* v, const float* descale,
                     const fm_mask* mask, void* o, float* lse, void* ws, size_t ws_bytes, hipStream_t stream,
                     int32_t max_split = 8) {
  fm_status st = check_problem(p);
  if (st != FM_OK) return st;
  const bool fp8 = descale != nullptr;
  if (fp8 != (p->dtype == FM_FP8_E4M3))
    return fail(FM_ERR_INVALID_ARGUMENT, fp8 ? "fm_attn_fwd_fp8 needs dtype FM_FP8_E4M3"
                                             : "FP8 inputs go to fm_attn_fwd_fp8");
  if (fp8)
    for (int i = 0; i < 3; ++i)
      if (!(descale[i] > 0.f) || !std::isfinite(descale[i]))
        return fail(FM_ERR_INVALID_ARGUMENT, "descale %d must be positive and finite", i);
  fm::MaskArgs mk;
  st = check_mask(mask, p->batch, p->heads, &mk);
  if (st != FM_OK) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(o, "o")) || (st = check_ptr(lse, "lse")))
    return st;
  const Layout L = workspace_layout(p, mask, false, max_split);
  if (!ws || reinterpret_cast<uintptr_t>(ws) % 256)
    return fail(FM_ERR_WORKSPACE, "workspace is NULL or not 256-byte aligned");
  if (ws_bytes < L.total)
    return fail(FM_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L.total);
  const int32_t tq = (int32_t)ceil_div(p->seqlen_q, fm::kFwdBlockQ);
  const int32_t tk = (int32_t)ceil_div(p->seqlen_k, fm::kFwdBlockK);
  if (tq > 65535) return fail(FM_ERR_INVALID_ARGUMENT, "seqlen_q too large");
  char* w = static_cast<char*>(ws);
  int32_t* summary = reinterpret_cast<int32_t*>(w + L.summary);
  uint8_t* classes = reinterpret_cast<uint8_t*>(w + L.map);
  int32_t* counts = reinterpret_cast<int32_t*>(w + L.counts);
  st = classify_into(mk, p->seqlen_q, p->seqlen_k, fm::kFwdBlockQ, fm::kFwdBlockK, 0, summary, classes, stream,
                     counts);
  if (st != FM_OK) return st;

  fm::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.q_sb = p->q_stride[0]; a.q_ss = p->q_stride[1]; a.q_sh = p->q_stride[2];
  a.k_sb = p->k_stride[0]; a.k_ss = p->k_stride[1]; a.k_sh = p->k_stride[2];
  a.v_sb = p->v_stride[0]; a.v_ss = p->v_stride[1]; a.v_sh = p->v_stride[2];
  a.o_sb = p->o_stride[0]; a.o_ss = p->o_stride[1]; a.o_sh = p->o_stride[2];
  a.batch = p->batch;
  a.heads = p->heads;
  a.seq_q = p->seqlen_q;
  a.seq_k = p->seqlen_k;
  a.scale = p->softmax_scale;
  a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  a.mask = mk;
  a.classes = classes;
  a.tq = tq;
  a.tk = tk;
  fm::OrderArgs oa{};
  oa.counts = counts;
  oa.rows = (int32_t)((int64_t)mk.bm * mk.hm * tq);
  oa.len = tk;
  oa.inner = oa.rows;
  oa.group = 1;
  oa.order = reinterpret_cast<int32_t*>(w + L.order);
  hipError_t e = run_stage(FM_STAGE_ORDER, stream, [&] { return fm::launch_order(oa, stream); });
  if (e != hipSuccess) return hip_fail(e, "forward order launch");
  a.order = oa.order;
  a.rep = (mk.bm > 1 ? 1 : p->batch) * (mk.hm > 1 ? 1 : p->heads);
  a.heads_kv = kv_heads(p);
  a.group = p->heads / a.heads_kv;
  a.o_scale = 1.f;
  a.ksplit = L.ksplit;
  if (L.ksplit > 1) {
    a.opart = reinterpret_cast<float*>(w + L.opart);
    a.lpart = reinterpret_cast<float*>(w + L.lpart);
  }
  if (fp8) {
    if ((int64_t)p->batch * a.heads_kv * tk > INT32_MAX) return fail(FM_ERR_INVALID_ARGUMENT, "problem too large");
    fm::VtArgs va{};
    va.v = static_cast<const uint8_t*>(v);
    va.v_sb = p->v_stride[0]; va.v_ss = p->v_stride[1]; va.v_sh = p->v_stride[2];
    va.batch = p->batch;
    va.heads_kv = a.heads_kv;
    va.seq_k = p->seqlen_k;
    va.tk = tk;
    va.vt = reinterpret_cast<uint8_t*>(w + L.vt);
    e = run_stage(FM_STAGE_VT, stream, [&] { return fm::launch_vt(va, p->head_dim, stream); });
    if (e != hipSuccess) return hip_fail(e, "V transpose launch");
    a.vt = va.vt;
    a.scale_log2 = p->softmax_scale * descale[0] * descale[1] * 1.4426950408889634f;
    a.o_scale = descale[2];
    e = run_stage(FM_STAGE_FWD, stream, [&] { return fm::launch_fwd_fp8(a, p->head_dim, stream); });
  } else {
    e = run_stage(FM_STAGE_FWD, stream,
                  [&] { return fm::launch_fwd(a, p->head_dim, p->dtype == FM_FP32, stream); });
  }
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  return FM_OK;
}

}  // namespace

extern "C" {

fm_status fm_attn_fwd(const fm_problem* p, const void* q, const void* k, const void* v, const fm_mask* mask,
                      void* o, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return fwd_common(p, q, k, v, nullptr, mask, o, lse, ws, ws_bytes, stream);
}

fm_status fm_attn_fwd_noalloc(const fm_problem* p, const void* q, const void* k, const void* v, const fm_mask* mask,
                              void* o, float* lse, hipStream_t stream) {
  fm_status st = check_problem(p);
  if (st != FM_OK) return st;
  fm::MaskArgs mk;
  if ((st = check_mask(mask, p->batch, p->heads, &mk)) != FM_OK) return st;
  // as many list parts as the scratch holds (fewer parts change only the
  // rounding order of the merge)
  int32_t split = 8;
  while (split > 1 && workspace_layout(p, mask, false, split).total > kScratchBytes) split /= 2;
  const size_t need = workspace_layout(p, mask, false, split).total;
  if (need > kScratchBytes)
    return fail(FM_ERR_WORKSPACE, "the allocation-free forward needs %zu bytes of scratch; it holds at most %zu",
                need, kScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_address(stream, &ws)) != FM_OK) return st;
  return fwd_common(p, q, k, v, nullptr, mask, o, lse, ws, kScratchBytes, stream, split);
}

fm_status fm_attn_fwd_fp8(const fm_problem* p, const void* q, const void* k, const void* v, const float* descale,
                          const fm_mask* mask, void* o, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!descale) return fail(FM_ERR_INVALID_ARGUMENT, "descale is NULL");
  return fwd_common(p, q, k, v, descale, mask, o, lse, ws, ws_bytes, stream);
}

fm_status fm_attn_bwd(const fm_problem* p, const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, const fm_mask* mask, void* dq, void* dk, void* dv,
                      void* ws, size_t ws_bytes, hipStream_t stream) {
  fm_status st = check_problem(p);
  if (st != FM_OK) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(o, "o")) || (st = check_ptr(lse, "lse")) || (st = check_ptr(dout, "dout")) ||
      (st = check_ptr(dq, "dq")) || (st = check_ptr(dk, "dk")) || (st = check_ptr(dv, "dv")))
    return st;
  fm::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  Layout L;
  if ((st = bwd_setup(p, mask, ws, ws_bytes, stream, true, false, &a, &L)) != FM_OK) return st;
  const bool maybe_ds = a.plan != nullptr;
  const bool f32 = p->dtype == FM_FP32;
  hipError_t e = run_stage(FM_STAGE_BWD, stream, [&] { return fm::launch_bwd_dkdv(a, p->head_dim, f32, stream); });
  if (e != hipSuccess) return hip_fail(e, "dK/dV launch");
  // both dQ kernels are launched when the dS store may be in use; each exits
  // at once unless the plan selected its path
  e = run_stage(FM_STAGE_BWD_DQ, stream, [&] { return fm::launch_bwd_dq(a, p->head_dim, f32, stream); });
  if (e != hipSuccess) return hip_fail(e, "dQ launch");
  if (maybe_ds) {
    e = run_stage(FM_STAGE_BWD_DQ_DS, stream, [&] { return fm::launch_bwd_dq_ds(a, p->head_dim, f32, stream); });
    if (e != hipSuccess) return hip_fail(e, "dQ (stored dS) launch");
  }
  return FM_OK;
}

fm_status fm_bwd_dq_path(const fm_problem* p, const fm_mask* mask, const void* ws, size_t ws_bytes,
                         hipStream_t stream, int32_t* stored_ds) {
  if (!stored_ds) return fail(FM_ERR_INVALID_ARGUMENT, "stored_ds is NULL");
  fm_status st = check_problem(p);
  if (st != FM_OK) return st;
  if (p->dtype == FM_FP8_E4M3) return fail(FM_ERR_UNSUPPORTED, "the backward takes bf16 or float32 inputs");
  fm::MaskArgs mk;
  if ((st = check_mask(mask, p->batch, p->heads, &mk)) != FM_OK) return st;
  const Layout L = workspace_layout(p, mask, true);
  if (!ws || reinterpret_cast<uintptr_t>(ws) % 256)
    return fail(FM_ERR_WORKSPACE, "workspace is NULL or not 256-byte aligned");
  if (ws_bytes < L.total)
    return fail(FM_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L.total);
  *stored_ds = 0;
  if (ws_bytes < L.ds) return FM_OK;   // no room for the slot map: recompute is certain
  int32_t flag = 0;
  const int32_t* plan = reinterpret_cast<const int32_t*>(static_cast<const char*>(ws) + L.plan);
  hipError_t e;
  if ((e = hipMemcpyAsync(&flag, plan + 1, sizeof(flag), hipMemcpyDeviceToHost, stream)) != hipSuccess ||
      (e = hipStreamSynchronize(stream)) != hipSuccess)
    return hip_fail(e, "reading the dQ path flag");
  *stored_ds = flag != 0;
  return FM_OK;
}

fm_status fm_bwd_workspace_size_ds(const fm_problem* p, const fm_mask* mask, void* ws, size_t ws_bytes,
                                   hipStream_t stream, size_t* bytes) {
  if (!bytes) return fail(FM_ERR_INVALID_ARGUMENT, "bytes is NULL");
  fm::BwdArgs a{};
  Layout L;
  fm_status st = bwd_setup(p, mask, ws, ws_bytes, stream, false, true, &a, &L);
  if (st != FM_OK) return st;
  hipError_t e;
  int32_t total = 0;
  if ((e = hipMemcpyAsync(&total, a.plan, sizeof(total), hipMemcpyDeviceToHost, stream)) != hipSuccess ||
      (e = hipStreamSynchronize(stream)) != hipSuccess)
    return hip_fail(e, "reading the tile count");
  if (total == INT32_MAX) return fail(FM_ERR_UNSUPPORTED, "too many non-SKIP tiles for the dS store");
  *bytes = L.ds + (size_t)total * (size_t)a.rep * (size_t)fm::kBwdBlockQ * fm::kBwdBlockK * 2;
  return FM_OK;
}

fm_status fm_mask_localize(const fm_mask* global, int32_t seqlen_k, int32_t seqlen_q_global,
                           const int32_t* chunk_start, const int32_t* chunk_len, int32_t num_chunks,
                           int32_t* const out[4], hipStream_t stream) {
  fm::MaskArgs mk;
  if (!global) return fail(FM_ERR_INVALID_ARGUMENT, "mask is NULL");
  fm_status st = check_mask(global, global->batch, global->heads, &mk);
  if (st != FM_OK) return st;
  if (global->batch < 1 || global->heads < 1 || (int64_t)global->batch * global->heads > 65535)
    return fail(FM_ERR_INVALID_ARGUMENT, "mask batch*heads must be in [1, 65535]");
  if (seqlen_k < 1 || seqlen_k > kMaxSeq) return fail(FM_ERR_INVALID_ARGUMENT, "seqlen_k out of range");
  if (seqlen_q_global < 1 || seqlen_q_global > kMaxSeq)
    return fail(FM_ERR_INVALID_ARGUMENT, "seqlen_q_global out of range");
  if (num_chunks < 1 || num_chunks > fm::kMaxChunks)
    return fail(FM_ERR_INVALID_ARGUMENT, "num_chunks must be in [1, %d]", fm::kMaxChunks);
  if (!chunk_start || !chunk_len) return fail(FM_ERR_INVALID_ARGUMENT, "chunk list is NULL");
  if (!out) return fail(FM_ERR_INVALID_ARGUMENT, "out is NULL");
  fm::LocalizeArgs a{};
  a.mask = mk;
  a.seq_k = seqlen_k;
  a.seq_q_global = seqlen_q_global;
  a.num_chunks = num_chunks;
  int64_t prev_end = 0, off = 0;
  for (int c = 0; c < num_chunks; ++c) {
    const int64_t s = chunk_start[c], l = chunk_len[c];
    if (l < 1) return fail(FM_ERR_INVALID_ARGUMENT, "chunk %d has length %lld", c, (long long)l);
    if (s < prev_end)
      return fail(FM_ERR_INVALID_ARGUMENT, "chunk %d starts at %lld: chunks must ascend without overlap", c,
                  (long long)s);
    if (s + l > seqlen_q_global)
      return fail(FM_ERR_INVALID_ARGUMENT, "chunk %d ends past seqlen_q_global", c);
    a.chunk_start[c] = (int32_t)s;
    a.chunk_len[c] = (int32_t)l;
    a.chunk_off[c] = (int32_t)off;
    off += l;
    prev_end = s + l;
  }
  for (int i = 0; i < 4; ++i) {
    const bool need = i < 2 ? mk.has_lower : mk.has_upper;
    if (need && !out[i]) return fail(FM_ERR_INVALID_ARGUMENT, "out[%d] is NULL", i);
    if (need && reinterpret_cast<uintptr_t>(out[i]) % 4)
      return fail(FM_ERR_INVALID_ARGUMENT, "out[%d] not 4-byte aligned", i);
    a.out[i] = out[i];
  }
  hipError_t e = run_stage(FM_STAGE_LOCALIZE, stream, [&] { return fm::launch_localize(a, stream); });
  if (e != hipSuccess) return hip_fail(e, "localize launch");
  return FM_OK;
}

fm_status fm_chunk_work(const fm_mask* global, int32_t seqlen_k, int32_t seqlen_q_global,
                        const int32_t* chunk_start, const int32_t* chunk_len, int32_t num_chunks, int64_t* work,
                        hipStream_t stream) {
  fm::MaskArgs mk;
  if (!global) return fail(FM_ERR_INVALID_ARGUMENT, "mask is NULL");
  fm_status st = check_mask(global, global->batch, global->heads, &mk);
  if (st != FM_OK) return st;
  if (global->batch < 1 || global->heads < 1 || (int64_t)global->batch * global->heads > 65535)
    return fail(FM_ERR_INVALID_ARGUMENT, "mask batch*heads must be in [1, 65535]");
  if (seqlen_k < 1 || seqlen_k > kMaxSeq) return fail(FM_ERR_INVALID_ARGUMENT, "seqlen_k out of range");
  if (seqlen_q_global < 1 || seqlen_q_global > kMaxSeq)
    return fail(FM_ERR_INVALID_ARGUMENT, "seqlen_q_global out of range");
  if (num_chunks < 1 || num_chunks > fm::kMaxChunks)
    return fail(FM_ERR_INVALID_ARGUMENT, "num_chunks must be in [1, %d]", fm::kMaxChunks);
  if (!chunk_start || !chunk_len) return fail(FM_ERR_INVALID_ARGUMENT, "chunk list is NULL");
  if (!work || reinterpret_cast<uintptr_t>(work) % 8) return fail(FM_ERR_INVALID_ARGUMENT, "work is NULL or not 8-byte aligned");
  fm::ChunkWorkArgs a{};
  a.mask = mk;
  a.seq_k = seqlen_k;
  a.num_chunks = num_chunks;
  int64_t prev_end = 0;
  for (int c = 0; c < num_chunks; ++c) {
    const int64_t s = chunk_start[c], l = chunk_len[c];
    if (l < 1) return fail(FM_ERR_INVALID_ARGUMENT, "chunk %d has length %lld", c, (long long)l);
    if (s < prev_end)
      return fail(FM_ERR_INVALID_ARGUMENT, "chunk %d starts at %lld: chunks must ascend without overlap", c,
                  (long long)s);
    if (s + l > seqlen_q_global) return fail(FM_ERR_INVALID_ARGUMENT, "chunk %d ends past seqlen_q_global", c);
    a.chunk_start[c] = (int32_t)s;
    a.chunk_len[c] = (int32_t)l;
    prev_end = s + l;
  }
  a.work = work;
  hipError_t e = run_stage(FM_STAGE_CHUNK_WORK, stream, [&] { return fm::launch_chunk_work(a, stream); });
  if (e != hipSuccess) return hip_fail(e, "chunk work launch");
  return FM_OK;
}

fm_status fm_cp_plan(const int64_t* chunk_work, int32_t num_chunks, int32_t num_ranks, int32_t* rank_of_chunk,
                     int64_t* max_load) {
  if (!chunk_work || !rank_of_chunk) return fail(FM_ERR_INVALID_ARGUMENT, "chunk_work or rank_of_chunk is NULL");
  if (num_ranks < 1 || num_chunks < 1 || num_chunks > 4096 || num_chunks % num_ranks)
    return fail(FM_ERR_INVALID_ARGUMENT, "num_chunks (%d) must be a multiple of num_ranks (%d), at most 4096",
                num_chunks, num_ranks);
  for (int c = 0; c < num_chunks; ++c)
    if (chunk_work[c] < 0) return fail(FM_ERR_INVALID_ARGUMENT, "chunk_work[%d] is negative", c);
  const int64_t m = fm::plan_chunks(chunk_work, num_chunks, num_ranks, rank_of_chunk);
  if (max_load) *max_load = m;
  return FM_OK;
}

fm_status fm_kv_transfer_set(const fm_mask* mask, int32_t seqlen_q, int32_t seqlen_k, int32_t block_k,
                             uint8_t* need, int32_t* count, hipStream_t stream) {
  fm::MaskArgs mk;
  if (!mask) return fail(FM_ERR_INVALID_ARGUMENT, "mask is NULL");
  fm_status st = check_mask(mask, mask->batch, mask->heads, &mk);
  if (st != FM_OK) return st;
  if (mask->batch < 1 || mask->heads < 1 || (int64_t)mask->batch * mask->heads > 65535)
    return fail(FM_ERR_INVALID_ARGUMENT, "mask batch*heads must be in [1, 65535]");
  if (seqlen_q < 1 || seqlen_q > kMaxSeq) return fail(FM_ERR_INVALID_ARGUMENT, "seqlen_q out of range");
  if (seqlen_k < 1 || seqlen_k > kMaxSeq) return fail(FM_ERR_INVALID_ARGUMENT, "seqlen_k out of range");
  if (block_k < 1 || block_k > (1 << 30)) return fail(FM_ERR_INVALID_ARGUMENT, "block_k must be in [1, 2^30]");
  if (!need) return fail(FM_ERR_INVALID_ARGUMENT, "need is NULL");
  if (count && reinterpret_cast<uintptr_t>(count) % 4) return fail(FM_ERR_INVALID_ARGUMENT, "count not 4-byte aligned");
  fm::TransferArgs a{};
  a.mask = mk;
  a.seq_q = seqlen_q;
  a.seq_k = seqlen_k;
  a.block_k = block_k;
  a.tk = (int32_t)ceil_div(seqlen_k, block_k);
  a.need = need;
  a.count = count;
  hipError_t e = run_stage(FM_STAGE_TRANSFER, stream, [&] { return fm::launch_transfer_set(a, stream); });
  if (e != hipSuccess) return hip_fail(e, "transfer set launch");
  return FM_OK;
}

fm_status fm_profile_begin(int32_t max_launches) {
  if (max_launches < 1 || max_launches > (1 << 20))
    return fail(FM_ERR_INVALID_ARGUMENT, "max_launches must be in [1, 2^20]");
  if ((int)g_prof.ev.size() < 2 * max_launches) {
    for (hipEvent_t e : g_prof.ev)
      if (e) (void)hipEventDestroy(e);
    g_prof.ev.assign(2 * max_launches, nullptr);
    for (auto& e : g_prof.ev) {
      hipError_t err = hipEventCreate(&e);
      if (err != hipSuccess) return hip_fail(err, "hipEventCreate");
    }
  }
  g_prof.stage.assign(max_launches, 0);
  g_prof.cap = max_launches;
  g_prof.used = 0;
  g_prof.enabled = true;
  return FM_OK;
}

fm_status fm_profile_end(float* total_ms, int32_t* launches) {
  if (!g_prof.enabled) return fail(FM_ERR_INVALID_ARGUMENT, "profiling was not started");
  g_prof.enabled = false;
  float tot[FM_NUM_STAGES] = {0};
  int32_t cnt[FM_NUM_STAGES] = {0};
  for (int i = 0; i < g_prof.used; ++i) {
    hipError_t e = hipEventSynchronize(g_prof.ev[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    tot[g_prof.stage[i]] += ms;
    cnt[g_prof.stage[i]] += 1;
  }
  for (int s = 0; s < FM_NUM_STAGES; ++s) {
    if (total_ms) total_ms[s] = tot[s];
    if (launches) launches[s] = cnt[s];
  }
  return FM_OK;
}

}  // extern "C"
