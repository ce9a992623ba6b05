// zl_api.cpp -- the C ABI of libzl_attn.so: argument validation, workspace
// layout and kernel dispatch.  Validation runs before any HIP call, so a bad
// argument never touches the device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "zl_attn.h"
#include "zl_kernels.h"

namespace {

using zl::Layout;

constexpr int kMaxBatch = 1 << 22;
constexpr int kMaxHeads = 1 << 12;
constexpr int kMaxWorkers = 1 << 16;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WsLayout {
  size_t lse_off, out_off, total;
};

// Workspace: [part_lse 2P*32 f32][part_o 2P*cols*Dv f32], each part 256-byte
// aligned: two fp32 partial slots of `cols` query columns per worker (16; 32
// for MLA, whose tiles may serve 32 query rows; see zl_split.h for which run
// writes which slot).
int max_slot_cols(int dv) { return dv == 512 ? zl::kMlaSlotCols : zl::kHeadsPerUnit; }

WsLayout ws_layout(int workers, int dv) {
  WsLayout w;
  w.lse_off = 0;
  w.out_off = round_up((size_t)2 * workers * zl::kLseSlot * 4, 256);
  w.total = w.out_off + round_up((size_t)2 * workers * max_slot_cols(dv) * dv * 4, 256);
  return w;
}

int head_blocks(int group) { return group <= zl::kHeadsPerUnit ? 1 : group / zl::kHeadsPerUnit; }

bool group_ok(int group) {
  return group >= 1 && (group <= zl::kHeadsPerUnit || group % zl::kHeadsPerUnit == 0);
}

int pick_workers(int requested, Layout layout) {
  return requested > 0 ? requested : zl::default_workers(layout);
}

bool workers_ok(int w) { return w >= 8 && w <= kMaxWorkers && w % 8 == 0; }

// Shared shape checks; returns ZL_OK or the status to report.
zl_status_t check_common(int batch, int num_q_heads, int num_kv_heads, int max_seqlen_k,
                         int dtype, int workers) {
  if (batch < 0 || batch > kMaxBatch) return ZL_ERR_INVALID_ARGUMENT;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads > kMaxHeads) return ZL_ERR_INVALID_ARGUMENT;
  if (num_q_heads % num_kv_heads != 0) return ZL_ERR_INVALID_ARGUMENT;
  if (max_seqlen_k < 0) return ZL_ERR_INVALID_ARGUMENT;
  if (dtype != ZL_DTYPE_F16 && dtype != ZL_DTYPE_BF16) return ZL_ERR_INVALID_ARGUMENT;
  if (!workers_ok(workers)) return ZL_ERR_INVALID_ARGUMENT;
  if (!group_ok(num_q_heads / num_kv_heads)) return ZL_ERR_UNSUPPORTED;
  return ZL_OK;
}

size_t gqa_ws_size(int batch, int num_q_heads, int num_kv_heads, int head_dim, int max_seqlen_k,
                   int dtype, int num_workers) {
  if (head_dim != 64 && head_dim != 128) return 0;
  const Layout layout = head_dim == 128 ? zl::kGqaD128 : zl::kGqaD64;
  const int P = pick_workers(num_workers, layout);
  if (check_common(batch, num_q_heads, num_kv_heads, max_seqlen_k, dtype, P) != ZL_OK) return 0;
  return ws_layout(P, head_dim).total;
}

size_t mla_ws_size(int batch, int num_q_heads, int kv_lora_rank, int rope_dim, int max_seqlen_k,
                   int dtype, int num_workers) {
  if (kv_lora_rank != 512 || rope_dim != 64) return 0;
  const int P = pick_workers(num_workers, zl::kMla576);
  if (check_common(batch, num_q_heads, 1, max_seqlen_k, dtype, P) != ZL_OK) return 0;
  return ws_layout(P, kv_lora_rank).total;
}

zl_status_t run_decode(zl::DecodeArgs a, Layout layout, int dv, int dtype, int phases,
                       void* workspace, size_t workspace_bytes, zl_stream_t stream, int max_vseqs = 0) {
  const WsLayout wl = ws_layout(a.P, dv);
  if (workspace == nullptr || !aligned(workspace, 256)) return ZL_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < wl.total) return ZL_ERR_WORKSPACE_TOO_SMALL;
  char* ws = static_cast<char*>(workspace);
  a.part_lse = reinterpret_cast<float*>(ws + wl.lse_off);
  a.part_o = reinterpret_cast<float*>(ws + wl.out_off);
  a.seg_cost = layout == zl::kMla576 ? zl::kSegCostMla : zl::kSegCostGqa;
  // Slot width the kernels write: 32 columns only for MLA with several new
  // tokens per sequence (the workspace is sized for the widest).
  const bool wide = layout == zl::kMla576 && a.cu_q != nullptr;
  a.slot_cols = wide ? zl::kMlaSlotCols : zl::kHeadsPerUnit;
  a.rows_log2 = wide ? zl::kMlaMqRowsLog2 : zl::kMqRowsLog2;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (phases & 1) e = zl::launch_decode(a, layout, dtype, st);
  if (e == hipSuccess && (phases & 2)) e = zl::launch_merge(a, dv, dtype, max_vseqs, st);
  return e == hipSuccess ? ZL_OK : ZL_ERR_HIP;
}

}  // namespace

extern "C" {

size_t zl_decode_attn_workspace_size(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                     int max_seqlen_k, int dtype) {
  return gqa_ws_size(batch, num_q_heads, num_kv_heads, head_dim, max_seqlen_k, dtype, 0);
}

size_t zl_decode_attn_workspace_size_ex(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                        int max_seqlen_k, int dtype, int num_workers) {
  if (num_workers < 0) return 0;
  return gqa_ws_size(batch, num_q_heads, num_kv_heads, head_dim, max_seqlen_k, dtype, num_workers);
}

}  // extern "C"

namespace {

// Paging parameters: a block table, its row length and the page size (a power
// of two, 16 .. 256 tokens; tiles of 32 tokens then touch at most 3 pages).
struct Paging {
  const int32_t* table = nullptr;
  int max_pages = 0;
  int page_size = 0;
};

// Several new query tokens per sequence: their bounds, count and mask.
struct Varlen {
  const int32_t* cu_q = nullptr;
  int total_q = 0;
  int causal = 0;
};

// Upper bound on the virtual sequences (blocks of R = 2^rows_log2 query rows
// of one sequence) of a call: sum over b of ceil(nq_b * G / R).
long long max_virtual_seqs(const Varlen& vl, int batch, int group, int rows_log2) {
  const long long R = 1LL << rows_log2;
  return ((long long)vl.total_q * group + (R - 1) * batch + R - 1) / R;
}

// Positions of the work line (tokens, or virtual tokens, plus the
// per-sequence cost) are 32-bit inside the kernels.  The kernels clamp every
// cache length to max_seqlen_k, so the bound holds whatever cu_seqlens holds.
zl_status_t check_varlen(const Varlen& vl, int batch, int group, int max_seqlen_k, int seg_cost,
                         int rows_log2) {
  if (!vl.cu_q)
    return (long long)batch * ((long long)max_seqlen_k + seg_cost) >= (1LL << 31) ? ZL_ERR_UNSUPPORTED : ZL_OK;
  if (!aligned(vl.cu_q, 4) || vl.total_q < 0 || (vl.causal != 0 && vl.causal != 1))
    return ZL_ERR_INVALID_ARGUMENT;
  const long long V = max_virtual_seqs(vl, batch, group, rows_log2);
  if (V * ((long long)max_seqlen_k + seg_cost) >= (1LL << 31)) return ZL_ERR_UNSUPPORTED;
  return ZL_OK;
}

zl_status_t check_paging(const Paging& pg, int max_seqlen_k, int& shift) {
  shift = 0;
  if (!pg.table) return ZL_OK;
  if (!aligned(pg.table, 4)) return ZL_ERR_INVALID_ARGUMENT;
  if (pg.page_size < 16 || pg.page_size > 256 || (pg.page_size & (pg.page_size - 1)) != 0)
    return ZL_ERR_UNSUPPORTED;
  if (pg.max_pages < 1 || pg.max_pages > (1 << 24)) return ZL_ERR_INVALID_ARGUMENT;
  if ((long long)max_seqlen_k > (long long)pg.max_pages * pg.page_size) return ZL_ERR_INVALID_ARGUMENT;
  while ((1 << shift) < pg.page_size) ++shift;
  return ZL_OK;
}

zl_status_t gqa_impl(const void* q, const void* k_cache, const void* v_cache, const Paging& pg, const Varlen& vl,
                     const int32_t* cu_seqlens, int batch, int num_q_heads, int num_kv_heads, int head_dim,
                     int max_seqlen_k, float softmax_scale, int dtype, void* out, float* lse,
                     int num_workers, int phases, void* workspace, size_t workspace_bytes,
                     zl_stream_t stream) {
  if (num_workers < 0 || phases < 1 || phases > 3) return ZL_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) {
    if (head_dim <= 0) return ZL_ERR_INVALID_ARGUMENT;
    return ZL_ERR_UNSUPPORTED;
  }
  const Layout layout = head_dim == 128 ? zl::kGqaD128 : zl::kGqaD64;
  const int P = pick_workers(num_workers, layout);
  const zl_status_t st = check_common(batch, num_q_heads, num_kv_heads, max_seqlen_k, dtype, P);
  if (st != ZL_OK) return st;
  if (!std::isfinite(softmax_scale)) return ZL_ERR_INVALID_ARGUMENT;
  int shift = 0;
  const zl_status_t sp = check_paging(pg, max_seqlen_k, shift);
  if (sp != ZL_OK) return sp;
  const zl_status_t sv = check_varlen(vl, batch, num_q_heads / num_kv_heads, max_seqlen_k, zl::kSegCostGqa,
                                       zl::kMqRowsLog2);
  if (sv != ZL_OK) return sv;
  if (batch == 0 || (vl.cu_q && vl.total_q == 0)) return ZL_OK;
  // k_cache / v_cache may be NULL only when every sequence is empty (the
  // kernel never reads a cache row then); the host cannot see the lengths.
  if (!q || !cu_seqlens || !out) return ZL_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(cu_seqlens, 4) || !aligned(lse, 4))
    return ZL_ERR_INVALID_ARGUMENT;
  zl::DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.v = static_cast<const uint16_t*>(v_cache);
  a.cu = cu_seqlens;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.B = batch;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.G = num_q_heads / num_kv_heads;
  a.HB = vl.cu_q ? 1 : head_blocks(a.G);
  a.P = P;
  a.block_table = pg.table;
  a.max_pages = pg.max_pages;
  a.page_shift = shift;
  a.cu_q = vl.cu_q;
  a.causal = vl.causal;
  a.max_len = max_seqlen_k;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  return run_decode(a, layout, head_dim, dtype, phases, workspace, workspace_bytes, stream,
                    (int)max_virtual_seqs(vl, batch, a.G, zl::kMqRowsLog2));
}

}  // namespace

extern "C" {

zl_status_t zl_decode_attn_gqa_ex(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* cu_seqlens, int batch, int num_q_heads,
                                  int num_kv_heads, int head_dim, int max_seqlen_k,
                                  float softmax_scale, int dtype, void* out, float* lse,
                                  int num_workers, int phases, void* workspace,
                                  size_t workspace_bytes, zl_stream_t stream) {
  return gqa_impl(q, k_cache, v_cache, Paging{}, Varlen{}, cu_seqlens, batch, num_q_heads, num_kv_heads, head_dim,
                  max_seqlen_k, softmax_scale, dtype, out, lse, num_workers, phases, workspace,
                  workspace_bytes, stream);
}

zl_status_t zl_decode_attn_gqa_paged_ex(const void* q, const void* k_pages, const void* v_pages,
                                        const int32_t* block_table, int max_pages_per_seq, int page_size,
                                        const int32_t* cu_seqlens, int batch, int num_q_heads,
                                        int num_kv_heads, int head_dim, int max_seqlen_k,
                                        float softmax_scale, int dtype, void* out, float* lse,
                                        int num_workers, int phases, void* workspace,
                                        size_t workspace_bytes, zl_stream_t stream) {
  if (!block_table) return ZL_ERR_INVALID_ARGUMENT;
  Paging pg;
  pg.table = block_table;
  pg.max_pages = max_pages_per_seq;
  pg.page_size = page_size;
  return gqa_impl(q, k_pages, v_pages, pg, Varlen{}, cu_seqlens, batch, num_q_heads, num_kv_heads, head_dim,
                  max_seqlen_k, softmax_scale, dtype, out, lse, num_workers, phases, workspace,
                  workspace_bytes, stream);
}

zl_status_t zl_decode_attn_gqa_paged(const void* q, const void* k_pages, const void* v_pages,
                                     const int32_t* block_table, int max_pages_per_seq, int page_size,
                                     const int32_t* cu_seqlens, int batch, int num_q_heads,
                                     int num_kv_heads, int head_dim, int max_seqlen_k, float softmax_scale,
                                     int dtype, void* out, float* lse, void* workspace,
                                     size_t workspace_bytes, zl_stream_t stream) {
  return zl_decode_attn_gqa_paged_ex(q, k_pages, v_pages, block_table, max_pages_per_seq, page_size,
                                     cu_seqlens, batch, num_q_heads, num_kv_heads, head_dim, max_seqlen_k,
                                     softmax_scale, dtype, out, lse, 0, 3, workspace, workspace_bytes,
                                     stream);
}

zl_status_t zl_decode_attn_gqa(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* cu_seqlens, int batch, int num_q_heads,
                               int num_kv_heads, int head_dim, int max_seqlen_k,
                               float softmax_scale, int dtype, void* out, float* lse,
                               void* workspace, size_t workspace_bytes, zl_stream_t stream) {
  return zl_decode_attn_gqa_ex(q, k_cache, v_cache, cu_seqlens, batch, num_q_heads, num_kv_heads,
                               head_dim, max_seqlen_k, softmax_scale, dtype, out, lse, 0, 3,
                               workspace, workspace_bytes, stream);
}

size_t zl_decode_attn_mla_workspace_size(int batch, int num_q_heads, int kv_lora_rank, int rope_dim,
                                         int max_seqlen_k, int dtype) {
  return mla_ws_size(batch, num_q_heads, kv_lora_rank, rope_dim, max_seqlen_k, dtype, 0);
}

size_t zl_decode_attn_mla_workspace_size_ex(int batch, int num_q_heads, int kv_lora_rank,
                                            int rope_dim, int max_seqlen_k, int dtype,
                                            int num_workers) {
  if (num_workers < 0) return 0;
  return mla_ws_size(batch, num_q_heads, kv_lora_rank, rope_dim, max_seqlen_k, dtype, num_workers);
}

}  // extern "C"

namespace {

zl_status_t mla_impl(const void* q, const void* kv_cache, const Paging& pg, const Varlen& vl,
                     const int32_t* cu_seqlens, int batch,
                     int num_q_heads, int kv_lora_rank, int rope_dim, int max_seqlen_k, float softmax_scale,
                     int dtype, void* out, float* lse, int num_workers, int phases, void* workspace,
                     size_t workspace_bytes, zl_stream_t stream) {
  if (num_workers < 0 || phases < 1 || phases > 3) return ZL_ERR_INVALID_ARGUMENT;
  if (kv_lora_rank <= 0 || rope_dim < 0) return ZL_ERR_INVALID_ARGUMENT;
  if (kv_lora_rank != 512 || rope_dim != 64) return ZL_ERR_UNSUPPORTED;
  const int P = pick_workers(num_workers, zl::kMla576);
  const zl_status_t st = check_common(batch, num_q_heads, 1, max_seqlen_k, dtype, P);
  if (st != ZL_OK) return st;
  if (!std::isfinite(softmax_scale)) return ZL_ERR_INVALID_ARGUMENT;
  int shift = 0;
  const zl_status_t sp = check_paging(pg, max_seqlen_k, shift);
  if (sp != ZL_OK) return sp;
  const zl_status_t sv = check_varlen(vl, batch, num_q_heads, max_seqlen_k, zl::kSegCostMla, zl::kMlaMqRowsLog2);
  if (sv != ZL_OK) return sv;
  if (batch == 0 || (vl.cu_q && vl.total_q == 0)) return ZL_OK;
  if (!q || !cu_seqlens || !out) return ZL_ERR_INVALID_ARGUMENT;  // kv_cache: see above
  if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(out, 16) || !aligned(cu_seqlens, 4) ||
      !aligned(lse, 4))
    return ZL_ERR_INVALID_ARGUMENT;
  zl::DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(kv_cache);
  a.v = static_cast<const uint16_t*>(kv_cache);
  a.cu = cu_seqlens;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.B = batch;
  a.Hq = num_q_heads;
  a.Hkv = 1;
  a.G = num_q_heads;
  a.HB = vl.cu_q ? 1 : head_blocks(num_q_heads);
  a.P = P;
  a.block_table = pg.table;
  a.max_pages = pg.max_pages;
  a.page_shift = shift;
  a.cu_q = vl.cu_q;
  a.causal = vl.causal;
  a.max_len = max_seqlen_k;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  return run_decode(a, zl::kMla576, kv_lora_rank, dtype, phases, workspace, workspace_bytes, stream,
                    (int)max_virtual_seqs(vl, batch, num_q_heads, zl::kMlaMqRowsLog2));
}

// The prefill calls, packed (pg.table == nullptr) or paged.
zl_status_t prefill_impl(const void* q, const void* k_cache, const void* v_cache, const Paging& pg,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch, int total_q,
                         int num_q_heads, int num_kv_heads, int head_dim, int max_seqlen_k, float softmax_scale,
                         int causal, int dtype, void* out, float* lse, zl_stream_t stream) {
  if (batch < 0 || batch > kMaxBatch || total_q < 0 || max_seqlen_k < 0) return ZL_ERR_INVALID_ARGUMENT;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads > kMaxHeads || num_q_heads % num_kv_heads != 0)
    return ZL_ERR_INVALID_ARGUMENT;
  if (dtype != ZL_DTYPE_F16 && dtype != ZL_DTYPE_BF16) return ZL_ERR_INVALID_ARGUMENT;
  if (causal != 0 && causal != 1) return ZL_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(softmax_scale)) return ZL_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) return head_dim <= 0 ? ZL_ERR_INVALID_ARGUMENT : ZL_ERR_UNSUPPORTED;
  int shift = 0;
  const zl_status_t sp = check_paging(pg, max_seqlen_k, shift);
  if (sp != ZL_OK) return sp;
  const int group = num_q_heads / num_kv_heads;
  // Blocks of R = 2^kPrefillRowsLog2 query rows: sum over b of ceil(nq_b * G / R).
  const long long R = 1LL << zl::kPrefillRowsLog2;
  const long long blocks = ((long long)total_q * group + (R - 1) * batch + R - 1) / R;
  if (blocks * num_kv_heads >= (1LL << 31)) return ZL_ERR_UNSUPPORTED;
  if (batch == 0 || total_q == 0) return ZL_OK;
  if (!q || !cu_seqlens_q || !cu_seqlens_k || !out) return ZL_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4) || !aligned(lse, 4))
    return ZL_ERR_INVALID_ARGUMENT;
  zl::DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.v = static_cast<const uint16_t*>(v_cache);
  a.cu = cu_seqlens_k;
  a.cu_q = cu_seqlens_q;
  a.causal = causal;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.B = batch;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.G = group;
  a.HB = 1;
  a.max_len = max_seqlen_k;
  a.block_table = pg.table;
  a.max_pages = pg.max_pages;
  a.page_shift = shift;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  const hipError_t e =
      zl::launch_prefill(a, head_dim, dtype, (int)blocks, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ZL_OK : ZL_ERR_HIP;
}

}  // namespace

extern "C" {

zl_status_t zl_decode_attn_mla_ex(const void* q, const void* kv_cache, const int32_t* cu_seqlens,
                                  int batch, int num_q_heads, int kv_lora_rank, int rope_dim,
                                  int max_seqlen_k, float softmax_scale, int dtype,
                                  void* out, float* lse, int num_workers, int phases,
                                  void* workspace, size_t workspace_bytes, zl_stream_t stream) {
  return mla_impl(q, kv_cache, Paging{}, Varlen{}, cu_seqlens, batch, num_q_heads, kv_lora_rank, rope_dim, max_seqlen_k,
                  softmax_scale, dtype, out, lse, num_workers, phases, workspace, workspace_bytes, stream);
}

zl_status_t zl_decode_attn_mla_paged_ex(const void* q, const void* kv_pages, const int32_t* block_table,
                                        int max_pages_per_seq, int page_size, const int32_t* cu_seqlens,
                                        int batch, int num_q_heads, int kv_lora_rank, int rope_dim,
                                        int max_seqlen_k, float softmax_scale, int dtype, void* out,
                                        float* lse, int num_workers, int phases, void* workspace,
                                        size_t workspace_bytes, zl_stream_t stream) {
  if (!block_table) return ZL_ERR_INVALID_ARGUMENT;
  Paging pg;
  pg.table = block_table;
  pg.max_pages = max_pages_per_seq;
  pg.page_size = page_size;
  return mla_impl(q, kv_pages, pg, Varlen{}, cu_seqlens, batch, num_q_heads, kv_lora_rank, rope_dim, max_seqlen_k,
                  softmax_scale, dtype, out, lse, num_workers, phases, workspace, workspace_bytes, stream);
}

zl_status_t zl_decode_attn_mla_paged(const void* q, const void* kv_pages, const int32_t* block_table,
                                     int max_pages_per_seq, int page_size, const int32_t* cu_seqlens,
                                     int batch, int num_q_heads, int kv_lora_rank, int rope_dim,
                                     int max_seqlen_k, float softmax_scale, int dtype, void* out,
                                     float* lse, void* workspace, size_t workspace_bytes, zl_stream_t stream) {
  return zl_decode_attn_mla_paged_ex(q, kv_pages, block_table, max_pages_per_seq, page_size, cu_seqlens, batch,
                                     num_q_heads, kv_lora_rank, rope_dim, max_seqlen_k, softmax_scale, dtype, out,
                                     lse, 0, 3, workspace, workspace_bytes, stream);
}

zl_status_t zl_decode_attn_mla(const void* q, const void* kv_cache, const int32_t* cu_seqlens,
                               int batch, int num_q_heads, int kv_lora_rank, int rope_dim,
                               int max_seqlen_k, float softmax_scale, int dtype, void* out,
                               float* lse, void* workspace, size_t workspace_bytes,
                               zl_stream_t stream) {
  return zl_decode_attn_mla_ex(q, kv_cache, cu_seqlens, batch, num_q_heads, kv_lora_rank, rope_dim,
                               max_seqlen_k, softmax_scale, dtype, out, lse, 0, 3, workspace,
                               workspace_bytes, stream);
}

zl_status_t zl_attn_varlen_gqa_ex(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch, int total_q,
                                  int num_q_heads, int num_kv_heads, int head_dim, int max_seqlen_k,
                                  float softmax_scale, int causal, int dtype, void* out, float* lse,
                                  int num_workers, int phases, void* workspace, size_t workspace_bytes,
                                  zl_stream_t stream) {
  if (!cu_seqlens_q) return ZL_ERR_INVALID_ARGUMENT;
  Varlen vl;
  vl.cu_q = cu_seqlens_q;
  vl.total_q = total_q;
  vl.causal = causal;
  return gqa_impl(q, k_cache, v_cache, Paging{}, vl, cu_seqlens_k, batch, num_q_heads, num_kv_heads, head_dim,
                  max_seqlen_k, softmax_scale, dtype, out, lse, num_workers, phases, workspace, workspace_bytes,
                  stream);
}

zl_status_t zl_attn_varlen_gqa(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch, int total_q,
                               int num_q_heads, int num_kv_heads, int head_dim, int max_seqlen_k,
                               float softmax_scale, int causal, int dtype, void* out, float* lse,
                               void* workspace, size_t workspace_bytes, zl_stream_t stream) {
  return zl_attn_varlen_gqa_ex(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, batch, total_q, num_q_heads,
                               num_kv_heads, head_dim, max_seqlen_k, softmax_scale, causal, dtype, out, lse, 0, 3,
                               workspace, workspace_bytes, stream);
}

zl_status_t zl_attn_varlen_mla_ex(const void* q, const void* kv_cache, const int32_t* cu_seqlens_q,
                                  const int32_t* cu_seqlens_k, int batch, int total_q, int num_q_heads,
                                  int kv_lora_rank, int rope_dim, int max_seqlen_k, float softmax_scale, int causal,
                                  int dtype, void* out, float* lse, int num_workers, int phases,
                                  void* workspace, size_t workspace_bytes, zl_stream_t stream) {
  if (!cu_seqlens_q) return ZL_ERR_INVALID_ARGUMENT;
  Varlen vl;
  vl.cu_q = cu_seqlens_q;
  vl.total_q = total_q;
  vl.causal = causal;
  return mla_impl(q, kv_cache, Paging{}, vl, cu_seqlens_k, batch, num_q_heads, kv_lora_rank, rope_dim,
                  max_seqlen_k, softmax_scale, dtype, out, lse, num_workers, phases, workspace, workspace_bytes,
                  stream);
}

zl_status_t zl_attn_varlen_gqa_paged_ex(const void* q, const void* k_pages, const void* v_pages,
                                        const int32_t* block_table, int max_pages_per_seq, int page_size,
                                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                                        int total_q, int num_q_heads, int num_kv_heads, int head_dim,
                                        int max_seqlen_k, float softmax_scale, int causal, int dtype,
                                        void* out, float* lse, int num_workers, int phases, void* workspace,
                                        size_t workspace_bytes, zl_stream_t stream) {
  if (!cu_seqlens_q || !block_table) return ZL_ERR_INVALID_ARGUMENT;
  Paging pg;
  pg.table = block_table;
  pg.max_pages = max_pages_per_seq;
  pg.page_size = page_size;
  Varlen vl;
  vl.cu_q = cu_seqlens_q;
  vl.total_q = total_q;
  vl.causal = causal;
  return gqa_impl(q, k_pages, v_pages, pg, vl, cu_seqlens_k, batch, num_q_heads, num_kv_heads, head_dim,
                  max_seqlen_k, softmax_scale, dtype, out, lse, num_workers, phases, workspace, workspace_bytes,
                  stream);
}

zl_status_t zl_attn_varlen_gqa_paged(const void* q, const void* k_pages, const void* v_pages,
                                     const int32_t* block_table, int max_pages_per_seq, int page_size,
                                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                                     int total_q, int num_q_heads, int num_kv_heads, int head_dim, int max_seqlen_k,
                                     float softmax_scale, int causal, int dtype, void* out, float* lse,
                                     void* workspace, size_t workspace_bytes, zl_stream_t stream) {
  return zl_attn_varlen_gqa_paged_ex(q, k_pages, v_pages, block_table, max_pages_per_seq, page_size, cu_seqlens_q,
                                     cu_seqlens_k, batch, total_q, num_q_heads, num_kv_heads, head_dim,
                                     max_seqlen_k, softmax_scale, causal, dtype, out, lse, 0, 3, workspace,
                                     workspace_bytes, stream);
}

zl_status_t zl_attn_varlen_mla_paged_ex(const void* q, const void* kv_pages, const int32_t* block_table,
                                        int max_pages_per_seq, int page_size, const int32_t* cu_seqlens_q,
                                        const int32_t* cu_seqlens_k, int batch, int total_q, int num_q_heads,
                                        int kv_lora_rank, int rope_dim, int max_seqlen_k, float softmax_scale,
                                        int causal, int dtype, void* out, float* lse, int num_workers,
                                        int phases, void* workspace, size_t workspace_bytes, zl_stream_t stream) {
  if (!cu_seqlens_q || !block_table) return ZL_ERR_INVALID_ARGUMENT;
  Paging pg;
  pg.table = block_table;
  pg.max_pages = max_pages_per_seq;
  pg.page_size = page_size;
  Varlen vl;
  vl.cu_q = cu_seqlens_q;
  vl.total_q = total_q;
  vl.causal = causal;
  return mla_impl(q, kv_pages, pg, vl, cu_seqlens_k, batch, num_q_heads, kv_lora_rank, rope_dim, max_seqlen_k,
                  softmax_scale, dtype, out, lse, num_workers, phases, workspace, workspace_bytes, stream);
}

zl_status_t zl_attn_varlen_mla_paged(const void* q, const void* kv_pages, const int32_t* block_table,
                                     int max_pages_per_seq, int page_size, const int32_t* cu_seqlens_q,
                                     const int32_t* cu_seqlens_k, int batch, int total_q, int num_q_heads,
                                     int kv_lora_rank, int rope_dim, int max_seqlen_k, float softmax_scale,
                                     int causal, int dtype, void* out, float* lse, void* workspace,
                                     size_t workspace_bytes, zl_stream_t stream) {
  return zl_attn_varlen_mla_paged_ex(q, kv_pages, block_table, max_pages_per_seq, page_size, cu_seqlens_q,
                                     cu_seqlens_k, batch, total_q, num_q_heads, kv_lora_rank, rope_dim,
                                     max_seqlen_k, softmax_scale, causal, dtype, out, lse, 0, 3, workspace,
                                     workspace_bytes, stream);
}

zl_status_t zl_attn_varlen_mla(const void* q, const void* kv_cache, const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k, int batch, int total_q, int num_q_heads,
                               int kv_lora_rank, int rope_dim, int max_seqlen_k, float softmax_scale, int causal,
                               int dtype, void* out, float* lse, void* workspace, size_t workspace_bytes,
                               zl_stream_t stream) {
  return zl_attn_varlen_mla_ex(q, kv_cache, cu_seqlens_q, cu_seqlens_k, batch, total_q, num_q_heads, kv_lora_rank,
                               rope_dim, max_seqlen_k, softmax_scale, causal, dtype, out, lse, 0, 3, workspace,
                               workspace_bytes, stream);
}

zl_status_t zl_attn_prefill_gqa(const void* q, const void* k_cache, const void* v_cache, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_k, int batch, int total_q, int num_q_heads, int num_kv_heads,
                                int head_dim, int max_seqlen_k, float softmax_scale, int causal, int dtype,
                                void* out, float* lse, zl_stream_t stream) {
  return prefill_impl(q, k_cache, v_cache, Paging{}, cu_seqlens_q, cu_seqlens_k, batch, total_q, num_q_heads,
                      num_kv_heads, head_dim, max_seqlen_k, softmax_scale, causal, dtype, out, lse, stream);
}

zl_status_t zl_attn_prefill_gqa_paged(const void* q, const void* k_pages, const void* v_pages,
                                      const int32_t* block_table, int max_pages_per_seq, int page_size,
                                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                                      int total_q, int num_q_heads, int num_kv_heads, int head_dim, int max_seqlen_k,
                                      float softmax_scale, int causal, int dtype, void* out, float* lse,
                                      zl_stream_t stream) {
  if (!block_table) return ZL_ERR_INVALID_ARGUMENT;  // (the packed call serves that case)
  return prefill_impl(q, k_pages, v_pages, Paging{block_table, max_pages_per_seq, page_size}, cu_seqlens_q,
                      cu_seqlens_k, batch, total_q, num_q_heads, num_kv_heads, head_dim, max_seqlen_k, softmax_scale,
                      causal, dtype, out, lse, stream);
}

zl_status_t zl_attn_combine(const float* partial_out, const float* partial_lse, int num_splits,
                            int batch, int num_heads, int head_dim_v, int out_dtype,
                            void* out, float* lse, zl_stream_t stream) {
  if (num_splits < 1 || num_splits > 1024) return ZL_ERR_INVALID_ARGUMENT;
  if (batch < 0 || batch > kMaxBatch || num_heads <= 0 || num_heads > kMaxHeads)
    return ZL_ERR_INVALID_ARGUMENT;
  if (head_dim_v < 4 || head_dim_v > 4096 || head_dim_v % 4 != 0) return ZL_ERR_INVALID_ARGUMENT;
  if (out_dtype != ZL_DTYPE_F16 && out_dtype != ZL_DTYPE_BF16) return ZL_ERR_INVALID_ARGUMENT;
  if (batch == 0) return ZL_OK;
  if (!partial_out || !partial_lse || !out) return ZL_ERR_INVALID_ARGUMENT;
  if (!aligned(partial_out, 16) || !aligned(partial_lse, 4) || !aligned(out, 8) || !aligned(lse, 4))
    return ZL_ERR_INVALID_ARGUMENT;
  const long long rows = (long long)batch * num_heads;
  if (rows > (1LL << 30)) return ZL_ERR_INVALID_ARGUMENT;
  zl::CombineArgs a{};
  a.part_o = partial_out;
  a.part_lse = partial_lse;
  a.out = out;
  a.lse = lse;
  a.S = num_splits;
  a.rows = (int)rows;
  a.Dv = head_dim_v;
  const hipError_t e = zl::launch_combine(a, out_dtype, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ZL_OK : ZL_ERR_HIP;
}

}  // extern "C"

namespace {

constexpr long long kMaxCodecElems = 1LL << 40;

bool codec_chunk_ok(int chunk) { return chunk == 256 || chunk == 512 || chunk == 1024; }

zl_status_t run_codec(const zl::CodecArgs& a, int op, int chunk, int dtype, zl_stream_t stream) {
  const hipError_t e = zl::launch_codec(a, op, chunk, dtype, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ZL_OK : ZL_ERR_HIP;
}

}  // namespace

extern "C" {

zl_status_t zl_int8_quantize(const void* x, int dtype, long long n, int chunk, int8_t* codes,
                             float* scales, zl_stream_t stream) {
  if (dtype != ZL_DTYPE_F16 && dtype != ZL_DTYPE_BF16) return ZL_ERR_INVALID_ARGUMENT;
  if (n < 0 || n > kMaxCodecElems) return ZL_ERR_INVALID_ARGUMENT;
  if (!codec_chunk_ok(chunk)) return ZL_ERR_UNSUPPORTED;
  if (n == 0) return ZL_OK;
  if (!x || !codes || !scales) return ZL_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4)) return ZL_ERR_INVALID_ARGUMENT;
  zl::CodecArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.codes_out = codes;
  a.scales_out = scales;
  a.n = n;
  return run_codec(a, zl::kCodecQuantize, chunk, dtype, stream);
}

zl_status_t zl_int8_dequantize(const int8_t* codes, const float* scales, long long n, int chunk, int dtype,
                               void* out, zl_stream_t stream) {
  if (dtype != ZL_DTYPE_F16 && dtype != ZL_DTYPE_BF16) return ZL_ERR_INVALID_ARGUMENT;
  if (n < 0 || n > kMaxCodecElems) return ZL_ERR_INVALID_ARGUMENT;
  if (!codec_chunk_ok(chunk)) return ZL_ERR_UNSUPPORTED;
  if (n == 0) return ZL_OK;
  if (!codes || !scales || !out) return ZL_ERR_INVALID_ARGUMENT;
  if (!aligned(codes, 16) || !aligned(scales, 4) || !aligned(out, 16)) return ZL_ERR_INVALID_ARGUMENT;
  zl::CodecArgs a{};
  a.codes_in = codes;
  a.scales_in = scales;
  a.out16 = static_cast<uint16_t*>(out);
  a.n = n;
  return run_codec(a, zl::kCodecDequantize, chunk, dtype, stream);
}

zl_status_t zl_int8_reduce_step(const int8_t* codes_in, const float* scales_in, const void* local, int dtype,
                                long long n, int chunk, int8_t* codes_out, float* scales_out, void* sum_out,
                                zl_stream_t stream) {
  if (dtype != ZL_DTYPE_F16 && dtype != ZL_DTYPE_BF16) return ZL_ERR_INVALID_ARGUMENT;
  if (n < 0 || n > kMaxCodecElems) return ZL_ERR_INVALID_ARGUMENT;
  if (!codec_chunk_ok(chunk)) return ZL_ERR_UNSUPPORTED;
  if ((codes_out == nullptr) != (scales_out == nullptr)) return ZL_ERR_INVALID_ARGUMENT;
  if (!codes_out && !sum_out) return ZL_ERR_INVALID_ARGUMENT;
  if (n == 0) return ZL_OK;
  if (!codes_in || !scales_in || !local) return ZL_ERR_INVALID_ARGUMENT;
  if (!aligned(codes_in, 16) || !aligned(scales_in, 4) || !aligned(local, 16) || !aligned(codes_out, 16) ||
      !aligned(scales_out, 4) || !aligned(sum_out, 16))
    return ZL_ERR_INVALID_ARGUMENT;
  zl::CodecArgs a{};
  a.x = static_cast<const uint16_t*>(local);
  a.codes_in = codes_in;
  a.scales_in = scales_in;
  a.codes_out = codes_out;
  a.scales_out = scales_out;
  a.out16 = static_cast<uint16_t*>(sum_out);
  a.n = n;
  return run_codec(a, zl::kCodecReduce, chunk, dtype, stream);
}

zl_status_t zl_hbm_read_probe(const void* src, size_t bytes, int head_dim_k, int workgroups, uint32_t* sink,
                              zl_stream_t stream) {
  if (head_dim_k != 64 && head_dim_k != 128 && head_dim_k != 576) return ZL_ERR_UNSUPPORTED;
  const int wg = workgroups == 0 ? zl::read_probe_default_workgroups(head_dim_k) : workgroups;
  if (!workers_ok(wg)) return ZL_ERR_INVALID_ARGUMENT;
  if (bytes > ((size_t)1 << 46)) return ZL_ERR_INVALID_ARGUMENT;
  if (bytes < 1024) return ZL_OK;
  if (!src || !sink || !aligned(src, 16) || !aligned(sink, 4)) return ZL_ERR_INVALID_ARGUMENT;
  const hipError_t e =
      zl::launch_read_probe(src, (long long)bytes, head_dim_k, wg, sink, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ZL_OK : ZL_ERR_HIP;
}

const char* zl_status_string(int status) {
  switch (status) {
    case ZL_OK: return "ZL_OK";
    case ZL_ERR_INVALID_ARGUMENT: return "ZL_ERR_INVALID_ARGUMENT";
    case ZL_ERR_UNSUPPORTED: return "ZL_ERR_UNSUPPORTED";
    case ZL_ERR_WORKSPACE_TOO_SMALL: return "ZL_ERR_WORKSPACE_TOO_SMALL";
    case ZL_ERR_HIP: return "ZL_ERR_HIP";
  }
  return "unknown zl_status_t";
}

}  // extern "C"
