// zl_kernels.h -- argument blocks and launchers of the decode kernels
// (internal to libzl_attn.so; the public ABI is include/zl_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace zl {

// Sizes shared by host planning and the kernels.
constexpr int kHeadsPerUnit = 16;  // query heads packed into one MFMA N dimension
// Floats per partial-lse slot: one 128-byte cache line, so no two slots (which
// different XCDs write and read) ever share a line.
constexpr int kLseSlot = 32;
// Rows per virtual sequence with several new tokens per sequence (zl_split.h):
// 16 for the GQA kernels, 32 for MLA, whose tiles then serve two blocks of 16
// query columns.  The MLA partial slots hold 32 columns in every mode.
constexpr int kMqRowsLog2 = 4;
constexpr int kMlaMqRowsLog2 = 5;
constexpr int kMlaSlotCols = 32;
static_assert(kMlaSlotCols <= kLseSlot, "a slot's lse values fit its line");

enum Layout {
  kGqaD64 = 0,   // K, V [T, Hkv, 64]
  kGqaD128 = 1,  // K, V [T, Hkv, 128]
  kMla576 = 2,   // latent [T, 576]; K = row[0:576], V = row[0:512]
};

// One decode call.  For MLA: Hkv = 1, G = Hq, v == k == latent.
struct DecodeArgs {
  const uint16_t* q;    // [B, Hq, Dk]
  const uint16_t* k;    // K rows
  const uint16_t* v;    // V rows
  const int32_t* cu;    // [B + 1]
  uint16_t* out;        // [B, Hq, Dv]
  float* lse;           // [B, Hq] or nullptr
  float* part_o;        // [2P, slot_cols, Dv]
  float* part_lse;      // [2P, kLseSlot] (first slot_cols used)
  // Paged caches (block table): k / v are page pools [pages, 2^page_shift,
  // row]; token i of sequence b lives in page block_table[b*max_pages +
  // (i >> page_shift)], row i & (2^page_shift - 1).  block_table == nullptr:
  // packed caches, token t (cu numbering) is row t.
  const int32_t* block_table;
  int max_pages, page_shift;
  // Several new query tokens per sequence (cu_q != nullptr): q, out are
  // [cu_q[B], Hq, D] and lse [cu_q[B], Hq]; cu holds the cache bounds; the
  // work units are the key/value heads (HB = 1) and the batch is cut into
  // virtual sequences of 2^rows_log2 query rows (zl_split.h).  causal: new token i of
  // nq sees cache rows 0 .. lk - nq + i.
  const int32_t* cu_q;
  int causal;
  int rows_log2;        // rows per virtual sequence: 2^rows_log2 (16 or 32)
  int slot_cols;        // query columns per partial slot (16, or 32 for MLA)
  int B, Hq, Hkv, G, HB, P;
  int seg_cost;         // phantom positions per sequence (zl_split.h)
  int max_len;          // max_seqlen_k: cache lengths are clamped to [0, max_len]
  float scale_log2;     // softmax_scale * log2(e)
};

// Phantom positions per sequence on the work line (the fixed cost of starting
// a sequence in a run, in tokens): measured per-segment overheads of the two
// kernels, rounded.
constexpr int kSegCostGqa = 32;
constexpr int kSegCostMla = 64;

struct CombineArgs {
  const float* part_o;   // [S, rows, Dv]
  const float* part_lse; // [S, rows]
  void* out;             // [rows, Dv] 16-bit
  float* lse;            // [rows] or nullptr
  int S, rows, Dv;
};

// Long runs of new tokens (prefill_attn.hip): blocks of (key/value head,
// 2^kPrefillRowsLog2 query rows), taken in rounds by at most two persistent
// workgroups per CU; max_blocks bounds the blocks of the batch per head.
constexpr int kPrefillRowsLog2 = 7;
hipError_t launch_prefill(const DecodeArgs& a, int head_dim, int dtype, int max_blocks, hipStream_t stream);

// INT8 coding of an all-reduce payload (int8_codec.hip).
enum CodecOp { kCodecQuantize = 0, kCodecDequantize = 1, kCodecReduce = 2 };

struct CodecArgs {
  const uint16_t* x;        // quantize: the payload; reduce: the local values
  const int8_t* codes_in;   // dequantize, reduce
  const float* scales_in;
  int8_t* codes_out;        // quantize; reduce (nullptr: no coding)
  float* scales_out;
  uint16_t* out16;          // dequantize: the values; reduce: the sum (or nullptr)
  long long n;              // elements
};

hipError_t launch_codec(const CodecArgs& a, int op, int chunk, int dtype, hipStream_t stream);

// Workers (one wavefront each, a multiple of 8) a decode call launches.
int default_workers(Layout layout);
int mla_default_workers();
hipError_t launch_mla(const DecodeArgs& a, int dtype, hipStream_t stream);

hipError_t launch_decode(const DecodeArgs& a, Layout layout, int dtype, hipStream_t stream);
// max_vseqs: with several new tokens per sequence, an upper bound on the
// virtual sequences (ignored otherwise).
hipError_t launch_merge(const DecodeArgs& a, int dv, int dtype, int max_vseqs, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, int dtype, hipStream_t stream);

// Plain streaming read at a decode kernel's launch shape (hbm_read.hip):
// head_dim_k 64 / 128 (GQA) or 576 (MLA) picks the shape; workgroups is a
// multiple of 8; sink holds one word per workgroup.
int read_probe_default_workgroups(int head_dim_k);
hipError_t launch_read_probe(const void* src, long long bytes, int head_dim_k, int workgroups, uint32_t* sink,
                             hipStream_t stream);

}  // namespace zl
