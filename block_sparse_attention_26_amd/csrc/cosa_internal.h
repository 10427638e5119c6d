// Internal interface between the C-ABI host layer (cosa_api.cpp) and the HIP
// kernels (osk.hip, kap.hip). Not installed; the public ABI is include/cosa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cosa {

// Workgroups are dispatched round-robin over the MI355X's 8 XCDs (each with
// its own L2); launch mappings group units that share K/V pages per XCD.
constexpr int kNumXcd = 8;
constexpr int kNumCu = 256;  // compute units of one MI355X
// KV groups the attention walks at a time (its launch order): every XCD works
// on each group of a phase instead of owning one group for the whole launch,
// which evens the XCDs' shares; at 128K tokens four groups' bf16 K and V
// (256 MB) also fit the MI355X's last-level cache.
constexpr int kPhaseGroups = 4;

// Largest KV-block count per sequence the proxy's in-LDS sort handles.
constexpr int kMaxSortBlocks = 4096;

struct SeqArgs {
  const int32_t* cu_seqlens_q;  // [batch+1]
  const int32_t* seqlens_k;     // [batch]
  const int32_t* block_table;   // [batch, max_blocks_k]
  int32_t batch, h_q, h_kv, group, max_blocks_k, num_pages;
  int32_t max_nq, max_nk;
  // element strides of q and o: token, head (head_dim is contiguous)
  int64_t q_tok, q_head, o_tok, o_head;
};

// Ordered-skip / dense attention launch.
struct OskArgs {
  SeqArgs seq;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const int32_t* order;  // [batch, h_kv, max_nq, kmax] (null for dense)
  const int32_t* count;  // [batch, h_kv, max_nq]      (null for dense)
  int32_t* visited;      // [batch, h_q, max_nq]       (null for dense)
  int32_t* skipped;      // [batch, h_q, max_nq]       (null for dense)
  uint8_t* skip_bits;    // [batch, h_q, max_nq, kmax] (nullable)
  float* lse;            // [h_q, total_q]             (nullable)
  const uint64_t* mask;  // [batch, h_kv, max_nq, mask_words] binary block mask (mask walk only)
  int32_t mask_words;
  int32_t total_q;
  int32_t kmax;
  float scale;           // softmax scale
  float scale_log2;      // softmax scale * log2(e)
  float skip_thr_raw;    // ln(tau) / scale: threshold on raw q.k differences
  int32_t skip_on;       // tau > 0
  int64_t n_units;       // batch * h_q * max_nq
};

// Proxy launches.
struct KapArgs {
  SeqArgs seq;
  const void* q;
  const void* k;
  void* q_pool;          // [batch, max_nr, h_q, d]   (dtype)
  void* k_pool;          // [num_pages, h_kv, B/p, d] (dtype)
  float* scores;         // P: [batch, h_q, max_nr, max_nk] fp32
  int32_t fill_scores;   // 1: write -inf into every non-visible entry of P
  float* block_scores;   // nullable [batch, h_kv, max_nq, max_nk]
  float* row_max;        // nullable [batch, h_q, max_nr]: row maxima of P from the score pass
  int32_t* order;        // [batch, h_kv, max_nq, kmax]
  uint8_t* hrm;          // [batch, h_kv, max_nq, kmax]
  int32_t* count;        // [batch, h_kv, max_nq]
  int32_t pool;
  int32_t max_nr;
  int32_t kmax;
  double budget;
  float scale;
  int32_t keys_pooled;     // k_pool already holds the pooled keys: skip key pooling
  int32_t pool_last_only;  // key pooling: only the last KV block of each sequence
  int32_t score_splits;    // score pass: workgroups sharing one key range (set by the launcher)
};

// The proxy scores a problem with one pooled query row per sequence (a decode
// step) with the group's query heads as MFMA columns; that pass leaves the
// row maxima to the rank pass.
inline bool kap_decode_scores(int max_nr, int group, int per, int dtype) {
  return max_nr == 1 && group <= 32 && per >= 4 && per <= 32 && dtype == 1;
}

// Mask <-> list conversions (one wave per row of batch * h_kv * max_nq).
struct MaskArgs {
  SeqArgs seq;
  int32_t block;
  int64_t n_rows;
  int32_t mask_words;        // <= 64
  int32_t kmax;
  const int32_t* order;      // list -> mask input
  const int32_t* count;
  uint64_t* mask_out;
  const uint64_t* mask_in;   // mask -> list input (null: every causal block)
  int32_t* order_out;
  int32_t* count_out;
  int32_t kmax_out;          // union tables: width of order_out
};

// Exact block attention mass (one workgroup per batch * h_q * max_nq unit).
struct MassArgs {
  SeqArgs seq;
  const void* q;
  const void* k;
  const float* lse;   // [h_q, total_q] natural-log sum-exp per row
  float* mass;        // [batch, h_q, max_nq, max_nk]
  int32_t total_q;
  float scale_log2;
  int64_t n_units;
};

// Decode-stage walk: one workgroup per (sequence, KV group, list segment),
// then one wave per (sequence, query head) merging the segments.
struct DecodeArgs {
  SeqArgs seq;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const int32_t* order;    // [batch, h_kv, max_nq (= 1), kmax]
  const int32_t* count;    // [batch, h_kv, max_nq]
  int32_t* visited;        // [batch, h_q, max_nq]
  int32_t* skipped;        // [batch, h_q, max_nq]
  float* lse;              // [h_q, total_q] (nullable)
  float* part;             // [batch, h_q, n_splits, D + 2]: acc, running max, sum
  int32_t* part_counts;    // [batch, h_q, n_splits, 2]: visited, skipped
  int32_t total_q;
  int32_t kmax;
  int32_t n_splits;
  float scale;
  float scale_log2;
  float skip_thr_raw;
  int32_t skip_on;
};

// Each launcher returns hipSuccess or the launch error. `dtype` is cosa_dtype.
hipError_t launch_osk(const OskArgs& a, int dtype, int head_dim, int block, bool dense,
                      hipStream_t stream);
hipError_t launch_osk_bf16(const OskArgs& a, int head_dim, int block, bool dense, hipStream_t stream);
hipError_t launch_kap(const KapArgs& a, int dtype, int head_dim, int block, hipStream_t stream);
// single stages: query pooling (bf16) and the rank/sort pass over given scores
hipError_t launch_kap_pool_q(const KapArgs& a, int dtype, int head_dim, hipStream_t stream);
hipError_t launch_kap_rank(const KapArgs& a, int block, hipStream_t stream);
hipError_t launch_kap_pool_k(const KapArgs& a, int dtype, int head_dim, int block, hipStream_t stream);
hipError_t launch_cobs_scores(const KapArgs& a, int head_dim, int block, hipStream_t stream);
hipError_t launch_mask_from_order(const MaskArgs& a, hipStream_t stream);
hipError_t launch_order_from_mask(const MaskArgs& a, hipStream_t stream);
hipError_t launch_union_order(const MaskArgs& a, hipStream_t stream);
hipError_t launch_block_mass(const MassArgs& a, int head_dim, int block, hipStream_t stream);
hipError_t launch_osk_decode(const DecodeArgs& a, int head_dim, int block, hipStream_t stream);

}  // namespace cosa
