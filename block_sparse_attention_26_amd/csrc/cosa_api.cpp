// Host side of libcosa: argument validation, closed-form extents, workspace
// layout and kernel launches. Declarations and contracts: include/cosa.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "../../include/cosa.h"
#include "cosa_internal.h"

// Fixed device scratch of the allocation-free decode entry point
// (cosa_osk_decode_noalloc): each GPU the library runs on holds its own copy
// of this array, at its own address, from the module's load until the process
// ends. Host code never passes `scratch` itself to a kernel (on the host the
// name is only a stand-in); it passes the device address looked up below.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local std::string g_last_error;

cosa_status fail(cosa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

cosa_status ok() {
  g_last_error.clear();
  return COSA_OK;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Budget rule: k = clamp(ceil(beta * n - 1e-9), 1, n) in IEEE double.
int budget_count(int n, double beta) {
  int k = (int)ceil(beta * (double)n - 1e-9);
  return std::max(1, std::min(n, k));
}

// Causal KV blocks of query block qb (kb = 0 .. n-1).
int n_causal(int qb, int B, int Lq, int Lk) {
  const int off = Lk - Lq;
  return (off + std::min(qb * B + B - 1, Lq - 1)) / B + 1;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Element strides of q and o (0 = contiguous).
int64_t q_tok(const cosa_problem* p) { return p->q_stride_tok ? p->q_stride_tok : (int64_t)p->h_q * p->head_dim; }
int64_t q_head(const cosa_problem* p) { return p->q_stride_head ? p->q_stride_head : p->head_dim; }
int64_t o_tok(const cosa_problem* p) { return p->o_stride_tok ? p->o_stride_tok : (int64_t)p->h_q * p->head_dim; }
int64_t o_head(const cosa_problem* p) { return p->o_stride_head ? p->o_stride_head : p->head_dim; }

// Strides in 16-byte units (the kernels move q and o rows in 16-byte pieces)
// and an o layout in which no two elements share memory.
cosa_status check_strides(const cosa_problem* p) {
  const int64_t unit = p->dtype == COSA_BF16 ? 8 : 4;
  const int64_t v[4] = {p->q_stride_tok, p->q_stride_head, p->o_stride_tok, p->o_stride_head};
  const char* name[4] = {"q_stride_tok", "q_stride_head", "o_stride_tok", "o_stride_head"};
  for (int i = 0; i < 4; ++i)
    if (v[i] < 0 || v[i] % unit != 0)
      return fail(COSA_ERR_INVALID_ARG, "%s (%lld) must be >= 0 and a multiple of %lld elements (16 bytes)",
                  name[i], (long long)v[i], (long long)unit);
  // the output dimensions with more than one entry, by increasing stride
  struct Dim { int64_t stride, n; } dims[2] = {{o_tok(p), p->host_cu_seqlens_q[p->batch]}, {o_head(p), p->h_q}};
  if (dims[0].stride > dims[1].stride) std::swap(dims[0], dims[1]);
  int nd = 0;
  Dim live[2];
  for (const Dim& d : dims)
    if (d.n > 1) live[nd++] = d;
  if (nd >= 1 && live[0].stride < p->head_dim)
    return fail(COSA_ERR_INVALID_ARG, "o strides overlap: a stride (%lld) below head_dim (%d)",
                (long long)live[0].stride, p->head_dim);
  if (nd == 2 && live[1].stride < live[0].stride * live[0].n)
    return fail(COSA_ERR_INVALID_ARG, "o strides overlap: stride %lld < %lld x %lld", (long long)live[1].stride,
                (long long)live[0].stride, (long long)live[0].n);
  return COSA_OK;
}

cosa_status check_aligned(const void* ptr, const char* what) {
  if (((uintptr_t)ptr & 15) != 0) return fail(COSA_ERR_INVALID_ARG, "%s must be 16-byte aligned", what);
  return COSA_OK;
}

cosa_status validate(const cosa_problem* p) {
  if (!p) return fail(COSA_ERR_INVALID_ARG, "problem is NULL");
  if (p->batch < 1) return fail(COSA_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", p->batch);
  if (p->h_q < 1 || p->h_kv < 1)
    return fail(COSA_ERR_INVALID_ARG, "h_q and h_kv must be >= 1 (got %d, %d)", p->h_q, p->h_kv);
  if (p->h_q % p->h_kv != 0)
    return fail(COSA_ERR_INVALID_ARG, "h_kv (%d) must divide h_q (%d)", p->h_kv, p->h_q);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(COSA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", p->head_dim);
  if (p->block != 64 && p->block != 128)
    return fail(COSA_ERR_UNSUPPORTED, "block must be 64 or 128 (got %d)", p->block);
  if (p->dtype != COSA_F32 && p->dtype != COSA_BF16)
    return fail(COSA_ERR_INVALID_ARG, "dtype must be COSA_F32 or COSA_BF16 (got %d)", p->dtype);
  if (!(p->softmax_scale > 0.f) || !isfinite(p->softmax_scale))
    return fail(COSA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (p->num_pages < 1) return fail(COSA_ERR_INVALID_ARG, "num_pages must be >= 1");
  if (p->max_blocks_k < 1) return fail(COSA_ERR_INVALID_ARG, "max_blocks_k must be >= 1");
  if (!p->cu_seqlens_q || !p->seqlens_k || !p->block_table)
    return fail(COSA_ERR_INVALID_ARG, "cu_seqlens_q, seqlens_k and block_table must be non-NULL");
  if (!p->host_cu_seqlens_q || !p->host_seqlens_k)
    return fail(COSA_ERR_INVALID_ARG, "host_cu_seqlens_q and host_seqlens_k must be non-NULL");
  if (p->host_cu_seqlens_q[0] != 0) return fail(COSA_ERR_INVALID_ARG, "cu_seqlens_q[0] must be 0");
  for (int b = 0; b < p->batch; ++b) {
    const int64_t lq = (int64_t)p->host_cu_seqlens_q[b + 1] - p->host_cu_seqlens_q[b];
    const int64_t lk = p->host_seqlens_k[b];
    if (lq < 0) return fail(COSA_ERR_INVALID_ARG, "cu_seqlens_q decreases at sequence %d", b);
    if (lk < lq)
      return fail(COSA_ERR_INVALID_ARG, "sequence %d: seqlens_k (%lld) < query length (%lld)", b,
                  (long long)lk, (long long)lq);
    if (cdiv(lk, p->block) > p->max_blocks_k)
      return fail(COSA_ERR_INVALID_ARG, "sequence %d needs %lld KV blocks > max_blocks_k (%d)", b,
                  (long long)cdiv(lk, p->block), p->max_blocks_k);
  }
  return check_strides(p);
}

void compute_dims(const cosa_problem* p, int pool, double budget, cosa_dims_t* d) {
  d->total_q = p->host_cu_seqlens_q[p->batch];
  d->max_nq = d->max_nk = d->max_nr = 0;
  d->kmax = 0;
  for (int b = 0; b < p->batch; ++b) {
    const int lq = p->host_cu_seqlens_q[b + 1] - p->host_cu_seqlens_q[b];
    const int lk = p->host_seqlens_k[b];
    const int nq = (int)cdiv(lq, p->block);
    d->max_nq = std::max(d->max_nq, nq);
    d->max_nk = std::max(d->max_nk, (int)cdiv(lk, p->block));
    if (pool > 0) d->max_nr = std::max(d->max_nr, (int)cdiv(lq, pool));
    if (budget > 0.0 && nq > 0)
      d->kmax = std::max(d->kmax, budget_count(n_causal(nq - 1, p->block, lq, lk), budget));
  }
  if (budget > 0.0) d->kmax = std::max(d->kmax, 1);
}

cosa_status check_pool(const cosa_problem* p, int pool) {
  if (pool < 1 || pool > p->block || p->block % pool != 0)
    return fail(COSA_ERR_INVALID_ARG, "pool (%d) must divide block (%d)", pool, p->block);
  return COSA_OK;
}

size_t kap_ws_size(const cosa_problem* p, int pool, bool with_scores) {
  cosa_dims_t d;
  compute_dims(p, pool, 0.0, &d);
  const size_t es = p->dtype == COSA_BF16 ? 2 : 4;
  size_t sz = align256((size_t)p->batch * d.max_nr * p->h_q * p->head_dim * es);
  sz += align256((size_t)p->num_pages * p->h_kv * (p->block / pool) * p->head_dim * es);
  sz += align256((size_t)p->batch * p->h_q * d.max_nr * sizeof(float));  // row maxima of P
  if (with_scores) sz += align256((size_t)p->batch * p->h_q * d.max_nr * d.max_nk * sizeof(float));
  return sz;
}

size_t decode_ws_size(const cosa_problem* p, int n_splits) {
  return align256((size_t)p->batch * p->h_q * n_splits * (p->head_dim + 2) * sizeof(float)) +
         align256((size_t)p->batch * p->h_q * n_splits * 2 * sizeof(int32_t));
}

cosa::SeqArgs seq_args(const cosa_problem* p, const cosa_dims_t& d) {
  cosa::SeqArgs s;
  s.cu_seqlens_q = p->cu_seqlens_q;
  s.seqlens_k = p->seqlens_k;
  s.block_table = p->block_table;
  s.batch = p->batch;
  s.h_q = p->h_q;
  s.h_kv = p->h_kv;
  s.group = p->h_q / p->h_kv;
  s.max_blocks_k = p->max_blocks_k;
  s.num_pages = p->num_pages;
  s.max_nq = d.max_nq;
  s.max_nk = d.max_nk;
  s.q_tok = q_tok(p);
  s.q_head = q_head(p);
  s.o_tok = o_tok(p);
  s.o_head = o_head(p);
  return s;
}

cosa_status hip_result(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(COSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

cosa_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(COSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(COSA_ERR_UNSUPPORTED, "device %d is beyond the %d devices the scratch table holds", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(COSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return COSA_OK;
}

int32_t min_mask_words(const cosa_problem* p) {
  cosa_dims_t d;
  compute_dims(p, 0, 0.0, &d);
  return (int32_t)cdiv(d.max_nk, 64);
}

cosa_status check_mask_words(const cosa_problem* p, int32_t mask_words, bool capped) {
  const int32_t need = min_mask_words(p);
  if (mask_words < std::max(need, 1))
    return fail(COSA_ERR_INVALID_ARG, "mask_words (%d) must be >= ceil(max_nk / 64) = %d", mask_words,
                std::max(need, 1));
  if (capped && mask_words > 64)
    return fail(COSA_ERR_UNSUPPORTED, "mask_words (%d) exceeds 64 (4096 KV blocks)", mask_words);
  return COSA_OK;
}

// list walk (order/count), mask walk (mask) or dense walk
cosa_status run_attention(const cosa_problem* p, const void* q, const void* k, const void* v,
                          const int32_t* order, const int32_t* count, int32_t kmax,
                          const uint64_t* mask, int32_t mask_words, int32_t group,
                          float tau, void* o, int32_t* visited, int32_t* skipped,
                          uint8_t* skip_bits, float* lse, void* stream, bool dense) {
  cosa_status st = validate(p);
  if (st != COSA_OK) return st;
  if (!q || !k || !v || !o) return fail(COSA_ERR_INVALID_ARG, "q, k_pages, v_pages and o must be non-NULL");
  if ((st = check_aligned(q, "q")) != COSA_OK || (st = check_aligned(o, "o")) != COSA_OK) return st;
  const bool masked = !dense && mask_words > 0;
  if (masked) {
    if (!mask || !visited || !skipped)
      return fail(COSA_ERR_INVALID_ARG, "mask, visited and skipped must be non-NULL");
    if ((st = check_mask_words(p, mask_words, false)) != COSA_OK) return st;
    if (p->dtype != COSA_BF16)
      return fail(COSA_ERR_UNSUPPORTED, "the mask walk is built for bf16 only");
  }
  if (!dense) {
    if (!masked && (!order || !count || !visited || !skipped))
      return fail(COSA_ERR_INVALID_ARG, "order, count, visited and skipped must be non-NULL");
    if (!masked && kmax < 1) return fail(COSA_ERR_INVALID_ARG, "kmax must be >= 1 (got %d)", kmax);
    if (group != p->h_q / p->h_kv)
      return fail(COSA_ERR_INVALID_ARG, "group (%d) must equal h_q / h_kv (%d)", group, p->h_q / p->h_kv);
    if (!(tau >= 0.f && tau < 1.f))
      return fail(COSA_ERR_INVALID_ARG, "skip_threshold must lie in [0, 1) (got %g)", (double)tau);
  }
  cosa_dims_t d;
  compute_dims(p, 0, 0.0, &d);
  if (d.total_q == 0 || d.max_nq == 0) return ok();
  cosa::OskArgs a{};
  a.seq = seq_args(p, d);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.order = order;
  a.count = count;
  a.visited = visited;
  a.skipped = skipped;
  a.skip_bits = skip_bits;
  a.lse = lse;
  a.mask = masked ? mask : nullptr;
  a.mask_words = masked ? mask_words : 0;
  a.total_q = d.total_q;
  a.kmax = kmax;
  a.scale = p->softmax_scale;
  a.scale_log2 = (float)((double)p->softmax_scale * 1.4426950408889634);
  a.skip_on = (!dense && tau > 0.f) ? 1 : 0;
  a.skip_thr_raw = a.skip_on ? (float)(log((double)tau) / (double)p->softmax_scale) : 0.f;
  a.n_units = (int64_t)p->batch * p->h_q * d.max_nq;
  return hip_result(cosa::launch_osk(a, p->dtype, p->head_dim, p->block, dense, (hipStream_t)stream),
                    dense ? "dense attention launch" : (masked ? "masked OSK launch" : "OSK launch"));
}

cosa_status run_mask_conversion(const cosa_problem* p, const int32_t* order, const int32_t* count,
                                int32_t kmax, uint64_t* mask_out, const uint64_t* mask_in,
                                int32_t mask_words, int32_t* order_out, int32_t* count_out,
                                void* stream, bool to_mask) {
  cosa_status st = validate(p);
  if (st != COSA_OK) return st;
  if (to_mask ? (!order || !count || !mask_out) : (!order_out || !count_out))
    return fail(COSA_ERR_INVALID_ARG, to_mask ? "order, count and mask must be non-NULL"
                                              : "order and count must be non-NULL");
  if (kmax < 1) return fail(COSA_ERR_INVALID_ARG, "kmax must be >= 1 (got %d)", kmax);
  if ((to_mask || mask_in) && (st = check_mask_words(p, mask_words, true)) != COSA_OK) return st;
  if (!to_mask && !mask_in && min_mask_words(p) > 64)
    return fail(COSA_ERR_UNSUPPORTED, "more than 4096 KV blocks per sequence");
  cosa_dims_t d;
  compute_dims(p, 0, 0.0, &d);
  cosa::MaskArgs a{};
  a.seq = seq_args(p, d);
  a.block = p->block;
  a.n_rows = (int64_t)p->batch * p->h_kv * d.max_nq;
  if (a.n_rows == 0) return ok();
  a.mask_words = mask_words;
  a.kmax = kmax;
  a.order = order;
  a.count = count;
  a.mask_out = mask_out;
  a.mask_in = mask_in;
  a.order_out = order_out;
  a.count_out = count_out;
  return hip_result(to_mask ? cosa::launch_mask_from_order(a, (hipStream_t)stream)
                            : cosa::launch_order_from_mask(a, (hipStream_t)stream),
                    to_mask ? "mask-from-order launch" : "order-from-mask launch");
}

}  // namespace

extern "C" {

cosa_status cosa_validate(const cosa_problem* problem) {
  cosa_status st = validate(problem);
  return st == COSA_OK ? ok() : st;
}

cosa_status cosa_dims(const cosa_problem* problem, int32_t pool, double budget, cosa_dims_t* out) {
  cosa_status st = validate(problem);
  if (st != COSA_OK) return st;
  if (!out) return fail(COSA_ERR_INVALID_ARG, "out is NULL");
  if (pool != 0 && (st = check_pool(problem, pool)) != COSA_OK) return st;
  if (!(budget >= 0.0 && budget <= 1.0))
    return fail(COSA_ERR_INVALID_ARG, "budget must lie in (0, 1] (or 0 to skip kmax)");
  compute_dims(problem, pool, budget, out);
  return ok();
}

size_t cosa_kap_kmax(const cosa_problem* problem, double budget) {
  if (validate(problem) != COSA_OK || !(budget > 0.0 && budget <= 1.0)) return 0;
  cosa_dims_t d;
  compute_dims(problem, 0, budget, &d);
  return (size_t)d.kmax;
}

size_t cosa_kap_workspace_size(const cosa_problem* problem, int32_t pool, int32_t with_scores) {
  if (validate(problem) != COSA_OK || check_pool(problem, pool) != COSA_OK) return 0;
  return kap_ws_size(problem, pool, with_scores != 0);
}

// the proxy with its own key pooling (k_pages) or over caller-pooled keys
static cosa_status run_kap(const cosa_problem* problem, const void* q, const void* k_pages, const void* pooled_keys,
                           int32_t pool, double budget, int32_t* order, uint8_t* hrm, int32_t* count, int32_t kmax,
                    float* proxy_scores, float* block_scores, void* workspace, size_t workspace_bytes,
                    void* stream) {
  cosa_status st = validate(problem);
  if (st != COSA_OK) return st;
  if ((st = check_pool(problem, pool)) != COSA_OK) return st;
  if (!(budget > 0.0 && budget <= 1.0))
    return fail(COSA_ERR_INVALID_ARG, "budget must lie in (0, 1] (got %g)", budget);
  if (!q || !(k_pages || pooled_keys) || !order || !hrm || !count)
    return fail(COSA_ERR_INVALID_ARG, pooled_keys ? "q, pooled_keys, order, hrm and count must be non-NULL"
                                                  : "q, k_pages, order, hrm and count must be non-NULL");
  if ((st = check_aligned(q, "q")) != COSA_OK) return st;
  cosa_dims_t d;
  compute_dims(problem, pool, budget, &d);
  if (kmax < d.kmax)
    return fail(COSA_ERR_INVALID_ARG, "kmax (%d) is smaller than the widest list (%d)", kmax, d.kmax);
  if (d.max_nk > cosa::kMaxSortBlocks)
    return fail(COSA_ERR_UNSUPPORTED, "max KV blocks per sequence %d exceeds %d", d.max_nk,
                cosa::kMaxSortBlocks);
  if ((int64_t)(problem->h_q / problem->h_kv) * (problem->block / pool) > 4096)
    return fail(COSA_ERR_UNSUPPORTED, "group * block / pool exceeds 4096 pooled rows per list");
  const bool own_scores = proxy_scores == nullptr;
  const size_t need = kap_ws_size(problem, pool, own_scores);
  if (!workspace || workspace_bytes < need)
    return fail(COSA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if (((uintptr_t)workspace & 255) != 0)
    return fail(COSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (d.total_q == 0 || d.max_nq == 0) return ok();

  const size_t es = problem->dtype == COSA_BF16 ? 2 : 4;
  unsigned char* ws = (unsigned char*)workspace;
  cosa::KapArgs a{};
  a.seq = seq_args(problem, d);
  a.q = q;
  a.k = k_pages;
  a.q_pool = ws;
  ws += align256((size_t)problem->batch * d.max_nr * problem->h_q * problem->head_dim * es);
  a.k_pool = pooled_keys ? const_cast<void*>(pooled_keys) : (void*)ws;  // read only when given
  a.keys_pooled = pooled_keys ? 1 : 0;
  ws += align256((size_t)problem->num_pages * problem->h_kv * (problem->block / pool) *
                 problem->head_dim * es);
  // the score pass reduces rows of P to their maxima when blocks hold 4..32
  // pooled keys (not in its decode shape); otherwise the rank pass does
  const int per = problem->block / pool;
  const bool decode_scores = cosa::kap_decode_scores(d.max_nr, problem->h_q / problem->h_kv, per, problem->dtype);
  a.row_max = (per >= 4 && per <= 32 && !decode_scores) ? (float*)ws : nullptr;
  ws += align256((size_t)problem->batch * problem->h_q * d.max_nr * sizeof(float));
  a.scores = own_scores ? (float*)ws : proxy_scores;
  a.fill_scores = own_scores ? 0 : 1;
  a.block_scores = block_scores;
  a.order = order;
  a.hrm = hrm;
  a.count = count;
  a.pool = pool;
  a.max_nr = d.max_nr;
  a.kmax = kmax;
  a.budget = budget;
  a.scale = problem->softmax_scale;
  return hip_result(cosa::launch_kap(a, problem->dtype, problem->head_dim, problem->block,
                                     (hipStream_t)stream),
                    "KAP launch");
}

cosa_status cosa_kap_order(const cosa_problem* problem, const void* q, const void* k_pages,
                           int32_t pool, double budget, int32_t* order, uint8_t* hrm,
                           int32_t* count, int32_t kmax, float* proxy_scores,
                           float* block_scores, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return run_kap(problem, q, k_pages, nullptr, pool, budget, order, hrm, count, kmax, proxy_scores,
                 block_scores, workspace, workspace_bytes, stream);
}

cosa_status cosa_kap_order_pooled(const cosa_problem* problem, const void* q, const void* pooled_keys,
                                  int32_t pool, double budget, int32_t* order, uint8_t* hrm,
                                  int32_t* count, int32_t kmax, float* proxy_scores,
                                  float* block_scores, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (!pooled_keys) return fail(COSA_ERR_INVALID_ARG, "pooled_keys must be non-NULL");
  return run_kap(problem, q, nullptr, pooled_keys, pool, budget, order, hrm, count, kmax, proxy_scores,
                 block_scores, workspace, workspace_bytes, stream);
}

cosa_status cosa_kap_pool_keys(const cosa_problem* problem, const void* k_pages, int32_t pool,
                               void* pooled_keys, int32_t last_block_only, void* stream) {
  cosa_status st = validate(problem);
  if (st != COSA_OK) return st;
  if ((st = check_pool(problem, pool)) != COSA_OK) return st;
  if (!k_pages || !pooled_keys) return fail(COSA_ERR_INVALID_ARG, "k_pages and pooled_keys must be non-NULL");
  cosa_dims_t d;
  compute_dims(problem, pool, 0.0, &d);
  if (d.max_nk == 0) return ok();
  cosa::KapArgs a{};
  a.seq = seq_args(problem, d);
  a.k = k_pages;
  a.k_pool = pooled_keys;
  a.pool = pool;
  a.pool_last_only = last_block_only ? 1 : 0;
  return hip_result(cosa::launch_kap_pool_k(a, problem->dtype, problem->head_dim, problem->block,
                                            (hipStream_t)stream),
                    "key pooling launch");
}

cosa_status cosa_osk_attention(const cosa_problem* problem, const void* q, const void* k_pages,
                               const void* v_pages, const int32_t* order, const int32_t* count,
                               int32_t kmax, int32_t group, float skip_threshold, void* o,
                               int32_t* visited, int32_t* skipped, uint8_t* skip_bits, float* lse,
                               void* stream) {
  return run_attention(problem, q, k_pages, v_pages, order, count, kmax, nullptr, 0, group,
                       skip_threshold, o, visited, skipped, skip_bits, lse, stream, false);
}

cosa_status cosa_osk_attention_masked(const cosa_problem* problem, const void* q, const void* k_pages,
                                      const void* v_pages, const uint64_t* mask, int32_t mask_words,
                                      int32_t group, float skip_threshold, void* o, int32_t* visited,
                                      int32_t* skipped, float* lse, void* stream) {
  if (mask_words < 1) return fail(COSA_ERR_INVALID_ARG, "mask_words must be >= 1 (got %d)", mask_words);
  return run_attention(problem, q, k_pages, v_pages, nullptr, nullptr, 0, mask, mask_words, group,
                       skip_threshold, o, visited, skipped, nullptr, lse, stream, false);
}

cosa_status cosa_mask_from_order(const cosa_problem* problem, const int32_t* order, const int32_t* count,
                                 int32_t kmax, uint64_t* mask, int32_t mask_words, void* stream) {
  return run_mask_conversion(problem, order, count, kmax, mask, nullptr, mask_words, nullptr, nullptr,
                             stream, true);
}

cosa_status cosa_union_order(const cosa_problem* problem, const int32_t* order, const int32_t* count,
                             int32_t kmax, int32_t* union_order, int32_t* union_count,
                             int32_t union_kmax, void* stream) {
  cosa_status st = validate(problem);
  if (st != COSA_OK) return st;
  if (!order || !count || !union_order || !union_count)
    return fail(COSA_ERR_INVALID_ARG, "order, count, union_order and union_count must be non-NULL");
  if (kmax < 1 || union_kmax < 1)
    return fail(COSA_ERR_INVALID_ARG, "kmax and union_kmax must be >= 1 (got %d, %d)", kmax, union_kmax);
  if (min_mask_words(problem) > 64)
    return fail(COSA_ERR_UNSUPPORTED, "more than 4096 KV blocks per sequence");
  cosa_dims_t d;
  compute_dims(problem, 0, 0.0, &d);
  cosa::MaskArgs a{};
  a.seq = seq_args(problem, d);
  a.block = problem->block;
  a.n_rows = (int64_t)problem->batch * problem->h_kv * d.max_nq;
  if (a.n_rows == 0) return ok();
  a.kmax = kmax;
  a.order = order;
  a.count = count;
  a.order_out = union_order;
  a.count_out = union_count;
  a.kmax_out = union_kmax;
  return hip_result(cosa::launch_union_order(a, (hipStream_t)stream), "union-order launch");
}

size_t cosa_cobs_workspace_size(const cosa_problem* problem, int32_t pool) {
  if (validate(problem) != COSA_OK || check_pool(problem, pool) != COSA_OK) return 0;
  cosa_dims_t d;
  compute_dims(problem, pool, 0.0, &d);
  return align256((size_t)problem->batch * d.max_nr * problem->h_q * problem->head_dim * 2);
}

cosa_status cosa_cobs_scores(const cosa_problem* problem, const void* q, const void* k_pages, int32_t pool,
                             float* scores, void* workspace, size_t workspace_bytes, void* stream) {
  cosa_status st = validate(problem);
  if (st != COSA_OK) return st;
  if ((st = check_pool(problem, pool)) != COSA_OK) return st;
  if (!q || !k_pages || !scores) return fail(COSA_ERR_INVALID_ARG, "q, k_pages and scores must be non-NULL");
  if ((st = check_aligned(q, "q")) != COSA_OK) return st;
  if (problem->dtype != COSA_BF16) return fail(COSA_ERR_UNSUPPORTED, "second-order scores are built for bf16 only");
  const size_t need = cosa_cobs_workspace_size(problem, pool);
  if (!workspace || workspace_bytes < need)
    return fail(COSA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if (((uintptr_t)workspace & 255) != 0) return fail(COSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  cosa_dims_t d;
  compute_dims(problem, pool, 0.0, &d);
  if (d.total_q == 0 || d.max_nr == 0) return ok();
  cosa::KapArgs a{};
  a.seq = seq_args(problem, d);
  a.q = q;
  a.k = k_pages;
  a.q_pool = workspace;
  a.scores = scores;
  a.pool = pool;
  a.max_nr = d.max_nr;
  a.scale = problem->softmax_scale;
  hipError_t e = cosa::launch_kap_pool_q(a, problem->dtype, problem->head_dim, (hipStream_t)stream);
  if (e == hipSuccess) e = cosa::launch_cobs_scores(a, problem->head_dim, problem->block, (hipStream_t)stream);
  return hip_result(e, "second-order score launch");
}

cosa_status cosa_kap_rank(const cosa_problem* problem, int32_t pool, double budget, const float* scores,
                          int32_t* order, uint8_t* hrm, int32_t* count, int32_t kmax, float* block_scores,
                          void* stream) {
  cosa_status st = validate(problem);
  if (st != COSA_OK) return st;
  if ((st = check_pool(problem, pool)) != COSA_OK) return st;
  if (!(budget > 0.0 && budget <= 1.0))
    return fail(COSA_ERR_INVALID_ARG, "budget must lie in (0, 1] (got %g)", budget);
  if (!scores || !order || !hrm || !count)
    return fail(COSA_ERR_INVALID_ARG, "scores, order, hrm and count must be non-NULL");
  cosa_dims_t d;
  compute_dims(problem, pool, budget, &d);
  if (kmax < d.kmax)
    return fail(COSA_ERR_INVALID_ARG, "kmax (%d) is smaller than the widest list (%d)", kmax, d.kmax);
  if (d.max_nk > cosa::kMaxSortBlocks)
    return fail(COSA_ERR_UNSUPPORTED, "max KV blocks per sequence %d exceeds %d", d.max_nk, cosa::kMaxSortBlocks);
  if ((int64_t)(problem->h_q / problem->h_kv) * (problem->block / pool) > 4096)
    return fail(COSA_ERR_UNSUPPORTED, "group * block / pool exceeds 4096 pooled rows per list");
  if (d.total_q == 0 || d.max_nq == 0) return ok();
  cosa::KapArgs a{};
  a.seq = seq_args(problem, d);
  a.scores = const_cast<float*>(scores);  // read only
  a.row_max = nullptr;                    // the rank pass takes the row maxima itself
  a.block_scores = block_scores;
  a.order = order;
  a.hrm = hrm;
  a.count = count;
  a.pool = pool;
  a.max_nr = d.max_nr;
  a.kmax = kmax;
  a.budget = budget;
  a.scale = problem->softmax_scale;
  return hip_result(cosa::launch_kap_rank(a, problem->block, (hipStream_t)stream), "rank launch");
}

size_t cosa_osk_decode_workspace_size(const cosa_problem* problem, int32_t n_splits) {
  if (validate(problem) != COSA_OK || n_splits < 1) return 0;
  return decode_ws_size(problem, n_splits);
}

// The decode step over a caller's workspace, or (fixed_scratch) over this
// library's static per-device scratch array.
static cosa_status run_decode(const cosa_problem* problem, const void* q, const void* k_pages,
                              const void* v_pages, const int32_t* order, const int32_t* count,
                              int32_t kmax, int32_t group, float skip_threshold, int32_t n_splits,
                              void* o, int32_t* visited, int32_t* skipped, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream, bool fixed_scratch) {
  cosa_status st = validate(problem);
  if (st != COSA_OK) return st;
  const cosa_problem* p = problem;
  if (!q || !k_pages || !v_pages || !o || !order || !count || !visited || !skipped)
    return fail(COSA_ERR_INVALID_ARG, "q, k_pages, v_pages, o, order, count, visited and skipped must be non-NULL");
  if (p->dtype != COSA_BF16) return fail(COSA_ERR_UNSUPPORTED, "the decode walk is built for bf16 only");
  if ((st = check_aligned(q, "q")) != COSA_OK || (st = check_aligned(o, "o")) != COSA_OK) return st;
  if (kmax < 1) return fail(COSA_ERR_INVALID_ARG, "kmax must be >= 1 (got %d)", kmax);
  if (group != p->h_q / p->h_kv)
    return fail(COSA_ERR_INVALID_ARG, "group (%d) must equal h_q / h_kv (%d)", group, p->h_q / p->h_kv);
  if (group > 32) return fail(COSA_ERR_UNSUPPORTED, "the decode walk handles up to 32 query heads per KV head");
  if (!(skip_threshold >= 0.f && skip_threshold < 1.f))
    return fail(COSA_ERR_INVALID_ARG, "skip_threshold must lie in [0, 1) (got %g)", (double)skip_threshold);
  if (n_splits < 1 || n_splits > 1024)
    return fail(COSA_ERR_INVALID_ARG, "n_splits must lie in [1, 1024] (got %d)", n_splits);
  for (int b = 0; b < p->batch; ++b)
    if (p->host_cu_seqlens_q[b + 1] - p->host_cu_seqlens_q[b] > 1)
      return fail(COSA_ERR_INVALID_ARG, "sequence %d has %d query tokens; a decode step has at most one", b,
                  p->host_cu_seqlens_q[b + 1] - p->host_cu_seqlens_q[b]);
  const size_t need = decode_ws_size(p, n_splits);
  if (fixed_scratch) {
    if (need > kScratchBytes)
      return fail(COSA_ERR_UNSUPPORTED,
                  "the decode step needs %zu bytes of scratch (batch %d x h_q %d x n_splits %d partial "
                  "results), more than the fixed %zu-byte scratch of the allocation-free entry point; "
                  "use cosa_osk_decode with a workspace",
                  need, p->batch, p->h_q, n_splits, kScratchBytes);
  } else {
    if (!workspace || workspace_bytes < need)
      return fail(COSA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    if (((uintptr_t)workspace & 255) != 0) return fail(COSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  cosa_dims_t d;
  compute_dims(p, 0, 0.0, &d);
  if (d.total_q == 0 || d.max_nq == 0) return ok();
  if (fixed_scratch && (st = scratch_of_current_device(&workspace)) != COSA_OK) return st;
  cosa::DecodeArgs a{};
  a.seq = seq_args(p, d);
  a.q = q;
  a.k = k_pages;
  a.v = v_pages;
  a.o = o;
  a.order = order;
  a.count = count;
  a.visited = visited;
  a.skipped = skipped;
  a.lse = lse;
  unsigned char* ws = (unsigned char*)workspace;
  a.part = (float*)ws;
  ws += align256((size_t)p->batch * p->h_q * n_splits * (p->head_dim + 2) * sizeof(float));
  a.part_counts = (int32_t*)ws;
  a.total_q = d.total_q;
  a.kmax = kmax;
  a.n_splits = n_splits;
  a.scale = p->softmax_scale;
  a.scale_log2 = (float)((double)p->softmax_scale * 1.4426950408889634);
  a.skip_on = skip_threshold > 0.f ? 1 : 0;
  a.skip_thr_raw = a.skip_on ? (float)(log((double)skip_threshold) / (double)p->softmax_scale) : 0.f;
  return hip_result(cosa::launch_osk_decode(a, p->head_dim, p->block, (hipStream_t)stream), "decode launch");
}

cosa_status cosa_osk_decode(const cosa_problem* problem, const void* q, const void* k_pages,
                            const void* v_pages, const int32_t* order, const int32_t* count,
                            int32_t kmax, int32_t group, float skip_threshold, int32_t n_splits,
                            void* o, int32_t* visited, int32_t* skipped, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return run_decode(problem, q, k_pages, v_pages, order, count, kmax, group, skip_threshold, n_splits, o,
                    visited, skipped, lse, workspace, workspace_bytes, stream, false);
}

cosa_status cosa_osk_decode_noalloc(const cosa_problem* problem, const void* q, const void* k_pages,
                                    const void* v_pages, const int32_t* order, const int32_t* count,
                                    int32_t kmax, int32_t group, float skip_threshold, int32_t n_splits,
                                    void* o, int32_t* visited, int32_t* skipped, float* lse, void* stream) {
  return run_decode(problem, q, k_pages, v_pages, order, count, kmax, group, skip_threshold, n_splits, o,
                    visited, skipped, lse, nullptr, 0, stream, true);
}

cosa_status cosa_block_mass(const cosa_problem* problem, const void* q, const void* k_pages,
                            const float* lse, float* mass, void* stream) {
  cosa_status st = validate(problem);
  if (st != COSA_OK) return st;
  if (!q || !k_pages || !lse || !mass)
    return fail(COSA_ERR_INVALID_ARG, "q, k_pages, lse and mass must be non-NULL");
  if ((st = check_aligned(q, "q")) != COSA_OK) return st;
  if (problem->dtype != COSA_BF16) return fail(COSA_ERR_UNSUPPORTED, "block mass is built for bf16 only");
  cosa_dims_t d;
  compute_dims(problem, 0, 0.0, &d);
  cosa::MassArgs a{};
  a.seq = seq_args(problem, d);
  a.q = q;
  a.k = k_pages;
  a.lse = lse;
  a.mass = mass;
  a.total_q = d.total_q;
  a.scale_log2 = (float)((double)problem->softmax_scale * 1.4426950408889634);
  a.n_units = (int64_t)problem->batch * problem->h_q * d.max_nq;
  if (a.n_units == 0 || d.max_nk == 0) return ok();
  return hip_result(cosa::launch_block_mass(a, problem->head_dim, problem->block, (hipStream_t)stream),
                    "block-mass launch");
}

cosa_status cosa_order_from_mask(const cosa_problem* problem, const uint64_t* mask, int32_t mask_words,
                                 int32_t* order, int32_t* count, int32_t kmax, void* stream) {
  return run_mask_conversion(problem, nullptr, nullptr, kmax, nullptr, mask, mask_words, order, count,
                             stream, false);
}

cosa_status cosa_dense_attention(const cosa_problem* problem, const void* q, const void* k_pages,
                                 const void* v_pages, void* o, float* lse, void* stream) {
  return run_attention(problem, q, k_pages, v_pages, nullptr, nullptr, 1, nullptr, 0,
                       problem ? problem->h_q / std::max(problem->h_kv, 1) : 1, 0.f, o, nullptr,
                       nullptr, nullptr, lse, stream, true);
}

const char* cosa_status_string(cosa_status status) {
  switch (status) {
    case COSA_OK: return "success";
    case COSA_ERR_INVALID_ARG: return "invalid argument";
    case COSA_ERR_UNSUPPORTED: return "unsupported size or layout";
    case COSA_ERR_WORKSPACE: return "workspace missing or too small";
    case COSA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* cosa_last_error(void) { return g_last_error.c_str(); }

int32_t cosa_version(void) { return 100; }

}  // extern "C"
