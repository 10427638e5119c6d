// Binary block masks <-> computation-order lists.
//
// The CoSA technical summary (gist.science, "CoSA: Accelerating Long-Context
// Inference via Proxy-Kernel Co-Designed Sparse Attention") contrasts its
// computation-order list (§2.1) with the binary masks of earlier proxies, and
// its page-remapped walk (§2.3, "mask-skipped") with the control-flow skipping
// of standard sparse kernels. These conversions let the same selection run
// either way: a list becomes a mask (its order is dropped), and a mask becomes
// an ascending list (the visit order of a fixed-order kernel).
//
// One wave per row (sequence, KV head, query block); a row's mask has at most
// 64 words (4096 KV blocks), one per lane.
#include "cosa_internal.h"

namespace cosa {
namespace {

struct RowInfo {
  int n;      // causal KV blocks of the row (0 past the sequence's last query block)
  bool live;  // row inside the padded grid
};

__device__ RowInfo row_info(const MaskArgs& a, int64_t row) {
  RowInfo r{0, row < a.n_rows};
  if (!r.live) return r;
  const SeqArgs& sq = a.seq;
  const int qb = (int)(row % sq.max_nq);
  const int b = (int)(row / sq.max_nq / sq.h_kv);
  const int q0 = sq.cu_seqlens_q[b];
  const int Lq = sq.cu_seqlens_q[b + 1] - q0;
  const int Lk = sq.seqlens_k[b];
  if (qb * a.block < Lq) r.n = (Lk - Lq + min(qb * a.block + a.block - 1, Lq - 1)) / a.block + 1;
  return r;
}

// bit kb of the row's mask for every listed entry with 0 <= kb < n
__global__ __launch_bounds__(256) void mask_from_order_kernel(MaskArgs a) {
  __shared__ unsigned long long words[4][64];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + w;
  const RowInfo ri = row_info(a, row);
  words[w][lane] = 0ull;
  __syncthreads();
  if (ri.live && ri.n > 0) {
    const int cnt = max(0, min(a.count[row], a.kmax));
    const int32_t* lst = a.order + row * a.kmax;
    for (int t = lane; t < cnt; t += 64) {
      const int kb = lst[t];
      if (kb >= 0 && kb < ri.n) atomicOr(&words[w][kb >> 6], 1ull << (kb & 63));
    }
  }
  __syncthreads();
  if (ri.live && lane < a.mask_words) a.mask_out[row * a.mask_words + lane] = words[w][lane];
}

// ascending list of the set causal bits (every causal block without a mask),
// truncated to kmax entries
__global__ __launch_bounds__(256) void order_from_mask_kernel(MaskArgs a) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + w;
  const RowInfo ri = row_info(a, row);
  if (!ri.live) return;
  uint64_t bits = 0;
  const int base = lane * 64;
  if (base < ri.n) {
    bits = a.mask_in ? a.mask_in[row * a.mask_words + lane] : ~0ull;
    if (ri.n - base < 64) bits &= (1ull << (ri.n - base)) - 1ull;
  }
  // exclusive prefix sum of the per-word counts across the wave
  const int pc = __popcll(bits);
  int incl = pc;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  const int total = __shfl(incl, 63, 64);
  const int n_out = min(total, a.kmax);
  int pos = incl - pc;
  int32_t* lst = a.order_out + row * a.kmax;
  while (bits && pos < n_out) {
    const int bit = __builtin_ctzll(bits);
    lst[pos++] = base + bit;
    bits &= bits - 1ull;
  }
  for (int t = n_out + lane; t < a.kmax; t += 64) lst[t] = -1;
  if (lane == 0) a.count_out[row] = n_out;
}

// Block-union tables (CompactAttention page, selection stage): for a
// (sequence, KV group), OR the listed causal blocks of all its query blocks
// into one table, then write, for every query block, the table's blocks that
// are causal for it, ascending. Each of kUnionSlices workgroups of a
// (sequence, KV group) builds the table (a cheap pass over the lists) and
// writes every kUnionSlices-th query block's list.
constexpr int kUnionSlices = 16;

__global__ __launch_bounds__(256) void union_order_kernel(MaskArgs a) {
  __shared__ unsigned long long u[64];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int64_t bg = blockIdx.x / kUnionSlices;  // b * h_kv + g
  const int slice = blockIdx.x % kUnionSlices;
  const SeqArgs& sq = a.seq;
  const int b = (int)(bg / sq.h_kv);
  const int q0 = sq.cu_seqlens_q[b];
  const int Lq = sq.cu_seqlens_q[b + 1] - q0;
  const int Lk = sq.seqlens_k[b];
  const int nq = (Lq + a.block - 1) / a.block;  // query blocks of this sequence
  auto n_of = [&](int qb) { return (Lk - Lq + min(qb * a.block + a.block - 1, Lq - 1)) / a.block + 1; };
  const int64_t row0 = bg * sq.max_nq;
  if (tid < 64) u[tid] = 0ull;
  __syncthreads();
  for (int64_t i = tid; i < (int64_t)nq * a.kmax; i += 256) {
    const int qb = (int)(i / a.kmax), t = (int)(i % a.kmax);
    const int cnt = max(0, min(a.count[row0 + qb], a.kmax));
    if (t >= cnt) continue;
    const int kb = a.order[(row0 + qb) * a.kmax + t];
    if (kb >= 0 && kb < n_of(qb)) atomicOr(&u[kb >> 6], 1ull << (kb & 63));
  }
  __syncthreads();
  for (int qb = slice + kUnionSlices * w; qb < sq.max_nq; qb += kUnionSlices * 4) {
    const int64_t row = row0 + qb;
    const int n = qb < nq ? n_of(qb) : 0;
    uint64_t bits = 0;
    const int base = lane * 64;
    if (base < n) {
      bits = u[lane];
      if (n - base < 64) bits &= (1ull << (n - base)) - 1ull;
    }
    const int pc = __popcll(bits);
    int incl = pc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d, 64);
      if (lane >= d) incl += y;
    }
    const int total = __shfl(incl, 63, 64);
    const int n_out = min(total, a.kmax_out);
    int pos = incl - pc;
    int32_t* lst = a.order_out + row * a.kmax_out;
    while (bits && pos < n_out) {
      lst[pos++] = base + __builtin_ctzll(bits);
      bits &= bits - 1ull;
    }
    for (int t = n_out + lane; t < a.kmax_out; t += 64) lst[t] = -1;
    if (lane == 0) a.count_out[row] = n_out;
  }
}

}  // namespace

hipError_t launch_union_order(const MaskArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.seq.batch * a.seq.h_kv * kUnionSlices;
  hipLaunchKernelGGL(union_order_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_mask_from_order(const MaskArgs& a, hipStream_t stream) {
  const int64_t grid = (a.n_rows + 3) / 4;
  hipLaunchKernelGGL(mask_from_order_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_order_from_mask(const MaskArgs& a, hipStream_t stream) {
  const int64_t grid = (a.n_rows + 3) / 4;
  hipLaunchKernelGGL(order_from_mask_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace cosa
