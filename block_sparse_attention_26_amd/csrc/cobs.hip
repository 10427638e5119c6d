// Second-order block scores (COBS page, §2.2-2.3) as an alternative proxy
// ranking, bf16 inputs.
//
// For pooled query row r and KV block kb, with s_j = scale * q_pooled[r] . k_j
// over the raw keys j of the block that the row's window may see:
//     P2[b, h, r, kb] = mean_j s_j + 1/2 var_j s_j
// (population variance; -inf when no key is visible) - the page's
// q.k_mean + 1/2 q^T Sigma q with the exact per-block key covariance. The
// proxy's MaxNorm, HRM, sort and budget then rank P2 as they rank P.
//
// One workgroup per (sequence, query head, 128 pooled rows): 4 waves of 32
// rows. Per KV block the K slab is staged through registers (one block
// ahead) into LDS with rows padded by 16 bytes; S^T = K Q_pooled^T runs on
// v_mfma_f32_32x32x16_bf16 (4 key tiles per wave); each lane then forms the
// mean over its row's visible keys and, in a second pass over the same
// registers, the variance (no cancellation between large sums). Results are
// staged in LDS and written 32 blocks of a row (128 bytes) at a time.
#include <math.h>

#include "cosa_internal.h"

namespace cosa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int BLK>
__global__ __launch_bounds__(256) void cobs_score_kernel(KapArgs a) {
  constexpr int ROWS = 128;                 // pooled rows per workgroup
  constexpr int KT = BLK / 32;              // 32-key tiles per block
  constexpr int QREGS = D / 16;
  constexpr int PITCH = D * 2 + 16;         // bytes per K row in LDS
  constexpr int CHUNKS = BLK * D / 8;       // 16-byte chunks per K slab
  constexpr int CPT = CHUNKS / 256;         // per thread
  constexpr int CB = 32;                    // blocks per staged output chunk
  static_assert(CPT * 256 == CHUNKS, "whole chunks per thread");
  __shared__ __attribute__((aligned(16))) unsigned char kt_lds[BLK * PITCH];
  __shared__ float pst[ROWS][CB + 1];

  const SeqArgs& sq = a.seq;
  const int G = sq.group;
  const int ntile = (a.max_nr + ROWS - 1) / ROWS;
  const int64_t bid = blockIdx.x;
  const int h = (int)(bid % sq.h_q);
  const int b = (int)(bid / sq.h_q % sq.batch);
  const int rt = (int)(bid / sq.h_q / sq.batch);
  const int g = h / G;
  const int q0 = sq.cu_seqlens_q[b];
  const int Lq = sq.cu_seqlens_q[b + 1] - q0;
  const int Lk = sq.seqlens_k[b];
  const int off = Lk - Lq;
  const int p = a.pool;
  const int R = (Lq + p - 1) / p;
  const int nk = (Lk + BLK - 1) / BLK;
  const int r0 = rt * ROWS;
  float* P = a.scores + (((int64_t)b * sq.h_q + h) * a.max_nr) * sq.max_nk;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hl = lane >> 5;
  (void)ntile;

  // blocks computed: the causal blocks of the tile's last row; the rest -inf
  const int r_last = min(r0 + ROWS, R) - 1;
  const int kb_end = r0 < R ? min((off + min(r_last * p + p - 1, Lq - 1)) / BLK + 1, nk) : 0;
  for (int i = tid; i < ROWS * sq.max_nk; i += 256) {
    const int r = r0 + i / sq.max_nk, kb = i % sq.max_nk;
    if (r < a.max_nr && (r >= R || kb >= kb_end)) P[(int64_t)r * sq.max_nk + kb] = kNegInf;
  }
  if (kb_end == 0) return;

  const int my_r = r0 + w * 32 + l32;
  const bool r_ok = my_r < R;
  const int jmax = r_ok ? off + min(my_r * p + p - 1, Lq - 1) : -1;  // last visible key
  bf16x8 qf[QREGS];
  {
    const uint16_t* qp = (const uint16_t*)a.q_pool + (((size_t)b * a.max_nr + (r_ok ? my_r : r0)) * sq.h_q + h) * D + hl * 8;
#pragma unroll
    for (int ks = 0; ks < QREGS; ++ks) {
      const uint4 x = r_ok ? *(const uint4*)(qp + ks * 16) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }
  const int32_t* table = sq.block_table + (int64_t)b * sq.max_blocks_k;
  const size_t page_elems = (size_t)sq.h_kv * BLK * D;
  uint4 stg[CPT];
  auto fetch = [&](int kb) {
    int page = table[kb];
    const bool page_ok = (unsigned)page < (unsigned)sq.num_pages;
    const int nvalid = min(BLK, Lk - kb * BLK);
    const uint16_t* src = (const uint16_t*)a.k + (size_t)(page_ok ? page : 0) * page_elems + (size_t)g * BLK * D;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int i = tid + 256 * j, r = i / (D / 8), c = i % (D / 8);
      // rows past the sequence end stay finite (they are never visible)
      stg[j] = (page_ok && r < nvalid) ? *(const uint4*)(src + (size_t)r * D + c * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int i = tid + 256 * j, r = i / (D / 8), c = i % (D / 8);
      *(uint4*)(kt_lds + r * PITCH + c * 16) = stg[j];
    }
  };

  const float sc = a.scale;
  fetch(0);
  for (int kb = 0; kb < kb_end; ++kb) {
    __syncthreads();  // the previous block's LDS reads are done
    stage();
    if (kb + 1 < kb_end) fetch(kb + 1);
    __syncthreads();
    f32x16 s[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kt][v] = 0.f;
      const unsigned char* kp = kt_lds + (kt * 32 + l32) * PITCH + hl * 16;
#pragma unroll
      for (int ks = 0; ks < QREGS; ++ks)
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(kp + ks * 32), qf[ks], s[kt], 0, 0, 0);
    }
    // element (kt, v) is key kb*B + kt*32 + 8*(v/4) + 4*hl + v%4 of this lane's row
    const int thr = min(jmax, Lk - 1) - kb * BLK - 4 * hl;
    float n = 0.f, sum = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (kt * 32 + 8 * (v >> 2) + (v & 3) <= thr) {
          n += 1.f;
          sum += s[kt][v];
        }
    n = xor32_sum(n);
    sum = xor32_sum(sum);
    const float mean = n > 0.f ? sum / n : 0.f;
    float dev = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (kt * 32 + 8 * (v >> 2) + (v & 3) <= thr) {
          const float e = s[kt][v] - mean;
          dev += e * e;
        }
    dev = xor32_sum(dev);
    const float p2 = n > 0.f ? sc * mean + 0.5f * sc * sc * (dev / n) : kNegInf;
    const int cb = kb % CB;
    if (hl == 0) pst[w * 32 + l32][cb] = p2;
    if (cb == CB - 1 || kb == kb_end - 1) {  // write the chunk's rows
      __syncthreads();
      const int c0 = kb - cb;
      for (int i = tid; i < ROWS * CB; i += 256) {
        const int rr = i / CB, c = i % CB, r = r0 + rr;
        if (r < R && c <= cb) P[(int64_t)r * sq.max_nk + c0 + c] = pst[rr][c];
      }
    }
  }
}

template <int D, int BLK>
hipError_t launch_one(const KapArgs& a, hipStream_t stream) {
  const int64_t ntile = (a.max_nr + 127) / 128;
  const int64_t grid = ntile * a.seq.batch * a.seq.h_q;
  hipLaunchKernelGGL((cobs_score_kernel<D, BLK>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cobs_scores(const KapArgs& a, int head_dim, int block, hipStream_t stream) {
  if (head_dim == 128 && block == 128) return launch_one<128, 128>(a, stream);
  if (head_dim == 128 && block == 64) return launch_one<128, 64>(a, stream);
  if (head_dim == 64 && block == 128) return launch_one<64, 128>(a, stream);
  if (head_dim == 64 && block == 64) return launch_one<64, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace cosa
