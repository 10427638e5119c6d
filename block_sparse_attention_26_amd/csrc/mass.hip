// Exact attention mass of every causal block (a diagnostic, bf16 inputs).
//
// The COBS page ("Oracle Sparse Attention") ranks KV blocks by the exact
// softmax mass they hold, an upper bound for any proxy at the same budget.
// Given each row's log-sum-exp over its visible keys (from the dense kernel),
// this kernel writes, for each (sequence, query head, query block, KV block),
// the sum over the valid rows and visible keys of exp(scale * q.k - lse).
//
// One workgroup per (sequence, query head, query block): BLK/32 waves of 32
// rows. Per causal block the K tile is copied into LDS (rows padded by 16
// bytes), S^T = K Q^T runs on v_mfma_f32_32x32x16_bf16 as in the attention
// kernels, and the probabilities are summed per lane, across the wave with
// cross-lane adds, then across waves in a fixed order, so results are
// deterministic.
#include <math.h>

#include "cosa_internal.h"

namespace cosa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  return x;
}

template <int D, int BLK>
__global__ __launch_bounds__(2 * BLK) void block_mass_kernel(MassArgs a) {
  constexpr int NW = BLK / 32, THREADS = 64 * NW, KT = BLK / 32, QREGS = D / 16;
  constexpr int PITCH = D * 2 + 16;  // bytes per K row in LDS
  __shared__ __attribute__((aligned(16))) unsigned char kt_lds[BLK * PITCH];
  __shared__ float part[NW];

  const SeqArgs& sq = a.seq;
  const int64_t u = blockIdx.x;
  const int qb = (int)(u % sq.max_nq);
  const int h = (int)(u / sq.max_nq % sq.h_q);
  const int b = (int)(u / sq.max_nq / sq.h_q);
  const int g = h / sq.group;
  const int q0 = sq.cu_seqlens_q[b];
  const int Lq = sq.cu_seqlens_q[b + 1] - q0;
  const int Lk = sq.seqlens_k[b];
  float* out = a.mass + u * sq.max_nk;
  const int tid = threadIdx.x;
  if (qb * BLK >= Lq) {  // past the sequence's end: an all-zero row
    for (int kb = tid; kb < sq.max_nk; kb += THREADS) out[kb] = 0.f;
    return;
  }
  const int off = Lk - Lq;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, hl = lane >> 5;
  const int row = w * 32 + l32;
  const bool row_valid = qb * BLK + row < Lq;
  const int my_pos = off + qb * BLK + row;
  const int n_causal = (off + min(qb * BLK + BLK - 1, Lq - 1)) / BLK + 1;
  for (int kb = n_causal + tid; kb < sq.max_nk; kb += THREADS) out[kb] = 0.f;

  bf16x8 qf[QREGS];
  {
    // rows past the sequence end load nothing; their address is the block's first row
    const int qrow = row_valid ? row : 0;
    const uint16_t* qp = (const uint16_t*)a.q + (int64_t)(q0 + qb * BLK + qrow) * sq.q_tok + (int64_t)h * sq.q_head + hl * 8;
#pragma unroll
    for (int ks = 0; ks < QREGS; ++ks) {
      const uint4 x = row_valid ? *(const uint4*)(qp + ks * 16) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }
  // exp(scale*s - lse) = exp2(s*c2 - lse*log2(e))
  const float c2 = a.scale_log2;
  const float lse2 = row_valid ? a.lse[(size_t)h * a.total_q + q0 + qb * BLK + row] * 1.4426950408889634f : 0.f;
  const int32_t* table = sq.block_table + (int64_t)b * sq.max_blocks_k;
  const size_t page_elems = (size_t)sq.h_kv * BLK * D;

  for (int kb = 0; kb < n_causal; ++kb) {
    const int page = table[kb];
    const int nvalid = min(BLK, Lk - kb * BLK);
    __syncthreads();  // the previous tile's reads are done
    if ((unsigned)page < (unsigned)sq.num_pages) {
      const uint16_t* src = (const uint16_t*)a.k + (size_t)page * page_elems + (size_t)g * BLK * D;
      for (int i = tid; i < BLK * D / 8; i += THREADS) {
        const int r = i / (D / 8), c = i % (D / 8);
        // rows past the sequence end are masked below; keep them finite
        const uint4 x = r < nvalid ? *(const uint4*)(src + (size_t)r * D + c * 8) : make_uint4(0, 0, 0, 0);
        *(uint4*)(kt_lds + r * PITCH + c * 16) = x;
      }
    }
    __syncthreads();
    float acc = 0.f;
    if ((unsigned)page < (unsigned)sq.num_pages) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        f32x16 s;
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] = 0.f;
        const unsigned char* kp = kt_lds + (kt * 32 + l32) * PITCH + hl * 16;
#pragma unroll
        for (int ks = 0; ks < QREGS; ++ks)
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(kp + ks * 32), qf[ks], s, 0, 0, 0);
        // element v is key kb*B + kt*32 + 8*(v/4) + 4*hl + v%4 of this lane's row
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kb * BLK + kt * 32 + 8 * (v >> 2) + 4 * hl + (v & 3);
          if (row_valid && key <= my_pos) acc += __builtin_amdgcn_exp2f(__builtin_fmaf(s[v], c2, -lse2));
        }
      }
    } else {
      acc = __builtin_nanf("");  // a page outside the pool
    }
    acc = wave_sum(acc);
    if (lane == 0) part[w] = acc;
    __syncthreads();
    if (tid == 0) {
      float m = part[0];
#pragma unroll
      for (int i = 1; i < NW; ++i) m += part[i];
      out[kb] = m;
    }
  }
}

template <int D, int BLK>
hipError_t launch_one(const MassArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((block_mass_kernel<D, BLK>), dim3((unsigned)a.n_units), dim3(2 * BLK), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_mass(const MassArgs& a, int head_dim, int block, hipStream_t stream) {
  if (head_dim == 128 && block == 128) return launch_one<128, 128>(a, stream);
  if (head_dim == 128 && block == 64) return launch_one<128, 64>(a, stream);
  if (head_dim == 64 && block == 128) return launch_one<64, 128>(a, stream);
  if (head_dim == 64 && block == 64) return launch_one<64, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace cosa
