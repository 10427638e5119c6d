// Decode-stage ordered walk: one new query token per sequence (bf16, gfx950).
//
// The CoSA pages name decoding as future work without a method; this keeps
// the prefill walk's rules (technical summary §2.3: listed pages only, in list
// order, in-kernel skip from local vs running maxima; §1: the skip is decided
// per query head) and parallelises a (sequence, KV group) list by cutting it
// into contiguous segments that separate workgroups walk, merged afterwards by
// log-sum-exp (online softmax is order invariant, §2.1).
//
// Walk kernel: one workgroup per (sequence, KV group, segment), BLK/32 waves;
// wave w owns keys 32w..32w+31 of every KV block. The group's G query heads
// are the columns of S^T = K Q^T (v_mfma_f32_32x32x16_bf16, G <= 32 of 32
// columns used; decode is bandwidth-bound). K and V pages are loaded into
// registers one block ahead and written to LDS in the XOR-swizzled layouts of
// the prefill kernel, so V^T fragments come from ds_read_b64_tr_b16. The
// block's per-head maxima are combined across waves in LDS; each wave then
// runs the online-softmax update and O^T += V^T P^T over its own 32 keys, and
// the waves' partial sums are added once at the end of the segment.
// Merge kernel: one wave per (sequence, query head) combines the segments.
#include <math.h>

#include "cosa_internal.h"

namespace cosa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kNegInf = -__builtin_huge_valf();

// x combined with lane l ^ 32's x
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int BLK>
struct DecGeo {
  static constexpr int NW = BLK / 32;                // one wave per 32-key tile
  static constexpr int THREADS = 64 * NW;
  static constexpr int DT = D / 32;                  // 32-column tiles of O^T
  static constexpr int QREGS = D / 16;               // k-steps of S
  static constexpr int CH = D / 8;                   // 16-byte chunks per row
  static constexpr int ROWB = D * 2;                 // bytes per row
  static constexpr int TILE = BLK * ROWB;            // bytes per K or V tile
  static constexpr int CPT = TILE / 16 / THREADS;    // 16-byte chunks per thread per tile
  static constexpr int ACCB = DT * 16 * 64 * 4;      // bytes of one wave's O^T partial
  __device__ static constexpr int swz_k(int r) { return r % CH; }
  __device__ static constexpr int swz_v(int r) { return D == 128 ? 4 * (r % 4) : 4 * (r % 2); }
};

template <int D, int BLK>
__global__ __launch_bounds__(2 * BLK, 2) void osk_decode_kernel(DecodeArgs a) {
  using Gm = DecGeo<D, BLK>;
  constexpr int NW = Gm::NW, DT = Gm::DT, QREGS = Gm::QREGS, CH = Gm::CH, ROWB = Gm::ROWB;
  constexpr int TILE = Gm::TILE, CPT = Gm::CPT, THREADS = Gm::THREADS;
  static_assert(CPT * 16 * THREADS == TILE, "whole chunks per thread");
  static_assert((NW - 1) * Gm::ACCB <= 2 * TILE, "wave partials fit in the tiles");
  __shared__ __attribute__((aligned(16))) unsigned char kbuf[TILE];
  __shared__ __attribute__((aligned(16))) unsigned char vbuf[TILE];
  __shared__ float red[NW][32];

  const SeqArgs& sq = a.seq;
  const int G = sq.group;
  const int S = a.n_splits;
  const int64_t u = blockIdx.x;
  const int s = (int)(u % S);
  const int g = (int)(u / S % sq.h_kv);
  const int b = (int)(u / S / sq.h_kv);
  const int q0 = __builtin_amdgcn_readfirstlane(sq.cu_seqlens_q[b]);
  const int Lq = __builtin_amdgcn_readfirstlane(sq.cu_seqlens_q[b + 1]) - q0;
  const int Lk = __builtin_amdgcn_readfirstlane(sq.seqlens_k[b]);
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool col_ok = l32 < G && Lq > 0;  // column l32 is query head g*G + l32

  int n_list = 0;
  const int32_t* lst = nullptr;
  if (Lq > 0) {
    const int64_t list_row = ((int64_t)b * sq.h_kv + g) * sq.max_nq;  // the single query block
    n_list = max(0, min(__builtin_amdgcn_readfirstlane(a.count[list_row]), a.kmax));
    lst = a.order + list_row * a.kmax;
  }
  const int t0 = (int)(((int64_t)s * n_list) / S), t1 = (int)(((int64_t)(s + 1) * n_list) / S);
  const int my_pos = Lk - 1;  // the query token's absolute position
  const int n_causal = Lq > 0 ? my_pos / BLK + 1 : 0;

  bf16x8 qf[QREGS];
  {
    // columns past the group's heads load nothing; their address is the group's first head
    const uint16_t* qp = (const uint16_t*)a.q + (int64_t)q0 * sq.q_tok + (int64_t)(g * G + (col_ok ? l32 : 0)) * sq.q_head + hl * 8;
#pragma unroll
    for (int ks = 0; ks < QREGS; ++ks) {
      const uint4 x = col_ok ? *(const uint4*)(qp + ks * 16) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // ---- register staging of one block's K and V slabs ----------------------
  const int32_t* table = sq.block_table + (int64_t)b * sq.max_blocks_k;
  const size_t page_bytes = (size_t)sq.h_kv * TILE;
  const unsigned char* kg = (const unsigned char*)a.k + (size_t)g * TILE;
  const unsigned char* vg = (const unsigned char*)a.v + (size_t)g * TILE;
  uint4 sk[CPT], sv[CPT];
  int bad = 0;
  // entry t: validates it, loads its rows (rows past the sequence end as
  // zeros, so NaN-filled slots never reach the MFMAs), returns its block
  auto fetch = [&](int t) -> int {
    int kb = __builtin_amdgcn_readfirstlane(lst[t]);
    if (kb < 0 || kb >= n_causal) {
      bad = 1;
      kb = 0;
    }
    int page = __builtin_amdgcn_readfirstlane(table[kb]);
    if ((unsigned)page >= (unsigned)sq.num_pages) {
      bad = 1;
      page = 0;
    }
    const int nvalid = min(BLK, Lk - kb * BLK);
    const unsigned char* kp = kg + (size_t)page * page_bytes;
    const unsigned char* vp = vg + (size_t)page * page_bytes;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int i = tid + THREADS * j, r = i / CH, c = i % CH;
      const bool ok = r < nvalid;
      sk[j] = ok ? *(const uint4*)(kp + r * ROWB + c * 16) : make_uint4(0, 0, 0, 0);
      sv[j] = ok ? *(const uint4*)(vp + r * ROWB + c * 16) : make_uint4(0, 0, 0, 0);
    }
    return kb;
  };
  auto stage = [&]() {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int i = tid + THREADS * j, r = i / CH, c = i % CH;
      *(uint4*)(kbuf + r * ROWB + ((c ^ Gm::swz_k(r)) << 4)) = sk[j];
      *(uint4*)(vbuf + r * ROWB + ((c ^ Gm::swz_v(r)) << 4)) = sv[j];
    }
  };

  // K (A operand of S^T): row 32w + l32, logical chunk 2ks + hl
  const unsigned char* k_lane = kbuf + (w * 32 + l32) * ROWB;
  const int k_swz = Gm::swz_k(l32);
  // V^T (A operand of O^T) via ds_read_b64_tr_b16, as in the prefill kernel
  int v_addr[DT];
  {
    const int i = lane & 15, gi = lane >> 4, hh = gi >> 1, dg = gi & 1;
    const int q = i >> 2;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = dt * 32 + 16 * dg + 4 * (i & 3);
      v_addr[dt] = (4 * hh + q) * ROWB + (((d >> 3) ^ Gm::swz_v(q)) << 4) + (d & 7) * 2;
    }
  }

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[dt][v] = 0.f;
  float m_run = kNegInf;  // running max of raw q.k for this column's head
  float l_run = 0.f;      // this lane's share of the running sum
  int n_skip = 0;
  const float c2 = a.scale_log2;
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};

  int kb_next = 0;
  if (t0 < t1) kb_next = fetch(t0);
  for (int t = t0; t < t1; ++t) {
    __syncthreads();  // every wave is done with the previous block's tiles
    stage();
    const int kb = kb_next;
    if (t + 1 < t1) kb_next = fetch(t + 1);  // in flight while this block computes
    __syncthreads();  // block t visible

    f32x16 sc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sc[v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < QREGS; ++ks)
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(k_lane + (((2 * ks + hl) ^ k_swz) << 4)),
                                                   qf[ks], sc, 0, 0, 0);
    // element v is key kb*B + 32w + 8*(v/4) + 4*hl + v%4
    if (kb * BLK + BLK - 1 > my_pos) {
      const int thr = my_pos - kb * BLK - w * 32 - 4 * hl;
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (8 * (v >> 2) + (v & 3) > thr) sc[v] = kNegInf;
    }
    float mw = sc[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mw = fmaxf(mw, sc[v]);
    mw = xor32_max(mw);
    if (hl == 0) red[w][l32] = mw;
    __syncthreads();  // the block's per-wave maxima are visible
    float m_loc = red[0][l32];
#pragma unroll
    for (int i = 1; i < NW; ++i) m_loc = fmaxf(m_loc, red[i][l32]);

    // skip per query head; the block is skipped outright when every head skips
    const float diff = m_loc != kNegInf ? m_loc - m_run : kNegInf;
    const bool skip_col = a.skip_on && diff < a.skip_thr_raw;
    n_skip += skip_col ? 1 : 0;
    if (__all(skip_col || !col_ok)) continue;
    const float m_new = skip_col ? m_run : fmaxf(m_run, m_loc);
    const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * c2);
    const float mc = (m_new == kNegInf) ? 0.f : m_new * c2;
    bf16x8 pt[2];
#pragma unroll
    for (int v = 0; v < 16; ++v)
      pt[v >> 3][v & 7] = skip_col ? (__bf16)0.f : (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[v], c2, -mc));
    // the row sum adds the same rounded weights that enter P.V
    float rs = 0.f;
    rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pt[0], pt[0], 0, 1), ones, rs, false);
    rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pt[0], pt[0], 2, 3), ones, rs, false);
    rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pt[0], pt[0], 4, 5), ones, rs, false);
    rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pt[0], pt[0], 6, 7), ones, rs, false);
    rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pt[1], pt[1], 0, 1), ones, rs, false);
    rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pt[1], pt[1], 2, 3), ones, rs, false);
    rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pt[1], pt[1], 4, 5), ones, rs, false);
    rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pt[1], pt[1], 6, 7), ones, rs, false);
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[dt][v] *= alpha;
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int st = 2 * w + s2;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vbuf + v_addr[dt] + (st * 16) * ROWB));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vbuf + v_addr[dt] + (st * 16 + 8) * ROWB));
        const bf16x8 vv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pt[s2], acc[dt], 0, 0, 0);
      }
    }
  }

  // ---- the waves' partial sums of this segment (same running max) ---------
  const float lw = xor32_sum(l_run);
  __syncthreads();  // every wave is done with the tiles and the maxima
  if (hl == 0) red[w][l32] = lw;
  if (w > 0) {
    float* slot = (float*)((w - 1) * Gm::ACCB < TILE ? kbuf + (w - 1) * Gm::ACCB : vbuf + (w - 1) * Gm::ACCB - TILE);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) slot[(dt * 16 + v) * 64 + lane] = acc[dt][v];
  }
  __syncthreads();
  if (w == 0 && col_ok) {
    float l_tot = red[0][l32];
    for (int i = 1; i < NW; ++i) {
      l_tot += red[i][l32];
      const float* slot =
          (const float*)((i - 1) * Gm::ACCB < TILE ? kbuf + (i - 1) * Gm::ACCB : vbuf + (i - 1) * Gm::ACCB - TILE);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[dt][v] += slot[(dt * 16 + v) * 64 + lane];
    }
    const int h = g * G + l32;
    const int64_t slot_id = ((int64_t)b * sq.h_q + h) * S + s;
    float* part = a.part + slot_id * (D + 2);
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) part[dt * 32 + 8 * (v >> 2) + 4 * hl + (v & 3)] = bad ? nan : acc[dt][v];
    if (hl == 0) {
      part[D] = m_run;
      part[D + 1] = bad ? nan : l_tot;
      a.part_counts[slot_id * 2] = t1 - t0;
      a.part_counts[slot_id * 2 + 1] = n_skip;
    }
  }
}

// one wave per (sequence, query head): merge the segments by log-sum-exp
template <int D>
__global__ __launch_bounds__(256) void osk_decode_merge(DecodeArgs a) {
  const SeqArgs& sq = a.seq;
  const int lane = threadIdx.x & 63;
  const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // b * h_q + h
  if (unit >= (int64_t)sq.batch * sq.h_q) return;
  const int b = (int)(unit / sq.h_q), h = (int)(unit % sq.h_q);
  const int q0 = sq.cu_seqlens_q[b];
  const int Lq = sq.cu_seqlens_q[b + 1] - q0;
  const int S = a.n_splits;
  const float* part = a.part + unit * S * (D + 2);
  const int32_t* pc = a.part_counts + unit * S * 2;
  if (Lq == 0) {
    if (lane == 0) {
      a.visited[unit * sq.max_nq] = 0;
      a.skipped[unit * sq.max_nq] = 0;
    }
    return;
  }
  float m_star = kNegInf;
  int vis = 0, skp = 0;
  for (int s = 0; s < S; ++s) {
    m_star = fmaxf(m_star, part[s * (D + 2) + D]);
    vis += pc[2 * s];
    skp += pc[2 * s + 1];
  }
  const float c2 = a.scale_log2;
  float l_star = 0.f;
  float o[(D + 63) / 64];
#pragma unroll
  for (int i = 0; i < (D + 63) / 64; ++i) o[i] = 0.f;
  if (m_star != kNegInf) {
    for (int s = 0; s < S; ++s) {
      const float* ps = part + s * (D + 2);
      const float m_s = ps[D];
      if (m_s == kNegInf) continue;
      const float wgt = __builtin_amdgcn_exp2f((m_s - m_star) * c2);
      l_star += wgt * ps[D + 1];
#pragma unroll
      for (int i = 0; i < (D + 63) / 64; ++i)
        if (lane + 64 * i < D) o[i] += wgt * ps[lane + 64 * i];
    }
  } else {
    // no computed key: l stays 0 (or NaN when a segment met a corrupt entry)
    for (int s = 0; s < S; ++s) l_star += part[s * (D + 2) + D + 1];
  }
  const float inv = l_star > 0.f ? 1.f / l_star : (l_star == l_star ? 0.f : l_star);
  uint16_t* orow = (uint16_t*)a.o + (int64_t)q0 * sq.o_tok + (int64_t)h * sq.o_head;
#pragma unroll
  for (int i = 0; i < (D + 63) / 64; ++i)
    if (lane + 64 * i < D) orow[lane + 64 * i] = __builtin_bit_cast(uint16_t, (__bf16)(o[i] * inv));
  if (lane == 0) {
    a.visited[unit * sq.max_nq] = vis;
    a.skipped[unit * sq.max_nq] = skp;
    if (a.lse)
      a.lse[(size_t)h * a.total_q + q0] =
          l_star > 0.f ? m_star * a.scale + logf(l_star) : (l_star == l_star ? kNegInf : l_star);
  }
}

template <int D, int BLK>
hipError_t launch_one(const DecodeArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.seq.batch * a.seq.h_kv * a.n_splits;
  hipLaunchKernelGGL((osk_decode_kernel<D, BLK>), dim3((unsigned)grid), dim3(2 * BLK), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t mgrid = ((int64_t)a.seq.batch * a.seq.h_q + 3) / 4;
  hipLaunchKernelGGL((osk_decode_merge<D>), dim3((unsigned)mgrid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_osk_decode(const DecodeArgs& a, int head_dim, int block, hipStream_t stream) {
  if (head_dim == 128 && block == 128) return launch_one<128, 128>(a, stream);
  if (head_dim == 128 && block == 64) return launch_one<128, 64>(a, stream);
  if (head_dim == 64 && block == 128) return launch_one<64, 128>(a, stream);
  if (head_dim == 64 && block == 64) return launch_one<64, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace cosa
