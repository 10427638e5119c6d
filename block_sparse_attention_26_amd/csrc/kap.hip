// Kernel-Aware Proxy (KAP) for gfx950.
//
// Method: CoSA technical summary (gist.science, "CoSA: Accelerating
// Long-Context Inference via Proxy-Kernel Co-Designed Sparse Attention"),
// §2.2 Stage 1, in the page's order:
//   block ranking - downsample Q and K (kap_pool_q / kap_pool_k: mean over p
//       tokens), approximate scores and MaxPool over the keys of each KV block
//       (kap_score_grp / kap_score: MFMA GEMM with the per-block max fused
//       into its epilogue),
//       MaxNorm (kap_rank_sort: exp(P - row max));
//   HRM flag generation - blocks that attain some pooled row's max, united
//       over the query heads of a KV group (the GQA union follows the
//       CompactAttention page, selection stage);
//   flag-grouped sorting - HRM blocks first, then by block score, cut to the
//       row's budget (kap_rank_sort: bitonic sort of 64-bit keys in LDS).
// §2.1 defines the result as a computation order, not a binary mask.
//
// Bit-exact contract: from the fp32 proxy scores P onwards every operation
// is one IEEE binary32 operation in a fixed order (row max, P - max, exp32,
// a sequential sum over heads then rows, exact comparisons), so order, HRM
// flags and block scores equal those of any other IEEE implementation given
// the same P. Floating-point contraction is disabled for that code.
#include <math.h>

#include <algorithm>

#include <type_traits>

#include "cosa_internal.h"
#include "kap_common.h"

namespace cosa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;


__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) {
  return __builtin_bit_cast(float, h16 << 16);
}

// 8 consecutive elements -> fp32 (the pooling passes read each element once:
// bf16 loads are non-temporal, which keeps the stream out of the way of cached data)
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, size_t elem, float* out) {
  if constexpr (BF16) {
    typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
    const u32x4_nt x = __builtin_nontemporal_load((const u32x4_nt*)((const uint16_t*)base + elem));
    const uint32_t w[4] = {x[0], x[1], x[2], x[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
      out[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  } else {
    const float4 x0 = *(const float4*)((const float*)base + elem);
    const float4 x1 = *(const float4*)((const float*)base + elem + 4);
    out[0] = x0.x; out[1] = x0.y; out[2] = x0.z; out[3] = x0.w;
    out[4] = x1.x; out[5] = x1.y; out[6] = x1.z; out[7] = x1.w;
  }
}

template <bool BF16>
__device__ __forceinline__ void store8(void* base, size_t elem, const float* v) {
  if constexpr (BF16) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[2 * i]) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[2 * i + 1]) << 16);
    *(uint4*)((uint16_t*)base + elem) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    *(float4*)((float*)base + elem) = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)((float*)base + elem + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// ---- pooling (reading R1: mean over p consecutive tokens) ------------------
// One workgroup per (sequence, pooled row); 8-element chunks over h_q * D.
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void kap_pool_q(KapArgs a) {
  const SeqArgs& sq = a.seq;
  const int b = blockIdx.x / a.max_nr, r = blockIdx.x % a.max_nr;
  const int q0 = sq.cu_seqlens_q[b];
  const int Lq = sq.cu_seqlens_q[b + 1] - q0;
  const int lo = r * a.pool;
  if (lo >= Lq) return;
  const int hi = min(lo + a.pool, Lq);
  const float inv_cnt = 1.f / (float)(hi - lo);
  const int chunks = sq.h_q * D / 8;
  for (int c = threadIdx.x; c < chunks; c += kThreads) {
    const int64_t cin = (int64_t)(c / (D / 8)) * sq.q_head + (c % (D / 8)) * 8;  // this chunk within a token
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // eight tokens' loads in flight at a time; the sum stays in token order
    int tok = lo;
    for (; tok + 8 <= hi; tok += 8) {
      float x[8][8];
#pragma unroll
      for (int u = 0; u < 8; ++u) load8<BF16>(a.q, (size_t)((int64_t)(q0 + tok + u) * sq.q_tok + cin), x[u]);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += x[u][i];
    }
    for (; tok < hi; ++tok) {
      float x[8];
      load8<BF16>(a.q, (size_t)((int64_t)(q0 + tok) * sq.q_tok + cin), x);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += x[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= inv_cnt;
    store8<BF16>(a.q_pool, ((size_t)b * a.max_nr + r) * sq.h_q * D + (size_t)c * 8, acc);
  }
}

// One workgroup per (sequence, KV block): pools the page into B/p slots.
template <bool BF16, int D, int BLK>
__global__ __launch_bounds__(kThreads) void kap_pool_k(KapArgs a) {
  const SeqArgs& sq = a.seq;
  // every block (one workgroup per (sequence, block)), or, in decode, only
  // the last block of each sequence (one workgroup per (sequence, KV head))
  const bool last = a.pool_last_only != 0;
  const int b = last ? blockIdx.x / sq.h_kv : blockIdx.x / sq.max_nk;
  const int Lk = sq.seqlens_k[b];
  const int kb = last ? (Lk - 1) / BLK : blockIdx.x % sq.max_nk;
  if (Lk <= 0 || kb * BLK >= Lk) return;
  const int page = sq.block_table[(int64_t)b * sq.max_blocks_k + kb];
  if ((unsigned)page >= (unsigned)sq.num_pages) return;
  const int nvalid = min(BLK, Lk - kb * BLK);
  const int per = BLK / a.pool;  // pooled slots per page
  constexpr int CH = D / 8;
  const int chunks = (last ? 1 : sq.h_kv) * per * CH;
  for (int c = threadIdx.x; c < chunks; c += kThreads) {
    const int dch = c % CH;
    const int slot = (c / CH) % per;
    const int g = last ? (int)(blockIdx.x % sq.h_kv) : c / (CH * per);
    const int lo = slot * a.pool;
    const int hi = min(lo + a.pool, nvalid);
    const size_t row0 = ((size_t)page * sq.h_kv + g) * BLK;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // four tokens' loads in flight at a time; the sum stays in token order
    int tok = lo;
    for (; tok + 4 <= hi; tok += 4) {
      float x[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) load8<BF16>(a.k, (row0 + tok + u) * D + dch * 8, x[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += x[u][i];
    }
    for (; tok < hi; ++tok) {
      float x[8];
      load8<BF16>(a.k, (row0 + tok) * D + dch * 8, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += x[i];
    }
    const float inv_cnt = hi > lo ? 1.f / (float)(hi - lo) : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= inv_cnt;
    store8<BF16>(a.k_pool, (((size_t)page * sq.h_kv + g) * per + slot) * D + dch * 8, acc);
  }
}

// llvm.maximum (v_maximum3_f32 on gfx950): unlike fmaxf it needs no quieting
// copy of operands the compiler cannot prove free of signaling NaNs
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// ---- proxy scores with fused MaxPool (readings R2-R4) ----------------------
// One workgroup per (sequence, query head, tile of 32*RT pooled rows), longest
// tiles first. Each of the 4 waves computes 32-key x 32-row tiles of
// S^T = Kpool . Qpool^T per step (128 pooled keys per step), one per row tile
// against the same K fragments (loaded one step ahead). Blocks of 4..32 pooled
// keys are reduced to their maxima in registers (RT = 2; the fp32 path, bf16
// takes the group form below); other block sizes go through LDS (RT = 1).
constexpr int kScoreRows = 32;
constexpr int kScoreKeys = 128;

template <bool BF16, int D, int BLK, int RT>
__global__ __launch_bounds__(kThreads) void kap_score(KapArgs a) {
  constexpr int ROWS = kScoreRows * RT;  // pooled query rows per workgroup
  // LDS reduction (blocks of 1, 2, 64 or 128 pooled keys), double-buffered
  __shared__ float tile[RT == 1 ? 2 : 1][RT == 1 ? kScoreRows : 1][kScoreKeys + 1];
  // RT > 1: block maxima staged per chunk of CB blocks (double-buffered) so
  // that P is written in whole 128-byte row segments
  constexpr int CB = 32;
  __shared__ float pst[RT > 1 ? 2 : 1][RT > 1 ? ROWS : 1][CB + 1];
  const SeqArgs& sq = a.seq;
  const int G = sq.group;
  const int ntile = (a.max_nr + ROWS - 1) / ROWS;
  const int64_t bid = blockIdx.x;
  const int h = (int)(bid % sq.h_q);
  int64_t rest = bid / sq.h_q;
  const int b = (int)(rest % sq.batch);
  const int rt = ntile - 1 - (int)(rest / sq.batch);
  const int g = h / G;
  const int q0 = sq.cu_seqlens_q[b];
  const int Lq = sq.cu_seqlens_q[b + 1] - q0;
  const int Lk = sq.seqlens_k[b];
  const int off = Lk - Lq;
  const int p = a.pool;
  const int per = BLK / p;  // pooled keys per KV block
  const int R = (Lq + p - 1) / p;
  const int Rk = (Lk + p - 1) / p;
  const int nk = (Lk + BLK - 1) / BLK;
  const int r0 = rt * ROWS;
  float* P = a.scores + (((int64_t)b * sq.h_q + h) * a.max_nr) * sq.max_nk;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;

  if (r0 >= R) {
    if (a.fill_scores)
      for (int i = tid; i < ROWS * sq.max_nk; i += kThreads) {
        const int r = r0 + i / sq.max_nk;
        if (r < a.max_nr) P[(int64_t)r * sq.max_nk + i % sq.max_nk] = kNegInf;
      }
    return;
  }
  // Blocks computed: every causal block of the query block holding the
  // tile's last row (a superset of what any row of the tile can see).
  const int r_last = min(r0 + ROWS, R) - 1;
  const int qb_last = r_last / per;
  const int kb_end = min((off + min(qb_last * BLK + BLK - 1, Lq - 1)) / BLK + 1, nk);

  // this lane's query rows (B operands), one per row tile
  int my_jmax[RT];
  constexpr int QREGS = BF16 ? D / 16 : D / 2;
  bf16x8 qf16[RT][BF16 ? QREGS : 1];
  float qf32[RT][BF16 ? 1 : QREGS];
#pragma unroll
  for (int u = 0; u < RT; ++u) {
    const int my_r = r0 + u * kScoreRows + l32;
    const bool r_ok = my_r < R;
    my_jmax[u] = r_ok ? (off + min(my_r * p + p - 1, Lq - 1)) / p : -1;
    const size_t qoff = (((size_t)b * a.max_nr + (r_ok ? my_r : r0)) * sq.h_q + h) * D;
    if constexpr (BF16) {
      const uint16_t* qp = (const uint16_t*)a.q_pool + qoff + hl * 8;
#pragma unroll
      for (int ks = 0; ks < QREGS; ++ks) {
        uint4 x = r_ok ? *(const uint4*)(qp + ks * 16) : make_uint4(0, 0, 0, 0);
        qf16[u][ks] = __builtin_bit_cast(bf16x8, x);
      }
    } else {
      const float* qp = (const float*)a.q_pool + qoff + hl;
#pragma unroll
      for (int ks = 0; ks < QREGS; ++ks) qf32[u][ks] = r_ok ? qp[2 * ks] : 0.f;
    }
  }

  const int jend = kb_end * per;  // pooled keys covered
  // the sequence's block table row, staged once (the fragment addresses of a
  // step then need no dependent global load)
  __shared__ int32_t ptab[kMaxSortBlocks];
  for (int i = tid; i < kb_end; i += kThreads) ptab[i] = sq.block_table[(int64_t)b * sq.max_blocks_k + i];
  __syncthreads();
  // this lane's key row (A operand) of the step at j0: element offset, or -1
  auto key_off = [&](int j0) -> int64_t {
    const int jk = j0 + w * 32 + l32;
    if (!(jk < Rk && jk < jend)) return -1;
    const int page = ptab[jk / per];
    return (int64_t)((((size_t)page * sq.h_kv + g) * per) + jk % per) * D;
  };
  // the next step's K fragments are loaded while the current step computes
  constexpr int KREGS = BF16 ? QREGS : 1;
  uint4 kc[KREGS], kn[KREGS];
  int64_t koff_c = key_off(0);
  if constexpr (BF16) {
    const uint16_t* kp = (const uint16_t*)a.k_pool + (koff_c < 0 ? 0 : koff_c) + hl * 8;
#pragma unroll
    for (int ks = 0; ks < QREGS; ++ks) kc[ks] = *(const uint4*)(kp + ks * 16);  // masked when invalid
  }
  float rmx[RT];  // running row maxima over this wave's keys (RT > 1)
#pragma unroll
  for (int u = 0; u < RT; ++u) rmx[u] = kNegInf;
  int it = 0;
  // the tile's first row sees the fewest keys
  const int jmax_first = (off + min(r0 * p + p - 1, Lq - 1)) / p;
  // one 128-key step on the current fragments, loading the next step's; the
  // loop runs two steps per trip with the fragment buffers swapped, so the
  // prefetched fragments are never copied
  auto step = [&](int j0, int it, uint4 (&cur)[KREGS], uint4 (&nxt)[KREGS]) {
      const int64_t koff_n = j0 + kScoreKeys < jend ? key_off(j0 + kScoreKeys) : -1;
      const bool edge = j0 + kScoreKeys - 1 > jmax_first || j0 + kScoreKeys > Rk;
      if constexpr (BF16) {
        const uint16_t* kp = (const uint16_t*)a.k_pool + (koff_n < 0 ? 0 : koff_n) + hl * 8;
#pragma unroll
        for (int ks = 0; ks < QREGS; ++ks) nxt[ks] = *(const uint4*)(kp + ks * 16);  // an invalid key is masked
      }
      // ---- per row tile, one 32x32 MFMA tile per wave: keys j0 + w*32 + [0,32)
      f32x16 sc[RT];
#pragma unroll
      for (int u = 0; u < RT; ++u)
#pragma unroll
        for (int v = 0; v < 16; ++v) sc[u][v] = 0.f;
      if constexpr (BF16) {
#pragma unroll
        for (int ks = 0; ks < QREGS; ++ks)
#pragma unroll
          for (int u = 0; u < RT; ++u)
            sc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cur[ks]), qf16[u][ks], sc[u], 0, 0, 0);
      } else {
        const bool k_ok = koff_c >= 0;
        const float* kp = (const float*)a.k_pool + (k_ok ? koff_c : 0) + hl;
#pragma unroll
        for (int ks = 0; ks < QREGS; ++ks) {
          const float kv = k_ok ? kp[2 * ks] : 0.f;
#pragma unroll
          for (int u = 0; u < RT; ++u) sc[u] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv, qf32[u][ks], sc[u], 0, 0, 0);
        }
      }
#pragma unroll
      for (int u = 0; u < RT; ++u) {
        // element v of this lane: key jj = w*32 + 8*(v/4) + 4*hl + v%4 of the step
        float x[16];
        if constexpr (RT > 1) {
          // Raw dot products; the scale is applied after the max-pool (rounding
          // of scale*x is monotone in x, so max then scale gives the same bits).
          // Only steps that reach the first row's causal edge or the key range
          // end need the mask.
          if (edge) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int j = j0 + w * 32 + 8 * (v >> 2) + 4 * hl + (v & 3);
              x[v] = (j <= my_jmax[u] && j < Rk) ? sc[u][v] : kNegInf;
            }
          } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) x[v] = sc[u][v];
          }
        } else {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int j = j0 + w * 32 + 8 * (v >> 2) + 4 * hl + (v & 3);
            x[v] = (j <= my_jmax[u] && j < Rk) ? sc[u][v] * a.scale : kNegInf;
          }
        }
        if constexpr (RT > 1) {
          // blocks of 4..32 keys lie inside one wave's 32 keys: maxima in
          // registers, the two lane halves exchanged with v_permlane32_swap
          float g4[4], o4[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) g4[q] = vmax(vmax(x[4 * q], x[4 * q + 1]), vmax(x[4 * q + 2], x[4 * q + 3]));
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(g4[q]), __float_as_uint(g4[q]), false, false);
            o4[q] = __uint_as_float(hl ? sw[0] : sw[1]);  // the other half's value
          }
          const int r = r0 + u * kScoreRows + l32;
          rmx[u] = vmax(rmx[u], vmax(vmax(vmax(g4[0], o4[0]), vmax(g4[1], o4[1])),
                                       vmax(vmax(g4[2], o4[2]), vmax(g4[3], o4[3]))));
          if (hl == 0 && r < R) {
            const int kbase = (j0 + w * 32) / per;
            float* srow = pst[(kbase / CB) & 1][u * kScoreRows + l32] + kbase % CB;
            float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            int nb;
            if (per == 4) {  // block 2q + half
              nb = 8;
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                m[2 * q] = g4[q];
                m[2 * q + 1] = o4[q];
              }
            } else if (per == 8) {  // block q
              nb = 4;
#pragma unroll
              for (int q = 0; q < 4; ++q) m[q] = vmax(g4[q], o4[q]);
            } else if (per == 16) {  // block q/2
              nb = 2;
              m[0] = vmax(vmax(g4[0], o4[0]), vmax(g4[1], o4[1]));
              m[1] = vmax(vmax(g4[2], o4[2]), vmax(g4[3], o4[3]));
            } else {  // per == 32
              nb = 1;
              m[0] = vmax(vmax(vmax(g4[0], o4[0]), vmax(g4[1], o4[1])),
                           vmax(vmax(g4[2], o4[2]), vmax(g4[3], o4[3])));
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
              if (i < nb) srow[i] = m[i];
          }
        } else {
          float (*tl)[kScoreKeys + 1] = tile[it & 1];
#pragma unroll
          for (int v = 0; v < 16; ++v) tl[l32][w * 32 + 8 * (v >> 2) + 4 * hl + (v & 3)] = x[v];
          __syncthreads();
          // ---- per-block maxima of the 128-key step --------------------------
          const int nblk = kScoreKeys / per < 1 ? 1 : kScoreKeys / per;
          for (int i = tid; i < kScoreRows * nblk; i += kThreads) {
            const int rr = i / nblk, bi = i % nblk;
            const int kb = (j0 + bi * per) / per;
            const int r = r0 + rr;
            if (r >= R || kb >= kb_end) continue;
            float m = kNegInf;
            for (int e = 0; e < per; ++e) m = fmaxf(m, tl[rr][bi * per + e]);
            P[(int64_t)r * sq.max_nk + kb] = m;
          }
        }
      }
      if constexpr (RT > 1) {
        // last step of a chunk of CB blocks: write the chunk's rows, scaled
        const int cks = CB * per;  // keys per chunk
        if ((j0 + kScoreKeys) % cks == 0 || j0 + kScoreKeys >= jend) {
          const int ch = j0 / cks;
          __syncthreads();
          for (int i = tid; i < ROWS * CB; i += kThreads) {
            const int rr = i / CB, c = i % CB;
            const int r = r0 + rr, kb = ch * CB + c;
            if (r < R && kb < kb_end) P[(int64_t)r * sq.max_nk + kb] = pst[ch & 1][rr][c] * a.scale;
          }
        }
      }
    koff_c = koff_n;
  };
  for (int j0 = 0; j0 < jend; j0 += 2 * kScoreKeys, it += 2) {
    step(j0, it, kc, kn);
    if (j0 + kScoreKeys < jend) step(j0 + kScoreKeys, it + 1, kn, kc);
  }
  if constexpr (RT > 1) {
    // Row maxima of P: each wave saw a quarter of every step's keys, so the
    // four partial maxima are combined through LDS. Blocks past a row's causal
    // range are all -inf for that row, so the maximum equals the one over its
    // causal blocks.
    if (a.row_max) {
      __shared__ float part[kThreads / 64][ROWS];
      if (hl == 0)
#pragma unroll
        for (int u = 0; u < RT; ++u) part[w][u * kScoreRows + l32] = rmx[u] * a.scale;
      __syncthreads();
      for (int i = tid; i < ROWS; i += kThreads) {
        const int r = r0 + i;
        float m = part[0][i];
#pragma unroll
        for (int ww = 1; ww < kThreads / 64; ++ww) m = fmaxf(m, part[ww][i]);
        if (r < R) a.row_max[((int64_t)b * sq.h_q + h) * a.max_nr + r] = m;
      }
    }
  }
  if (a.fill_scores) {
    // -inf for blocks past this tile's reach and for padding rows
    for (int i = tid; i < ROWS * sq.max_nk; i += kThreads) {
      const int r = r0 + i / sq.max_nk, kb = i % sq.max_nk;
      if (r >= a.max_nr) continue;
      if (r >= R || kb >= kb_end) P[(int64_t)r * sq.max_nk + kb] = kNegInf;
    }
  }
}

// ---- proxy scores, group form (bf16, blocks of 4..32 pooled keys) ----------
// One workgroup per (sequence, KV group, four (query head, 32-row tile)
// pairs), pairs numbered tile-major so a workgroup's waves share a row tile
// when G >= 4 and hold adjacent tiles otherwise; longest tiles first. Each
// step's 128 pooled keys are copied once into LDS (global_load_lds, rows
// XOR-swizzled by (row mod 16) through the choice of each lane's source
// chunk) and shared by the four waves. Each wave forms S^T = Kpool . Qpool^T for its 32 rows
// against all keys of a step (two 32-key tiles), so its row maxima need no
// combining across waves, and writes the step's block maxima (times the
// scale: rounding of scale * x is monotone in x) straight from registers.
// When the pairs alone give too few workgroups for the chip (a short query
// chunk over a long cache), score_splits workgroups share a pair set, each
// taking a contiguous share of its steps, and the row maxima are left to the
// rank pass.
// Steps are 64 keys in a ring of NSTAGE LDS stages: the copy of step
// t + NSTAGE - 1 is issued when step t starts.
template <int D, int BLK>
__global__ __launch_bounds__(kThreads, 2) void kap_score_grp(KapArgs a) {
  constexpr int STEP = 64;               // pooled keys per step
  constexpr int NSTAGE = 3;              // LDS ring (three workgroups per CU at d = 128)
  constexpr int ROWB = D * 2;            // bytes per pooled key row
  constexpr int STAGE = STEP * ROWB;     // bytes per step tile
  constexpr int CH = D / 8;              // 16-byte chunks per row
  constexpr int RPC = 1024 / ROWB;       // rows per 1 KB copy
  constexpr int CPW = STAGE / 1024 / 4;  // copies per wave per step
  constexpr int QREGS = D / 16;
  constexpr int KT = STEP / 32;
  __shared__ __attribute__((aligned(1024))) unsigned char kst[NSTAGE][STAGE];
  extern __shared__ int32_t ptab[];      // the sequence's block-table row (dynamic)
  const SeqArgs& sq = a.seq;
  const int G = sq.group;
  const int ntile = (a.max_nr + 31) / 32;
  const int npb = (G * ntile + 3) / 4;   // pair blocks per (sequence, group)
  const int nsplit = a.score_splits;
  const int split = (int)(blockIdx.x % nsplit);
  const int64_t bid = blockIdx.x / nsplit;
  const int g = (int)(bid % sq.h_kv);
  int64_t rest = bid / sq.h_kv;
  const int b = (int)(rest % sq.batch);
  const int pb = npb - 1 - (int)(rest / sq.batch);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int q0 = __builtin_amdgcn_readfirstlane(sq.cu_seqlens_q[b]);
  const int Lq = __builtin_amdgcn_readfirstlane(sq.cu_seqlens_q[b + 1]) - q0;
  const int Lk = __builtin_amdgcn_readfirstlane(sq.seqlens_k[b]);
  const int off = Lk - Lq;
  const int p = a.pool;
  const int per = BLK / p;               // pooled keys per KV block: 4, 8, 16 or 32
  const int lper = __builtin_ctz(per);
  const int R = (Lq + p - 1) / p;
  const int Rk = (Lk + p - 1) / p;
  const int nk = (Lk + BLK - 1) / BLK;
  // this wave's pair
  const int pair = pb * 4 + w;
  const int rt = pair / G;
  const int h = g * G + pair % G;
  const bool wave_on = pair < G * ntile;
  const int r0 = rt * 32;
  float* P = a.scores + (((int64_t)b * sq.h_q + h) * a.max_nr) * sq.max_nk;
  // -inf for a wave's rows and blocks it does not compute (export mode)
  auto fill_rest = [&](int kb_from) {
    if (!a.fill_scores || !wave_on || split != 0) return;
    for (int i = lane; i < 32 * sq.max_nk; i += 64) {
      const int r = r0 + i / sq.max_nk, kb = i % sq.max_nk;
      if (r < a.max_nr && (r >= R || kb >= kb_from)) P[(int64_t)r * sq.max_nk + kb] = kNegInf;
    }
  };
  // the workgroup's last pair holds its furthest rows
  const int rt_last = min(pb * 4 + 3, G * ntile - 1) / G;
  const int r_last = min(rt_last * 32 + 32, R) - 1;
  if (pb * 4 / G * 32 >= R) {  // no row of this sequence here
    fill_rest(0);
    return;
  }
  const int qb_last = r_last >> lper;
  const int kb_end = min((off + min(qb_last * BLK + BLK - 1, Lq - 1)) / BLK + 1, nk);
  const int jend = kb_end * per;  // pooled keys covered
  // this workgroup's share of the steps
  const int nsteps = (jend + STEP - 1) / STEP;
  const int j_lo = (int)((int64_t)split * nsteps / nsplit) * STEP;
  const int j_hi = min((int)((int64_t)(split + 1) * nsteps / nsplit) * STEP, jend);
  if (j_lo >= j_hi) {
    fill_rest(kb_end);
    return;
  }

  for (int i = tid; i < kb_end; i += kThreads) ptab[i] = sq.block_table[(int64_t)b * sq.max_blocks_k + i];

  // query fragments (B operand) of this wave's 32 rows
  const int my_r = r0 + l32;
  const bool r_ok = wave_on && my_r < R;
  const int my_jmax = r_ok ? (off + min(my_r * p + p - 1, Lq - 1)) / p : -1;
  const int jmax_first = wave_on && r0 < R ? (off + min(r0 * p + p - 1, Lq - 1)) / p : -1;
  bf16x8 qf[QREGS];
  {
    const size_t qoff = (((size_t)b * a.max_nr + (r_ok ? my_r : 0)) * sq.h_q + (wave_on ? h : 0)) * D;
    const uint16_t* qp = (const uint16_t*)a.q_pool + qoff + hl * 8;
#pragma unroll
    for (int ks = 0; ks < QREGS; ++ks) {
      const uint4 x = r_ok ? *(const uint4*)(qp + ks * 16) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }
  __syncthreads();  // ptab staged

  // copy n of this wave fills stage bytes [(w*CPW + n) * 1024, +1024): row
  // cr = (w*CPW + n)*RPC + lane/CH of the step, physical chunk lane%CH holding
  // logical chunk (lane%CH) ^ (cr % CH). A row past the covered blocks reads
  // the last covered block (its scores are masked).
  const unsigned char* kpool = (const unsigned char*)a.k_pool + (size_t)g * per * ROWB;
  const size_t page_bytes = (size_t)sq.h_kv * per * ROWB;
  uint32_t c_off[CPW];
  int c_blk[CPW];
#pragma unroll
  for (int n = 0; n < CPW; ++n) {
    const int cr = (w * CPW + n) * RPC + lane / CH;
    c_off[n] = (uint32_t)((cr & (per - 1)) * ROWB + (((lane % CH) ^ (cr % CH)) << 4));
    c_blk[n] = cr >> lper;
  }
  auto issue = [&](int j0, int stage) {
#pragma unroll
    for (int n = 0; n < CPW; ++n) {
      const int kbq = min((j0 >> lper) + c_blk[n], kb_end - 1);
      const unsigned page = min((unsigned)ptab[kbq], (unsigned)sq.num_pages - 1u);  // a corrupt entry stays in the pool
      const unsigned char* src = kpool + (size_t)page * page_bytes + c_off[n];
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(kst[stage] + (w * CPW + n) * 1024), 16, 0, 0);
    }
  };

  // A operand: key row kt*32 + l32, logical chunk 2*ks + hl
  const int k_swz = l32 % CH;
  float rmx = kNegInf;       // raw row maximum over the computed keys
  float pend[16];            // scaled block maxima waiting for their row segment to complete
  int npend = 0;             // steps in the ring since the last write
  // s_waitcnt with vmcnt <= (NSTAGE-2)*CPW (expcnt and lgkmcnt at their
  // maxima): vector memory operations complete in issue order, and when the
  // copies of the NSTAGE-2 following steps were issued after this step's, at
  // least that many operations are newer than it
  constexpr int AHEAD = NSTAGE - 2;
  constexpr int kWaitAhead = (AHEAD * CPW) | (7 << 4) | (0xF << 8);
  static_assert(AHEAD * CPW < 16, "vmcnt field");
#pragma unroll
  for (int t = 0; t < NSTAGE - 1; ++t)
    if (j_lo + t * STEP < j_hi) issue(j_lo + t * STEP, t);
  int stage = 0;
  for (int j0 = j_lo; j0 < j_hi; j0 += STEP, stage = stage + 1 == NSTAGE ? 0 : stage + 1) {
    if (j0 + AHEAD * STEP < j_hi)
      __builtin_amdgcn_s_waitcnt(kWaitAhead);
    else
      __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // this step's tile landed; every wave is done with the previous step's stage
    if (j0 + (NSTAGE - 1) * STEP < j_hi) issue(j0 + (NSTAGE - 1) * STEP, stage == 0 ? NSTAGE - 1 : stage - 1);
    if (!wave_on) continue;
    const unsigned char* kl = kst[stage] + l32 * ROWB;
    f32x16 sc[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[kt][v] = 0.f;
    // fragments of k-step ks+1 are read while the MFMAs of k-step ks run (order
    // pinned: without it the reads were placed just before their MFMAs)
    {
      bf16x8 kf[2][KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) kf[0][kt] = *(const bf16x8*)(kl + kt * 32 * ROWB + (((hl) ^ k_swz) << 4));
#pragma unroll
      for (int ks = 0; ks < QREGS; ++ks) {
        if (ks + 1 < QREGS) {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
            kf[(ks + 1) & 1][kt] = *(const bf16x8*)(kl + kt * 32 * ROWB + (((2 * (ks + 1) + hl) ^ k_swz) << 4));
        }
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) sc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks & 1][kt], qf[ks], sc[kt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, KT, 0);
#pragma unroll
      for (int ks = 0; ks < QREGS; ++ks) {
        if (ks + 1 < QREGS) __builtin_amdgcn_sched_group_barrier(0x100, KT, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, KT, 0);
      }
    }
    // element v of tile kt: key j0 + kt*32 + 8*(v/4) + 4*hl + v%4; only steps
    // that reach the first row's causal edge or the key range end need the mask
    const bool edge = j0 + STEP - 1 > jmax_first || j0 + STEP > Rk;
    float bm[STEP / 4];  // block maxima of the step (NB used)
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      if (edge) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = j0 + kt * 32 + 8 * (v >> 2) + 4 * hl + (v & 3);
          if (!(j <= my_jmax && j < Rk)) sc[kt][v] = kNegInf;
        }
      }
      // maxima of the lane's four groups of 4 keys, and of the other half's
      float g4[4], o4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) g4[q] = vmax(vmax(sc[kt][4 * q], sc[kt][4 * q + 1]), vmax(sc[kt][4 * q + 2], sc[kt][4 * q + 3]));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(g4[q]), __float_as_uint(g4[q]), false, false);
        o4[q] = __uint_as_float(hl ? sw[0] : sw[1]);
      }
      // keys 8q..8q+3 and 8q+4..8q+7 of the tile
      float lo[4], hi[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        lo[q] = hl ? o4[q] : g4[q];
        hi[q] = hl ? g4[q] : o4[q];
      }
      const float t01 = vmax(vmax(lo[0], hi[0]), vmax(lo[1], hi[1]));
      const float t23 = vmax(vmax(lo[2], hi[2]), vmax(lo[3], hi[3]));
      rmx = vmax(rmx, vmax(t01, t23));
      if (per == 4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bm[kt * 8 + 2 * q] = lo[q];
          bm[kt * 8 + 2 * q + 1] = hi[q];
        }
      } else if (per == 8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) bm[kt * 4 + q] = vmax(lo[q], hi[q]);
      } else if (per == 16) {
        bm[kt * 2] = t01;
        bm[kt * 2 + 1] = t23;
      } else {
        bm[kt] = vmax(t01, t23);
      }
    }
    // the step's NB block maxima of this lane's row (the two lane halves hold
    // one half each) wait in a register ring until a 32-block (128-byte)
    // segment of the row is complete, which both halves then write in the
    // same store instructions: lines of P are written whole, not a few bytes
    // per step (partly written lines evicted early were written twice)
    auto stash = [&](auto nb_c) {
      constexpr int NB = decltype(nb_c)::value;  // blocks per step
      constexpr int HALF = NB / 2;
      constexpr int F = 32 / NB;                 // steps per segment
      static_assert(F * HALF == 16, "ring size");
#pragma unroll
      for (int t = 0; t < F - 1; ++t)
#pragma unroll
        for (int i = 0; i < HALF; ++i) pend[t * HALF + i] = pend[(t + 1) * HALF + i];
#pragma unroll
      for (int i = 0; i < HALF; ++i) pend[(F - 1) * HALF + i] = (hl ? bm[HALF + i] : bm[i]) * a.scale;
      ++npend;
      const int kb_next = (j0 >> lper) + NB;  // the first block after this step
      if ((kb_next & 31) == 0 || j0 + STEP >= j_hi) {
        if (r_ok) {
#pragma unroll
          for (int t = 0; t < F; ++t) {
            if (t >= F - npend) {  // slot t: the step starting at block kb_next - (F - t) * NB
              const int kb = kb_next - (F - t) * NB + hl * HALF;
              float* dst = P + (int64_t)my_r * sq.max_nk + kb;
              const int room = kb_end - kb;  // blocks of this half still covered
              if (HALF % 4 == 0 && room >= HALF && ((uintptr_t)dst & 15) == 0) {
#pragma unroll
                for (int i = 0; i < HALF; i += 4)
                  *(float4*)(dst + i) = make_float4(pend[t * HALF + i], pend[t * HALF + i + 1],
                                                    pend[t * HALF + i + 2], pend[t * HALF + i + 3]);
              } else {
#pragma unroll
                for (int i = 0; i < HALF; ++i)
                  if (i < room) dst[i] = pend[t * HALF + i];
              }
            }
          }
        }
        npend = 0;
      }
    };
    if (per == 4) stash(std::integral_constant<int, STEP / 4>{});
    else if (per == 8) stash(std::integral_constant<int, STEP / 8>{});
    else if (per == 16) stash(std::integral_constant<int, STEP / 16>{});
    else stash(std::integral_constant<int, STEP / 32>{});
  }
  if (wave_on) {
    if (a.row_max && hl == 0 && r_ok) a.row_max[((int64_t)b * sq.h_q + h) * a.max_nr + my_r] = rmx * a.scale;
    fill_rest(kb_end);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no copy is in flight when the workgroup's LDS is released
}

// ---- MaxNorm, HRM, block score, flag-grouped sort, budget (R5-R10) ---------
// One workgroup per (sequence, KV group, query block), longest rows first.

// ---- proxy scores for decode problems (one pooled query row per sequence) --
// The G query heads of a KV group are the MFMA columns (Kpool . Qpool^T with
// G of 32 columns used), so one workgroup scores a chunk of kDecodeKeys
// pooled keys for the whole group; blocks of 4..32 pooled keys are reduced in
// registers as in kap_score. Row maxima are left to the rank pass.
constexpr int kDecodeKeys = 512;

template <int D, int BLK>
__global__ __launch_bounds__(kThreads) void kap_score_decode(KapArgs a) {
  const SeqArgs& sq = a.seq;
  const int G = sq.group;
  const int p = a.pool;
  const int per = BLK / p;
  const int nchunk = (sq.max_nk * per + kDecodeKeys - 1) / kDecodeKeys;
  const int64_t bid = blockIdx.x;
  const int chunk = (int)(bid % nchunk);
  const int g = (int)(bid / nchunk % sq.h_kv);
  const int b = (int)(bid / nchunk / sq.h_kv);
  const int q0 = sq.cu_seqlens_q[b];
  const int Lq = sq.cu_seqlens_q[b + 1] - q0;
  const int Lk = sq.seqlens_k[b];
  const int off = Lk - Lq;
  const int Rk = (Lk + p - 1) / p;
  const int nk = (Lk + BLK - 1) / BLK;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hl = lane >> 5;
  const bool col_ok = l32 < G && Lq > 0;  // column l32 is query head g*G + l32
  const int h = g * G + (l32 < G ? l32 : 0);
  const int jmax = Lq > 0 ? (off + min(p - 1, Lq - 1)) / p : -1;  // last pooled key row 0 sees
  const int kb0 = chunk * (kDecodeKeys / per);
  const int kb1 = min(kb0 + kDecodeKeys / per, sq.max_nk);
  const int kb_end = Lq > 0 ? min(min(jmax / per + 1, nk), kb1) : kb0;  // computed: [kb0, kb_end)
  if (a.fill_scores && lane < 32 && l32 < G)
    for (int kb = max(kb_end, kb0) + w * 1; kb < kb1; kb += kThreads / 64)  // blocks no key of which is seen
      a.scores[(((int64_t)b * sq.h_q + g * G + l32) * a.max_nr) * sq.max_nk + kb] = kNegInf;
  if (kb_end <= kb0) return;

  constexpr int QREGS = D / 16;
  bf16x8 qf[QREGS];
  {
    const uint16_t* qp = (const uint16_t*)a.q_pool + (((size_t)b * a.max_nr) * sq.h_q + h) * D + hl * 8;
#pragma unroll
    for (int ks = 0; ks < QREGS; ++ks) {
      const uint4 x = col_ok ? *(const uint4*)(qp + ks * 16) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }
  const int jend = kb_end * per;
  auto key_off = [&](int j0) -> int64_t {
    const int jk = j0 + w * 32 + l32;
    if (!(jk < Rk && jk < jend)) return -1;
    const int page = sq.block_table[(int64_t)b * sq.max_blocks_k + jk / per];
    return (int64_t)((((size_t)page * sq.h_kv + g) * per) + jk % per) * D;
  };
  uint4 kc[QREGS], kn[QREGS];
  int64_t koff = key_off(kb0 * per);
  {
    const uint16_t* kp = (const uint16_t*)a.k_pool + (koff < 0 ? 0 : koff) + hl * 8;
#pragma unroll
    for (int ks = 0; ks < QREGS; ++ks) kc[ks] = koff >= 0 ? *(const uint4*)(kp + ks * 16) : make_uint4(0, 0, 0, 0);
  }
  float* P = a.scores + (((int64_t)b * sq.h_q + h) * a.max_nr) * sq.max_nk;
  for (int j0 = kb0 * per; j0 < jend; j0 += kScoreKeys) {
    const int64_t koff_n = j0 + kScoreKeys < jend ? key_off(j0 + kScoreKeys) : -1;
    {
      const uint16_t* kp = (const uint16_t*)a.k_pool + (koff_n < 0 ? 0 : koff_n) + hl * 8;
#pragma unroll
      for (int ks = 0; ks < QREGS; ++ks)
        kn[ks] = koff_n >= 0 ? *(const uint4*)(kp + ks * 16) : make_uint4(0, 0, 0, 0);
    }
    f32x16 sc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sc[v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < QREGS; ++ks)
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kc[ks]), qf[ks], sc, 0, 0, 0);
    // element v: pooled key j0 + w*32 + 8*(v/4) + 4*hl + v%4 (raw dot; scaled after the max)
    float x[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int j = j0 + w * 32 + 8 * (v >> 2) + 4 * hl + (v & 3);
      x[v] = (j <= jmax && j < Rk) ? sc[v] : kNegInf;
    }
    float g4[4], o4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) g4[q] = fmaxf(fmaxf(x[4 * q], x[4 * q + 1]), fmaxf(x[4 * q + 2], x[4 * q + 3]));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(g4[q]), __float_as_uint(g4[q]), false, false);
      o4[q] = __uint_as_float(hl ? sw[0] : sw[1]);
    }
    if (hl == 0 && col_ok) {
      const int kbase = (j0 + w * 32) / per;
      float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      int nb;
      if (per == 4) {
        nb = 8;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          m[2 * q] = g4[q];
          m[2 * q + 1] = o4[q];
        }
      } else if (per == 8) {
        nb = 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) m[q] = fmaxf(g4[q], o4[q]);
      } else if (per == 16) {
        nb = 2;
        m[0] = fmaxf(fmaxf(g4[0], o4[0]), fmaxf(g4[1], o4[1]));
        m[1] = fmaxf(fmaxf(g4[2], o4[2]), fmaxf(g4[3], o4[3]));
      } else {
        nb = 1;
        m[0] = fmaxf(fmaxf(fmaxf(g4[0], o4[0]), fmaxf(g4[1], o4[1])), fmaxf(fmaxf(g4[2], o4[2]), fmaxf(g4[3], o4[3])));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < nb && kbase + i < kb_end) P[kbase + i] = m[i] * a.scale;
    }
#pragma unroll
    for (int ks = 0; ks < QREGS; ++ks) kc[ks] = kn[ks];
  }
}

// the rank pass's sort size for lists of up to max_nk blocks (a power of two,
// at least one key per thread) and its dynamic LDS: keys, then row maxima
__host__ __device__ inline int rank_sort_size(int max_nk) {
  int n = kThreads;
  while (n < max_nk) n <<= 1;
  return n;
}
// (the row maxima padded to a whole number of the key loop's 16-row chunks)
constexpr int kRankChunk = 16;
inline size_t rank_lds_bytes(const KapArgs& a, int block) {
  const int nr = a.seq.group * (block / a.pool);  // G * (B/p) pooled rows per list
  const int nr_pad = (nr + kRankChunk - 1) / kRankChunk * kRankChunk;
  return (size_t)rank_sort_size(a.seq.max_nk) * sizeof(unsigned long long) + (size_t)nr_pad * sizeof(float);
}

template <int BLK>
__global__ __launch_bounds__(kThreads) void kap_rank_sort(KapArgs a) {
  // keys (the sort network's size) and row maxima in LDS sized at launch
  // (rank_lds_bytes), so short lists leave room for more workgroups per CU
  extern __shared__ unsigned long long rank_dyn[];
  unsigned long long* keys = rank_dyn;
  float* rmax = (float*)(rank_dyn + rank_sort_size(a.seq.max_nk));
  const SeqArgs& sq = a.seq;
  const int G = sq.group;
  const int64_t bid = blockIdx.x;
  const int g = (int)(bid % sq.h_kv);
  int64_t rest = bid / sq.h_kv;
  const int b = (int)(rest % sq.batch);
  const int qb = sq.max_nq - 1 - (int)(rest / sq.batch);
  const int q0 = sq.cu_seqlens_q[b];
  const int Lq = sq.cu_seqlens_q[b + 1] - q0;
  const int Lk = sq.seqlens_k[b];
  const int off = Lk - Lq;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t list_row = ((int64_t)b * sq.h_kv + g) * sq.max_nq + qb;
  int32_t* order = a.order + list_row * a.kmax;
  uint8_t* hrm = a.hrm + list_row * a.kmax;
  float* bs = a.block_scores ? a.block_scores + list_row * sq.max_nk : nullptr;

  if (qb * BLK >= Lq) {  // past this sequence's end: empty list
    for (int t = tid; t < a.kmax; t += kThreads) {
      order[t] = -1;
      hrm[t] = 0;
    }
    if (bs)
      for (int kb = tid; kb < sq.max_nk; kb += kThreads) bs[kb] = 0.f;
    if (tid == 0) a.count[list_row] = 0;
    return;
  }
  const int n = (off + min(qb * BLK + BLK - 1, Lq - 1)) / BLK + 1;
  const int p = a.pool, per = BLK / p;
  const int R = (Lq + p - 1) / p;
  const int r0 = qb * per;
  const int nrow = min(r0 + per, R) - r0;
  const int NR = G * nrow;
  const float* Pb = a.scores + ((int64_t)b * sq.h_q) * a.max_nr * sq.max_nk;

  // row maxima over the row's causal blocks (max is exact in any order):
  // from the score pass when it produced them
  if (a.row_max) {
    for (int ri = tid; ri < NR; ri += kThreads) {
      const int h = g * G + ri / nrow, r = r0 + ri % nrow;
      rmax[ri] = a.row_max[((int64_t)b * sq.h_q + h) * a.max_nr + r];
    }
  } else
  for (int ri = w; ri < NR; ri += kThreads / 64) {
    const int h = g * G + ri / nrow, r = r0 + ri % nrow;
    const float* row = Pb + ((int64_t)h * a.max_nr + r) * sq.max_nk;
    float m = kNegInf;
    int kb = lane;
    for (; kb + 192 < n; kb += 256) {  // four independent loads in flight
      const float x0 = row[kb], x1 = row[kb + 64], x2 = row[kb + 128], x3 = row[kb + 192];
      m = fmaxf(m, fmaxf(fmaxf(x0, x1), fmaxf(x2, x3)));
    }
    for (; kb < n; kb += 64) m = fmaxf(m, row[kb]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (lane == 0) rmax[ri] = m;
  }
  __syncthreads();

  int npad = kThreads;  // the sort network's size: a power of two, at least one key per thread
  while (npad < n) npad <<= 1;
  for (int kb = tid; kb < npad; kb += kThreads) {
    unsigned long long key = 0ull;
    if (kb < n) {
      float s = 0.0f;
      bool flag = false;
      // heads ascending, then rows ascending; the loads of a chunk of rows are
      // issued together, and so are the chunk's row maxima (four 16-byte LDS
      // reads, one wait per chunk instead of one per term); the sum stays
      // sequential
      constexpr int CHUNK = kRankChunk;
      // element offset of row (head g*G + ri / nrow, pooled row r0 + ri % nrow),
      // advanced row by row (no division per term)
      int64_t roff = ((int64_t)g * G * a.max_nr + r0) * sq.max_nk;
      int rr = 0;
      const int64_t next_head = (int64_t)(a.max_nr - nrow + 1) * sq.max_nk;
      for (int r0c = 0; r0c < NR; r0c += CHUNK) {
        float xs[CHUNK], rm[CHUNK];
#pragma unroll
        for (int c = 0; c < CHUNK; ++c) {
          const int ri = r0c + c;
          if (ri < NR) {
            xs[c] = __builtin_nontemporal_load(Pb + roff + kb);  // P is read once: non-temporal
            if (++rr == nrow) {
              rr = 0;
              roff += next_head;
            } else {
              roff += sq.max_nk;
            }
          }
        }
#pragma unroll
        for (int q = 0; q < CHUNK / 4; ++q) {
          const float4 m4 = *(const float4*)(rmax + r0c + 4 * q);  // padded: in bounds
          rm[4 * q] = m4.x;
          rm[4 * q + 1] = m4.y;
          rm[4 * q + 2] = m4.z;
          rm[4 * q + 3] = m4.w;
        }
#pragma unroll
        for (int c = 0; c < CHUNK; ++c) {
          const int ri = r0c + c;
          if (ri < NR) {
            float dlt;
            {
#pragma clang fp contract(off)
              dlt = xs[c] - rm[c];
              s = s + exp32(dlt);
            }
            flag |= (dlt == 0.0f);
          }
        }
      }
      key = rank_key(flag, s, kb);
      if (bs) bs[kb] = s;
    }
    keys[kb] = key;
  }
  if (bs)
    for (int kb = n + tid; kb < sq.max_nk; kb += kThreads) bs[kb] = 0.f;
  __syncthreads();

  // descending sort (padding keys are 0, below every real key)
  sort_keys_desc_any(keys, npad, tid);

  int kcnt = (int)ceil(a.budget * (double)n - 1e-9);
  kcnt = max(1, min(n, kcnt));
  for (int t = tid; t < a.kmax; t += kThreads) {
    if (t < kcnt) {
      const unsigned long long key = keys[t];
      order[t] = (int32_t)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull));
      hrm[t] = (uint8_t)(key >> 63);
    } else {
      order[t] = -1;
      hrm[t] = 0;
    }
  }
  if (tid == 0) a.count[list_row] = kcnt;
}

template <bool BF16, int D, int BLK>
hipError_t launch_all(const KapArgs& a, hipStream_t stream) {
  const SeqArgs& sq = a.seq;
  KapArgs ra = a;  // the score and rank passes' arguments (split score pass: no row maxima)
  ra.score_splits = 1;
  const int64_t g1 = (int64_t)sq.batch * a.max_nr;
  hipLaunchKernelGGL((kap_pool_q<BF16, D>), dim3((unsigned)g1), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!a.keys_pooled) {
    const int64_t g2 = (int64_t)sq.batch * sq.max_nk;
    hipLaunchKernelGGL((kap_pool_k<BF16, D, BLK>), dim3((unsigned)g2), dim3(kThreads), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int per = BLK / a.pool;
  if (BF16 && kap_decode_scores(a.max_nr, sq.group, per, 1)) {  // one pooled row: heads as columns
    const int64_t nchunk = ((int64_t)sq.max_nk * per + kDecodeKeys - 1) / kDecodeKeys;
    const int64_t g3 = nchunk * sq.h_kv * sq.batch;
    if constexpr (BF16)
      hipLaunchKernelGGL((kap_score_decode<D, BLK>), dim3((unsigned)g3), dim3(kThreads), 0, stream, a);
  } else if (BF16 && per >= 4 && per <= 32) {  // group form: pooled K staged once per KV group
    const int64_t ntile = (a.max_nr + 31) / 32;
    const int64_t npb = (sq.group * ntile + 3) / 4;
    const int64_t g3 = npb * sq.batch * sq.h_kv;
    // a grid of fewer than two workgroups per CU splits each pair set's keys
    // (at most 8 ways); the rank pass then takes the row maxima from P
    const int64_t nsplit = std::min<int64_t>(8, std::max<int64_t>(1, (2 * kNumCu + g3 - 1) / g3));
    if (nsplit > 1) {
      ra.row_max = nullptr;
      ra.score_splits = (int32_t)nsplit;
    }
    if constexpr (BF16)
      hipLaunchKernelGGL((kap_score_grp<D, BLK>), dim3((unsigned)(g3 * nsplit)), dim3(kThreads),
                         (size_t)sq.max_nk * sizeof(int32_t), stream, ra);
  } else if (per >= 4 && per <= 32) {  // fp32: block maxima in registers, two row tiles share each K load
    const int64_t ntile = (a.max_nr + 2 * kScoreRows - 1) / (2 * kScoreRows);
    const int64_t g3 = ntile * sq.batch * sq.h_q;
    if constexpr (!BF16)
      hipLaunchKernelGGL((kap_score<BF16, D, BLK, 2>), dim3((unsigned)g3), dim3(kThreads), 0, stream, a);
  } else {
    const int64_t ntile = (a.max_nr + kScoreRows - 1) / kScoreRows;
    const int64_t g3 = ntile * sq.batch * sq.h_q;
    hipLaunchKernelGGL((kap_score<BF16, D, BLK, 1>), dim3((unsigned)g3), dim3(kThreads), 0, stream, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t g4 = (int64_t)sq.max_nq * sq.batch * sq.h_kv;
  hipLaunchKernelGGL((kap_rank_sort<BLK>), dim3((unsigned)g4), dim3(kThreads), rank_lds_bytes(ra, BLK), stream, ra);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kap_pool_q(const KapArgs& a, int dtype, int head_dim, hipStream_t stream) {
  const int64_t g1 = (int64_t)a.seq.batch * a.max_nr;
  if (dtype == 1 && head_dim == 128)
    hipLaunchKernelGGL((kap_pool_q<true, 128>), dim3((unsigned)g1), dim3(kThreads), 0, stream, a);
  else if (dtype == 1 && head_dim == 64)
    hipLaunchKernelGGL((kap_pool_q<true, 64>), dim3((unsigned)g1), dim3(kThreads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_kap_pool_k(const KapArgs& a, int dtype, int head_dim, int block, hipStream_t stream) {
  const int64_t g2 = a.pool_last_only ? (int64_t)a.seq.batch * a.seq.h_kv : (int64_t)a.seq.batch * a.seq.max_nk;
#define COSA_POOLK_CASE(BF, DD, BB)                                                                   \
  if ((dtype == 1) == BF && head_dim == DD && block == BB) {                                           \
    hipLaunchKernelGGL((kap_pool_k<BF, DD, BB>), dim3((unsigned)g2), dim3(kThreads), 0, stream, a); \
    return hipGetLastError();                                                                          \
  }
  COSA_POOLK_CASE(true, 128, 128)
  COSA_POOLK_CASE(true, 128, 64)
  COSA_POOLK_CASE(true, 64, 128)
  COSA_POOLK_CASE(true, 64, 64)
  COSA_POOLK_CASE(false, 128, 128)
  COSA_POOLK_CASE(false, 128, 64)
  COSA_POOLK_CASE(false, 64, 128)
  COSA_POOLK_CASE(false, 64, 64)
#undef COSA_POOLK_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_kap_rank(const KapArgs& a, int block, hipStream_t stream) {
  const int64_t g4 = (int64_t)a.seq.max_nq * a.seq.batch * a.seq.h_kv;
  if (block == 128)
    hipLaunchKernelGGL((kap_rank_sort<128>), dim3((unsigned)g4), dim3(kThreads), rank_lds_bytes(a, 128), stream, a);
  else if (block == 64)
    hipLaunchKernelGGL((kap_rank_sort<64>), dim3((unsigned)g4), dim3(kThreads), rank_lds_bytes(a, 64), stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_kap(const KapArgs& a, int dtype, int head_dim, int block, hipStream_t stream) {
  const bool bf = dtype == 1;
#define COSA_KAP_CASE(BF, DD, BB) \
  if (bf == BF && head_dim == DD && block == BB) return launch_all<BF, DD, BB>(a, stream);
  COSA_KAP_CASE(true, 128, 128)
  COSA_KAP_CASE(true, 128, 64)
  COSA_KAP_CASE(true, 64, 128)
  COSA_KAP_CASE(true, 64, 64)
  COSA_KAP_CASE(false, 128, 128)
  COSA_KAP_CASE(false, 128, 64)
  COSA_KAP_CASE(false, 64, 128)
  COSA_KAP_CASE(false, 64, 64)
#undef COSA_KAP_CASE
  return hipErrorInvalidValue;
}

}  // namespace cosa
