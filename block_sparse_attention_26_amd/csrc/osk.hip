// Ordered-Skipping Kernel (OSK) and the dense causal baseline for gfx950:
// the generic register-staged kernel, used for fp32 inputs (the bf16 path is
// osk_bf16.hip).
//
// Method: CoSA technical summary (gist.science, "CoSA: Accelerating
// Long-Context Inference via Proxy-Kernel Co-Designed Sparse Attention"):
//  §2.3 Stage 2 - blocks missing from the proxy's list are never touched (the
//       walk follows the list and gathers pages through the block table);
//       listed blocks may be skipped in-kernel from the local vs running row
//       maxima; the rest gets the full online-softmax update and P.V.
//  §2.1 - the online-softmax accumulation is independent of the visit order,
//       so the list order only changes which blocks can be skipped.
//  §1   - the skip decision is taken for the whole tile: one row whose local
//       max is close to its running max keeps the block (the "bucket
//       effect"), so the kernel reduces the per-row margins over all rows of
//       the query block before deciding.
//
// Work decomposition (one workgroup per (sequence b, query head h, query
// block qb)): B/32 waves, each owning 32 query rows. Scores are computed
// transposed, S^T = K . Q^T, with v_mfma_f32_32x32x16_bf16 (fp32 inputs use
// v_mfma_f32_32x32x2_f32), so every lane holds one query row and 16 keys per
// 32-key tile; the row max needs one cross-half exchange and the softmax
// scalars (running max, sum, rescale factor) are per-lane registers. The
// output is accumulated transposed as well, O^T += V^T . P^T, which lets the
// bf16 P registers feed the MFMA B operand directly (the contraction order of
// keys inside a 16-key step is permuted identically in V^T and P^T).
// K tiles are staged in LDS row-major; V tiles are transposed in registers
// (8x8 bf16 blocks, v_perm_b32) while being staged, so the V^T operand is two
// 8-byte LDS reads per lane. LDS pitches are padded so that these reads are
// bank-conflict free.
//
// Launch order: query blocks from the last (longest list) to the first, and
// the G query heads of a KV group on the same XCD, back to back, so their
// identical K/V page gathers hit that XCD's L2.
#include <math.h>

#include "cosa_internal.h"

namespace cosa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kNegInf = -__builtin_huge_valf();

template <bool BF16, int D, int BLK>
struct Cfg {
  static constexpr int NW = BLK / 32;  // waves; 32 query rows each
  static constexpr int THREADS = 64 * NW;
  static constexpr int KT = BLK / 32;  // 32-key tiles per KV block
  static constexpr int DT = D / 32;    // 32-wide head-dim tiles of O
  // bf16: K [BLK][D] pitch 2D+16 bytes, V^T [D][BLK] pitch 2*BLK+8 bytes.
  // fp32: K and V [BLK][D] pitch 4D+4 bytes.
  static constexpr int K_PITCH = BF16 ? (D * 2 + 16) : (D * 4 + 4);
  static constexpr int V_PITCH = BF16 ? (BLK * 2 + 8) : (D * 4 + 4);
  static constexpr int K_BYTES = BLK * K_PITCH;
  static constexpr int V_BYTES = BF16 ? D * V_PITCH : BLK * V_PITCH;
  static constexpr int QREGS = BF16 ? D / 16 : D / 2;
};

__device__ __forceinline__ float wave_max32(float x) {
  // max over lanes 0..31 (and, identically, 32..63)
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 8));
  x = fmaxf(x, __shfl_xor(x, 4));
  x = fmaxf(x, __shfl_xor(x, 2));
  x = fmaxf(x, __shfl_xor(x, 1));
  return x;
}

// Pack two 16-bit halves: lo from a, hi from b; `hi_half` selects the upper
// halves of both sources instead of the lower ones.
__device__ __forceinline__ uint32_t pack_halves(uint32_t a, uint32_t b, bool hi_half) {
  return __builtin_amdgcn_perm(b, a, hi_half ? 0x07060302u : 0x05040100u);
}

// Per-thread register staging of one K or V tile (global -> registers -> LDS).
// bf16: K as 16-byte row chunks; V as one 8-key x 8-column block per thread,
// transposed in registers on the way into the V^T tile. fp32: both row-major.
template <bool BF16, int D, int BLK>
struct Stage {
  using C = Cfg<BF16, D, BLK>;
  static constexpr int THREADS = C::THREADS;
  static constexpr int CH = BF16 ? D / 8 : D / 4;           // 16-byte chunks per key row
  static constexpr int KPT = BLK * CH / THREADS;            // chunks per thread (K, and fp32 V)
  static constexpr int VBLK = BF16 ? (BLK / 8) * (D / 8) : 0;  // bf16 V: 8x8 blocks
  static constexpr int REGS = BF16 ? (KPT > 8 ? KPT : 8) : KPT;
  uint4 r[REGS];

  __device__ __forceinline__ void load_k(const void* base, int nvalid, int tid) {
    const uint4* g = (const uint4*)base;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = i * THREADS + tid;
      r[i] = (c / CH) < nvalid ? g[c] : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store_k(unsigned char* k_lds, int tid) const {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = i * THREADS + tid;
      if constexpr (BF16) {
        *(uint4*)(k_lds + (c / CH) * C::K_PITCH + (c % CH) * 16) = r[i];
      } else {
        uint32_t* dst = (uint32_t*)(k_lds + (c / CH) * C::K_PITCH) + (c % CH) * 4;
        dst[0] = r[i].x; dst[1] = r[i].y; dst[2] = r[i].z; dst[3] = r[i].w;
      }
    }
  }
  __device__ __forceinline__ void load_v(const void* base, int nvalid, int tid) {
    if constexpr (BF16) {
      const uint4* g = (const uint4*)base;
      const int dch = tid % (D / 8), kg = tid / (D / 8);
      if (tid < VBLK) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int key = kg * 8 + i;
          r[i] = key < nvalid ? g[key * (D / 8) + dch] : make_uint4(0, 0, 0, 0);
        }
      }
    } else {
      load_k(base, nvalid, tid);
    }
  }
  __device__ __forceinline__ void store_v(unsigned char* v_lds, int tid) const {
    if constexpr (BF16) {
      const int dch = tid % (D / 8), kg = tid / (D / 8);
      if (tid < VBLK) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // row d = dch*8 + j of V^T: keys kg*8 .. kg*8+7
          uint32_t o4[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t lo = (&r[2 * p].x)[j / 2], hi = (&r[2 * p + 1].x)[j / 2];
            o4[p] = pack_halves(lo, hi, j & 1);
          }
          unsigned char* dst = v_lds + (dch * 8 + j) * C::V_PITCH + kg * 16;
          *(uint2*)dst = make_uint2(o4[0], o4[1]);
          *(uint2*)(dst + 8) = make_uint2(o4[2], o4[3]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int c = i * THREADS + tid;
        uint32_t* dst = (uint32_t*)(v_lds + (c / CH) * C::V_PITCH) + (c % CH) * 4;
        dst[0] = r[i].x; dst[1] = r[i].y; dst[2] = r[i].z; dst[3] = r[i].w;
      }
    }
  }
};

// The ordered walk. Per listed block t (K and V tiles single-buffered in LDS,
// one staging buffer in registers cycled through three phases):
//   barrier A  - every wave is done with PV(t-1): write V(t) from registers;
//                start loading K(t+1) into the registers
//   S(t) = K(t) Q^T, causal mask, row maxima, per-wave skip margin
//   barrier C  - every wave is done reading K(t): write K(t+1) to LDS, start
//                loading V(t+1); all margins visible -> skip decision
//   unless skipped: online-softmax update and O^T += V(t)^T P^T
// Two workgroups share a CU, so one's MFMA work overlaps the other's loads and
// softmax.
template <bool BF16, int D, int BLK, bool DENSE>
__global__ __launch_bounds__(2 * BLK, 1) void osk_kernel(OskArgs a) {  // 2*BLK == Cfg::THREADS
  using C = Cfg<BF16, D, BLK>;
  using S = Stage<BF16, D, BLK>;
  __shared__ __attribute__((aligned(16))) unsigned char k_lds[C::K_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds[C::V_BYTES];
  __shared__ float red[C::NW];

  const SeqArgs& sq = a.seq;
  const int G = sq.group;
  // ---- unit decode: XCD-grouped, longest query block first --------------
  // KV groups are walked in phases of kPhaseGroups; inside a phase the group
  // index runs fastest, so every XCD shares in each group of the phase and
  // only that phase's pages are live in the last-level cache.
  const int64_t bid = blockIdx.x;
  const int64_t xcd = bid % kNumXcd, slot = bid / kNumXcd;
  const int64_t lam = ((slot / G) * kNumXcd + xcd) * G + slot % G;
  if (lam >= a.n_units) return;
  const int hig = (int)(lam % G);
  const int64_t rest = lam / G;
  const int64_t per_group = (int64_t)sq.batch * sq.max_nq;
  const int phase = (int)(rest / ((int64_t)kPhaseGroups * per_group));
  const int in_phase = min(kPhaseGroups, sq.h_kv - phase * kPhaseGroups);
  const int64_t within = rest - (int64_t)phase * kPhaseGroups * per_group;
  const int g = phase * kPhaseGroups + (int)(within % in_phase);
  const int64_t w2 = within / in_phase;
  const int b = (int)(w2 % sq.batch);
  const int qb = sq.max_nq - 1 - (int)(w2 / sq.batch);
  const int h = g * G + hig;
  const int q0 = sq.cu_seqlens_q[b];
  const int Lq = sq.cu_seqlens_q[b + 1] - q0;
  const int Lk = sq.seqlens_k[b];
  const int tid = threadIdx.x;
  if (qb * BLK >= Lq) {  // past this sequence's end: an empty row
    if constexpr (!DENSE) {
      const int64_t out_row = ((int64_t)b * sq.h_q + h) * sq.max_nq + qb;
      if (tid == 0) {
        a.visited[out_row] = 0;
        a.skipped[out_row] = 0;
      }
      if (a.skip_bits)
        for (int t = tid; t < a.kmax; t += C::THREADS) a.skip_bits[out_row * a.kmax + t] = 255;
    }
    return;
  }
  const int off = Lk - Lq;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hl = lane >> 5;  // which half of the wave
  const int row = w * 32 + l32;
  const bool row_valid = qb * BLK + row < Lq;
  const int my_pos = off + qb * BLK + row;
  const int n_causal = (off + min(qb * BLK + BLK - 1, Lq - 1)) / BLK + 1;

  // ---- query fragments (B operand of S^T = K Q^T) -------------------------
  bf16x8 qf16[BF16 ? C::QREGS : 1];
  float qf32[BF16 ? 1 : C::QREGS];
  {
    // rows past the sequence end load nothing; their address is the block's first row
    const int64_t qoff = (int64_t)(q0 + qb * BLK + (row_valid ? row : 0)) * sq.q_tok + (int64_t)h * sq.q_head;
    if constexpr (BF16) {
      const uint16_t* qp = (const uint16_t*)a.q + qoff + hl * 8;
#pragma unroll
      for (int ks = 0; ks < C::QREGS; ++ks) {
        uint4 x = row_valid ? *(const uint4*)(qp + ks * 16) : make_uint4(0, 0, 0, 0);
        qf16[ks] = __builtin_bit_cast(bf16x8, x);
      }
    } else {
      const float* qp = (const float*)a.q + qoff + hl;
#pragma unroll
      for (int ks = 0; ks < C::QREGS; ++ks) qf32[ks] = row_valid ? qp[ks * 2] : 0.f;
    }
  }

  int n_list;
  const int32_t* lst = nullptr;
  if constexpr (DENSE) {
    n_list = n_causal;
  } else {
    const int64_t list_row = ((int64_t)b * sq.h_kv + g) * sq.max_nq + qb;
    n_list = max(0, min(a.count[list_row], a.kmax));  // a corrupt count can neither overrun nor underrun the row
    lst = a.order + list_row * a.kmax;
  }
  const int64_t out_row = ((int64_t)b * sq.h_q + h) * sq.max_nq + qb;
  bool bad = false;
  const int32_t* table = sq.block_table + (int64_t)b * sq.max_blocks_k;
  const size_t tile_elems = (size_t)BLK * D;
  const size_t head_off = (size_t)g * tile_elems;
  const size_t page_elems = (size_t)sq.h_kv * tile_elems;
  // list entry t -> (first key, element offset of its page slab for this KV head)
  auto locate = [&](int t, int& key0, size_t& elem) {
    int kb = DENSE ? t : lst[t];
    if (kb < 0 || kb >= n_causal) {
      bad = true;
      kb = 0;
    }
    int page = table[kb];
    if ((unsigned)page >= (unsigned)sq.num_pages) {
      bad = true;
      page = 0;
    }
    key0 = kb * BLK;
    elem = (size_t)page * page_elems + head_off;
  };
  const unsigned char* kbase = (const unsigned char*)a.k;
  const unsigned char* vbase = (const unsigned char*)a.v;
  constexpr int ES = BF16 ? 2 : 4;

  f32x16 acc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[dt][v] = 0.f;
  float m_run = kNegInf;  // running max of raw q.k (unscaled)
  float l_run = 0.f;      // this lane's share of the running sum
  int n_skip = 0;
  const float c2 = a.scale_log2;

  // ---- prologue: K(0) into LDS, V(0) into the staging registers -----------
  S stg;
  int key0 = 0;
  size_t elem = 0;
  if (n_list > 0) {  // an empty list touches no entry
    locate(0, key0, elem);
    stg.load_k(kbase + elem * ES, min(BLK, Lk - key0), tid);
    stg.store_k(k_lds, tid);
    stg.load_v(vbase + elem * ES, min(BLK, Lk - key0), tid);
  }

  for (int t = 0; t < n_list; ++t) {
    int nkey0 = 0;
    size_t nelem = 0;
    const bool more = t + 1 < n_list;
    if (more) locate(t + 1, nkey0, nelem);

    __syncthreads();  // A: PV(t-1) done everywhere; K(t) visible
    stg.store_v(v_lds, tid);
    if (more) stg.load_k(kbase + nelem * ES, min(BLK, Lk - nkey0), tid);

    // ---- S^T = K Q^T for this wave's 32 rows ------------------------------
    // k-step outer, key tile inner: KT independent accumulators per k-step.
    f32x16 s[C::KT];
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kt][v] = 0.f;
    if constexpr (BF16) {
      const unsigned char* kp = k_lds + l32 * C::K_PITCH + hl * 16;
#pragma unroll
      for (int ks = 0; ks < C::QREGS; ++ks) {
#pragma unroll
        for (int kt = 0; kt < C::KT; ++kt) {
          const bf16x8 kf = *(const bf16x8*)(kp + kt * 32 * C::K_PITCH + ks * 32);
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf16[ks], s[kt], 0, 0, 0);
        }
      }
    } else {
      const float* kp = (const float*)(k_lds + l32 * C::K_PITCH) + hl;
#pragma unroll
      for (int ks = 0; ks < C::QREGS; ++ks)
#pragma unroll
        for (int kt = 0; kt < C::KT; ++kt)
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x2f32(kp[kt * 32 * (C::K_PITCH / 4) + 2 * ks], qf32[ks],
                                                       s[kt], 0, 0, 0);
    }
    // causal mask: element (kt, v) is key kt*32 + 8*(v/4) + 4*hl + v%4
    if (key0 + BLK - 1 > off + qb * BLK) {
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = key0 + kt * 32 + 8 * (v >> 2) + 4 * hl + (v & 3);
          if (key > my_pos) s[kt][v] = kNegInf;
        }
    }
    float m_loc = kNegInf;
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) m_loc = fmaxf(m_loc, s[kt][v]);
    m_loc = fmaxf(m_loc, __shfl_xor(m_loc, 32));

    // ---- per-tile skip margin: max over the wave's valid rows --------------
    if constexpr (!DENSE) {
      if (a.skip_on) {
        float diff = (row_valid && m_loc != kNegInf) ? m_loc - m_run : kNegInf;
        diff = wave_max32(diff);
        if (lane == 0) red[w] = diff;
      }
    }
    __syncthreads();  // C: K(t) reads done everywhere; V(t) and margins visible
    if (more) {
      stg.store_k(k_lds, tid);
      stg.load_v(vbase + nelem * ES, min(BLK, Lk - nkey0), tid);
    }
    key0 = nkey0;  // for the next iteration's mask (set before a possible skip)
    bool skip = false;
    if constexpr (!DENSE) {
      if (a.skip_on) {
        float worst = red[0];
#pragma unroll
        for (int i = 1; i < C::NW; ++i) worst = fmaxf(worst, red[i]);
        skip = worst < a.skip_thr_raw;
      }
    }
    n_skip += skip ? 1 : 0;
    if (!skip) {
    // ---- online-softmax update ---------------------------------------------
    const float m_new = fmaxf(m_run, m_loc);
    const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * c2);
    const float mc = (m_new == kNegInf) ? 0.f : m_new * c2;
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][v], c2, -mc));
        s[kt][v] = p;
        rs += p;
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
    if (__any(alpha != 1.f)) {  // rescale only when some row's max moved
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[dt][v] *= alpha;
    }

    // ---- O^T += V^T P^T ----------------------------------------------------
    if constexpr (BF16) {
      bf16x8 pb[C::KT][2];
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int i = 0; i < 8; ++i) pb[kt][s2][i] = (__bf16)s[kt][8 * s2 + i];
      // k-step outer (16 keys), head-dim tile inner: DT independent accumulators
      const unsigned char* vp = v_lds + l32 * C::V_PITCH + hl * 8;
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt) {
            const unsigned char* vr = vp + dt * 32 * C::V_PITCH + (kt * 32 + 16 * s2) * 2;
            const uint2 lo = *(const uint2*)vr;
            const uint2 hi = *(const uint2*)(vr + 16);
            const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[kt][s2], acc[dt], 0, 0, 0);
          }
    } else {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = kt * 32 + 8 * (v >> 2) + 4 * hl + (v & 3);
            const float vf = *((const float*)(v_lds + key * C::V_PITCH) + dt * 32 + l32);
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf, s[kt][v], acc[dt], 0, 0, 0);
          }
    }
    }  // !skip
    if constexpr (!DENSE) {
      if (tid == 0 && a.skip_bits) a.skip_bits[out_row * a.kmax + t] = skip ? 1 : 0;
    }
  }

  // ---- epilogue -------------------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (bad) inv = __builtin_nanf("");
  if (row_valid) {
    const int64_t ooff = (int64_t)(q0 + qb * BLK + row) * sq.o_tok + (int64_t)h * sq.o_head;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = dt * 32 + 8 * g4 + 4 * hl;
        const float o0 = acc[dt][4 * g4 + 0] * inv, o1 = acc[dt][4 * g4 + 1] * inv;
        const float o2 = acc[dt][4 * g4 + 2] * inv, o3 = acc[dt][4 * g4 + 3] * inv;
        if constexpr (BF16) {
          const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o0) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o1) << 16);
          const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o2) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o3) << 16);
          *(uint2*)((uint16_t*)a.o + ooff + d0) = make_uint2(lo, hi);
        } else {
          *(float4*)((float*)a.o + ooff + d0) = make_float4(o0, o1, o2, o3);
        }
      }
    if (a.lse && hl == 0) {
      a.lse[(size_t)h * a.total_q + q0 + qb * BLK + row] =
          bad ? __builtin_nanf("") : (l_tot > 0.f ? m_run * a.scale + logf(l_tot) : kNegInf);
    }
  }
  if constexpr (!DENSE) {
    if (tid == 0) {
      a.visited[out_row] = n_list;
      a.skipped[out_row] = n_skip;
    }
    if (a.skip_bits)
      for (int t = n_list + tid; t < a.kmax; t += C::THREADS) a.skip_bits[out_row * a.kmax + t] = 255;
  }
}

template <bool BF16, int D, int BLK>
hipError_t launch_one(const OskArgs& a, bool dense, hipStream_t stream) {
  using C = Cfg<BF16, D, BLK>;
  const int64_t per = (int64_t)kNumXcd * a.seq.group;
  const int64_t grid = (a.n_units + per - 1) / per * per;
  if (dense)
    hipLaunchKernelGGL((osk_kernel<BF16, D, BLK, true>), dim3((unsigned)grid), dim3(C::THREADS), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((osk_kernel<BF16, D, BLK, false>), dim3((unsigned)grid), dim3(C::THREADS), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_osk(const OskArgs& a, int dtype, int head_dim, int block, bool dense,
                      hipStream_t stream) {
  if (dtype == 1) return launch_osk_bf16(a, head_dim, block, dense, stream);
#define COSA_OSK_CASE(DD, BB) \
  if (head_dim == DD && block == BB) return launch_one<false, DD, BB>(a, dense, stream);
  COSA_OSK_CASE(128, 128)
  COSA_OSK_CASE(128, 64)
  COSA_OSK_CASE(64, 128)
  COSA_OSK_CASE(64, 64)
#undef COSA_OSK_CASE
  return hipErrorInvalidValue;
}

}  // namespace cosa
