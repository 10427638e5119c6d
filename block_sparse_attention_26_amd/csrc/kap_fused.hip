// Fused Kernel-Aware Proxy pass for gfx950: scores, MaxPool, MaxNorm, HRM
// flags, block scores, flag-grouped sort and budget of one order list in one
// workgroup, with the proxy scores P kept in registers (never in memory
// unless the caller asks for them).
//
// Method: CoSA technical summary (gist.science, "CoSA: Accelerating
// Long-Context Inference via Proxy-Kernel Co-Designed Sparse Attention"),
// §2.2 Stage 1 (block ranking: approximate scores of the downsampled queries
// and keys, MaxPool over the keys of each block, MaxNorm; HRM flag
// generation; flag-grouped sorting under a budget), after the pooling passes
// of kap.hip. The results equal those of the two-pass route (score pass, then
// rank pass) bit for bit: the same MFMA sequence forms P, and from P on every
// operation is the same single IEEE binary32 operation in the same order.
//
// One workgroup per list row (sequence, KV group, query block), longest rows
// first, the KV group fastest so that each XCD's L2 serves one group's pooled
// keys. Its G*p' rows (G query heads x p' = B/p pooled rows, at most 32) are
// the 32 columns of S^T = Kpool . Qpool^T on v_mfma_f32_32x32x16_bf16, so each
// lane owns one row. The four waves take interleaved 32-key steps of the
// row's causal pooled keys, each through its own two-stage LDS ring filled by
// global_load_lds (no barrier in the score phase). Per step the block maxima
// of the lane's row stay in registers (n/8 values per lane for n blocks).
// Then: row maxima across the waves (one barrier), c = exp32(P - rowmax) and
// the HRM test in registers, a transposition through LDS in chunks of 256
// blocks so that one thread per block sums its column in the specified order
// (heads, then rows), and the bitonic sort of the 64-bit keys in LDS.
#include "cosa_internal.h"
#include "kap_common.h"

namespace cosa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

template <int D, int PER, int NB>
struct FusedGeo {
  static constexpr int NW = 4;                          // waves
  static constexpr int STEP = 32;                       // pooled keys per MFMA tile
  static constexpr int BPS = STEP / PER;                // blocks per step: 8, 4 or 2
  static constexpr int BPL = BPS / 2;                   // blocks kept per lane half
  static constexpr int NSW = NB * PER / (STEP * NW);    // steps per wave, at most
  static constexpr int PV = NSW * BPL;                  // P values per lane (NB / 8)
  static constexpr int ROWB = D * 2;                    // bytes per pooled key row
  static constexpr int STAGE = STEP * ROWB;             // bytes per step tile
  static constexpr int NST = 2;                         // per-wave ring
  static constexpr int CPS = STAGE / 1024;              // 1 KB copies per step
  static constexpr int RPC = 1024 / ROWB;               // key rows per copy
  static constexpr int CH = D / 8;                      // 16-byte chunks per row
  static constexpr int QREGS = D / 16;
  static constexpr int CB = 256;                        // blocks per transposition chunk
  static constexpr int CBP = CB + 1;                    // padded chunk row (floats)
  static constexpr int NCH = NB / CB;                   // chunks, at most
  static constexpr int SPC = CB / BPS;                  // steps per chunk (multiple of NW)
  static constexpr int RING_BYTES = NW * NST * STAGE;
  static constexpr int SUM_BYTES = 32 * CBP * 4 + NB * 8;  // chunk + keys
  static constexpr int WORK_BYTES = RING_BYTES > SUM_BYTES ? RING_BYTES : SUM_BYTES;
  static_assert(NB % CB == 0 && SPC % NW == 0, "chunking");
  static_assert(STEP % PER == 0 && BPS % 2 == 0, "two lane halves per step");
};

template <int D, int PER, int NB>
__global__ __launch_bounds__(kThreads, 2) void kap_fused(KapArgs a) {
  using Gm = FusedGeo<D, PER, NB>;
  constexpr int STEP = Gm::STEP, BPS = Gm::BPS, BPL = Gm::BPL, NSW = Gm::NSW, PV = Gm::PV;
  constexpr int ROWB = Gm::ROWB, STAGE = Gm::STAGE, CPS = Gm::CPS, RPC = Gm::RPC, CH = Gm::CH;
  constexpr int QREGS = Gm::QREGS, CB = Gm::CB, CBP = Gm::CBP, NCH = Gm::NCH, SPC = Gm::SPC;
  // LDS: the waves' rings in the score phase, then the transposition chunk
  // and the sort keys (same bytes); the block-table row; the row maxima
  __shared__ __attribute__((aligned(1024))) unsigned char work[Gm::WORK_BYTES];
  __shared__ int32_t ptab[NB];
  __shared__ float red[Gm::NW][32];

  const SeqArgs& sq = a.seq;
  const int G = sq.group;
  const int64_t bid = blockIdx.x;
  const int g = (int)(bid % sq.h_kv);
  const int64_t rest = bid / sq.h_kv;
  const int b = (int)(rest % sq.batch);
  const int qb = sq.max_nq - 1 - (int)(rest / sq.batch);
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q0 = __builtin_amdgcn_readfirstlane(sq.cu_seqlens_q[b]);
  const int Lq = __builtin_amdgcn_readfirstlane(sq.cu_seqlens_q[b + 1]) - q0;
  const int Lk = __builtin_amdgcn_readfirstlane(sq.seqlens_k[b]);
  const int p = a.pool;
  const int BLK = PER * p;
  const int off = Lk - Lq;
  const int R = (Lq + p - 1) / p;
  const int Rk = (Lk + p - 1) / p;
  const int r0 = qb * PER;
  const int64_t list_row = ((int64_t)b * sq.h_kv + g) * sq.max_nq + qb;
  int32_t* order = a.order + list_row * a.kmax;
  uint8_t* hrm = a.hrm + list_row * a.kmax;
  float* bs = a.block_scores ? a.block_scores + list_row * sq.max_nk : nullptr;
  const bool export_p = a.fill_scores != 0;
  // this lane's row: query head g*G + ri / PER, pooled row r0 + ri % PER
  const int ri = l32;
  const int hloc = ri / PER;
  const int my_r = r0 + ri % PER;
  const bool head_ok = hloc < G;
  const bool row_ok = head_ok && my_r < R;
  const int h = g * G + (head_ok ? hloc : 0);
  // P rows of this lane that exist in the exported tensor
  const bool p_row = export_p && head_ok && my_r < a.max_nr;
  float* prow = p_row ? a.scores + (((int64_t)b * sq.h_q + h) * a.max_nr + my_r) * sq.max_nk : nullptr;

  if (qb * BLK >= Lq) {  // past this sequence's end: an empty list
    for (int t = tid; t < a.kmax; t += kThreads) {
      order[t] = -1;
      hrm[t] = 0;
    }
    if (bs)
      for (int kb = tid; kb < sq.max_nk; kb += kThreads) bs[kb] = 0.f;
    if (tid == 0) a.count[list_row] = 0;
    if (prow)
      for (int kb = w * 2 + hl; kb < sq.max_nk; kb += 2 * Gm::NW) prow[kb] = kNegInf;
    return;
  }
  const int n = (off + min(qb * BLK + BLK - 1, Lq - 1)) / BLK + 1;  // causal blocks (<= NB)
  const int jend = n * PER;                                           // pooled keys covered
  const int nsteps = (jend + STEP - 1) / STEP;
  const int nmine = nsteps > w ? (nsteps - 1 - w) / Gm::NW + 1 : 0;   // this wave's steps
  const int my_jmax = row_ok ? (off + min(my_r * p + p - 1, Lq - 1)) / p : -1;
  const int jmin = (off + min(r0 * p + p - 1, Lq - 1)) / p;           // the first row's limit

  for (int i = tid; i < n; i += kThreads) ptab[i] = sq.block_table[(int64_t)b * sq.max_blocks_k + i];

  // query fragments (B operand): row ri, columns ks*16 + hl*8 .. +8
  bf16x8 qf[QREGS];
  {
    const size_t qoff = (((size_t)b * a.max_nr + (row_ok ? my_r : 0)) * sq.h_q + h) * D;
    const uint16_t* qp = (const uint16_t*)a.q_pool + qoff + hl * 8;
#pragma unroll
    for (int ks = 0; ks < QREGS; ++ks) {
      const uint4 x = row_ok ? *(const uint4*)(qp + ks * 16) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }
  __syncthreads();  // ptab staged

  // copy c of a step fills ring bytes [c * 1024, +1024): key row
  // cr = c*RPC + lane/CH of the step (block cr / PER of the step, slot
  // cr % PER of its page), physical chunk lane%CH holding logical chunk
  // (lane%CH) ^ (cr % CH). A row past the covered blocks reads the last
  // covered block (its scores are masked).
  const unsigned char* kpool = (const unsigned char*)a.k_pool + (size_t)g * PER * ROWB;
  const size_t page_bytes = (size_t)sq.h_kv * PER * ROWB;
  unsigned char* ring = work + w * Gm::NST * STAGE;
  uint32_t c_off[CPS];
  int c_blk[CPS];
#pragma unroll
  for (int c = 0; c < CPS; ++c) {
    const int cr = c * RPC + lane / CH;
    c_off[c] = (uint32_t)((cr % PER) * ROWB + (((lane % CH) ^ (cr % CH)) << 4));
    c_blk[c] = cr / PER;
  }
  auto issue = [&](int st, int stage) {
#pragma unroll
    for (int c = 0; c < CPS; ++c) {
      const int kbq = min(st * BPS + c_blk[c], n - 1);
      const unsigned page = min((unsigned)ptab[kbq], (unsigned)sq.num_pages - 1u);  // a corrupt entry stays in the pool
      const unsigned char* src = kpool + (size_t)page * page_bytes + c_off[c];
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(ring + stage * STAGE + c * 1024), 16, 0, 0);
    }
  };

  // ---- scores and block maxima (raw q.k; the scale is applied after the max,
  // which rounding keeps exact since it is monotone) ------------------------
  float pv[PV];
  float rmx = kNegInf;
  const int k_swz = l32 % CH;
  if (nmine > 0) issue(w, 0);
#pragma unroll
  for (int i = 0; i < NSW; ++i) {
    if (i < nmine) {
      const int st = w + Gm::NW * i;
      __builtin_amdgcn_s_waitcnt(0);  // this step's copies (the only ones in flight) landed
      asm volatile("" ::: "memory");
      if (i + 1 < nmine) issue(st + Gm::NW, (i + 1) & 1);  // into the stage the previous step read
      const unsigned char* kl = ring + (i & 1) * STAGE + l32 * ROWB;
      f32x16 sc;
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[v] = 0.f;
      bf16x8 kf[2];
      kf[0] = *(const bf16x8*)(kl + ((hl ^ k_swz) << 4));
#pragma unroll
      for (int ks = 0; ks < QREGS; ++ks) {
        if (ks + 1 < QREGS) kf[(ks + 1) & 1] = *(const bf16x8*)(kl + (((2 * (ks + 1) + hl) ^ k_swz) << 4));
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks & 1], qf[ks], sc, 0, 0, 0);
      }
      // element v: pooled key st*32 + 8*(v/4) + 4*hl + v%4
      const int j0 = st * STEP;
      if (j0 + STEP - 1 > jmin || j0 + STEP > Rk) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = j0 + 8 * (v >> 2) + 4 * hl + (v & 3);
          if (!(j <= my_jmax && j < Rk)) sc[v] = kNegInf;
        }
      }
      float g4[4], lo[4], hi[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) g4[q] = vmax(vmax(sc[4 * q], sc[4 * q + 1]), vmax(sc[4 * q + 2], sc[4 * q + 3]));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(g4[q]), __float_as_uint(g4[q]), false, false);
        const float o = __uint_as_float(hl ? sw[0] : sw[1]);
        lo[q] = hl ? o : g4[q];  // keys 8q .. 8q+3 of the step
        hi[q] = hl ? g4[q] : o;  // keys 8q+4 .. 8q+7
      }
      float bm[BPS];
      if constexpr (PER == 4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bm[2 * q] = lo[q];
          bm[2 * q + 1] = hi[q];
        }
      } else if constexpr (PER == 8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) bm[q] = vmax(lo[q], hi[q]);
      } else {
        bm[0] = vmax(vmax(lo[0], hi[0]), vmax(lo[1], hi[1]));
        bm[1] = vmax(vmax(lo[2], hi[2]), vmax(lo[3], hi[3]));
      }
#pragma unroll
      for (int u = 0; u < BPS; ++u) rmx = vmax(rmx, bm[u]);
      // this half keeps blocks hl*BPL .. hl*BPL + BPL - 1 of the step
#pragma unroll
      for (int u = 0; u < BPL; ++u) pv[i * BPL + u] = hl ? bm[BPL + u] : bm[u];
    }
  }

  // ---- row maxima across the waves ----------------------------------------
  __syncthreads();  // every wave is done with its ring: `work` is free
  if (hl == 0) red[w][l32] = rmx;
  __syncthreads();
  float m_raw = red[0][l32];
#pragma unroll
  for (int i = 1; i < Gm::NW; ++i) m_raw = vmax(m_raw, red[i][l32]);
  float m;
  {
#pragma clang fp contract(off)
    m = m_raw * a.scale;
  }
  // P for the caller (parity checks): the lane's blocks, -inf past the causal
  // ones and in rows past the sequence end (whose scores are masked only in
  // edge steps: the score phase needs no row that does not exist)
  if (prow) {
#pragma unroll
    for (int i = 0; i < NSW; ++i)
      if (i < nmine) {
        const int kb0 = (w + Gm::NW * i) * BPS + hl * BPL;
#pragma unroll
        for (int u = 0; u < BPL; ++u)
          if (kb0 + u < n) prow[kb0 + u] = row_ok ? pv[i * BPL + u] * a.scale : kNegInf;
      }
    for (int kb = n + w * 2 + hl; kb < sq.max_nk; kb += 2 * Gm::NW) prow[kb] = kNegInf;
  }

  // ---- MaxNorm and HRM in registers: c = exp32(P - m), stored negated when
  // P attains the row maximum (c is then exactly 1; otherwise c >= +0) ------
  if (row_ok) {
#pragma unroll
    for (int i = 0; i < NSW; ++i)
      if (i < nmine) {
#pragma unroll
        for (int u = 0; u < BPL; ++u) {
#pragma clang fp contract(off)
          const float P = pv[i * BPL + u] * a.scale;
          const float dlt = P - m;
          const float c = exp32(dlt);
          pv[i * BPL + u] = dlt == 0.0f ? -c : c;
        }
      }
  }

  // ---- block scores: per chunk of 256 blocks, the waves' values go through
  // LDS and thread t sums block t's column over the rows in order ----------
  float* cb = (float*)work;
  unsigned long long* keys = (unsigned long long*)(work + 32 * CBP * 4);
  uint32_t rows_valid = 0;  // bit ri: row ri exists (the same in every lane)
  for (int x = 0; x < 32; ++x)
    if (x / PER < G && r0 + x % PER < R) rows_valid |= 1u << x;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    if (ch * CB < n) {
#pragma unroll
      for (int ii = 0; ii < SPC / Gm::NW; ++ii) {
        const int i = ch * (SPC / Gm::NW) + ii;
        if (i < nmine) {
          const int kl0 = (w + Gm::NW * i) * BPS + hl * BPL - ch * CB;
#pragma unroll
          for (int u = 0; u < BPL; ++u) cb[ri * CBP + kl0 + u] = pv[i * BPL + u];
        }
      }
      __syncthreads();
      const int kb = ch * CB + tid;
      if (kb < n) {
        float s = 0.0f;
        bool flag = false;
        for (int x = 0; x < 32; ++x) {
          if ((rows_valid >> x) & 1u) {
            const float v = cb[x * CBP + tid];
            {
#pragma clang fp contract(off)
              s = s + __builtin_fabsf(v);
            }
            flag |= v < 0.0f;
          }
        }
        keys[kb] = rank_key(flag, s, kb);
        if (bs) bs[kb] = s;
      }
      __syncthreads();  // the chunk is read before the next one overwrites it
    }
  }
  int npad = kThreads;  // the sort network's size: a power of two, at least one key per thread
  while (npad < n) npad <<= 1;
  for (int kb = n + tid; kb < npad; kb += kThreads) keys[kb] = 0ull;  // below every real key
  if (bs)
    for (int kb = n + tid; kb < sq.max_nk; kb += kThreads) bs[kb] = 0.f;
  __syncthreads();
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

template <int D, int PER>
hipError_t launch_per(const KapArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.seq.max_nq * a.seq.batch * a.seq.h_kv;
  if (a.seq.max_nk <= 256)
    hipLaunchKernelGGL((kap_fused<D, PER, 256>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((kap_fused<D, PER, 1024>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

bool kap_fused_eligible(const KapArgs& a, int dtype, int block) {
  return kap_fused_shape(dtype, block / a.pool, a.seq.group, a.seq.max_nk, a.max_nr);
}

hipError_t launch_kap_fused(const KapArgs& a, int head_dim, int block, hipStream_t stream) {
  const int per = block / a.pool;
#define COSA_FUSED_CASE(DD, PP) \
  if (head_dim == DD && per == PP) return launch_per<DD, PP>(a, stream);
  COSA_FUSED_CASE(128, 8)
  COSA_FUSED_CASE(128, 4)
  COSA_FUSED_CASE(128, 16)
  COSA_FUSED_CASE(64, 8)
  COSA_FUSED_CASE(64, 4)
  COSA_FUSED_CASE(64, 16)
#undef COSA_FUSED_CASE
  return hipErrorInvalidValue;
}

}  // namespace cosa
