// Ordered-Skipping Kernel, two-tile form: head_dim 128, block 128, bf16, gfx950.
//
// Method: CoSA technical summary (gist.science, "CoSA: Accelerating
// Long-Context Inference via Proxy-Kernel Co-Designed Sparse Attention"),
// §2.3 (walk only the listed pages, in order; skip a retained block in-kernel
// from the local vs running row maxima; otherwise compute it), §2.1 (the
// online-softmax result does not depend on the visit order) and §1 (the skip
// veto is per tile: every row of the query block must agree). Same results as
// the one-tile kernel in osk_bf16.hip; only the work split differs.
//
// One workgroup of four waves per (sequence, KV group, query block, pair of
// query heads of the group): wave w holds the 64 query rows 64*(w%2) .. +63 of
// head 2*pair + w/2 as two 32-row tiles A and B. Both heads of the pair walk
// the group's one list, so each listed K and V page is copied into LDS once
// for two heads. Tile B runs half a block behind tile A; iteration t is
//   1. S_A(t) = K(t) Q_A^T         (MFMA)  beside B's weights for block t-1
//   2. O_B^T += V(t-1)^T P_B^T     (MFMA)  beside A's row maxima and the
//                                          first half of A's weights
//   3. S_B(t) = K(t) Q_B^T         (MFMA)  beside the rest of A's weights
//   4. B's row maxima, the per-head skip vote, barrier X(t), then
//      O_A^T += V(t)^T P_A^T       (MFMA)  beside the copies of K(t+2), V(t+1)
// so the weights a wave forms never feed the MFMAs they run beside: the
// matrix pipe and the VALU work on independent instruction streams of one
// wave (one wave per SIMD). Weights are formed before the vote and dropped
// when the head skips the block.
//
// Registers: the outputs O_A, O_B (MFMA accumulators) and the query fragments
// (MFMA operands only) live in AGPRs, scores and weights in VGPRs. The MFMAs
// are written as inline assembly to get that split, so the waits the
// compiler would insert around them are explicit here: after a score pass
// before VALU reads the scores, before the first MFMA that reads a new weight
// tile, and around the (rare) rescale of O and the epilogue's reads of O.
//
// LDS: K and V tiles double-buffered (2 x 2 x 32 KB, one workgroup per CU).
// After barrier X(t) every wave issues its share of the copies of K(t+2)
// (into the buffer K(t) leaves) and V(t+1) (into the buffer V(t-1) left);
// barrier X(t+1) waits for them. List entries and their pages are held in two
// 64-entry register windows (one entry per lane) read with readlane.
#include <math.h>

#include "cosa_internal.h"

namespace cosa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kNegInf = -__builtin_huge_valf();

// maxima as llvm.maximum (v_maximum3_f32), no operand quieting (a NaN score
// only comes from a NaN input, and then the row's result is NaN either way)
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max16(const f32x16& v) {
  const float t0 = vmax3(v[0], v[1], v[2]), t1 = vmax3(v[3], v[4], v[5]), t2 = vmax3(v[6], v[7], v[8]);
  const float t3 = vmax3(v[9], v[10], v[11]), t4 = vmax3(v[12], v[13], v[14]);
  return vmax(vmax3(t0, t1, t2), vmax3(t3, t4, v[15]));
}

constexpr int D = 128, BLK = 128;
constexpr int NWAVE = 4, THREADS = 64 * NWAVE;
constexpr int KT = BLK / 32;        // 32-key tiles per block
constexpr int DT = D / 32;          // 32-column tiles of O
constexpr int QREGS = D / 16;       // k-steps of S
constexpr int CH = D / 8;           // 16-byte chunks per row
constexpr int ROWB = D * 2;         // bytes per row
constexpr int TILE = BLK * ROWB;    // bytes per K or V tile
constexpr int NL = TILE / 1024 / NWAVE;  // 1 KB copies per wave per tile
constexpr int RPC = 1024 / ROWB;    // rows per 1 KB copy
static_assert(RPC == 4 && CH == 16 && NL == 8, "copy geometry");

// K rows XOR-swizzled by (row mod 16), V rows by 4*(row mod 4) (16-byte chunks)
__device__ constexpr int swz_k(int r) { return r % CH; }
__device__ constexpr int swz_v(int r) { return 4 * (r % 4); }

enum PpMode { kPpList = 0, kPpDense = 1 };

// ---- MFMAs as inline assembly ------------------------------------------------
// scores: accumulator in VGPRs, query fragment in AGPRs
__device__ __forceinline__ void mma_s0(f32x16& d, const bf16x8& k, const bf16x8& q) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(k), "a"(q));
}
__device__ __forceinline__ void mma_s(f32x16& d, const bf16x8& k, const bf16x8& q) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(k), "a"(q));
}
// outputs: accumulator in AGPRs; the first MFMA that reads a weight register
// freshly written by the VALU waits two states first
__device__ __forceinline__ void mma_o(f32x16& acc, const bf16x8& v, const bf16x8& p, bool fresh) {
  if (fresh)
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(v), "v"(p));
  else
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(v), "v"(p));
}
// the MFMA results of a score pass are complete before the VALU reads them
__device__ __forceinline__ void settle_s(f32x16 (&s)[KT]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(s[0]), "+v"(s[1]), "+v"(s[2]), "+v"(s[3]));
}
// outputs complete before the epilogue's VALU reads them
__device__ __forceinline__ void settle_o(f32x16 (&o)[DT]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]));
}
// o *= alpha in place in AGPRs: wait for the MFMAs that wrote o, then read,
// scale and write back each register; the MFMAs that next read o come after
// enough other instructions (a score pass or the vote and barrier)
#define PP_SCALE1(i) "v_accvgpr_read_b32 %16, %" #i "\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %" #i ", %16\n\t"
__device__ __forceinline__ void scale_o(f32x16& o, float alpha) {
  float tmp;
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4\n\t" PP_SCALE1(0) PP_SCALE1(1) PP_SCALE1(2) PP_SCALE1(3) PP_SCALE1(4)
               PP_SCALE1(5) PP_SCALE1(6) PP_SCALE1(7) PP_SCALE1(8) PP_SCALE1(9) PP_SCALE1(10) PP_SCALE1(11)
               PP_SCALE1(12) PP_SCALE1(13) PP_SCALE1(14) PP_SCALE1(15) "s_nop 4"
               : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]),
                 "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]), "+a"(o[14]),
                 "+a"(o[15]), "=&v"(tmp)
               : "v"(alpha));
}
#undef PP_SCALE1
__device__ __forceinline__ void settle_q(bf16x8 (&q)[QREGS]) {
  asm volatile("s_nop 4" : "+a"(q[0]), "+a"(q[1]), "+a"(q[2]), "+a"(q[3]), "+a"(q[4]), "+a"(q[5]), "+a"(q[6]),
               "+a"(q[7]));
}
__device__ __forceinline__ void pin() { __builtin_amdgcn_sched_barrier(0); }

// elements 4c..4c+3 of a score tile -> bf16 weights (into pd) and their sum
// (two bf16 dot products, continuing the tile's chain r)
__device__ __forceinline__ void pchunk(const f32x16& s, float c2, float mc, bf16x8 (&pd)[2], float& r, int c) {
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int v = 4 * c + j;
    pd[v >> 3][v & 7] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[v], c2, -mc));
  }
  // (pairs taken with constant shuffles: extracting them through a bit cast to
  // 32-bit lanes is miscompiled by this toolchain)
  switch (c) {
    case 0:
      r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pd[0], pd[0], 0, 1), ones, r, false);
      r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pd[0], pd[0], 2, 3), ones, r, false);
      break;
    case 1:
      r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pd[0], pd[0], 4, 5), ones, r, false);
      r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pd[0], pd[0], 6, 7), ones, r, false);
      break;
    case 2:
      r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pd[1], pd[1], 0, 1), ones, r, false);
      r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pd[1], pd[1], 2, 3), ones, r, false);
      break;
    default:
      r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pd[1], pd[1], 4, 5), ones, r, false);
      r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pd[1], pd[1], 6, 7), ones, r, false);
      break;
  }
}

// Softmax weights of one tile, formed in 16 chunks (4 per 32-key tile) that
// the passes place beside their MFMAs; the row sum adds the rounded weights
// tile by tile, each tile's chain in key order.
struct Weights {
  bf16x8 p[KT][2];
  float r[KT];
  float rs;
  float mc;
  __device__ __forceinline__ void start(float m_new, float c2) {
    mc = (m_new == kNegInf) ? 0.f : m_new * c2;
    rs = 0.f;
  }
  __device__ __forceinline__ void chunk(const f32x16 (&s)[KT], float c2, int i) {  // i in [0, 16)
    const int kt = i >> 2, c = i & 3;
    if (c == 0) r[kt] = 0.f;
    pchunk(s[kt], c2, mc, p[kt], r[kt], c);
    if (c == 3) rs += r[kt];
  }
};

template <int MODE>
__global__ __launch_bounds__(THREADS, 1) void osk_pp_kernel(OskArgs a) {
  constexpr bool DENSE = MODE == kPpDense;
  __shared__ __attribute__((aligned(1024))) unsigned char kbuf[2][TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vbuf[2][TILE];
  __shared__ uint32_t vote[2][NWAVE];  // per block parity and wave: all its rows vote to skip

  const SeqArgs& sq = a.seq;
  const int G = sq.group;
  const int GP = G / 2;  // head pairs per KV group
  // ---- unit decode: the one-tile kernel's order with head pairs for heads --
  // (the pairs of one (sequence, group, query block) are consecutive on one
  // XCD; KV groups walked in phases of kPhaseGroups; longest query blocks first)
  const int64_t bid = blockIdx.x;
  const int64_t xcd = bid % kNumXcd, slot = bid / kNumXcd;
  const int64_t lam = ((slot / GP) * kNumXcd + xcd) * GP + slot % GP;
  if (lam >= a.n_units / 2) return;
  const int pair = (int)(lam % GP);
  const int64_t rest = lam / GP;
  const int64_t per_group = (int64_t)sq.batch * sq.max_nq;
  const int phase = (int)(rest / ((int64_t)kPhaseGroups * per_group));
  const int in_phase = min(kPhaseGroups, sq.h_kv - phase * kPhaseGroups);
  const int64_t within = rest - (int64_t)phase * kPhaseGroups * per_group;
  const int g = phase * kPhaseGroups + (int)(within % in_phase);
  const int64_t w2 = within / in_phase;
  const int b = (int)(w2 % sq.batch);
  const int qb = sq.max_nq - 1 - (int)(w2 / sq.batch);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = w >> 1, part = w & 1;  // head of the pair, half of its query block
  const int h = g * G + 2 * pair + hw;
  const int l32 = lane & 31, hl = lane >> 5;
  const int q0 = __builtin_amdgcn_readfirstlane(sq.cu_seqlens_q[b]);
  const int Lq = __builtin_amdgcn_readfirstlane(sq.cu_seqlens_q[b + 1]) - q0;
  const int Lk = __builtin_amdgcn_readfirstlane(sq.seqlens_k[b]);
  const int64_t out_row = ((int64_t)b * sq.h_q + h) * sq.max_nq + qb;
  const bool head_lead = part == 0;  // this head's first wave writes its counters
  if (qb * BLK >= Lq) {  // past this sequence's end: an empty row for both heads
    if constexpr (!DENSE) {
      if (head_lead) {
        if (lane == 0) {
          a.visited[out_row] = 0;
          a.skipped[out_row] = 0;
        }
        if (a.skip_bits)
          for (int t = lane; t < a.kmax; t += 64) a.skip_bits[out_row * a.kmax + t] = 255;
      }
    }
    return;
  }
  const int off = Lk - Lq;
  const int rowA = part * 64 + l32, rowB = rowA + 32;
  const bool validA = qb * BLK + rowA < Lq, validB = qb * BLK + rowB < Lq;
  const int posA = off + qb * BLK + rowA, posB = posA + 32;
  const int n_causal = (off + min(qb * BLK + BLK - 1, Lq - 1)) / BLK + 1;
  const int diag_key0 = off + qb * BLK - (BLK - 1);  // blocks starting after this need the mask

  // ---- query fragments (B operand of S^T = K Q^T), kept in AGPRs -----------
  bf16x8 qa[QREGS], qc[QREGS];
  {
    const uint16_t* qbase = (const uint16_t*)a.q + (int64_t)h * sq.q_head + hl * 8;
    // rows past the sequence end load nothing; their address is the block's first row
    const uint16_t* pa = qbase + (int64_t)(q0 + qb * BLK + (validA ? rowA : 0)) * sq.q_tok;
    const uint16_t* pb = qbase + (int64_t)(q0 + qb * BLK + (validB ? rowB : 0)) * sq.q_tok;
#pragma unroll
    for (int ks = 0; ks < QREGS; ++ks) {
      qa[ks] = __builtin_bit_cast(bf16x8, validA ? *(const uint4*)(pa + ks * 16) : make_uint4(0, 0, 0, 0));
      qc[ks] = __builtin_bit_cast(bf16x8, validB ? *(const uint4*)(pb + ks * 16) : make_uint4(0, 0, 0, 0));
    }
    settle_q(qa);
    settle_q(qc);
  }

  int n_list;
  const int32_t* lst = nullptr;
  const int64_t list_row = ((int64_t)b * sq.h_kv + g) * sq.max_nq + qb;
  if constexpr (DENSE) {
    n_list = n_causal;
  } else {
    // clamped to [0, kmax]: a corrupt count can neither overrun nor underrun the row
    n_list = max(0, min(__builtin_amdgcn_readfirstlane(a.count[list_row]), a.kmax));
    lst = a.order + list_row * a.kmax;
  }
  const int32_t* table = sq.block_table + (int64_t)b * sq.max_blocks_k;
  const unsigned char* kglob = (const unsigned char*)a.k + (size_t)g * TILE;
  const unsigned char* vglob = (const unsigned char*)a.v + (size_t)g * TILE;
  const size_t page_bytes = (size_t)sq.h_kv * TILE;

  // ---- list entries: two 64-entry windows, entry base+lane in each lane ----
  // An entry that is not a causal block of the row, or whose page is out of
  // range, marks the output NaN (as in the one-tile kernel); it reads block 0
  // / page 0 so every copy stays inside the pool.
  int bad_lanes = 0;
  auto load_window = [&](int base, int& wkb, int& wpg) {
    const int t = base + lane;
    int kb = 0, pg = 0;
    if (t < n_list) {
      kb = DENSE ? t : lst[t];
      if (kb < 0 || kb >= n_causal) {
        bad_lanes = 1;
        kb = 0;
      }
      pg = table[kb];
      if ((unsigned)pg >= (unsigned)sq.num_pages) {
        bad_lanes = 1;
        pg = 0;
      }
    }
    wkb = kb;
    wpg = pg;
  };
  int cur_kb, cur_pg, nxt_kb, nxt_pg;
  int wbase = 0;
  load_window(0, cur_kb, cur_pg);
  load_window(64, nxt_kb, nxt_pg);
  // entry t's block and page (uniform); t in [wbase, wbase + 128)
  auto kb_of = [&](int t) -> int {
    const int i = t - wbase;
    return i < 64 ? __builtin_amdgcn_readlane(cur_kb, i) : __builtin_amdgcn_readlane(nxt_kb, i - 64);
  };
  auto page_of = [&](int t) -> int {
    const int i = t - wbase;
    return i < 64 ? __builtin_amdgcn_readlane(cur_pg, i) : __builtin_amdgcn_readlane(nxt_pg, i - 64);
  };

  // ---- per-lane DMA source offsets ----------------------------------------
  // Copy n of wave w fills LDS bytes [(w*NL + n) * 1024, +1024) of a tile: row
  // r = (w*NL + n)*4 + lane/16, physical chunk lane%16 holding logical chunk
  // (lane%16) ^ swz(r). For K, swz(r) = (lane/16) ^ 4*(n%4): copy 0's offset
  // with its chunk bits flipped by (n%4) << 6; for V it depends on the lane only.
  const uint32_t dma_lane = (uint32_t)((lane / CH) * ROWB);
  const uint32_t dma_k0 = dma_lane + (uint32_t)(((lane % CH) ^ swz_k(lane / CH)) * 16);
  const uint32_t dma_v0 = dma_lane + (uint32_t)(((lane % CH) ^ swz_v(lane / CH)) * 16);
  auto issue = [&](int page, bool is_k, unsigned char* tile, int n) {
    const unsigned char* src = (is_k ? kglob : vglob) + (size_t)page * page_bytes + (size_t)w * NL * 1024;
    uint32_t o = (is_k ? dma_k0 ^ (uint32_t)((n & 3) << 6) : dma_v0) + (uint32_t)(n * 1024);
    asm volatile("" : "+v"(o));  // a fresh 32-bit lane offset: scalar base + vector offset addressing
    __builtin_amdgcn_global_load_lds((const void*)(src + o), (lds_void*)(tile + w * NL * 1024 + n * 1024), 16, 0, 0);
  };

  // ---- operand addressing ---------------------------------------------------
  // K (A operand of S^T): row kt*32 + l32, logical chunk 2*ks + hl
  const int k_row = l32 * ROWB;
  const int k_swz = swz_k(l32);
  // V^T (A operand of O^T) via ds_read_b64_tr_b16: lane group gi = lane/16,
  // i = lane%16 reads key row 4*hh + i/4 (+ 16*step + 8*half), columns
  // dt*32 + 16*dg + 4*(i%4) .. +3
  int v_addr[DT];
  {
    const int i = lane & 15, gi = lane >> 4, hh = gi >> 1, dg = gi & 1;
    const int q = i >> 2;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = dt * 32 + 16 * dg + 4 * (i & 3);
      v_addr[dt] = (4 * hh + q) * ROWB + (((d >> 3) ^ swz_v(q)) << 4) + (d & 7) * 2;
    }
  }
  const float c2 = a.scale_log2;

  // score pass S^T = K Q^T over one K tile. Each fragment register is
  // re-read for k-step ks+1 right after the MFMA of k-step ks that used it,
  // four MFMAs before its next use; side(i) is the VALU work of slot i (32 slots)
  auto scores = [&](const unsigned char* kt_lds, const bf16x8 (&q)[QREGS], f32x16 (&s)[KT], auto&& side) {
    const unsigned char* kl = kt_lds + k_row;
    bf16x8 kf[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) kf[kt] = *(const bf16x8*)(kl + ((hl ^ k_swz) << 4) + kt * 32 * ROWB);
#pragma unroll
    for (int ks = 0; ks < QREGS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        if (ks == 0)
          mma_s0(s[kt], kf[kt], q[0]);
        else
          mma_s(s[kt], kf[kt], q[ks]);
        if (ks + 1 < QREGS)
          kf[kt] = *(const bf16x8*)(kl + (((2 * (ks + 1) + hl) ^ k_swz) << 4) + kt * 32 * ROWB);
        side(ks * KT + kt);
        pin();
      }
    }
    settle_s(s);
  };
  auto vread = [&](const unsigned char* vt_lds, int st, int dt, int e) -> s16x4 {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt_lds + v_addr[dt] + (st * 16 + 8 * e) * ROWB));
  };
  // O^T += V^T P^T over the block's 8 16-key steps, fragment registers
  // re-read for step st+1 right after the MFMA of step st; side(i) as above
  auto pv = [&](const unsigned char* vt_lds, f32x16 (&acc)[DT], const bf16x8 (&pt)[KT][2], auto&& side) {
    s16x4 vf[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      vf[dt][0] = vread(vt_lds, 0, dt, 0);
      vf[dt][1] = vread(vt_lds, 0, dt, 1);
    }
#pragma unroll
    for (int st = 0; st < 2 * KT; ++st) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 vv =
            __builtin_bit_cast(bf16x8, __builtin_shufflevector(vf[dt][0], vf[dt][1], 0, 1, 2, 3, 4, 5, 6, 7));
        mma_o(acc[dt], vv, pt[st >> 1][st & 1], dt == 0);
        if (st + 1 < 2 * KT) {
          vf[dt][0] = vread(vt_lds, st + 1, dt, 0);
          vf[dt][1] = vread(vt_lds, st + 1, dt, 1);
        }
        side(st * DT + dt);
        pin();
      }
    }
  };
  auto no_side = [](int) {};
  // causal mask of a tile (blocks past the query block's first row only):
  // element (kt, v) is key kb*B + kt*32 + 8*(v/4) + 4*hl + v%4
  auto mask_tile = [&](f32x16 (&s)[KT], int kb, int pos) {
    const int thr = pos - kb * BLK - 4 * hl;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (kt * 32 + 8 * (v >> 2) + (v & 3) > thr) s[kt][v] = kNegInf;
  };
  // rescale an output by alpha (only when some row's max moved)
  auto rescale = [&](f32x16 (&o)[DT], float alpha) {
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) scale_o(o[dt], alpha);
    }
  };

  f32x16 oa[DT], ob[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      oa[dt][v] = 0.f;
      ob[dt][v] = 0.f;
    }
  float mA = kNegInf, mB = kNegInf;  // running maxima of raw q.k (unscaled)
  float lA = 0.f, lB = 0.f;          // this lane's share of the running sums
  int n_skip = 0;

  // ---- prologue: K(0) -> kbuf[0], K(1) -> kbuf[1], V(0) -> vbuf[0] --------
  if (n_list > 0) {
    const int p0 = page_of(0);
#pragma unroll
    for (int n = 0; n < NL; ++n) issue(p0, true, kbuf[0], n);
    if (n_list > 1) {
      const int p1 = page_of(1);
#pragma unroll
      for (int n = 0; n < NL; ++n) issue(p1, true, kbuf[1], n);
    }
#pragma unroll
    for (int n = 0; n < NL; ++n) issue(p0, false, vbuf[0], n);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  f32x16 sa[KT], sb[KT];  // S_A(t); S_B(t-1) until B's weights are formed, then S_B(t)
  Weights wa, wb;
  bool b_pend = false;    // block t-1 was not skipped: B's weights and P.V are due
  float locB = kNegInf;   // B's local row maximum of block t-1
  for (int t = 0; t < n_list; ++t) {
    if (t - wbase == 64) {  // slide the windows: the next one becomes current
      wbase += 64;
      cur_kb = nxt_kb;
      cur_pg = nxt_pg;
      load_window(wbase + 64, nxt_kb, nxt_pg);
    }
    const int kb = kb_of(t);
    const unsigned char* kt_lds = kbuf[t & 1];
    unsigned char* vt_lds = vbuf[t & 1];
    const unsigned char* vp_lds = vbuf[(t + 1) & 1];  // V(t-1)
    const bool need_mask = kb * BLK > diag_key0;

    // ---- 1: S_A(t) beside B's weights for block t-1 ---------------------------
    float nB = mB;
    if (b_pend) {
      nB = vmax(mB, locB);
      wb.start(nB, c2);
    }
    scores(kt_lds, qa, sa, [&](int i) {
      if (b_pend && i >= 2 && i < 18) wb.chunk(sb, c2, i - 2);
    });
    if (b_pend) {
      const float alpha = (nB == mB) ? 1.f : __builtin_amdgcn_exp2f((mB - nB) * c2);
      rescale(ob, alpha);
      lB = lB * alpha + wb.rs;
      mB = nB;
    }

    // ---- 2: O_B += V(t-1) P_B beside A's maxima and first weights ------------
    if (need_mask) mask_tile(sa, kb, posA);
    float hA = kNegInf, locA = kNegInf, nA = kNegInf;
    auto side2 = [&](int i) {
      if (i < KT) hA = (i == 0) ? max16(sa[0]) : vmax(hA, max16(sa[i]));
      if (i == KT) {
        locA = max_xor32(hA);
        nA = vmax(mA, locA);
        wa.start(nA, c2);
      }
      if (i > KT && i <= KT + 8) wa.chunk(sa, c2, i - KT - 1);
    };
    if (b_pend) {
      pv(vp_lds, ob, wb.p, side2);
    } else {
#pragma unroll
      for (int i = 0; i <= KT + 8; ++i) side2(i);
    }

    // ---- 3: S_B(t) beside the rest of A's weights -------------------------------
    scores(kt_lds, qc, sb, [&](int i) {
      if (i >= 2 && i < 10) wa.chunk(sa, c2, i + 6);
    });

    // ---- 4: B's maxima, the vote, barrier X(t) -----------------------------------
    if (need_mask) mask_tile(sb, kb, posB);
    float hB = max16(sb[0]);
#pragma unroll
    for (int kt = 1; kt < KT; ++kt) hB = vmax(hB, max16(sb[kt]));
    if constexpr (!DENSE) {
      if (a.skip_on) {
        // a row's margin is below ln(tau) exactly when both of its halves' are
        // (subtracting the running max is monotone under rounding; a NaN margin
        // never votes to skip): one ballot per wave over both tiles' half-row
        // margins
        const float dA = (validA && hA != kNegInf) ? hA - mA : kNegInf;
        const float dB = (validB && hB != kNegInf) ? hB - mB : kNegInf;
        const bool wave_skips =
            __builtin_amdgcn_ballot_w64(!(dA < a.skip_thr_raw) || !(dB < a.skip_thr_raw)) == 0;
        if (lane == 0) vote[t & 1][w] = wave_skips ? 1u : 0u;
      }
    }
    locB = max_xor32(hB);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // X(t): K(t+1), V(t) landed; K(t), V(t-1) free; votes visible
    bool skip = false;
    if constexpr (!DENSE) {
      if (a.skip_on) skip = __builtin_amdgcn_readfirstlane(vote[t & 1][2 * hw] & vote[t & 1][2 * hw + 1]) != 0;
    }
    // next copies: K(t+2) into K(t)'s buffer, V(t+1) into V(t-1)'s
    const bool cp_k = t + 2 < n_list, cp_v = t + 1 < n_list;
    const int pgk = cp_k ? page_of(t + 2) : 0;
    const int pgv = cp_v ? page_of(t + 1) : 0;
    unsigned char* k_dst = kbuf[t & 1];
    unsigned char* v_dst = vbuf[(t + 1) & 1];
    // value rows past the sequence end are zeroed before P.V reads them
    // (uniform over the workgroup, whichever head skips)
    const int nvalid = min(BLK, Lk - kb * BLK);
    if (nvalid < BLK) {
      uint4* z = (uint4*)(vt_lds + nvalid * ROWB);
      for (int i = tid; i < (BLK - nvalid) * ROWB / 16; i += THREADS) z[i] = make_uint4(0, 0, 0, 0);
      __syncthreads();
    }
    n_skip += skip ? 1 : 0;
    if (!skip) {
      const float alpha = (nA == mA) ? 1.f : __builtin_amdgcn_exp2f((mA - nA) * c2);
      rescale(oa, alpha);
      lA = lA * alpha + wa.rs;
      mA = nA;
      // O_A += V(t) P_A beside the copies (one K and one V copy per 16-key step)
      pv(vt_lds, oa, wa.p, [&](int i) {
        if ((i & 3) == 1 && cp_k) issue(pgk, true, k_dst, i >> 2);
        if ((i & 3) == 3 && cp_v) issue(pgv, false, v_dst, i >> 2);
      });
    } else {
      if (cp_k)
#pragma unroll
        for (int n = 0; n < NL; ++n) issue(pgk, true, k_dst, n);
      if (cp_v)
#pragma unroll
        for (int n = 0; n < NL; ++n) issue(pgv, false, v_dst, n);
    }
    b_pend = !skip;
    if constexpr (!DENSE) {
      if (head_lead && lane == 0 && a.skip_bits) a.skip_bits[out_row * a.kmax + t] = skip ? 1 : 0;
    }
  }
  // ---- B's last block ---------------------------------------------------------
  if (b_pend) {
    const float nB = vmax(mB, locB);
    wb.start(nB, c2);
#pragma unroll
    for (int i = 0; i < 16; ++i) wb.chunk(sb, c2, i);
    const float alpha = (nB == mB) ? 1.f : __builtin_amdgcn_exp2f((mB - nB) * c2);
    rescale(ob, alpha);
    lB = lB * alpha + wb.rs;
    mB = nB;
    pv(vbuf[(n_list - 1) & 1], ob, wb.p, no_side);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no copy in flight when the workgroup's LDS is released
  settle_o(oa);
  settle_o(ob);

  // ---- epilogue ---------------------------------------------------------------
  const int bad = __builtin_amdgcn_ballot_w64(bad_lanes != 0) != 0 ? 1 : 0;
  auto store_tile = [&](const f32x16 (&acc)[DT], float l_run, float m_run, int row, bool valid) {
    const float l_tot = sum_xor32(l_run);
    float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (bad) inv = __builtin_nanf("");
    if (!valid) return;
    const int64_t ooff = (int64_t)(q0 + qb * BLK + row) * sq.o_tok + (int64_t)h * sq.o_head;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = dt * 32 + 8 * g4 + 4 * hl;
        const float o0 = acc[dt][4 * g4 + 0] * inv, o1 = acc[dt][4 * g4 + 1] * inv;
        const float o2 = acc[dt][4 * g4 + 2] * inv, o3 = acc[dt][4 * g4 + 3] * inv;
        const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o0) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o1) << 16);
        const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o2) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o3) << 16);
        *(uint2*)((uint16_t*)a.o + ooff + d0) = make_uint2(lo, hi);
      }
    if (a.lse && hl == 0) {
      a.lse[(size_t)h * a.total_q + q0 + qb * BLK + row] =
          bad ? __builtin_nanf("") : (l_tot > 0.f ? m_run * a.scale + logf(l_tot) : kNegInf);
    }
  };
  store_tile(oa, lA, mA, rowA, validA);
  store_tile(ob, lB, mB, rowB, validB);
  if constexpr (!DENSE) {
    if (head_lead) {
      if (lane == 0) {
        a.visited[out_row] = n_list;
        a.skipped[out_row] = n_skip;
      }
      if (a.skip_bits)
        for (int t = n_list + lane; t < a.kmax; t += 64) a.skip_bits[out_row * a.kmax + t] = 255;
    }
  }
}

}  // namespace

// The two-tile walk serves head_dim 128, block 128 and an even query-group
// size; other shapes take the one-tile kernel.
bool osk_pp_supported(int head_dim, int block, int group) {
  return head_dim == 128 && block == 128 && group % 2 == 0;
}

hipError_t launch_osk_pp(const OskArgs& a, bool dense, hipStream_t stream) {
  const int64_t units = a.n_units / 2;
  const int64_t per = (int64_t)kNumXcd * (a.seq.group / 2);
  const int64_t grid = (units + per - 1) / per * per;
  if (dense)
    hipLaunchKernelGGL((osk_pp_kernel<kPpDense>), dim3((unsigned)grid), dim3(THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((osk_pp_kernel<kPpList>), dim3((unsigned)grid), dim3(THREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace cosa
