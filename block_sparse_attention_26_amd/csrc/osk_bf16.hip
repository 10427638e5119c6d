// Ordered-Skipping Kernel (OSK) and dense baseline, bf16 path for gfx950.
//
// Method: CoSA technical summary (gist.science, "CoSA: Accelerating
// Long-Context Inference via Proxy-Kernel Co-Designed Sparse Attention"),
// §2.3 (walk only the listed pages, in order; skip a retained block in-kernel
// from the local vs running row maxima; otherwise compute it), §2.1 (the
// online-softmax result does not depend on the visit order) and §1 (the skip
// veto is per tile: every row of the query block must agree).
//
// One workgroup per (sequence, query head, query block): B/32 waves of 32
// query rows. Scores are formed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16, so each lane owns one query row; the output is
// accumulated transposed too, O^T += V^T P^T, with the bf16 P registers as the
// B operand.
//
// gfx950 data movement:
//  * K and V pages are copied global -> LDS by global_load_lds_dwordx4 (no
//    staging registers). Lane l of a load lands at LDS base + 16*l, so the
//    tiles are XOR-swizzled by choosing each lane's source chunk: K rows are
//    swizzled by (row mod 16) so the 32 rows read by one MFMA operand fetch
//    spread over all banks; V rows by 4*(row mod 4) for the transposed reads.
//  * V^T operands come from ds_read_b64_tr_b16: in each 16-lane group, lanes
//    4k..4k+3 address 4 consecutive head-dim columns of key row K_k and every
//    lane receives 4 keys of one column.
//  * Per listed block: barrier A (K(t) landed, V buffer free) -> copy V(t)
//    -> S(t) = K(t) Q^T, mask, row maxima, per-wave skip vote -> barrier C
//    (V(t) landed, K buffer free, votes visible) -> copy K(t+1) -> unless
//    skipped, softmax and O^T += V(t)^T P(t)^T. Tiles are single-buffered
//    (64 KB of LDS) so two workgroups share a CU: one's MFMA work overlaps the
//    other's softmax and copy waits.
// Tail keys (past the sequence end) are loaded from a valid key row of the
// same page and masked, so NaN-filled slots never reach the MFMAs.
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

// Maxima as llvm.maximum (v_maximum3_f32 on gfx950). Through fmaxf the
// compiler first quiets every operand it cannot prove free of signaling NaNs
// (an extra v_max_f32 x, x, x each); maximum needs no quieting because it
// propagates NaN, which the score maxima may do: a NaN score only comes from a
// NaN input, and then the row's result is NaN either way.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }

// x combined with lane l ^ 32's x (v_permlane32_swap exchanges the halves)
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max of x over lanes 0..31, valid in lane 0: within each row of 16 lanes a
// max of the 16 values of an accumulator, as a shallow tree
__device__ __forceinline__ float max16(const f32x16& v) {
  const float t0 = vmax3(v[0], v[1], v[2]), t1 = vmax3(v[3], v[4], v[5]), t2 = vmax3(v[6], v[7], v[8]);
  const float t3 = vmax3(v[9], v[10], v[11]), t4 = vmax3(v[12], v[13], v[14]);
  return vmax(vmax3(t0, t1, t2), vmax3(t3, t4, v[15]));
}

template <int D, int BLK>
struct Geo {
  static constexpr int NW = BLK / 32;
  static constexpr int THREADS = 64 * NW;
  static constexpr int KT = BLK / 32;         // 32-key tiles per block
  static constexpr int DT = D / 32;           // 32-column tiles of O
  static constexpr int QREGS = D / 16;        // k-steps of S
  static constexpr int CH = D / 8;            // 16-byte chunks per row
  static constexpr int ROWB = D * 2;          // bytes per row
  static constexpr int TILE = BLK * ROWB;     // bytes per K or V tile
  static constexpr int NL = TILE / 1024 / NW; // 1 KB DMA copies per wave per tile
  static constexpr int RPC = 1024 / ROWB;     // rows per 1 KB copy
  __device__ static constexpr int swz_k(int r) { return r % CH; }
  __device__ static constexpr int swz_v(int r) { return D == 128 ? 4 * (r % 4) : 4 * (r % 2); }
};

// Walk modes: the ordered list (the OSK), every causal block ascending (the
// dense baseline), or every causal block ascending under a binary block mask
// (control-flow skipping, for comparison with the list walk).
enum WalkMode { kList = 0, kDense = 1, kMask = 2 };

template <int D, int BLK, int MODE>
__global__ __launch_bounds__(2 * BLK, 2) void osk_bf16_kernel(OskArgs a) {
  constexpr bool DENSE = MODE == kDense;
  constexpr bool MASK = MODE == kMask;
  using Gm = Geo<D, BLK>;
  constexpr int NW = Gm::NW, KT = Gm::KT, DT = Gm::DT, QREGS = Gm::QREGS;
  constexpr int CH = Gm::CH, ROWB = Gm::ROWB, TILE = Gm::TILE, NL = Gm::NL, RPC = Gm::RPC;
  __shared__ __attribute__((aligned(1024))) unsigned char kbuf[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vbuf[TILE];
  __shared__ uint32_t vote[NW];  // per wave: 1 when all its rows vote to skip the block

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
  // sequence metadata is uniform: keep it in scalar registers
  const int q0 = __builtin_amdgcn_readfirstlane(sq.cu_seqlens_q[b]);
  const int Lq = __builtin_amdgcn_readfirstlane(sq.cu_seqlens_q[b + 1]) - q0;
  const int Lk = __builtin_amdgcn_readfirstlane(sq.seqlens_k[b]);
  const int tid = threadIdx.x;
  const int64_t out_row = ((int64_t)b * sq.h_q + h) * sq.max_nq + qb;
  if (qb * BLK >= Lq) {  // past this sequence's end: an empty row
    if constexpr (!DENSE) {
      if (tid == 0) {
        a.visited[out_row] = 0;
        a.skipped[out_row] = 0;
      }
      if (!MASK && a.skip_bits)
        for (int t = tid; t < a.kmax; t += Gm::THREADS) a.skip_bits[out_row * a.kmax + t] = 255;
    }
    return;
  }
  const int off = Lk - Lq;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int row = w * 32 + l32;
  const bool row_valid = qb * BLK + row < Lq;
  const int my_pos = off + qb * BLK + row;
  const int n_causal = (off + min(qb * BLK + BLK - 1, Lq - 1)) / BLK + 1;
  const int diag_key0 = off + qb * BLK - (BLK - 1);  // blocks starting after this need the mask

  // ---- query fragments (B operand of S^T = K Q^T) -------------------------
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

  int n_list;
  const int32_t* lst = nullptr;
  const uint64_t* mrow = nullptr;
  const int64_t list_row = ((int64_t)b * sq.h_kv + g) * sq.max_nq + qb;
  if constexpr (DENSE || MASK) {
    n_list = n_causal;
    if constexpr (MASK) mrow = a.mask + list_row * a.mask_words;
  } else {
    // clamped to [0, kmax]: a corrupt count can neither overrun nor underrun the row
    n_list = max(0, min(__builtin_amdgcn_readfirstlane(a.count[list_row]), a.kmax));
    lst = a.order + list_row * a.kmax;
  }
  int bad = 0;
  const int32_t* table = sq.block_table + (int64_t)b * sq.max_blocks_k;
  const unsigned char* kglob = (const unsigned char*)a.k + (size_t)g * TILE;
  const unsigned char* vglob = (const unsigned char*)a.v + (size_t)g * TILE;
  const size_t page_bytes = (size_t)sq.h_kv * TILE;

  // ---- per-lane DMA source offsets (bytes within a page slab) ------------
  // Copy n of wave w fills LDS bytes [(w*NL + n) * 1024, +1024): row
  // r = (w*NL + n)*RPC + lane/CH, physical chunk lane%CH, which must hold the
  // logical chunk (lane%CH) ^ swz(r). With d = 128 (RPC = 4, CH = 16, NL a
  // multiple of 4) the K swizzle of copy n is (lane%16) ^ (lane/16) ^ 4*(n%4),
  // i.e. copy 0's offset with its chunk bits flipped by (n%4) << 6; with d = 64
  // (RPC = CH = 8) it depends on the lane only. The V swizzle depends on the
  // lane only in both cases.
  static_assert(D == 64 || (RPC == 4 && CH == 16 && NL % 4 == 0), "K swizzle period");
  static_assert(D == 128 || RPC % CH == 0, "K swizzle period");
  static_assert(NL == QREGS, "one V copy per k-step of S");
  const uint32_t dma_lane = (uint32_t)((lane / CH) * ROWB);
  const uint32_t dma_k0 = dma_lane + (uint32_t)(((lane % CH) ^ Gm::swz_k(lane / CH)) * 16);
  const uint32_t dma_v0 = dma_lane + (uint32_t)(((lane % CH) ^ Gm::swz_v(lane / CH)) * 16);
  // ---- list walk --------------------------------------------------------------
  // Entry t names block kb_t, whose page comes from the block table. Both loads
  // for entry t+1 are issued a tile ahead (after barrier A of tile t) and read
  // after barrier C, so their latency hides under the tile's work. An entry
  // that is not a causal block of the row, or a page out of range, sets `bad`.
  auto entry_at = [&](int t) -> int { return MODE == kList ? lst[t] : t; };
  // mask word of block i (uniform; i < n_causal <= 64 * mask_words)
  auto mask_word = [&](int i) -> uint64_t {
    const uint64_t x = mrow[i >> 6];
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(x >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  };
  auto check_kb = [&](int raw) -> int {
    int kb = __builtin_amdgcn_readfirstlane(raw);  // uniform: keeps the mask branch scalar
    if (kb < 0 || kb >= n_causal) {
      bad = 1;
      kb = 0;
    }
    return kb;
  };
  auto check_page = [&](int raw) -> int {
    int page = __builtin_amdgcn_readfirstlane(raw);
    if ((unsigned)page >= (unsigned)sq.num_pages) {
      bad = 1;
      page = 0;
    }
    return page;
  };
  // A tile copy is issued as NL single-instruction copies that the loop spreads
  // over the MFMA k-steps, so their issue cost hides under matrix work. A
  // partial tile (the last block of a sequence) is copied whole from its page:
  // key rows past the sequence end only ever meet the causal mask, which
  // replaces their scores, and value rows past the end are zeroed in LDS before
  // P.V reads them.
  struct Copy {
    const unsigned char* src;  // this wave's part of the page slab
    unsigned char* dst;        // this wave's part of the LDS tile
  };
  auto copy_of = [&](int page, bool is_k) -> Copy {
    return Copy{(is_k ? kglob : vglob) + (size_t)page * page_bytes + (size_t)w * NL * 1024,
                (is_k ? kbuf : vbuf) + w * NL * 1024};
  };
  auto issue = [&](const Copy& c, bool is_k, int n) {
    uint32_t o = (is_k ? dma_k0 ^ (D == 128 ? (uint32_t)((n & 3) << 6) : 0u) : dma_v0) + (uint32_t)(n * 1024);
    asm volatile("" : "+v"(o));  // a fresh 32-bit lane offset: scalar base + vector offset addressing
    __builtin_amdgcn_global_load_lds((const void*)(c.src + o), (lds_void*)(c.dst + n * 1024), 16, 0, 0);
  };

  // ---- operand addressing ---------------------------------------------------
  // K (A operand of S^T): row kt*32 + l32, logical chunk 2*ks + hl.
  const unsigned char* k_lane = kbuf + l32 * ROWB;
  const int k_swz = Gm::swz_k(l32);
  // V^T (A operand of O^T) via ds_read_b64_tr_b16: lane group gi = lane/16,
  // i = lane%16 reads key row 4*hh + i/4 (+ 16*step + 8*half), columns
  // dt*32 + 16*dg + 4*(i%4) .. +3.
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
  float m_run = kNegInf;  // running max of raw q.k (unscaled)
  float l_run = 0.f;      // this lane's share of the running sum
  int n_skip = 0;
  const float c2 = a.scale_log2;

  int kb = 0, page = 0;  // entry t
  int raw_e = 0;         // entry t+1, loaded a tile ahead
  Copy ck{}, cv{};
  // mask walk: the block whose K copies are issued or pending (-1: none), the
  // mask word of the current block, selected blocks walked
  uint64_t mword = 0;
  int n_vis = 0;
  if (MASK) {
    kb = -1;
  } else if (n_list > 0) {  // an empty list touches no entry
    kb = check_kb(entry_at(0));
    page = check_page(table[kb]);
    ck = copy_of(page, true);
#pragma unroll
    for (int n = 0; n < NL; ++n) issue(ck, true, n);  // K(0)
    raw_e = entry_at(min(1, n_list - 1));
  }
  bool pend = false;  // K(t) still to be issued: the previous block was skipped
  for (int t = 0; t < n_list; ++t) {
    if constexpr (MASK) {
      // control-flow skipping: every causal block costs a bit test; a block
      // whose K was not prefetched (its predecessor unselected) is fetched
      // here, with its latency exposed
      for (;;) {
        if ((t & 63) == 0) mword = mask_word(t);
        if ((mword >> (t & 63)) & 1) break;
        if (++t == n_list) break;
      }
      if (t == n_list) break;
      ++n_vis;
      if (kb != t) {
        kb = t;
        page = check_page(table[t]);
        ck = copy_of(page, true);
        pend = true;
      }
    }
    if (pend) {
#pragma unroll 1
      for (int n = 0; n < NL; ++n) issue(ck, true, n);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // A: K(t) landed; every wave is done with V(t-1)
    // entry t+1 (the last entry again after the end, which keeps the K copies
    // of the next step unconditional) and its page; entry t+2
    int kb_next, raw_p;
    bool nsel = true;  // block t+1 is walked, so its K is prefetched during this block's P.V
    if constexpr (MASK) {
      kb_next = min(t + 1, n_list - 1);
      raw_p = table[kb_next];
      if (t + 1 < n_list) {
        const uint64_t wn = ((t + 1) & 63) ? mword : mask_word(t + 1);
        nsel = ((wn >> ((t + 1) & 63)) & 1) != 0;
      } else {
        nsel = false;
      }
    } else {
      kb_next = check_kb(raw_e);
      raw_p = table[kb_next];
      raw_e = entry_at(min(t + 2, n_list - 1));
    }
    const int nvalid = min(BLK, Lk - kb * BLK);
    cv = copy_of(page, false);  // V(t): copies issued during the S k-steps

    // ---- S^T = K Q^T for this wave's 32 rows -------------------------------
    // fragments of k-step ks+1 are read while the MFMAs of k-step ks run
    f32x16 s[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kt][v] = 0.f;
    {
      bf16x8 kf[2][KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) kf[0][kt] = *(const bf16x8*)(k_lane + ((hl ^ k_swz) << 4) + kt * 32 * ROWB);
#pragma unroll
      for (int ks = 0; ks < QREGS; ++ks) {
        issue(cv, false, ks);  // one V copy per k-step
        if (ks + 1 < QREGS) {
          const unsigned char* kp = k_lane + (((2 * (ks + 1) + hl) ^ k_swz) << 4);
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) kf[(ks + 1) & 1][kt] = *(const bf16x8*)(kp + kt * 32 * ROWB);
        }
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks & 1][kt], qf[ks], s[kt], 0, 0, 0);
      }
      // pin the order: per k-step, its V copies and the reads of step ks+1 are
      // issued ahead of the MFMAs of step ks
      __builtin_amdgcn_sched_group_barrier(0x100, KT, 0);  // DS reads (step 0)
#pragma unroll
      for (int ks = 0; ks < QREGS; ++ks) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // copy
        if (ks + 1 < QREGS) __builtin_amdgcn_sched_group_barrier(0x100, KT, 0);  // DS reads (step ks+1)
        __builtin_amdgcn_sched_group_barrier(0x008, KT, 0);                       // MFMA (step ks)
      }
    }
    // causal mask (only blocks that reach past the first row's position):
    // element (kt, v) is key kb*B + kt*32 + 8*(v/4) + 4*hl + v%4
    if (kb * BLK > diag_key0) {
      asm volatile("" ::: "memory");  // keep this a real branch (no if-conversion)
      const int thr = my_pos - kb * BLK - 4 * hl;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (kt * 32 + 8 * (v >> 2) + (v & 3) > thr) s[kt][v] = kNegInf;
    }
    float m_half = max16(s[0]);  // maximum over this lane's half of the row's keys
#pragma unroll
    for (int kt = 1; kt < KT; ++kt) m_half = vmax(m_half, max16(s[kt]));
    if constexpr (!DENSE) {
      if (a.skip_on) {
        // the largest margin is below the threshold exactly when every row's
        // is, and a row's margin is exactly when both of its halves' are
        // (subtracting the running max is monotone under rounding; a NaN
        // margin never votes to skip): one ballot per wave over the half-row
        // margins, before the halves are combined
        const float diff = (row_valid && m_half != kNegInf) ? m_half - m_run : kNegInf;
        const bool wave_skips = __builtin_amdgcn_ballot_w64(!(diff < a.skip_thr_raw)) == 0;
        if (lane == 0) vote[w] = wave_skips ? 1u : 0u;
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // C: V(t) landed; every wave is done with K(t); votes visible
    const float m_loc = max_xor32(m_half);
    bool skip = false;
    if constexpr (!DENSE) {
      if (a.skip_on) {
        uint32_t all = vote[0];
#pragma unroll
        for (int i = 1; i < NW; ++i) all &= vote[i];
        skip = __builtin_amdgcn_readfirstlane(all) != 0;
      }
    }
    // K(t+1): copies issued during P.V (drained before exit)
    const int page_next = check_page(raw_p);
    // (mask walk, next block unselected: the copies re-read this block's K
    // page, an L2 hit, so the copy sequence stays branch-free)
    ck = copy_of(nsel ? page_next : page, true);
    constexpr int KPS = (NL + 2 * KT - 1) / (2 * KT);  // K copies per P.V k-step

    // ---- online-softmax update and O^T += V^T P^T, one 32-key tile at a time:
    // the exps of tile kt+1 (VALU) run while the P.V MFMAs of tile kt execute
    n_skip += skip ? 1 : 0;
    if (!skip) {
      if (nvalid < BLK) {  // zero the value rows past the sequence end
        uint4* z = (uint4*)(vbuf + nvalid * ROWB);
        for (int i = tid; i < (BLK - nvalid) * ROWB / 16; i += Gm::THREADS) z[i] = make_uint4(0, 0, 0, 0);
        __syncthreads();
      }
      const float m_new = vmax(m_run, m_loc);
      const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * c2);
      const float mc = (m_new == kNegInf) ? 0.f : m_new * c2;
      if (__any(alpha != 1.f)) {  // rescale only when some row's max moved
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[dt][v] *= alpha;
      }
      m_run = m_new;
      float rs = 0.f;
      // P tile kt in bf16; the row sum adds the same rounded weights that
      // enter P.V, two per bf16 dot product, in a chain per tile
      const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
      auto ptile = [&](int kt, bf16x8 (&pd)[2]) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          pd[v >> 3][v & 7] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][v], c2, -mc));
        // (pairs taken with constant shuffles: extracting them through a
        // bit cast to 32-bit lanes is miscompiled by this toolchain)
        float r = 0.f;
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pd[0], pd[0], 0, 1), ones, r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pd[0], pd[0], 2, 3), ones, r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pd[0], pd[0], 4, 5), ones, r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pd[0], pd[0], 6, 7), ones, r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pd[1], pd[1], 0, 1), ones, r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pd[1], pd[1], 2, 3), ones, r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pd[1], pd[1], 4, 5), ones, r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pd[1], pd[1], 6, 7), ones, r, false);
        rs += r;
      };
      auto vread = [&](int st, int dt, int e) -> s16x4 {
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(vbuf + v_addr[dt] + (st * 16 + 8 * e) * ROWB));
      };
      s16x4 vf[2][DT][2];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        vf[0][dt][0] = vread(0, dt, 0);
        vf[0][dt][1] = vread(0, dt, 1);
      }
      bf16x8 pt[2][2];
      ptile(0, pt[0]);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT) ptile(kt + 1, pt[(kt + 1) & 1]);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int st = 2 * kt + s2;
#pragma unroll
          for (int n = st * KPS; n < (st + 1) * KPS && n < NL; ++n) issue(ck, true, n);
          if (st + 1 < 2 * KT)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              vf[(st + 1) & 1][dt][0] = vread(st + 1, dt, 0);
              vf[(st + 1) & 1][dt][1] = vread(st + 1, dt, 1);
            }
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const bf16x8 vv = __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(vf[st & 1][dt][0], vf[st & 1][dt][1], 0, 1, 2, 3, 4, 5, 6, 7));
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pt[kt & 1][s2], acc[dt], 0, 0, 0);
          }
        }
      }
      l_run = l_run * alpha + rs;
    }
    pend = skip && nsel;
    if constexpr (MODE == kList) {
      if (tid == 0 && a.skip_bits) a.skip_bits[out_row * a.kmax + t] = skip ? 1 : 0;
    }
    kb = nsel ? kb_next : -1;
    page = page_next;
  }

  __builtin_amdgcn_s_waitcnt(0);  // the trailing re-copy lands before the workgroup's LDS is released
  // ---- epilogue -------------------------------------------------------------
  const float l_tot = sum_xor32(l_run);
  float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (bad) inv = __builtin_nanf("");
  if (row_valid) {
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
  }
  if constexpr (!DENSE) {
    if (tid == 0) {
      a.visited[out_row] = MASK ? n_vis : n_list;
      a.skipped[out_row] = n_skip;
    }
    if (!MASK && a.skip_bits)
      for (int t = n_list + tid; t < a.kmax; t += Gm::THREADS) a.skip_bits[out_row * a.kmax + t] = 255;
  }
}

template <int D, int BLK>
hipError_t launch_one(const OskArgs& a, bool dense, hipStream_t stream) {
  const int64_t per = (int64_t)kNumXcd * a.seq.group;
  const int64_t grid = (a.n_units + per - 1) / per * per;
  if (dense)
    hipLaunchKernelGGL((osk_bf16_kernel<D, BLK, kDense>), dim3((unsigned)grid), dim3(2 * BLK), 0, stream, a);
  else if (a.mask)
    hipLaunchKernelGGL((osk_bf16_kernel<D, BLK, kMask>), dim3((unsigned)grid), dim3(2 * BLK), 0, stream, a);
  else
    hipLaunchKernelGGL((osk_bf16_kernel<D, BLK, kList>), dim3((unsigned)grid), dim3(2 * BLK), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_osk_bf16(const OskArgs& a, int head_dim, int block, bool dense, hipStream_t stream) {
  if (head_dim == 128 && block == 128) return launch_one<128, 128>(a, dense, stream);
  if (head_dim == 128 && block == 64) return launch_one<128, 64>(a, dense, stream);
  if (head_dim == 64 && block == 128) return launch_one<64, 128>(a, dense, stream);
  if (head_dim == 64 && block == 64) return launch_one<64, 64>(a, dense, stream);
  return hipErrorInvalidValue;
}

}  // namespace cosa
