// Device pieces shared by the proxy kernels (kap.hip, kap_fused.hip): the
// proxy's fp32 exponential and the descending bitonic sort of 64-bit keys.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cosa {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kThreads = 256;

// ---- exp32: the proxy's exponential, as specified ---------------------------
// 0 unless x >= -87; t = x*fp32(log2 e); n = rint(t); f = t - n;
// Horner over c_k = fp32(ln2^k / k!), k = 7..0; result p * 2^n.
__device__ inline float exp32(float x) {
#pragma clang fp contract(off)
  if (!(x >= -87.0f)) return 0.0f;
  const float t = x * __builtin_bit_cast(float, 0x3FB8AA3Bu);
  const float n = __builtin_rintf(t);
  const float f = t - n;
  float p = __builtin_bit_cast(float, 0x377FE5FEu);            // ln2^7/7!
  p = f * p; p = p + __builtin_bit_cast(float, 0x39218489u);   // ln2^6/6!
  p = f * p; p = p + __builtin_bit_cast(float, 0x3AAEC3FFu);   // ln2^5/5!
  p = f * p; p = p + __builtin_bit_cast(float, 0x3C1D955Bu);   // ln2^4/4!
  p = f * p; p = p + __builtin_bit_cast(float, 0x3D635847u);   // ln2^3/3!
  p = f * p; p = p + __builtin_bit_cast(float, 0x3E75FDF0u);   // ln2^2/2!
  p = f * p; p = p + __builtin_bit_cast(float, 0x3F317218u);   // ln2
  p = f * p; p = p + 1.0f;
  return __builtin_ldexpf(p, (int)n);
}

// ---- descending bitonic sort of 256*E unique 64-bit keys -------------------
// Thread t holds logical entries t*E .. t*E+E-1 in registers. Stages whose
// partner is in the same thread swap registers, stages within a wave exchange
// through cross-lane shuffles, and only stages across waves go through LDS
// (`lds` holds 256*E keys). In LDS, entry e of thread t sits at e*256 + t, so
// a wave's 64-bit accesses are consecutive (no bank conflicts); a partner
// across waves, logical (t ^ m)*E + e, is entry e of thread t ^ m. The
// network's result is the unique descending order.
__device__ __forceinline__ unsigned long long shfl_xor64(unsigned long long v, int m) {
  const int lo = __shfl_xor((int)(uint32_t)v, m, 64);
  const int hi = __shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

template <int E>
__device__ __forceinline__ void bitonic_desc(unsigned long long (&x)[E], unsigned long long* lds, int tid) {
  constexpr int N = kThreads * E;
  const int lane = tid & 63;
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j >= E; j >>= 1) {
      if (j < 64 * E) {  // partner: the same register of lane ^ (j / E)
        const int m = j / E;
        const bool lower = (lane & m) == 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const unsigned long long y = shfl_xor64(x[e], m);
          const bool desc = ((tid * E + e) & k) == 0;
          const bool take_max = lower == desc;
          x[e] = take_max ? (x[e] > y ? x[e] : y) : (x[e] < y ? x[e] : y);
        }
      } else {  // partner in another wave: entry e of thread tid ^ (j / E)
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) lds[e * kThreads + tid] = x[e];
        __syncthreads();
        const int pt = tid ^ (j / E);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = tid * E + e;
          const unsigned long long y = lds[e * kThreads + pt];
          const bool take_max = ((i & j) == 0) == ((i & k) == 0);
          x[e] = take_max ? (x[e] > y ? x[e] : y) : (x[e] < y ? x[e] : y);
        }
      }
    }
#pragma unroll
    for (int jj = E / 2; jj >= 1; jj >>= 1) {  // partner in the same thread
      if (jj <= (k >> 1)) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if ((e & jj) == 0) {
            const int q = e | jj;
            const bool desc = ((tid * E + e) & k) == 0;
            const unsigned long long lo = x[e], hi = x[q];
            const bool sw = desc ? (lo < hi) : (lo > hi);
            x[e] = sw ? hi : lo;
            x[q] = sw ? lo : hi;
          }
        }
      }
    }
  }
}

// sorts keys[0 .. N) (N = 256*E, key i at keys[i]) descending, leaving the
// result in keys
template <int E>
__device__ __forceinline__ void sort_keys_desc(unsigned long long* keys, int tid) {
  unsigned long long x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = keys[tid * E + e];
  bitonic_desc<E>(x, keys, tid);
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) keys[tid * E + e] = x[e];
  __syncthreads();
}

// sort of keys[0 .. npad), npad = 256 * (1, 2, 4, 8 or 16)
__device__ __forceinline__ void sort_keys_desc_any(unsigned long long* keys, int npad, int tid) {
  switch (npad / kThreads) {
    case 1: sort_keys_desc<1>(keys, tid); break;
    case 2: sort_keys_desc<2>(keys, tid); break;
    case 4: sort_keys_desc<4>(keys, tid); break;
    case 8: sort_keys_desc<8>(keys, tid); break;
    default: sort_keys_desc<16>(keys, tid); break;
  }
}

// 64-bit sort key of a block: HRM flag, then the block score's bits (a
// non-negative float orders like its bit pattern), then the smaller index
__device__ __forceinline__ unsigned long long rank_key(bool hrm, float s, int kb) {
  return ((unsigned long long)(hrm ? 1u : 0u) << 63) | ((unsigned long long)__builtin_bit_cast(uint32_t, s) << 32) |
         (unsigned long long)(0xFFFFFFFFu - (uint32_t)kb);
}

}  // namespace cosa
