// Device pieces shared by the decode kernels of both block images (64x128
// and 64x64 blocks): kernel arguments, the split-K hand-off, global->LDS
// loads, vmcnt waits, the subnormal-operand geometry of a bit plane and ring
// arithmetic.  Internal linkage: each source that includes this gets its own
// copy.
#pragma once
#include "device.h"
#include "internal.h"
#include "layout.h"

namespace gbb {

namespace {

struct DecodeArgs {
  const uint8_t* bits;
  const uint32_t* offs;
  const uint32_t* sz;
  const uint8_t* codes;
  const _Float16* x;
  _Float16* y;
  uint64_t* acc;   // split-K fixed-point accumulators [M][N] (zero between calls)
  float* facc;     // split-K overflow accumulators [M][N] (zero between calls)
  float* part;     // two-row kernel: K-segment partials [nseg][M][N] (zero between calls)
  int N, K, M, nbr, nbc, seg_cols, nseg;
};

// Split-K hand-off of one output element idx (of y and the accumulators).
// The 64-bit word is  v * 2^12 + poisoned * 2^6 + count  with v the sum of
// the partials rounded to multiples of 2^-28 (|partial| < 2^18, so 32 of
// them fit the 52-bit field exactly), count the contributions so far and
// poisoned those that went through the fp32 accumulator instead.  Every
// lane of the wave calls this together; `active` lanes contribute.
constexpr float kFixScale = 268435456.0f;   // 2^28
constexpr float kFixLimit = 262144.0f;      // 2^18
__device__ __forceinline__ void splitk_publish(const DecodeArgs& a, size_t idx, float p, bool active) {
  const bool big = active && !(__builtin_fabsf(p) < kFixLimit);   // also NaN
  uint64_t word = 1;
  if (big) {
    __hip_atomic_fetch_add(a.facc + idx, p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    word += 64;
  } else {
    word += uint64_t(int64_t(__builtin_rintf(p * kFixScale))) << 12;
  }
  // the overflow adds are visible before the counts that announce them
  if (__builtin_amdgcn_ballot_w64(big)) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  if (!active) return;
  const uint64_t tot = __hip_atomic_fetch_add(a.acc + idx, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + word;
  if (int(tot & 63) != a.nseg) return;
  // last contribution: the word holds the complete sum
  float r = float(double(int64_t(tot) >> 12) * (1.0 / 268435456.0));
  if ((tot >> 6) & 63) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    r += __hip_atomic_load(a.facc + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.facc + idx, 0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  a.y[idx] = (_Float16)r;
  __hip_atomic_store(a.acc + idx, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The same hand-off for P output elements per lane.  Every element's
// counting atomic is issued before any of their results is awaited, so the
// wave waits for one round trip to the memory-side atomics instead of P in
// a row (P = 16 for 32 tokens over two block rows).  Per element the
// arithmetic, the order of the overflow add before its count, and the last
// contribution's completion are those of splitk_publish.  Element 0 must be
// active whenever any element of the lane is.
template <int P>
__device__ __forceinline__ void splitk_publish_all(const DecodeArgs& a, const size_t (&idx)[P], const float (&p)[P],
                                                   const bool (&active)[P]) {
  uint64_t word[P];
  bool anybig = false;
#pragma unroll
  for (int k = 0; k < P; ++k) {
    const bool big = active[k] && !(__builtin_fabsf(p[k]) < kFixLimit);   // also NaN
    word[k] = 1;
    if (big) {
      __hip_atomic_fetch_add(a.facc + idx[k], p[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      word[k] += 64;
    } else {
      word[k] += uint64_t(int64_t(__builtin_rintf(p[k] * kFixScale))) << 12;
    }
    anybig = anybig || big;
  }
  if (__builtin_amdgcn_ballot_w64(anybig)) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  if (!active[0]) return;
  // An inactive element adds 0 to the lane's own element 0: with no branch
  // around each atomic, nothing makes the compiler await one before issuing
  // the next, and the extra adds meet no other lane's.
  uint64_t tot[P];
#pragma unroll
  for (int k = 0; k < P; ++k) {
    const uint64_t w = active[k] ? word[k] : 0;
    tot[k] = __hip_atomic_fetch_add(a.acc + (active[k] ? idx[k] : idx[0]), w, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) + w;
  }
#pragma unroll
  for (int k = 0; k < P; ++k) {
    if (!active[k] || int(tot[k] & 63) != a.nseg) continue;
    // last contribution: the word holds the complete sum
    float r = float(double(int64_t(tot[k]) >> 12) * (1.0 / 268435456.0));
    if ((tot[k] >> 6) & 63) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      r += __hip_atomic_load(a.facc + idx[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.facc + idx[k], 0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    a.y[idx[k]] = (_Float16)r;
    __hip_atomic_store(a.acc + idx[k], uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Default ring slots per wave (a power of two): a block takes 1 + nx + b
// slots (nx = ceil(M / 4) activation slots of four tokens each).  The
// launches for M <= 16 pass smaller rings (kRing8, kRing16) instead.
template <int MT>
struct Ring {
  static constexpr int kSlots = MT == 1 ? 16 : 32;
  static constexpr uint32_t kMask = kSlots * 1024 - 1;  // ring byte offsets wrap with this
  static_assert(1 + 4 * MT + 8 <= kSlots, "a block's records fit in the ring");
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const lds_void*)p));
}

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt left alone (gfx9 encoding), and
// a compiler barrier so no LDS read is moved above it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// s_waitcnt lgkmcnt(0): every LDS read of this wave has returned its data.
__device__ __forceinline__ void wait_lds() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until at most n (uniform, n >= 0) of this wave's loads are in
// flight; n is rounded down to a few levels, which only waits a little longer.
__device__ __forceinline__ void wait_vmcnt_at_most(int n) {
  if (n < 4) {
    if (n < 2) {
      if (n < 1) wait_vmcnt<0>(); else wait_vmcnt<1>();
    } else {
      if (n < 3) wait_vmcnt<2>(); else wait_vmcnt<3>();
    }
  } else if (n < 12) {
    if (n < 8) {
      if (n < 6) wait_vmcnt<4>(); else wait_vmcnt<6>();
    } else {
      if (n < 10) wait_vmcnt<8>(); else wait_vmcnt<10>();
    }
  } else {
    if (n < 16) wait_vmcnt<12>(); else wait_vmcnt<16>();
  }
}

// One global->LDS load of 16 or 4 bytes per lane from sbase + voff: lane l's
// bytes land at LDS address ring + off + l * size.  Inline assembly with no
// output registers (the data goes to LDS), so the compiler does not track it:
// every read of the ring is preceded by an explicit vmcnt wait instead, and a
// slot is only refilled after the reads of its previous record completed.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t ring, uint32_t off) {
  asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(ring), "s"(off)
               : "memory", "m0", "scc");
}
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t ring, uint32_t off) {
  asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(ring), "s"(off)
               : "memory", "m0", "scc");
}
// The same loads marked non-temporal, for the streams a launch reads exactly
// once (codes, scale/zero records): their lines are the first the caches give
// up, so the small data every launch revisits (bitwidths, offsets,
// activations) stays cached across the launches of a decoder step.  Measured
// on the Llama-3-8B layer set: 9.3 -> 8.6 us per launch.
__device__ __forceinline__ void dma16_once(const void* sbase, uint32_t voff, uint32_t ring, uint32_t off) {
  asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(ring), "s"(off)
               : "memory", "m0", "scc");
}
__device__ __forceinline__ void dma4_once(const void* sbase, uint32_t voff, uint32_t ring, uint32_t off) {
  asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dword %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(ring), "s"(off)
               : "memory", "m0", "scc");
}

template <int W>
struct PlaneGeom {
  static constexpr int NP = 16 / W;
  static constexpr int Q = W == 4 ? 2 : 4;
  static constexpr int off(int rt) { return W * (rt % Q); }  // o of row tile rt
};

// 2^e as a float, e a small compile-time integer.
__device__ __forceinline__ constexpr float pow2(int e) {
  return e >= 0 ? float(1ull << e) : 1.0f / float(1ull << -e);
}

// Byte offset off (below 2 RS slots) wrapped into a ring of RS slots of SB
// bytes (1 KiB, or 512 B for 64x64 blocks).
template <int RS, uint32_t SB = 1024>
__device__ __forceinline__ uint32_t wrap(uint32_t off) {
  if constexpr ((RS & (RS - 1)) == 0)
    return off & (RS * SB - 1u);
  else
    return off >= RS * SB ? off - RS * SB : off;
}

// Wait until at most n (uniform, n >= 0) loads are in flight, rounded down to
// 8, 4 or 0: two compares instead of a decision tree, at the price of waiting
// for a few later loads.
__device__ __forceinline__ void wait_vmcnt_coarse(int n) {
  if (n >= 8)
    wait_vmcnt<8>();
  else if (n >= 4)
    wait_vmcnt<4>();
  else
    wait_vmcnt<0>();
}

}  // namespace

}  // namespace gbb
