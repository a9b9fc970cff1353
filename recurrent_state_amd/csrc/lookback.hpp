// Decoupled look-back between the segments of a (sequence, head) pair, for the single-pass prefill
// kernels ("Expanding Attention", Huang, arXiv:2610.20637, Abstract: the states add across chunks, so
// prefill admits a parallel scan).  Workgroup (segment x, pair) publishes its segment's state sum
// (segment 0: already the inclusive prefix) with a flag, then the first wavefront reads the flags of
// x-1, x-2, ... (one lane each, 64 at a time) until the nearest inclusive prefix and every sum after
// it are published; the published values from there on are added in segment order (the same
// left-to-right sum whichever segments had published when, since an inclusive prefix is itself the
// left-to-right sum of the ones before it, so outputs are bitwise repeatable), and the inclusive
// prefix is published in turn.
//
// A flag is the call's tag (bits 2..63) plus kFlagAgg or kFlagIncl: a flag left by an earlier call, or
// whatever the workspace held, carries another tag and reads as not yet published.  Eager calls take a
// fresh nonzero tag each (lookback_tag); a call recorded into a HIP graph uses tag 0 and clears its
// flags first with a fill kernel.  Waits are only on lower segments of the same pair (lower linear
// workgroup ids, dispatched first), the form is used only where the whole grid is one round of one
// workgroup per CU, and every wait is bounded: after kSpinLimit polls the prefix is taken as NaN.
// Published values are stored and loaded at agent scope (the device's point of coherence), so no
// cache is written back or invalidated on either side.
#pragma once

#include <hip/hip_runtime.h>

namespace taylor {

constexpr unsigned long long kFlagAgg = 1, kFlagIncl = 2, kFlagMask = 3;
constexpr int kSpinLimit = 1 << 20;
constexpr int kFusedMaxGrid = 256;

// A fresh nonzero tag (bits 2..63) per eager single-pass call, from one process-wide counter.
unsigned long long lookback_tag();

// Whether the stream is recording a graph (or its state cannot be queried).
inline bool stream_recording(hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone;
}

// A state value that other workgroups of the same launch read (COH): stored through to the device's
// point of coherence (an agent-scope store), so that publishing needs no write-back of the XCD's L2,
// which would also flush every other workgroup's pending outputs.
template <bool COH>
__device__ __forceinline__ void put_state(float* p, float v) {
  if constexpr (COH)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// A value another workgroup of the same launch published (read from the point of coherence).
__device__ __forceinline__ float get_published(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Phase 2 of the single pass, for the E state elements of a pair (THREADS threads, element
// e = tid + THREADS i): `pre` (LDS) receives the segment's exclusive prefix (segment 0: the incoming
// state sin_p, or zero) and, for a middle segment, incl[slot] receives pre + own (own: the segment's
// sum, kept in LDS); the inclusive flag is then stored (not by the last segment, which nobody reads).
// Before this, the caller's state walk has written agg[slot] (a middle segment's sum) or incl[slot]
// (segment 0, which starts from the incoming state) and, after waiting for its stores and a barrier,
// published agg[slot] (segment 0: its inclusive flag).  `seen` is a workgroup-shared word.  Ends
// after a barrier, with the inclusive flag stored.
template <long long E, int THREADS>
__device__ __forceinline__ void lookback_prefix(float* pre, const float* own, const float* sin_p, const float* agg,
                                                float* incl, unsigned long long* flags, long long slot, int x,
                                                bool last, long long stride, unsigned long long tag,
                                                unsigned long long& seen, int tid) {
  constexpr int K = (int)((E + THREADS - 1) / THREADS);
  if (x == 0) {
    // segment 0's walk started from the incoming state, so it wrote its inclusive prefix itself; all
    // loads are issued before the first store (a load between stores would wait for each of them)
    float t[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const long long e = tid + (long long)THREADS * i;
      t[i] = sin_p && e < E ? sin_p[e] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const long long e = tid + (long long)THREADS * i;
      if (e < E) pre[e] = t[i];
    }
  } else {
    if (tid < 64) {
      // lane t reads the flag of slot base - t (segments x-1, x-2, ... of this pair, 64 at a time);
      // done once the nearest inclusive flag and every flag above it carry this call's tag
      const int t = tid;
      const long long lo = slot - x;  // segment 0 of this pair
      long long base = slot - 1, j0 = -1;
      for (int spin = 0;; ++spin) {
        const long long j = base - t;
        const bool in = j >= lo;
        const unsigned long long f = in ? __hip_atomic_load(flags + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
        const bool pub = in && (f & ~kFlagMask) == tag && (f & kFlagMask) != 0;
        const unsigned long long mpub = __ballot(pub), minc = __ballot(pub && (f & kFlagMask) == kFlagIncl),
                                 min_ = __ballot(in);
        if (minc != 0) {
          const int t0 = __builtin_ctzll(minc);
          const unsigned long long above = (1ull << t0) - 1;  // lanes nearer than the inclusive one
          if ((mpub & above) == above) {
            j0 = base - t0;
            break;
          }
        } else if (mpub == min_ && base - 64 >= lo) {
          base -= 64;  // a whole window of published sums: the inclusive prefix lies further back
          spin = 0;
          continue;
        }
        if (spin >= kSpinLimit) break;  // never published: give up (j0 = -1)
        __builtin_amdgcn_s_sleep(1);
      }
      if (t == 0) seen = (unsigned long long)j0;
    }
    __syncthreads();
    const long long j0 = (long long)seen;
    float acc[K];
    const float* first = incl + (j0 < 0 ? slot : j0) * stride;  // (not read when j0 < 0)
    // the inclusive prefix and up to three published sums after it: all loads issued before the
    // first add, then added in segment order
    long long m = j0 + 1;
    {
      const int cnt = j0 < 0 ? 0 : (int)min(3LL, slot - m);
      float t[3][K];
#pragma unroll
      for (int i = 0; i < K; ++i) {
        const long long e = tid + (long long)THREADS * i;
        acc[i] = j0 < 0 ? __builtin_nanf("") : (e < E ? get_published(first + e) : 0.f);
      }
#pragma unroll
      for (int u = 0; u < 3; ++u)
#pragma unroll
        for (int i = 0; i < K; ++i) {
          const long long e = tid + (long long)THREADS * i;
          t[u][i] = (u < cnt && e < E) ? get_published(agg + (m + u) * stride + e) : 0.f;
        }
#pragma unroll
      for (int u = 0; u < 3; ++u)
        if (u < cnt)
#pragma unroll
          for (int i = 0; i < K; ++i) acc[i] += t[u][i];
      m += cnt;
    }
    // further sums, three at a time (more than four segments per pair)
    for (; j0 >= 0 && m < slot; m += 3) {
      const int cnt = (int)min(3LL, slot - m);
      float t[3][K];
#pragma unroll
      for (int u = 0; u < 3; ++u)
#pragma unroll
        for (int i = 0; i < K; ++i) {
          const long long e = tid + (long long)THREADS * i;
          t[u][i] = (u < cnt && e < E) ? get_published(agg + (m + u) * stride + e) : 0.f;
        }
#pragma unroll
      for (int u = 0; u < 3; ++u)
        if (u < cnt)
#pragma unroll
          for (int i = 0; i < K; ++i) acc[i] += t[u][i];  // in segment order
    }
    float* inc = incl + slot * stride;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const long long e = tid + (long long)THREADS * i;
      if (e < E) {
        pre[e] = acc[i];
        if (!last) put_state<true>(inc + e, acc[i] + own[e]);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores acknowledged
  __syncthreads();
  if (x > 0 && !last && tid == 0)  // (segment 0 published its flag after its walk)
    __hip_atomic_store(flags + slot, tag | kFlagIncl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace taylor
