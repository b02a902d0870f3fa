// device_common.hpp — small device helpers shared by the gfx950 kernels:
// vector types, position searches, the cross-half-wave exchange, and the
// two-partial merge used both by the partial-attention epilogue and by the
// standalone merge kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

#define CPATTN_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }

// First index in the ascending array a[0, n) with a[idx] > x.
__device__ __forceinline__ int64_t upper_bound_i32(const int32_t* a, int64_t n, int32_t x) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    int64_t mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// First index in the ascending array a[0, n) with a[idx] >= x.
__device__ __forceinline__ int64_t lower_bound_i32(const int32_t* a, int64_t n, int32_t x) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    int64_t mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Wave-cooperative upper_bound: the first index of the ascending a[0, n) whose
// value exceeds x. Every lane of the wave must be active and pass the same
// arguments; the result is the same in every lane. Each round probes the last
// element of up to 64 equal segments of the remaining range with one gather
// and keeps the segment holding the boundary, so a search over n elements
// takes about log64(n) + 1 dependent loads instead of log2(n).
struct WaveSearch {
  int lo, hi;  // the answer lies in [lo, hi]
  int64_t step;
  // this lane's probe: the last element of segment `lane` of [lo, hi)
  __device__ __forceinline__ int probe_index(int lane, bool& probe) {
    step = ((int64_t)(hi - lo) + 63) >> 6;
    const int64_t first = (int64_t)lo + lane * step;
    probe = first < hi;
    return probe ? (int)(imin64(first + step, (int64_t)hi) - 1) : lo;
  }
  // Segments whose last element is <= x lie wholly at or below x (the array
  // is ascending), so they are a prefix; the boundary is in the next one.
  __device__ __forceinline__ void narrow(bool le) {
    const int c = __builtin_popcountll(__builtin_amdgcn_ballot_w64(le));
    const int64_t seg = (int64_t)lo + c * step;
    if (seg >= hi) {
      lo = hi;
    } else {
      hi = (int)(imin64(seg + step, (int64_t)hi) - 1);  // that segment's last element exceeds x
      lo = (int)seg;
    }
  }
};

__device__ __forceinline__ int wave_upper_bound(const int32_t* a, int n, int32_t x) {
  const int lane = threadIdx.x & 63;
  WaveSearch s{0, n, 0};
  while (s.lo < s.hi) {
    bool probe;
    const int i = s.probe_index(lane, probe);
    s.narrow(probe && a[i] <= x);
  }
  return s.lo;
}

// N wave-uniform upper bounds, search i in the ascending a[i][0, n[i]) for
// x[i], all searched together so that their rounds' loads overlap.
template <int N>
__device__ __forceinline__ void wave_upper_bounds(const int32_t* const (&a)[N], const int (&n)[N],
                                                  const int32_t (&x)[N], int (&r)[N]) {
  const int lane = threadIdx.x & 63;
  WaveSearch s[N];
#pragma unroll
  for (int i = 0; i < N; ++i) s[i] = WaveSearch{0, n[i], 0};
  for (;;) {
    bool any = false;
#pragma unroll
    for (int i = 0; i < N; ++i) any = any || s[i].lo < s[i].hi;
    if (!any) break;
    bool act[N], pr[N];
    int32_t v[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      act[i] = s[i].lo < s[i].hi;
      pr[i] = false;
      const int idx = act[i] ? s[i].probe_index(lane, pr[i]) : 0;
      v[i] = pr[i] ? a[i][idx] : 0;
    }
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (act[i]) s[i].narrow(pr[i] && v[i] <= x[i]);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) r[i] = s[i].lo;
}

// Two wave-uniform upper bounds in the same array, searched together so that
// their rounds' loads overlap.
__device__ __forceinline__ void wave_upper_bound2(const int32_t* a, int n, int32_t x1, int32_t x2, int& r1,
                                                  int& r2) {
  const int lane = threadIdx.x & 63;
  WaveSearch s1{0, n, 0}, s2{0, n, 0};
  while (s1.lo < s1.hi || s2.lo < s2.hi) {
    bool p1 = false, p2 = false;
    const bool a1 = s1.lo < s1.hi, a2 = s2.lo < s2.hi;
    const int i1 = a1 ? s1.probe_index(lane, p1) : 0;
    const int i2 = a2 ? s2.probe_index(lane, p2) : 0;
    const int32_t v1 = p1 ? a[i1] : 0;
    const int32_t v2 = p2 ? a[i2] : 0;
    if (a1) s1.narrow(p1 && v1 <= x1);
    if (a2) s2.narrow(p2 && v2 <= x2);
  }
  r1 = s1.lo;
  r2 = s2.lo;
}

// Start offset of the document holding global position p: the largest
// cu_seqlens entry <= p (cu_seqlens is ascending, cu_seqlens[0] == 0).
__device__ __forceinline__ int32_t doc_start(const int32_t* cu_seqlens, int32_t n_seqs, int32_t p) {
  int64_t idx = upper_bound_i32(cu_seqlens, (int64_t)n_seqs + 1, p) - 1;
  return cu_seqlens[idx < 0 ? 0 : idx];
}

// End of the document holding position p: the first offset > p (INT32_MAX
// past the last one).
__device__ __forceinline__ int32_t doc_end(const int32_t* cu_seqlens, int32_t n_seqs, int32_t p) {
  const int64_t idx = upper_bound_i32(cu_seqlens, (int64_t)n_seqs + 1, p);
  return idx <= n_seqs ? cu_seqlens[idx] : 0x7FFFFFFF;
}

// v_permlane32_swap exchanges the upper half-wave of its first operand with
// the lower half-wave of its second. Passing the same value twice leaves, in
// every lane, one result equal to the lane's own value and the other equal to
// the value of lane ^ 32, so a symmetric reduction needs no lane test.
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                            false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                            false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Merge weights of two partial results with natural-log normalisers la, lb:
// L = ln(e^la + e^lb), wa = e^(la-L), wb = e^(lb-L). A -inf side gets weight
// exactly 0 and the other side exactly 1; both -inf gives L = -inf, w = 0.
__device__ __forceinline__ void merge_weights(float la, float lb, float& wa, float& wb, float& L) {
  float mx = fmaxf(la, lb);
  if (mx == neg_inf()) {
    wa = 0.f; wb = 0.f; L = neg_inf();
    return;
  }
  float ea = __builtin_amdgcn_exp2f((la - mx) * kLog2e);   // one of ea, eb is exactly 1
  float eb = __builtin_amdgcn_exp2f((lb - mx) * kLog2e);
  float s = ea + eb;
  float inv = 1.0f / s;
  L = mx + __builtin_amdgcn_logf(s) * kLn2;
  wa = ea * inv;
  wb = eb * inv;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Round-to-nearest-even float32 -> bf16 bit pattern (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t f = {lo, hi};
  bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

}  // namespace cpattn
