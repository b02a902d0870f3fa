// api.cpp — the C ABI declared in include/cpattn.h: argument validation
// (always before any HIP call), the host-side index builder, and the kernel
// launches. No allocation, no state kept between calls.
#include "cpattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kernels.hpp"
#include "kernels_bwd.hpp"

static_assert(CPATTN_VARLEN_PLAN_RECORD == cpattn::kPlanRec, "plan record size");

namespace {

thread_local char g_err[512] = "";

cpattn_status fail(cpattn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

cpattn_status ok() {
  g_err[0] = '\0';
  return CPATTN_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

bool validate_env() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("CPATTN_VALIDATE");
    v = (e && e[0] == '1') ? 1 : 0;
  }
  return v == 1;
}

// Optional O(n) check that device positions ascend (synchronises `stream`).
cpattn_status check_sorted_device(const int32_t* dptr, int64_t n, const char* name, hipStream_t stream) {
  if (n <= 1) return CPATTN_OK;
  std::vector<int32_t> h((size_t)n);
  hipError_t e = hipMemcpyAsync(h.data(), dptr, sizeof(int32_t) * (size_t)n, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(CPATTN_ERR_HIP, "reading %s for validation: %s", name, hipGetErrorString(e));
  for (int64_t i = 1; i < n; ++i)
    if (h[(size_t)i] < h[(size_t)i - 1])
      return fail(CPATTN_ERR_UNSORTED, "%s is not ascending at index %lld", name, (long long)i);
  return CPATTN_OK;
}

// Optional check that a device plan is the one cpattn_varlen_plan makes for
// these positions (synchronises `stream`; copies the positions and the plan).
cpattn_status check_plan_device(const int32_t* dplan, const int32_t* q_pos, int64_t lq, const int32_t* k_pos,
                                int64_t lk, const int32_t* cu_seqlens, int32_t n_seqs, int32_t hq, int32_t hkv,
                                int in_bf16, int32_t head_dim, hipStream_t stream) {
  const int64_t n = cpattn::partial_workgroups(lq, hq, hkv) * cpattn::kPlanRec;
  std::vector<int32_t> plan((size_t)n), qp((size_t)lq), kp((size_t)lk), cu((size_t)n_seqs + 1), want((size_t)n);
  hipError_t e = hipMemcpyAsync(plan.data(), dplan, sizeof(int32_t) * (size_t)n, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(qp.data(), q_pos, sizeof(int32_t) * (size_t)lq, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess && lk > 0)
    e = hipMemcpyAsync(kp.data(), k_pos, sizeof(int32_t) * (size_t)lk, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(cu.data(), cu_seqlens, sizeof(int32_t) * ((size_t)n_seqs + 1), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(CPATTN_ERR_HIP, "reading the plan for validation: %s", hipGetErrorString(e));
  cpattn::plan_varlen(qp.data(), lq, kp.data(), lk, cu.data(), n_seqs, hq, hkv, in_bf16, head_dim, want.data());
  for (int64_t i = 0; i < n; ++i)
    if (plan[(size_t)i] != want[(size_t)i])
      return fail(CPATTN_ERR_RANGE, "the plan differs from cpattn_varlen_plan's at entry %lld (%d, expected %d)",
                  (long long)i, plan[(size_t)i], want[(size_t)i]);
  return CPATTN_OK;
}

size_t dsize(cpattn_dtype t) { return t == CPATTN_BF16 ? 2 : 4; }

cpattn_status check_partial_args(const void* q, const void* k, const void* v, cpattn_dtype in_dtype, int64_t lq,
                                 int64_t lk, int32_t hq, int32_t hkv, int32_t head_dim, const int32_t* q_pos,
                                 const int32_t* k_pos, int32_t causal, void* o, cpattn_dtype o_dtype,
                                 const float* lse, int32_t accumulate) {
  // zero-sized operands may be NULL (an empty tensor has no storage)
  if (lq != 0 && (!q || !o || !lse)) return fail(CPATTN_ERR_NULL, "q, o and lse must be non-NULL");
  if (lk != 0 && (!k || !v)) return fail(CPATTN_ERR_NULL, "k and v must be non-NULL");
  if (causal != 0 && causal != 1) return fail(CPATTN_ERR_RANGE, "causal must be 0 or 1, got %d", causal);
  if (accumulate != 0 && accumulate != 1) return fail(CPATTN_ERR_RANGE, "accumulate must be 0 or 1, got %d", accumulate);
  if (causal && ((lq != 0 && !q_pos) || (lk != 0 && !k_pos)))
    return fail(CPATTN_ERR_NULL, "q_pos and k_pos are required when causal");
  if (in_dtype != CPATTN_BF16 && in_dtype != CPATTN_F32) return fail(CPATTN_ERR_DTYPE, "in_dtype %d unsupported", (int)in_dtype);
  if (o_dtype != CPATTN_BF16 && o_dtype != CPATTN_F32) return fail(CPATTN_ERR_DTYPE, "o_dtype %d unsupported", (int)o_dtype);
  if (in_dtype == CPATTN_F32 && o_dtype != CPATTN_F32)
    return fail(CPATTN_ERR_DTYPE, "float32 inputs need a float32 output");
  if (head_dim != 64 && head_dim != 128) return fail(CPATTN_ERR_SHAPE, "head_dim must be 64 or 128, got %d", head_dim);
  if (hq < 1 || hkv < 1) return fail(CPATTN_ERR_SHAPE, "hq and hkv must be >= 1 (hq=%d hkv=%d)", hq, hkv);
  if (hq % hkv) return fail(CPATTN_ERR_SHAPE, "hq (%d) must be a multiple of hkv (%d)", hq, hkv);
  if (lq < 0 || lk < 0) return fail(CPATTN_ERR_SHAPE, "lq and lk must be >= 0");
  if (lq >= (int64_t)1 << 31 || lk >= (int64_t)1 << 31) return fail(CPATTN_ERR_SHAPE, "lq and lk must be < 2^31");
  if ((int64_t)hq * head_dim * lq >= (int64_t)1 << 40) return fail(CPATTN_ERR_SHAPE, "q is too large");
  // the kernel addresses a 64-key tile of one KV head with 32-bit buffer offsets
  if ((int64_t)hkv * head_dim * (int64_t)dsize(in_dtype) * 64 >= (int64_t)1 << 31)
    return fail(CPATTN_ERR_SHAPE, "hkv * head_dim too large (a 64-key KV tile must span < 2 GiB)");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(CPATTN_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
  if (!aligned(lse, 4) || (q_pos && !aligned(q_pos, 4)) || (k_pos && !aligned(k_pos, 4)))
    return fail(CPATTN_ERR_ALIGN, "lse and positions must be 4-byte aligned");
  const size_t nq = (size_t)lq * hq * head_dim * dsize(in_dtype);
  const size_t nk = (size_t)lk * hkv * head_dim * dsize(in_dtype);
  const size_t no = (size_t)lq * hq * head_dim * dsize(o_dtype);
  const size_t nl = (size_t)lq * hq * sizeof(float);
  if (overlaps(o, no, q, nq) || overlaps(o, no, k, nk) || overlaps(o, no, v, nk) || overlaps(lse, nl, q, nq) ||
      overlaps(lse, nl, k, nk) || overlaps(lse, nl, v, nk) || overlaps(o, no, lse, nl))
    return fail(CPATTN_ERR_ALIAS, "outputs must not overlap inputs or each other");
  return CPATTN_OK;
}

cpattn_status enqueue_partial(const void* q, const void* k, const void* v, cpattn_dtype in_dtype, int64_t lq,
                              int64_t lk, int32_t hq, int32_t hkv, int32_t head_dim, const int32_t* q_pos,
                              const int32_t* k_pos, const int32_t* cu_seqlens, int32_t n_seqs, int32_t causal,
                              float softmax_scale, void* o, cpattn_dtype o_dtype, float* lse, int32_t accumulate,
                              void* stream, const int32_t* plan = nullptr) {
  hipStream_t s = (hipStream_t)stream;
  if (validate_env() && causal) {
    cpattn_status st = check_sorted_device(q_pos, lq, "q_pos", s);
    if (st == CPATTN_OK) st = check_sorted_device(k_pos, lk, "k_pos", s);
    if (st == CPATTN_OK && cu_seqlens) st = check_sorted_device(cu_seqlens, (int64_t)n_seqs + 1, "cu_seqlens", s);
    if (st == CPATTN_OK && plan)
      st = check_plan_device(plan, q_pos, lq, k_pos, lk, cu_seqlens, n_seqs, hq, hkv, in_dtype == CPATTN_BF16,
                             head_dim, s);
    if (st != CPATTN_OK) return st;
  }
  if (lq == 0) return ok();
  cpattn::PartialParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.q_pos = q_pos; p.k_pos = k_pos; p.cu_seqlens = cu_seqlens; p.n_seqs = n_seqs;
  p.lq = lq; p.lk = lk; p.hq = hq; p.hkv = hkv;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  p.scale_log2 = scale * 1.4426950408889634f;
  p.causal = causal; p.accumulate = accumulate;
  p.wg_plan = plan;
  hipError_t e = cpattn::launch_partial(p, in_dtype == CPATTN_BF16, o_dtype == CPATTN_BF16, head_dim,
                                        cu_seqlens != nullptr, s);
  if (e != hipSuccess) return fail(CPATTN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

cpattn_status enqueue_partial_multi(const void* q, const void* const* k_blocks, const void* const* v_blocks,
                                    cpattn_dtype in_dtype, int64_t lq, const int64_t* lk_blocks, int32_t n_blocks,
                                    int32_t hq, int32_t hkv, int32_t head_dim, const int32_t* q_pos,
                                    const int32_t* const* k_pos_blocks, const int32_t* cu_seqlens, int32_t n_seqs,
                                    int32_t causal, float softmax_scale, void* o, cpattn_dtype o_dtype, float* lse,
                                    int32_t accumulate, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (validate_env() && causal) {
    cpattn_status st = check_sorted_device(q_pos, lq, "q_pos", s);
    for (int32_t b = 0; b < n_blocks && st == CPATTN_OK; ++b)
      st = check_sorted_device(k_pos_blocks[b], lk_blocks[b], "k_pos", s);
    if (st == CPATTN_OK && cu_seqlens) st = check_sorted_device(cu_seqlens, (int64_t)n_seqs + 1, "cu_seqlens", s);
    if (st != CPATTN_OK) return st;
  }
  if (lq == 0) return ok();
  cpattn::PartialParams p{};
  p.q = q; p.k = k_blocks[0]; p.v = v_blocks[0]; p.o = o; p.lse = lse;
  p.q_pos = q_pos; p.k_pos = k_pos_blocks[0]; p.cu_seqlens = cu_seqlens; p.n_seqs = n_seqs;
  p.lq = lq; p.lk = lk_blocks[0]; p.hq = hq; p.hkv = hkv;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  p.scale_log2 = scale * 1.4426950408889634f;
  p.causal = causal; p.accumulate = accumulate;
  cpattn::BlockTable bt{};
  bt.n = n_blocks;
  for (int32_t b = 0; b < n_blocks; ++b) {
    bt.k[b] = k_blocks[b];
    bt.v[b] = v_blocks[b];
    bt.k_pos[b] = k_pos_blocks[b];
    bt.lk[b] = (int32_t)lk_blocks[b];
  }
  hipError_t e = cpattn::launch_partial_multi(p, bt, in_dtype == CPATTN_BF16, o_dtype == CPATTN_BF16, head_dim,
                                              cu_seqlens != nullptr, s);
  if (e != hipSuccess) return fail(CPATTN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int cpattn_version(void) { return 100; }

const char* cpattn_last_error(void) { return g_err; }

cpattn_status cpattn_zigzag_index(int64_t total_len, int32_t cp_size, int32_t rank, cpattn_layout layout,
                                  const int32_t* cu_seqlens, int32_t n_seqs, int32_t* out_pos,
                                  int32_t* out_seq_start) {
  if (!out_pos) return fail(CPATTN_ERR_NULL, "out_pos must be non-NULL");
  if (cp_size < 1) return fail(CPATTN_ERR_RANGE, "cp_size must be >= 1, got %d", cp_size);
  if (rank < 0 || rank >= cp_size) return fail(CPATTN_ERR_RANGE, "rank %d outside [0, %d)", rank, cp_size);
  if (layout != CPATTN_CONTIGUOUS && layout != CPATTN_ZIGZAG && layout != CPATTN_STRIPED)
    return fail(CPATTN_ERR_RANGE, "unknown layout %d", (int)layout);
  if (total_len < 0 || total_len >= ((int64_t)1 << 31)) return fail(CPATTN_ERR_SHAPE, "total_len must be in [0, 2^31)");
  const int64_t unit = layout == CPATTN_ZIGZAG ? 2 * (int64_t)cp_size : cp_size;
  // documents: [start_t, end_t); one document when cu_seqlens is NULL
  int32_t nd = 1;
  if (cu_seqlens) {
    if (n_seqs < 1) return fail(CPATTN_ERR_SHAPE, "n_seqs must be >= 1 with cu_seqlens");
    if (cu_seqlens[0] != 0) return fail(CPATTN_ERR_SHAPE, "cu_seqlens[0] must be 0");
    if (cu_seqlens[n_seqs] != total_len)
      return fail(CPATTN_ERR_SHAPE, "cu_seqlens[n_seqs] (%d) must equal total_len (%lld)", cu_seqlens[n_seqs],
                  (long long)total_len);
    for (int32_t t = 0; t < n_seqs; ++t) {
      if (cu_seqlens[t + 1] < cu_seqlens[t]) return fail(CPATTN_ERR_UNSORTED, "cu_seqlens must ascend");
      if ((cu_seqlens[t + 1] - cu_seqlens[t]) % unit)
        return fail(CPATTN_ERR_SHAPE, "document %d length %d is not a multiple of %lld", t,
                    cu_seqlens[t + 1] - cu_seqlens[t], (long long)unit);
    }
    nd = n_seqs;
  } else if (total_len % unit) {
    return fail(CPATTN_ERR_SHAPE, "total_len %lld is not a multiple of %lld", (long long)total_len, (long long)unit);
  }
  int64_t n = 0;
  for (int32_t t = 0; t < nd; ++t) {
    const int64_t s0 = cu_seqlens ? cu_seqlens[t] : 0;
    const int64_t len = cu_seqlens ? (int64_t)cu_seqlens[t + 1] - s0 : total_len;
    const int64_t per = len / cp_size;  // tokens of this document on each rank
    for (int64_t u = 0; u < per; ++u) {
      int64_t pos;
      if (layout == CPATTN_CONTIGUOUS) {
        pos = (int64_t)rank * per + u;
      } else if (layout == CPATTN_STRIPED) {
        pos = u * cp_size + rank;
      } else {
        const int64_t c = len / (2 * (int64_t)cp_size);  // zig-zag chunk length
        pos = (u < c) ? (int64_t)rank * c + u : (int64_t)(2 * cp_size - 1 - rank) * c + (u - c);
      }
      out_pos[n] = (int32_t)(s0 + pos);
      if (out_seq_start) out_seq_start[n] = (int32_t)s0;
      ++n;
    }
  }
  return ok();
}

cpattn_status cpattn_partial(const void* q, const void* k, const void* v, cpattn_dtype in_dtype, int64_t lq,
                             int64_t lk, int32_t hq, int32_t hkv, int32_t head_dim, const int32_t* q_pos,
                             const int32_t* k_pos, int32_t causal, float softmax_scale, void* o,
                             cpattn_dtype o_dtype, float* lse, int32_t accumulate, void* stream) {
  cpattn_status st = check_partial_args(q, k, v, in_dtype, lq, lk, hq, hkv, head_dim, q_pos, k_pos, causal, o,
                                        o_dtype, lse, accumulate);
  if (st != CPATTN_OK) return st;
  if (!std::isfinite(softmax_scale)) return fail(CPATTN_ERR_RANGE, "softmax_scale must be finite");
  return enqueue_partial(q, k, v, in_dtype, lq, lk, hq, hkv, head_dim, q_pos, k_pos, nullptr, 0, causal,
                         softmax_scale, o, o_dtype, lse, accumulate, stream);
}

cpattn_status cpattn_varlen_partial(const void* q, const void* k, const void* v, cpattn_dtype in_dtype, int64_t lq,
                                    int64_t lk, int32_t hq, int32_t hkv, int32_t head_dim, const int32_t* q_pos,
                                    const int32_t* k_pos, const int32_t* cu_seqlens, int32_t n_seqs,
                                    float softmax_scale, void* o, cpattn_dtype o_dtype, float* lse,
                                    int32_t accumulate, void* stream) {
  cpattn_status st = check_partial_args(q, k, v, in_dtype, lq, lk, hq, hkv, head_dim, q_pos, k_pos, 1, o, o_dtype,
                                        lse, accumulate);
  if (st != CPATTN_OK) return st;
  if (!cu_seqlens) return fail(CPATTN_ERR_NULL, "cu_seqlens must be non-NULL");
  if (!aligned(cu_seqlens, 4)) return fail(CPATTN_ERR_ALIGN, "cu_seqlens must be 4-byte aligned");
  if (n_seqs < 1) return fail(CPATTN_ERR_SHAPE, "n_seqs must be >= 1, got %d", n_seqs);
  if (!std::isfinite(softmax_scale)) return fail(CPATTN_ERR_RANGE, "softmax_scale must be finite");
  return enqueue_partial(q, k, v, in_dtype, lq, lk, hq, hkv, head_dim, q_pos, k_pos, cu_seqlens, n_seqs, 1,
                         softmax_scale, o, o_dtype, lse, accumulate, stream);
}

int64_t cpattn_partial_workgroups(int64_t lq, int32_t hq, int32_t hkv) {
  if (lq < 0 || hq < 1 || hkv < 1 || hq % hkv != 0) return -1;
  return cpattn::partial_workgroups(lq, hq, hkv);
}

cpattn_status cpattn_varlen_plan(const int32_t* q_pos, int64_t lq, const int32_t* k_pos, int64_t lk,
                                 const int32_t* cu_seqlens, int32_t n_seqs, int32_t hq, int32_t hkv,
                                 int32_t head_dim, cpattn_dtype in_dtype, int32_t* plan, int64_t plan_len) {
  if (lq < 0 || lk < 0) return fail(CPATTN_ERR_SHAPE, "lq and lk must be >= 0");
  if (lq >= (int64_t)1 << 31 || lk >= (int64_t)1 << 31) return fail(CPATTN_ERR_SHAPE, "lq and lk must be < 2^31");
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(CPATTN_ERR_SHAPE, "hq must be a positive multiple of hkv (hq=%d, hkv=%d)", hq, hkv);
  if (head_dim != 64 && head_dim != 128) return fail(CPATTN_ERR_SHAPE, "head_dim must be 64 or 128, got %d", head_dim);
  if (in_dtype != CPATTN_BF16 && in_dtype != CPATTN_F32) return fail(CPATTN_ERR_DTYPE, "in_dtype must be bf16 or float32");
  if (n_seqs < 1) return fail(CPATTN_ERR_SHAPE, "n_seqs must be >= 1, got %d", n_seqs);
  const int64_t n = cpattn::partial_workgroups(lq, hq, hkv) * CPATTN_VARLEN_PLAN_RECORD;
  if (plan_len != n) return fail(CPATTN_ERR_SHAPE, "plan_len must be %lld (the call's workgroups x %d), got %lld",
                                 (long long)n, CPATTN_VARLEN_PLAN_RECORD, (long long)plan_len);
  if (n == 0) return ok();
  if (!q_pos || !cu_seqlens || !plan || (lk > 0 && !k_pos))
    return fail(CPATTN_ERR_NULL, "q_pos, k_pos, cu_seqlens and plan must be non-NULL");
  for (int64_t i = 1; i < lq; ++i)
    if (q_pos[i] < q_pos[i - 1]) return fail(CPATTN_ERR_UNSORTED, "q_pos is not ascending at index %lld", (long long)i);
  for (int64_t i = 1; i < lk; ++i)
    if (k_pos[i] < k_pos[i - 1]) return fail(CPATTN_ERR_UNSORTED, "k_pos is not ascending at index %lld", (long long)i);
  for (int32_t i = 1; i <= n_seqs; ++i)
    if (cu_seqlens[i] < cu_seqlens[i - 1])
      return fail(CPATTN_ERR_UNSORTED, "cu_seqlens is not ascending at index %d", i);
  cpattn::plan_varlen(q_pos, lq, k_pos, lk, cu_seqlens, n_seqs, hq, hkv, in_dtype == CPATTN_BF16, head_dim, plan);
  return ok();
}

cpattn_status cpattn_varlen_partial_planned(const void* q, const void* k, const void* v, cpattn_dtype in_dtype,
                                            int64_t lq, int64_t lk, int32_t hq, int32_t hkv, int32_t head_dim,
                                            const int32_t* q_pos, const int32_t* k_pos, const int32_t* cu_seqlens,
                                            int32_t n_seqs, float softmax_scale, void* o, cpattn_dtype o_dtype,
                                            float* lse, int32_t accumulate, const int32_t* plan, int64_t plan_len,
                                            void* stream) {
  cpattn_status st = check_partial_args(q, k, v, in_dtype, lq, lk, hq, hkv, head_dim, q_pos, k_pos, 1, o, o_dtype,
                                        lse, accumulate);
  if (st != CPATTN_OK) return st;
  if (!cu_seqlens) return fail(CPATTN_ERR_NULL, "cu_seqlens must be non-NULL");
  if (!aligned(cu_seqlens, 4)) return fail(CPATTN_ERR_ALIGN, "cu_seqlens must be 4-byte aligned");
  if (n_seqs < 1) return fail(CPATTN_ERR_SHAPE, "n_seqs must be >= 1, got %d", n_seqs);
  if (!std::isfinite(softmax_scale)) return fail(CPATTN_ERR_RANGE, "softmax_scale must be finite");
  const int64_t n = cpattn::partial_workgroups(lq, hq, hkv) * CPATTN_VARLEN_PLAN_RECORD;
  if (plan_len != n) return fail(CPATTN_ERR_SHAPE, "plan_len must be %lld (the call's workgroups x %d), got %lld",
                                 (long long)n, CPATTN_VARLEN_PLAN_RECORD, (long long)plan_len);
  if (n > 0 && !plan) return fail(CPATTN_ERR_NULL, "plan must be non-NULL");
  if (!aligned(plan, 4)) return fail(CPATTN_ERR_ALIGN, "plan must be 4-byte aligned");
  return enqueue_partial(q, k, v, in_dtype, lq, lk, hq, hkv, head_dim, q_pos, k_pos, cu_seqlens, n_seqs, 1,
                         softmax_scale, o, o_dtype, lse, accumulate, stream, n > 0 ? plan : nullptr);
}

cpattn_status cpattn_partial_multi(const void* q, const void* const* k_blocks, const void* const* v_blocks,
                                   cpattn_dtype in_dtype, int64_t lq, const int64_t* lk_blocks, int32_t n_blocks,
                                   int32_t hq, int32_t hkv, int32_t head_dim, const int32_t* q_pos,
                                   const int32_t* const* k_pos_blocks, const int32_t* cu_seqlens, int32_t n_seqs,
                                   int32_t causal, float softmax_scale, void* o, cpattn_dtype o_dtype, float* lse,
                                   int32_t accumulate, void* stream) {
  if (!k_blocks || !v_blocks || !lk_blocks || !k_pos_blocks)
    return fail(CPATTN_ERR_NULL, "the block arrays must be non-NULL");
  if (n_blocks < 1 || n_blocks > cpattn::kMaxBlocks)
    return fail(CPATTN_ERR_RANGE, "n_blocks must be in [1, %d], got %d", cpattn::kMaxBlocks, n_blocks);
  if (cu_seqlens) {
    if (causal != 1) return fail(CPATTN_ERR_RANGE, "documents (cu_seqlens) need causal = 1");
    if (!aligned(cu_seqlens, 4)) return fail(CPATTN_ERR_ALIGN, "cu_seqlens must be 4-byte aligned");
    if (n_seqs < 1) return fail(CPATTN_ERR_SHAPE, "n_seqs must be >= 1, got %d", n_seqs);
  }
  for (int32_t b = 0; b < n_blocks; ++b) {
    cpattn_status st = check_partial_args(q, k_blocks[b], v_blocks[b], in_dtype, lq, lk_blocks[b], hq, hkv,
                                          head_dim, q_pos, k_pos_blocks[b], causal, o, o_dtype, lse, accumulate);
    if (st != CPATTN_OK) return st;
  }
  if (!std::isfinite(softmax_scale)) return fail(CPATTN_ERR_RANGE, "softmax_scale must be finite");
  return enqueue_partial_multi(q, k_blocks, v_blocks, in_dtype, lq, lk_blocks, n_blocks, hq, hkv, head_dim, q_pos,
                               k_pos_blocks, cu_seqlens, cu_seqlens ? n_seqs : 0, causal, softmax_scale, o, o_dtype,
                               lse, accumulate, stream);
}

cpattn_status cpattn_bwd_delta(const void* o, cpattn_dtype o_dtype, const void* dout, cpattn_dtype dout_dtype,
                               int64_t lq, int32_t hq, int32_t head_dim, float* delta, void* stream) {
  if (lq != 0 && (!o || !dout || !delta)) return fail(CPATTN_ERR_NULL, "o, dout and delta must be non-NULL");
  if ((o_dtype != CPATTN_BF16 && o_dtype != CPATTN_F32) || (dout_dtype != CPATTN_BF16 && dout_dtype != CPATTN_F32))
    return fail(CPATTN_ERR_DTYPE, "o_dtype and dout_dtype must be bf16 or float32");
  if (head_dim != 64 && head_dim != 128) return fail(CPATTN_ERR_SHAPE, "head_dim must be 64 or 128, got %d", head_dim);
  if (lq < 0 || hq < 1) return fail(CPATTN_ERR_SHAPE, "lq must be >= 0 and hq >= 1");
  if (lq >= (int64_t)1 << 31) return fail(CPATTN_ERR_SHAPE, "lq must be < 2^31");
  if (!aligned(o, 16) || !aligned(dout, 16)) return fail(CPATTN_ERR_ALIGN, "o and dout must be 16-byte aligned");
  if (!aligned(delta, 4)) return fail(CPATTN_ERR_ALIGN, "delta must be 4-byte aligned");
  const size_t nd = (size_t)lq * hq * sizeof(float);
  if (overlaps(delta, nd, o, (size_t)lq * hq * head_dim * dsize(o_dtype)) ||
      overlaps(delta, nd, dout, (size_t)lq * hq * head_dim * dsize(dout_dtype)))
    return fail(CPATTN_ERR_ALIAS, "delta must not overlap o or dout");
  if (lq == 0) return ok();
  hipError_t e = cpattn::launch_bwd_delta(o, o_dtype == CPATTN_BF16, dout, dout_dtype == CPATTN_BF16, lq, hq,
                                          head_dim, delta, (hipStream_t)stream);
  if (e != hipSuccess) return fail(CPATTN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Everything cpattn_partial_bwd checks before it enqueues (one block's arguments).
static cpattn_status check_bwd_args(const void* q, const void* k, const void* v, const void* dout,
                                    cpattn_dtype in_dtype, int64_t lq, int64_t lk, int32_t hq, int32_t hkv,
                                    int32_t head_dim, const int32_t* q_pos, const int32_t* k_pos, int32_t causal,
                                    const int32_t* cu_seqlens, int32_t n_seqs, float softmax_scale, const float* lse,
                                    const float* delta, float* dq, int32_t accumulate_dq, float* dk, float* dv,
                                    int32_t accumulate_dkv, hipStream_t s) {
  if (lq != 0 && (!q || !dout || !lse || !delta || !dq))
    return fail(CPATTN_ERR_NULL, "q, dout, lse, delta and dq must be non-NULL");
  if (lk != 0 && (!k || !v || !dk || !dv)) return fail(CPATTN_ERR_NULL, "k, v, dk and dv must be non-NULL");
  if (causal != 0 && causal != 1) return fail(CPATTN_ERR_RANGE, "causal must be 0 or 1, got %d", causal);
  if ((accumulate_dq != 0 && accumulate_dq != 1) || (accumulate_dkv != 0 && accumulate_dkv != 1))
    return fail(CPATTN_ERR_RANGE, "accumulate_dq and accumulate_dkv must be 0 or 1");
  if (causal && ((lq != 0 && !q_pos) || (lk != 0 && !k_pos)))
    return fail(CPATTN_ERR_NULL, "q_pos and k_pos are required when causal");
  if (cu_seqlens) {
    if (causal != 1) return fail(CPATTN_ERR_RANGE, "documents (cu_seqlens) need causal = 1");
    if (!aligned(cu_seqlens, 4)) return fail(CPATTN_ERR_ALIGN, "cu_seqlens must be 4-byte aligned");
    if (n_seqs < 1) return fail(CPATTN_ERR_SHAPE, "n_seqs must be >= 1, got %d", n_seqs);
  }
  if (in_dtype != CPATTN_BF16 && in_dtype != CPATTN_F32)
    return fail(CPATTN_ERR_DTYPE, "q, k, v and dout must be bf16 or float32");
  if (head_dim != 64 && head_dim != 128) return fail(CPATTN_ERR_SHAPE, "head_dim must be 64 or 128, got %d", head_dim);
  if (hq < 1 || hkv < 1) return fail(CPATTN_ERR_SHAPE, "hq and hkv must be >= 1 (hq=%d hkv=%d)", hq, hkv);
  if (hq % hkv) return fail(CPATTN_ERR_SHAPE, "hq (%d) must be a multiple of hkv (%d)", hq, hkv);
  if (lq < 0 || lk < 0) return fail(CPATTN_ERR_SHAPE, "lq and lk must be >= 0");
  if (lq >= (int64_t)1 << 31 || lk >= (int64_t)1 << 31) return fail(CPATTN_ERR_SHAPE, "lq and lk must be < 2^31");
  // a 32-row tile of one head is addressed with 32-bit buffer offsets
  const int64_t esz = dsize(in_dtype);
  if ((int64_t)hq * head_dim * esz * 32 >= (int64_t)1 << 31)
    return fail(CPATTN_ERR_SHAPE, "hq * head_dim too large (a 32-row tile must span < 2 GiB)");
  if (!std::isfinite(softmax_scale)) return fail(CPATTN_ERR_RANGE, "softmax_scale must be finite");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) || !aligned(dq, 16) ||
      !aligned(dk, 16) || !aligned(dv, 16))
    return fail(CPATTN_ERR_ALIGN, "q, k, v, dout, dq, dk and dv must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(delta, 4) || (q_pos && !aligned(q_pos, 4)) || (k_pos && !aligned(k_pos, 4)))
    return fail(CPATTN_ERR_ALIGN, "lse, delta and positions must be 4-byte aligned");
  const size_t nq = (size_t)lq * hq * head_dim * esz, nk = (size_t)lk * hkv * head_dim * esz;
  const size_t ndq = (size_t)lq * hq * head_dim * 4, ndk = (size_t)lk * hkv * head_dim * 4;
  const size_t nl = (size_t)lq * hq * sizeof(float);
  const void* ins[] = {q, k, v, dout, lse, delta};
  const size_t nin[] = {nq, nk, nk, nq, nl, nl};
  void* outs[] = {dq, dk, dv};
  const size_t nout[] = {ndq, ndk, ndk};
  for (int a = 0; a < 3; ++a) {
    for (int b = 0; b < 6; ++b)
      if (overlaps(outs[a], nout[a], ins[b], nin[b]))
        return fail(CPATTN_ERR_ALIAS, "dq, dk and dv must not overlap the inputs");
    for (int b = a + 1; b < 3; ++b)
      if (overlaps(outs[a], nout[a], outs[b], nout[b])) return fail(CPATTN_ERR_ALIAS, "dq, dk and dv must not overlap");
  }
  if (validate_env() && causal) {
    cpattn_status st = check_sorted_device(q_pos, lq, "q_pos", s);
    if (st == CPATTN_OK) st = check_sorted_device(k_pos, lk, "k_pos", s);
    if (st == CPATTN_OK && cu_seqlens) st = check_sorted_device(cu_seqlens, (int64_t)n_seqs + 1, "cu_seqlens", s);
    if (st != CPATTN_OK) return st;
  }
  return CPATTN_OK;
}

static cpattn::BwdParams bwd_params(const void* q, const void* k, const void* v, const void* dout, int64_t lq,
                                    int64_t lk, int32_t hq, int32_t hkv, int32_t head_dim, const int32_t* q_pos,
                                    const int32_t* k_pos, int32_t causal, const int32_t* cu_seqlens, int32_t n_seqs,
                                    float softmax_scale, const float* lse, const float* delta, float* dq,
                                    int32_t accumulate_dq, float* dk, float* dv, int32_t accumulate_dkv) {
  cpattn::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.dout = dout; p.lse = lse; p.delta = delta;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.q_pos = q_pos; p.k_pos = k_pos; p.cu_seqlens = cu_seqlens; p.n_seqs = cu_seqlens ? n_seqs : 0;
  p.lq = (int32_t)lq; p.lk = (int32_t)lk; p.hq = hq; p.hkv = hkv;
  p.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  p.scale_log2 = p.scale * 1.4426950408889634f;
  p.causal = causal; p.acc_dq = accumulate_dq; p.acc_dkv = accumulate_dkv;
  return p;
}

cpattn_status cpattn_partial_bwd(const void* q, const void* k, const void* v, const void* dout, cpattn_dtype in_dtype,
                                 int64_t lq, int64_t lk, int32_t hq, int32_t hkv, int32_t head_dim,
                                 const int32_t* q_pos, const int32_t* k_pos, int32_t causal,
                                 const int32_t* cu_seqlens, int32_t n_seqs, float softmax_scale, const float* lse,
                                 const float* delta, float* dq, int32_t accumulate_dq, float* dk, float* dv,
                                 int32_t accumulate_dkv, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  cpattn_status st = check_bwd_args(q, k, v, dout, in_dtype, lq, lk, hq, hkv, head_dim, q_pos, k_pos, causal,
                                    cu_seqlens, n_seqs, softmax_scale, lse, delta, dq, accumulate_dq, dk, dv,
                                    accumulate_dkv, s);
  if (st != CPATTN_OK) return st;
  const cpattn::BwdParams p = bwd_params(q, k, v, dout, lq, lk, hq, hkv, head_dim, q_pos, k_pos, causal, cu_seqlens,
                                         n_seqs, softmax_scale, lse, delta, dq, accumulate_dq, dk, dv, accumulate_dkv);
  hipError_t e = in_dtype == CPATTN_F32 ? cpattn::launch_bwd_f32(p, head_dim, cu_seqlens != nullptr, s)
                                         : cpattn::launch_bwd(p, head_dim, cu_seqlens != nullptr, s);
  if (e != hipSuccess) return fail(CPATTN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int64_t cpattn_bwd_query_workgroups(int64_t lq, int32_t hq) {
  if (lq < 0 || hq < 1) return -1;
  return cpattn::bwd_query_workgroups(lq, hq);
}

cpattn_status cpattn_varlen_bwd_plan(const int32_t* q_pos, int64_t lq, const int32_t* k_pos, int64_t lk,
                                     const int32_t* cu_seqlens, int32_t n_seqs, int32_t hq, int32_t hkv,
                                     int32_t* plan, int64_t plan_len) {
  if (lq < 0 || lk < 0) return fail(CPATTN_ERR_SHAPE, "lq and lk must be >= 0");
  if (lq >= (int64_t)1 << 31 || lk >= (int64_t)1 << 31) return fail(CPATTN_ERR_SHAPE, "lq and lk must be < 2^31");
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(CPATTN_ERR_SHAPE, "hq must be a positive multiple of hkv (hq=%d, hkv=%d)", hq, hkv);
  if (n_seqs < 1) return fail(CPATTN_ERR_SHAPE, "n_seqs must be >= 1, got %d", n_seqs);
  const int64_t n = cpattn::bwd_query_workgroups(lq, hq);
  if (plan_len != n)
    return fail(CPATTN_ERR_SHAPE, "plan_len must be %lld (the query kernel's workgroups), got %lld", (long long)n,
                (long long)plan_len);
  if (n == 0) return ok();
  if (!q_pos || !cu_seqlens || !plan || (lk > 0 && !k_pos))
    return fail(CPATTN_ERR_NULL, "q_pos, k_pos, cu_seqlens and plan must be non-NULL");
  for (int64_t i = 1; i < lq; ++i)
    if (q_pos[i] < q_pos[i - 1]) return fail(CPATTN_ERR_UNSORTED, "q_pos is not ascending at index %lld", (long long)i);
  for (int64_t i = 1; i < lk; ++i)
    if (k_pos[i] < k_pos[i - 1]) return fail(CPATTN_ERR_UNSORTED, "k_pos is not ascending at index %lld", (long long)i);
  for (int32_t i = 1; i <= n_seqs; ++i)
    if (cu_seqlens[i] < cu_seqlens[i - 1])
      return fail(CPATTN_ERR_UNSORTED, "cu_seqlens is not ascending at index %d", i);
  cpattn::plan_bwd_query(q_pos, lq, k_pos, lk, cu_seqlens, n_seqs, hq, plan);
  return ok();
}

// Optional check that a device backward plan is the one cpattn_varlen_bwd_plan
// makes for these positions (synchronises `stream`).
static cpattn_status check_bwd_plan_device(const int32_t* dplan, const int32_t* q_pos, int64_t lq,
                                           const int32_t* k_pos, int64_t lk, const int32_t* cu_seqlens,
                                           int32_t n_seqs, int32_t hq, hipStream_t stream) {
  const int64_t n = cpattn::bwd_query_workgroups(lq, hq);
  std::vector<int32_t> plan((size_t)n), qp((size_t)lq), kp((size_t)lk), cu((size_t)n_seqs + 1), want((size_t)n);
  hipError_t e = hipMemcpyAsync(plan.data(), dplan, sizeof(int32_t) * (size_t)n, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(qp.data(), q_pos, sizeof(int32_t) * (size_t)lq, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess && lk > 0)
    e = hipMemcpyAsync(kp.data(), k_pos, sizeof(int32_t) * (size_t)lk, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(cu.data(), cu_seqlens, sizeof(int32_t) * ((size_t)n_seqs + 1), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(CPATTN_ERR_HIP, "reading the plan for validation: %s", hipGetErrorString(e));
  cpattn::plan_bwd_query(qp.data(), lq, kp.data(), lk, cu.data(), n_seqs, hq, want.data());
  for (int64_t i = 0; i < n; ++i)
    if (plan[(size_t)i] != want[(size_t)i])
      return fail(CPATTN_ERR_RANGE, "the plan differs from cpattn_varlen_bwd_plan's at entry %lld (%d, expected %d)",
                  (long long)i, plan[(size_t)i], want[(size_t)i]);
  return CPATTN_OK;
}

cpattn_status cpattn_varlen_partial_bwd_planned(const void* q, const void* k, const void* v, const void* dout,
                                                cpattn_dtype in_dtype, int64_t lq, int64_t lk, int32_t hq,
                                                int32_t hkv, int32_t head_dim, const int32_t* q_pos,
                                                const int32_t* k_pos, const int32_t* cu_seqlens, int32_t n_seqs,
                                                float softmax_scale, const float* lse, const float* delta, float* dq,
                                                int32_t accumulate_dq, float* dk, float* dv, int32_t accumulate_dkv,
                                                const int32_t* plan, int64_t plan_len, void* stream) {
  if (!cu_seqlens) return fail(CPATTN_ERR_NULL, "cu_seqlens must be non-NULL");
  hipStream_t s = (hipStream_t)stream;
  cpattn_status st = check_bwd_args(q, k, v, dout, in_dtype, lq, lk, hq, hkv, head_dim, q_pos, k_pos, 1, cu_seqlens,
                                    n_seqs, softmax_scale, lse, delta, dq, accumulate_dq, dk, dv, accumulate_dkv, s);
  if (st != CPATTN_OK) return st;
  const int64_t n = cpattn::bwd_query_workgroups(lq, hq);
  if (plan_len != n)
    return fail(CPATTN_ERR_SHAPE, "plan_len must be %lld (the query kernel's workgroups), got %lld", (long long)n,
                (long long)plan_len);
  if (n > 0 && !plan) return fail(CPATTN_ERR_NULL, "plan must be non-NULL");
  if (!aligned(plan, 4)) return fail(CPATTN_ERR_ALIGN, "plan must be 4-byte aligned");
  if (n > 0 && validate_env()) {
    st = check_bwd_plan_device(plan, q_pos, lq, k_pos, lk, cu_seqlens, n_seqs, hq, s);
    if (st != CPATTN_OK) return st;
  }
  cpattn::BwdParams p = bwd_params(q, k, v, dout, lq, lk, hq, hkv, head_dim, q_pos, k_pos, 1, cu_seqlens, n_seqs,
                                   softmax_scale, lse, delta, dq, accumulate_dq, dk, dv, accumulate_dkv);
  // (float32 inputs run their own kernels in the default order)
  p.dq_order = (in_dtype == CPATTN_BF16 && n > 0) ? plan : nullptr;
  hipError_t e = in_dtype == CPATTN_F32 ? cpattn::launch_bwd_f32(p, head_dim, true, s)
                                         : cpattn::launch_bwd(p, head_dim, true, s);
  if (e != hipSuccess) return fail(CPATTN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

cpattn_status cpattn_partial_bwd_multi(const void* q, const void* const* k_blocks, const void* const* v_blocks,
                                       const void* dout, cpattn_dtype in_dtype, int64_t lq, const int64_t* lk_blocks,
                                       int32_t n_blocks, int32_t hq, int32_t hkv, int32_t head_dim,
                                       const int32_t* q_pos, const int32_t* const* k_pos_blocks, int32_t causal,
                                       const int32_t* cu_seqlens, int32_t n_seqs, float softmax_scale,
                                       const float* lse, const float* delta, float* dq, int32_t accumulate_dq,
                                       float* const* dk_blocks, float* const* dv_blocks, int32_t accumulate_dkv,
                                       void* stream) {
  if (!k_blocks || !v_blocks || !lk_blocks || !k_pos_blocks || !dk_blocks || !dv_blocks)
    return fail(CPATTN_ERR_NULL, "the block arrays must be non-NULL");
  if (n_blocks < 1 || n_blocks > cpattn::kMaxBwdBlocks)
    return fail(CPATTN_ERR_RANGE, "n_blocks must be in [1, %d], got %d", cpattn::kMaxBwdBlocks, n_blocks);
  hipStream_t s = (hipStream_t)stream;
  for (int32_t b = 0; b < n_blocks; ++b) {
    cpattn_status st = check_bwd_args(q, k_blocks[b], v_blocks[b], dout, in_dtype, lq, lk_blocks[b], hq, hkv,
                                      head_dim, q_pos, k_pos_blocks[b], causal, cu_seqlens, n_seqs, softmax_scale,
                                      lse, delta, dq, accumulate_dq, dk_blocks[b], dv_blocks[b], accumulate_dkv, s);
    if (st != CPATTN_OK) return st;
  }
  // A block's dk, dv must not overlap any other block's inputs or outputs
  // (the key kernel writes them while other blocks' keys are still read).
  const int64_t esz = dsize(in_dtype);
  for (int32_t b = 0; b < n_blocks; ++b) {
    const size_t nkb = (size_t)lk_blocks[b] * hkv * head_dim;
    for (int32_t c = 0; c < n_blocks; ++c) {
      if (c == b) continue;
      const size_t nkc = (size_t)lk_blocks[c] * hkv * head_dim;
      const void* outs[] = {dk_blocks[b], dv_blocks[b]};
      for (const void* o : outs)
        if (overlaps(o, nkb * 4, k_blocks[c], nkc * esz) || overlaps(o, nkb * 4, v_blocks[c], nkc * esz) ||
            overlaps(o, nkb * 4, dk_blocks[c], nkc * 4) || overlaps(o, nkb * 4, dv_blocks[c], nkc * 4) ||
            (k_pos_blocks[c] && overlaps(o, nkb * 4, k_pos_blocks[c], (size_t)lk_blocks[c] * 4)))
          return fail(CPATTN_ERR_ALIAS, "dk and dv of block %d overlap the buffers of block %d", b, c);
    }
  }
  if (in_dtype == CPATTN_F32) {
    // float32 inputs: the single-block kernels, one block after another
    for (int32_t b = 0; b < n_blocks; ++b) {
      const cpattn::BwdParams p =
          bwd_params(q, k_blocks[b], v_blocks[b], dout, lq, lk_blocks[b], hq, hkv, head_dim, q_pos, k_pos_blocks[b],
                     causal, cu_seqlens, n_seqs, softmax_scale, lse, delta, dq, b > 0 || accumulate_dq,
                     dk_blocks[b], dv_blocks[b], accumulate_dkv);
      hipError_t e = cpattn::launch_bwd_f32(p, head_dim, cu_seqlens != nullptr, s);
      if (e != hipSuccess) return fail(CPATTN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    }
    return ok();
  }
  cpattn::BwdBlocks bt{};
  bt.n = n_blocks;
  int64_t wg = 0;
  for (int32_t b = 0; b < n_blocks; ++b) {
    wg += (lk_blocks[b] + 127) / 128 * hkv;
    if (wg >= (int64_t)1 << 31) return fail(CPATTN_ERR_SHAPE, "too many key tiles over the blocks (>= 2^31 workgroups)");
    bt.wg_end[b] = (int32_t)wg;
    bt.lk[b] = (int32_t)lk_blocks[b];
    bt.k[b] = k_blocks[b];
    bt.v[b] = v_blocks[b];
    bt.k_pos[b] = k_pos_blocks[b];
    bt.dk[b] = dk_blocks[b];
    bt.dv[b] = dv_blocks[b];
  }
  const cpattn::BwdParams p = bwd_params(q, nullptr, nullptr, dout, lq, 0, hq, hkv, head_dim, q_pos, nullptr, causal,
                                         cu_seqlens, n_seqs, softmax_scale, lse, delta, dq, accumulate_dq, nullptr,
                                         nullptr, accumulate_dkv);
  hipError_t e = cpattn::launch_bwd_multi(p, bt, head_dim, cu_seqlens != nullptr, s);
  if (e != hipSuccess) return fail(CPATTN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

cpattn_status cpattn_merge_lse(void* o_acc, float* lse_acc, const void* o_part, const float* lse_part,
                               cpattn_dtype o_dtype, int64_t lq, int32_t hq, int32_t head_dim, void* stream) {
  if (!o_acc || !lse_acc || !o_part || !lse_part) return fail(CPATTN_ERR_NULL, "all four buffers must be non-NULL");
  if (o_dtype != CPATTN_BF16 && o_dtype != CPATTN_F32) return fail(CPATTN_ERR_DTYPE, "o_dtype %d unsupported", (int)o_dtype);
  if (head_dim != 64 && head_dim != 128) return fail(CPATTN_ERR_SHAPE, "head_dim must be 64 or 128, got %d", head_dim);
  if (lq < 0 || hq < 1) return fail(CPATTN_ERR_SHAPE, "lq must be >= 0 and hq >= 1");
  if (lq >= (int64_t)1 << 31) return fail(CPATTN_ERR_SHAPE, "lq must be < 2^31");
  if (!aligned(o_acc, 16) || !aligned(o_part, 16)) return fail(CPATTN_ERR_ALIGN, "o buffers must be 16-byte aligned");
  if (!aligned(lse_acc, 4) || !aligned(lse_part, 4)) return fail(CPATTN_ERR_ALIGN, "lse buffers must be 4-byte aligned");
  const size_t no = (size_t)lq * hq * head_dim * dsize(o_dtype);
  const size_t nl = (size_t)lq * hq * sizeof(float);
  if (overlaps(o_acc, no, o_part, no) || overlaps(lse_acc, nl, lse_part, nl) || overlaps(o_acc, no, lse_acc, nl) ||
      overlaps(o_acc, no, lse_part, nl) || overlaps(lse_acc, nl, o_part, no))
    return fail(CPATTN_ERR_ALIAS, "o_part/lse_part must not overlap o_acc/lse_acc");
  if (lq == 0) return ok();
  hipError_t e = cpattn::launch_merge(o_acc, lse_acc, o_part, lse_part, o_dtype == CPATTN_BF16, lq, hq, head_dim,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return fail(CPATTN_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
