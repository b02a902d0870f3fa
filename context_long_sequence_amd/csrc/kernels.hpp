// kernels.hpp — host-visible launch interface between the C-ABI layer
// (api.cpp) and the gfx950 kernels. Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

struct PartialParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* q_pos;
  const int32_t* k_pos;
  const int32_t* cu_seqlens;
  int32_t n_seqs;
  int64_t lq, lk;
  int32_t hq, hkv;
  int32_t g_wg, r_wg;         // query heads / 32-row blocks per workgroup (set by launch_partial)
  int32_t n_qtiles, n_hgroups, n_wg;
  float scale_log2;           // softmax scale * log2(e)
  int32_t causal, accumulate;
  const int32_t* wg_plan;     // optional plan of a document call: kPlanRec int32 per workgroup id (see below)
};

// A document call's plan, one record per workgroup id (made on the host by
// plan_varlen): the logical tile it computes, its key range, and per wave the
// document starts of its first and last rows, its fully visible key range and
// whether its lanes must search their own document starts.
constexpr int kPlanRec = 48;
constexpr int kPlanTile = 0, kPlanKb = 1, kPlanKe = 2;
constexpr int kPlanSLast = 4, kPlanSFirst = 12, kPlanFLo = 20, kPlanFHi = 28, kPlanFlags = 36;

// The KV blocks of a multi-block call (passed by value as a kernel argument).
constexpr int kMaxBlocks = 32;
struct BlockTable {
  int32_t n;
  int32_t lk[kMaxBlocks];
  const void* k[kMaxBlocks];
  const void* v[kMaxBlocks];
  const int32_t* k_pos[kMaxBlocks];
};

// Enqueue the partial-attention kernel; arguments are already validated.
hipError_t launch_partial(PartialParams p, int in_bf16, int out_bf16, int head_dim, bool varlen, hipStream_t stream);

// Enqueue the kernel over the blocks of `bt` in order (p's k, v, k_pos, lk unused).
hipError_t launch_partial_multi(PartialParams p, const BlockTable& bt, int in_bf16, int out_bf16, int head_dim,
                                bool varlen, hipStream_t stream);

// Workgroups of a single-block call (the length of a dispatch order).
int64_t partial_workgroups(int64_t lq, int32_t hq, int32_t hkv);

// Host: the plan of a single-block call with documents (all arguments in
// host memory, already validated), kPlanRec int32 per workgroup: the dispatch
// order (within each XCD's set of logical tiles, the tiles that load the most
// key tiles first) and every range the kernel would otherwise search for.
void plan_varlen(const int32_t* q_pos, int64_t lq, const int32_t* k_pos, int64_t lk, const int32_t* cu_seqlens,
                 int32_t n_seqs, int32_t hq, int32_t hkv, int in_bf16, int head_dim, int32_t* plan);

// Enqueue the standalone merge (o_acc, lse_acc) <- merge(acc, part).
hipError_t launch_merge(void* o_acc, float* lse_acc, const void* o_part, const float* lse_part, int out_bf16,
                        int64_t lq, int32_t hq, int32_t head_dim, hipStream_t stream);

}  // namespace cpattn
