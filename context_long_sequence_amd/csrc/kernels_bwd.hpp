// kernels_bwd.hpp — host-visible launch interface of the gradient kernels
// (partial_bwd.hip, partial_bwd_f32.hip) for the C-ABI layer (api.cpp).
// Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

// Gradients of one KV block (partial_bwd.hip).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;           // [hq][lq], the rows' final log-normalisers
  const float* delta;         // [hq][lq], <dO, O>
  float* dq;                  // [lq][hq][d]
  float* dk;                  // [lk][hkv][d]
  float* dv;
  const int32_t* q_pos;
  const int32_t* k_pos;
  const int32_t* cu_seqlens;
  int32_t n_seqs;
  int32_t lq, lk, hq, hkv;
  float scale, scale_log2;
  int32_t causal, acc_dq, acc_dkv;
  int32_t n_tiles, n_wg;      // set per kernel by launch_bwd
  const int32_t* dq_order;    // query kernel: logical tile of each workgroup (a host plan), or NULL
};

// The KV blocks of a multi-block gradient call, in order (bf16 kernels only).
// The key kernel's grid covers every block's workgroups: block b takes
// workgroups wg_end[b-1] .. wg_end[b]-1 (wg_end[-1] = 0). The query kernel
// walks the blocks in order, dQ summed in registers across them.
constexpr int kMaxBwdBlocks = 32;
struct BwdBlocks {
  int32_t n;
  int32_t lk[kMaxBwdBlocks];
  int32_t wg_end[kMaxBwdBlocks];
  const void* k[kMaxBwdBlocks];
  const void* v[kMaxBwdBlocks];
  const int32_t* k_pos[kMaxBwdBlocks];
  float* dk[kMaxBwdBlocks];
  float* dv[kMaxBwdBlocks];
};

// Enqueue the key-gradient kernel over all blocks of `bt` (p's k, v, k_pos,
// lk, dk, dv unused), then the query-gradient kernel over the blocks in order.
hipError_t launch_bwd_multi(BwdParams p, const BwdBlocks& bt, int head_dim, bool varlen, hipStream_t stream);

// Enqueue the key-gradient kernel (if lk > 0) then the query-gradient kernel (if lq > 0):
// bf16 q, k, v, dout (partial_bwd.hip) or float32 ones (partial_bwd_f32.hip).
hipError_t launch_bwd(BwdParams p, int head_dim, bool varlen, hipStream_t stream);
hipError_t launch_bwd_f32(BwdParams p, int head_dim, bool varlen, hipStream_t stream);

// Workgroups of the query-gradient kernel (128 rows of one query head each).
int64_t bwd_query_workgroups(int64_t lq, int32_t hq);

// Host: the query kernel's dispatch order for a call with documents (all
// arguments in host memory, already validated): for each XCD, the logical
// tiles the default order gives it, those that load the most key tiles
// first (ties by logical id); plan[b] = the logical tile of workgroup b.
void plan_bwd_query(const int32_t* q_pos, int64_t lq, const int32_t* k_pos, int64_t lk, const int32_t* cu_seqlens,
                    int32_t n_seqs, int32_t hq, int32_t* plan);

// Enqueue delta[h][i] = <dout[i][h], o[i][h]>.
hipError_t launch_bwd_delta(const void* o, int o_bf16, const void* dout, int do_bf16, int64_t lq, int32_t hq,
                            int32_t head_dim, float* delta, hipStream_t stream);

}  // namespace cpattn
