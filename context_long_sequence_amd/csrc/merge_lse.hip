// merge_lse.hip — in-place merge of two partial attention results over
// disjoint key sets (PCP page "大模型长序列显存优化：PCP与DCP序列并行实战指南",
// §4.2: the global max / global sum normaliser, taken two partials at a
// time; FCP page "从固定环到自由拓扑：FCP到底在解决什么", §3.3: partials may be
// combined in any order).
//
// HBM-bound elementwise work: each lane moves 8 output elements (16 bytes of
// bf16 or 32 of float32) of both operands. The D/8 lanes of one row sit in
// one wave, so all of them read the row's stored LSE before the single lane
// that rewrites it stores (a wave executes its load before its store).
#include "device_common.hpp"
#include "kernels.hpp"

namespace cpattn {

template <typename TOut, int D>
__global__ __launch_bounds__(256) void merge_kernel(TOut* __restrict__ o_acc, float* __restrict__ lse_acc,
                                                    const TOut* __restrict__ o_part,
                                                    const float* __restrict__ lse_part, int64_t lq, int32_t hq) {
  constexpr int LPR = D / 8;  // lanes per row
  static_assert(64 % LPR == 0, "a row's lanes must share a wave");
  const int64_t n = lq * hq * LPR;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += stride) {
    const int64_t row = idx / LPR;  // row = token * hq + head
    const int part = (int)(idx % LPR);
    const int64_t tok = row / hq;
    const int h = (int)(row % hq);
    const int64_t li = (int64_t)h * lq + tok;
    float wa, wb, L;
    merge_weights(lse_acc[li], lse_part[li], wa, wb, L);
    const int64_t e0 = row * D + part * 8;
    if constexpr (sizeof(TOut) == 2) {
      uint4 a = *(const uint4*)(o_acc + e0);
      uint4 b = *(const uint4*)(o_part + e0);
      uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w}, ow[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float lo = wa * bf16_bits_to_f32((uint16_t)(aw[t] & 0xFFFF)) + wb * bf16_bits_to_f32((uint16_t)(bw[t] & 0xFFFF));
        float hi = wa * bf16_bits_to_f32((uint16_t)(aw[t] >> 16)) + wb * bf16_bits_to_f32((uint16_t)(bw[t] >> 16));
        ow[t] = pack_bf16x2(lo, hi);
      }
      *(uint4*)(o_acc + e0) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float4 a = *(const float4*)(o_acc + e0 + 4 * t);
        float4 b = *(const float4*)(o_part + e0 + 4 * t);
        *(float4*)(o_acc + e0 + 4 * t) =
            make_float4(wa * a.x + wb * b.x, wa * a.y + wb * b.y, wa * a.z + wb * b.z, wa * a.w + wb * b.w);
      }
    }
    if (part == 0) lse_acc[li] = L;
  }
}

template <typename TOut, int D>
static hipError_t launch_merge_typed(void* o_acc, float* lse_acc, const void* o_part, const float* lse_part,
                                     int64_t lq, int32_t hq, hipStream_t stream) {
  const int64_t n = lq * hq * (D / 8);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1 << 20) blocks = 1 << 20;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((merge_kernel<TOut, D>), dim3((unsigned)blocks), dim3(256), 0, stream, (TOut*)o_acc, lse_acc,
                     (const TOut*)o_part, lse_part, lq, hq);
  return hipGetLastError();
}

hipError_t launch_merge(void* o_acc, float* lse_acc, const void* o_part, const float* lse_part, int out_bf16,
                        int64_t lq, int32_t hq, int32_t head_dim, hipStream_t stream) {
  if (out_bf16) {
    return head_dim == 128 ? launch_merge_typed<__bf16, 128>(o_acc, lse_acc, o_part, lse_part, lq, hq, stream)
                           : launch_merge_typed<__bf16, 64>(o_acc, lse_acc, o_part, lse_part, lq, hq, stream);
  }
  return head_dim == 128 ? launch_merge_typed<float, 128>(o_acc, lse_acc, o_part, lse_part, lq, hq, stream)
                         : launch_merge_typed<float, 64>(o_acc, lse_acc, o_part, lse_part, lq, hq, stream);
}

}  // namespace cpattn
