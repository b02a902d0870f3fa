// partial_bwd_f32.hip — gradients of one KV block's part of a rank's
// attention for float32 inputs, on gfx950 (MI355X).
//
// The same gradients as partial_bwd.hip (PCP page "大模型长序列显存优化：PCP与
// DCP序列并行实战指南", §2.3: the backward runs over the same blocks; masks as
// in the forward): with each row's final LSE and D = <dO, O>,
//     P = exp(s - LSE),  dV = P^T dO,  dP = dO V^T,  dS = P (dP - D),
//     dQ = scale dS K,  dK = scale dS^T Q,
// accumulated in float32 from float32 operands with v_mfma_f32_32x32x2_f32.
//
// The structure is that of the bf16 kernels — a key kernel (dK, dV of 128
// keys of one KV head, walking the query tiles of every query head that
// reads it) and a query kernel (dQ of 128 rows of one head, walking the key
// tiles they see), no atomics, S and dP formed in both — with one role per
// wave and single-stage LDS tiles: this path serves float32 callers (small
// shapes, reference-precision runs), not the bf16 throughput path.
//
// Orientation (32x32x2 float32 MFMA: lane l supplies A[l % 32][l / 32] and
// B[l / 32][l % 32]; register r of the result is row 8(r/4) + 4(l/32) + r%4,
// column l % 32):
//  * key kernel: S = Q K^T and dP = dO V^T with each lane on ONE key (its K
//    and V rows in registers as the B operands) and 16 query rows in its
//    registers; P and dS, still in those registers, are then directly the B
//    operands of dV^T += dO^T P and dK^T += Q^T dS when the contraction over
//    query rows takes, at step r, row 8(r/4) + 4(l/32) + r%4 in lane l (a sum
//    over rows in any order is the same sum);
//  * query kernel: the mirror, S^T = K Q^T and dP^T = V dO^T with each lane
//    on one query row, and dQ^T += K^T dS^T.
// Tiles are row-major float32 in LDS with the 16-byte chunks of row r XORed
// with r % 16, so a column read across 16 rows hits 16 different chunks.
#include "device_common.hpp"
#include "kernels_bwd.hpp"
#include "tile_io.hpp"

namespace cpattn {

constexpr int kF32Threads = 256;  // four waves

template <int D>
struct F32Tile {
  static constexpr int kRowBytes = 4 * D;
  static constexpr int kChunks = D / 4;                      // 16-byte chunks per row
  static constexpr int kBytes = 32 * kRowBytes;              // a 32-row tile
  static constexpr int kUnits = kBytes / 16 / kF32Threads;   // 16-byte loads per thread per tile
  static constexpr int kNK = D / 2;                          // k-steps over the head dimension
  static constexpr int kNDT = D / 32;                        // 32-column blocks of the head dimension
  static constexpr int off(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 15)) << 4); }
  static constexpr int at(int row, int col) { return off(row, col >> 2) + ((col & 3) << 2); }
};

// 32 rows of one head of a [n_rows][heads][D] float32 tensor into registers
// (thread t: 16-byte units t, t + 256, ... of the row-major tile); rows at or
// past n_rows read as zeros.
template <int D>
__device__ __forceinline__ void fetch_rows_f32(u32x4_t* regs, const char* head_base, int row_stride, int r0,
                                               int n_rows, int tid) {
  using T = F32Tile<D>;
  const int rows = clamp_rows(n_rows - r0, 32);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(head_base + (int64_t)r0 * row_stride, (int64_t)rows * row_stride);
#pragma unroll
  for (int u = 0; u < T::kUnits; ++u) {
    const int unit = tid + kF32Threads * u;
    regs[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (unit / T::kChunks) * row_stride + (unit % T::kChunks) * 16,
                                                    0, 0);
  }
}

template <int D>
__device__ __forceinline__ void commit_rows_f32(char CPATTN_LDS* tile, const u32x4_t* regs, int tid) {
  using T = F32Tile<D>;
#pragma unroll
  for (int u = 0; u < T::kUnits; ++u) {
    const int unit = tid + kF32Threads * u;
    *(u32x4_t CPATTN_LDS*)(tile + T::off(unit / T::kChunks, unit % T::kChunks)) = regs[u];
  }
}

__device__ __forceinline__ float lds_f32(const char CPATTN_LDS* tile, int byte_off) {
  return *(const float CPATTN_LDS*)(tile + byte_off);
}

// ---------------------------------------------------------------------------
// Key kernel: dK, dV of 128 keys (32 per wave) of one KV head.

template <int D, bool VARLEN>
__global__ __launch_bounds__(kF32Threads, 1) void bwd_dkv_f32_kernel(BwdParams p) {
  using T = F32Tile<D>;
  constexpr int NK = T::kNK, NDT = T::kNDT;
  __shared__ __attribute__((aligned(16))) char q_s[T::kBytes], o_s[T::kBytes];
  __shared__ float l_s[32], d_s[32];
  __shared__ int32_t p_s[32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, li = lane & 31;
  const int L = tile_order(blockIdx.x, p.n_wg, p.hkv);
  const int hk = L / p.n_tiles;
  const int kt = L % p.n_tiles;
  const int G = p.hq / p.hkv;
  const int lq = p.lq, lk = p.lk;
  const int wg_j0 = kt * 128, wg_j1 = min(wg_j0 + 128, lk);
  const int j0 = wg_j0 + 32 * wave;
  const int kj = min(j0 + li, lk - 1);  // this lane's key (clamped)
  const bool key_valid = j0 + li < lk;

  // rows that see the workgroup's keys
  int i_lo = 0, i_hi = lq;
  if (p.causal) {
    i_lo = wave_upper_bound(p.q_pos, lq, p.k_pos[wg_j0] - 1);
    if constexpr (VARLEN) i_hi = wave_upper_bound(p.q_pos, lq, doc_end(p.cu_seqlens, p.n_seqs, p.k_pos[wg_j1 - 1]) - 1);
  }
  const int nqt = i_hi > i_lo ? (i_hi - i_lo + 31) / 32 : 0;
  const int n_it = G * nqt;

  // B operands of S = Q K^T and dP = dO V^T: the lane's key row, columns 2ks + g
  float kreg[NK], vreg[NK];
  {
    const float* krow = (const float*)p.k + ((int64_t)kj * p.hkv + hk) * D;
    const float* vrow = (const float*)p.v + ((int64_t)kj * p.hkv + hk) * D;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      kreg[ks] = krow[2 * ks + g];
      vreg[ks] = vrow[2 * ks + g];
    }
  }
  const int32_t my_kpos = p.causal ? p.k_pos[kj] : 0;
  const int32_t my_kend = VARLEN ? doc_end(p.cu_seqlens, p.n_seqs, my_kpos) : 0;

  // query tile it: head hk*G + it / nqt, rows i_lo + 32 (it % nqt) ..
  const int q_stride = p.hq * D * 4;
  u32x4_t qr[T::kUnits], dr[T::kUnits];
  float lr = 0.f, drow = 0.f;
  int32_t pr = 0;
  bool rv = false;
  auto fetch = [&](int it) __attribute__((always_inline)) {
    const int hh = hk * G + it / nqt;
    const int i0 = i_lo + 32 * (it % nqt);
    fetch_rows_f32<D>(qr, (const char*)p.q + (int64_t)hh * D * 4, q_stride, i0, lq, tid);
    fetch_rows_f32<D>(dr, (const char*)p.dout + (int64_t)hh * D * 4, q_stride, i0, lq, tid);
    if (tid < 32) {
      rv = i0 + tid < lq;
      const int64_t at = (int64_t)hh * lq + (rv ? i0 + tid : 0);
      lr = rv ? p.lse[at] : 0.f;
      drow = rv ? p.delta[at] : 0.f;
      pr = (rv && p.causal) ? p.q_pos[i0 + tid] : 0;
    }
  };
  auto commit = [&]() __attribute__((always_inline)) {
    commit_rows_f32<D>((char CPATTN_LDS*)q_s, qr, tid);
    commit_rows_f32<D>((char CPATTN_LDS*)o_s, dr, tid);
    if (tid < 32) {
      // base-2 LSE; rows past the end, or that see nothing, get +inf: P = 0
      l_s[tid] = (!rv || lr == neg_inf()) ? __builtin_inff() : lr * kLog2e;
      d_s[tid] = rv ? drow : 0.f;
      p_s[tid] = pr;
    }
  };

  f32x16_t dk_acc[NDT], dv_acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    dk_acc[dt] = f32x16_t{};
    dv_acc[dt] = f32x16_t{};
  }
  // At d 64 the next tile is fetched into registers while this one is
  // processed; at d 128 the key and value rows and both accumulators leave no
  // room for it, and it is fetched after.
  constexpr bool kAhead = D == 64;
  if (n_it > 0) {
    fetch(0);
    commit();
  }
  __syncthreads();
  for (int it = 0; it < n_it; ++it) {
    if (kAhead && it + 1 < n_it) fetch(it + 1);
    const char CPATTN_LDS* ql = (const char CPATTN_LDS*)q_s;
    const char CPATTN_LDS* ol = (const char CPATTN_LDS*)o_s;
    // S = Q K^T, dP = dO V^T (rows: the tile's queries; column: this lane's key)
    f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const int a = T::at(li, 2 * ks + g);
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(lds_f32(ql, a), kreg[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x2f32(lds_f32(ol, a), vreg[ks], dp, 0, 0, 0);
    }
    // P (into s) and dS (into dp) on visible pairs
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * g + (r & 3);
      bool vis = key_valid;
      if (p.causal) {
        const int32_t qp = p_s[row];
        vis = vis & (qp >= my_kpos);
        if (VARLEN) vis = vis & (qp < my_kend);
      }
      const float pv = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], p.scale_log2, -l_s[row])) : 0.f;
      s[r] = pv;
      dp[r] = pv * (dp[r] - d_s[row]);
    }
    // dV^T += dO^T P, dK^T += Q^T dS (contraction over the tile's rows: step r takes row(r, g))
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * g + (r & 3);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int a = T::at(row, 32 * dt + li);
        dv_acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(lds_f32(ol, a), s[r], dv_acc[dt], 0, 0, 0);
        dk_acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(lds_f32(ql, a), dp[r], dk_acc[dt], 0, 0, 0);
      }
    }
    __syncthreads();  // every wave is done with the stage
    if (it + 1 < n_it) {
      if (!kAhead) fetch(it + 1);
      commit();
      __syncthreads();
    }
  }

  // ---- store: lane li holds key j0 + li, head-dimension entries 32dt + 8rr + 4g + 0..3 ----
  if (!key_valid) return;
  float* dkrow = p.dk + ((int64_t)kj * p.hkv + hk) * D;
  float* dvrow = p.dv + ((int64_t)kj * p.hkv + hk) * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int d0 = 32 * dt + 8 * rr + 4 * g;
      float4 a = make_float4(dk_acc[dt][4 * rr] * p.scale, dk_acc[dt][4 * rr + 1] * p.scale,
                             dk_acc[dt][4 * rr + 2] * p.scale, dk_acc[dt][4 * rr + 3] * p.scale);
      float4 b = make_float4(dv_acc[dt][4 * rr], dv_acc[dt][4 * rr + 1], dv_acc[dt][4 * rr + 2], dv_acc[dt][4 * rr + 3]);
      if (p.acc_dkv) {
        const float4 oa = *(const float4*)(dkrow + d0), ob = *(const float4*)(dvrow + d0);
        a.x += oa.x; a.y += oa.y; a.z += oa.z; a.w += oa.w;
        b.x += ob.x; b.y += ob.y; b.z += ob.z; b.w += ob.w;
      }
      *(float4*)(dkrow + d0) = a;
      *(float4*)(dvrow + d0) = b;
    }
}

// ---------------------------------------------------------------------------
// Query kernel: dQ of 128 rows (32 per wave) of one query head.

template <int D, bool VARLEN>
__global__ __launch_bounds__(kF32Threads, 1) void bwd_dq_f32_kernel(BwdParams p) {
  using T = F32Tile<D>;
  constexpr int NK = T::kNK, NDT = T::kNDT;
  __shared__ __attribute__((aligned(16))) char k_s[T::kBytes], v_s[T::kBytes];
  __shared__ int32_t kp_s[32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, li = lane & 31;
  const int L = tile_order(blockIdx.x, p.n_wg, p.hq);
  const int h = L / p.n_tiles;
  const int qt = p.n_tiles - 1 - L % p.n_tiles;  // late rows (that see the most keys) first
  const int hk = h / (p.hq / p.hkv);
  const int lq = p.lq, lk = p.lk;
  const int wg_r0 = qt * 128, wg_r1 = min(wg_r0 + 128, lq);
  const int r0 = wg_r0 + 32 * wave;
  const int qi = min(r0 + li, lq - 1);  // this lane's row (clamped)
  const bool row_valid = r0 + li < lq;
  // Rows that see none of the block add nothing, and when accumulating dQ is
  // left as it is: the common case (the block's first key is after the
  // workgroup's last row) is decided by one load, before Q and dO are read.
  if (p.acc_dq && (lk == 0 || (p.causal && p.k_pos[0] > p.q_pos[wg_r1 - 1]))) return;

  // B operands of S^T = K Q^T and dP^T = V dO^T: the lane's row, columns 2ks + g
  float qreg[NK], dreg[NK];
  {
    const float* qrow = (const float*)p.q + ((int64_t)qi * p.hq + h) * D;
    const float* drow = (const float*)p.dout + ((int64_t)qi * p.hq + h) * D;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      qreg[ks] = qrow[2 * ks + g];
      dreg[ks] = drow[2 * ks + g];
    }
  }
  const float l_raw = p.lse[(int64_t)h * lq + qi];
  const float lse2 = (!row_valid || l_raw == neg_inf()) ? __builtin_inff() : l_raw * kLog2e;
  const float dlt = row_valid ? p.delta[(int64_t)h * lq + qi] : 0.f;
  const int32_t my_qpos = p.causal ? p.q_pos[qi] : 0;
  const int32_t my_start = VARLEN ? doc_start(p.cu_seqlens, p.n_seqs, my_qpos) : 0;

  // keys the workgroup's rows can see
  int kb = 0, ke = lk;
  if (p.causal) {
    ke = wave_upper_bound(p.k_pos, lk, p.q_pos[wg_r1 - 1]);
    if constexpr (VARLEN) kb = wave_upper_bound(p.k_pos, lk, doc_start(p.cu_seqlens, p.n_seqs, p.q_pos[wg_r0]) - 1);
  }
  const int nt = ke > kb ? (ke - kb + 31) / 32 : 0;
  // (with documents the rows may still see nothing)
  if (nt == 0 && p.acc_dq) return;

  const int kv_stride = p.hkv * D * 4;
  const char* kbase = (const char*)p.k + (int64_t)hk * D * 4;
  const char* vbase = (const char*)p.v + (int64_t)hk * D * 4;
  u32x4_t kr[T::kUnits], vr[T::kUnits];
  int32_t pr = 0;
  auto fetch = [&](int t) __attribute__((always_inline)) {
    const int j0 = kb + 32 * t;
    fetch_rows_f32<D>(kr, kbase, kv_stride, j0, lk, tid);
    fetch_rows_f32<D>(vr, vbase, kv_stride, j0, lk, tid);
    if (tid < 32) pr = (p.causal && j0 + tid < lk) ? p.k_pos[j0 + tid] : 0x7FFFFFFF;
  };
  auto commit = [&]() __attribute__((always_inline)) {
    commit_rows_f32<D>((char CPATTN_LDS*)k_s, kr, tid);
    commit_rows_f32<D>((char CPATTN_LDS*)v_s, vr, tid);
    if (tid < 32) kp_s[tid] = pr;
  };

  f32x16_t acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16_t{};
  if (nt > 0) {
    fetch(0);
    commit();
  }
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    if (t + 1 < nt) fetch(t + 1);
    const char CPATTN_LDS* kl = (const char CPATTN_LDS*)k_s;
    const char CPATTN_LDS* vl = (const char CPATTN_LDS*)v_s;
    // S^T = K Q^T, dP^T = V dO^T (rows: the tile's keys; column: this lane's row)
    f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const int a = T::at(li, 2 * ks + g);
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(lds_f32(kl, a), qreg[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x2f32(lds_f32(vl, a), dreg[ks], dp, 0, 0, 0);
    }
    // dS^T = P (dP - D) into dp; register r is key 8(r/4) + 4g + r%4 of the tile
    const int lim = min(lk - (kb + 32 * t), 32);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * g + (r & 3);
      bool vis = key < lim;
      if (p.causal) {
        const int32_t kp = kp_s[key];
        vis = vis & (kp <= my_qpos);
        if (VARLEN) vis = vis & (kp >= my_start);
      }
      const float pv = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], p.scale_log2, -lse2)) : 0.f;
      dp[r] = pv * (dp[r] - dlt);
    }
    // dQ^T += K^T dS^T (contraction over the tile's keys: step r takes key(r, g))
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * g + (r & 3);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(lds_f32(kl, T::at(key, 32 * dt + li)), dp[r], acc[dt], 0, 0, 0);
    }
    __syncthreads();
    if (t + 1 < nt) {
      commit();
      __syncthreads();
    }
  }

  // ---- store: lane holds row qi, head-dimension entries 32dt + 8rr + 4g + 0..3 ----
  if (!row_valid) return;
  float* dqrow = p.dq + ((int64_t)qi * p.hq + h) * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int d0 = 32 * dt + 8 * rr + 4 * g;
      float4 a = make_float4(acc[dt][4 * rr] * p.scale, acc[dt][4 * rr + 1] * p.scale, acc[dt][4 * rr + 2] * p.scale,
                             acc[dt][4 * rr + 3] * p.scale);
      if (p.acc_dq) {
        const float4 o = *(const float4*)(dqrow + d0);
        a.x += o.x; a.y += o.y; a.z += o.z; a.w += o.w;
      }
      *(float4*)(dqrow + d0) = a;
    }
}

// ---------------------------------------------------------------------------

template <int D, bool VARLEN>
static hipError_t launch_bwd_f32_typed(BwdParams p, hipStream_t stream) {
  if (p.lk > 0) {
    BwdParams a = p;
    a.n_tiles = (p.lk + 127) / 128;
    a.n_wg = a.n_tiles * p.hkv;
    hipLaunchKernelGGL((bwd_dkv_f32_kernel<D, VARLEN>), dim3(a.n_wg), dim3(kF32Threads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.lq > 0) {
    BwdParams a = p;
    a.n_tiles = (p.lq + 127) / 128;
    a.n_wg = a.n_tiles * p.hq;
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D, VARLEN>), dim3(a.n_wg), dim3(kF32Threads), 0, stream, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_bwd_f32(BwdParams p, int head_dim, bool varlen, hipStream_t stream) {
  if (head_dim == 128)
    return varlen ? launch_bwd_f32_typed<128, true>(p, stream) : launch_bwd_f32_typed<128, false>(p, stream);
  return varlen ? launch_bwd_f32_typed<64, true>(p, stream) : launch_bwd_f32_typed<64, false>(p, stream);
}

}  // namespace cpattn
