// Router gate projection in front of the route-sort path, MI355X (gfx950).
//
// The page "Kimi-K3 B1 route-sort + prepared-MoE handoff (stack)", Summary,
// puts a specialised batch-1 gate projection right before the route-sort
// kernel, which starts from FP32 router logits.  This file computes those
// logits, logits[t, e] = sum_i hidden[t, i] * W[e, i], for a small batch of
// tokens and hands them to the route-sort path on the same stream.
//
// At batch 1 the gate is a matrix-vector product: the E x H BF16 weight matrix
// (12.8 MB for 896 experts and H = 7168) is read once and every weight is used
// once per token, so it is bound by HBM, not by a matrix unit.  One workgroup
// per expert streams its weight row in 16-byte vectors, multiplies by the
// tokens' hidden rows (shared by all workgroups, so they stay in L2) and accumulates in
// float64: every BF16 x BF16 product is exact there and the sum is far more
// precise than FP32, so the one FP32 rounding at the end gives the correctly
// rounded dot product except where it lies within ~2^-40 (relative) of an
// FP32 rounding midpoint.  Tokens go four at a time, so each weight vector
// loaded serves four tokens.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_gate.h"
#include "moe_route_sort.h"
#include "route_internal.h"

namespace {

constexpr int kGateWaves = 4;   // waves per workgroup (one expert)
constexpr int kGateTok = 4;     // tokens per pass over a weight row
constexpr int kGateMaxM = 64;   // batch limit of this entry point

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ void unpack8(const uint4 q, double* f) {
  const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = (double)__uint_as_float(u[i] << 16);
    f[2 * i + 1] = (double)__uint_as_float(u[i] & 0xFFFF0000u);
  }
}

// One workgroup per expert: its 256 threads split the weight row (thread i
// takes vectors i, i + 256, ..., at most NJ of them).  Every weight vector of
// the thread, and the hidden vectors of the first TOK tokens, are requested
// before the first one is used, so a row's bytes are in flight together
// rather than one round trip per vector; the weight vectors stay in
// registers for the later tokens.  The partial sums meet in LDS.  Each
// thread accumulates its vectors in index order, as a plain loop would.
template <int NJ, int TOK>
__global__ __launch_bounds__(kGateWaves * 64) void k_gate(const uint16_t* __restrict__ hidden,
                                                          const uint16_t* __restrict__ w, float* logits, int M,
                                                          int E, int H) {
  constexpr int kT = kGateWaves * 64;
  __shared__ double part[TOK][kGateWaves];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int e = blockIdx.x;
  const int nv = H / 8;  // 16-byte vectors per row
  const uint4* wr = reinterpret_cast<const uint4*>(w + (size_t)e * H);
  uint4 wq[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) wq[j] = wr[min(tid + j * kT, nv - 1)];  // clamped: inside the row
  for (int t0 = 0; t0 < M; t0 += TOK) {
    uint4 hq[TOK][NJ];
#pragma unroll
    for (int q = 0; q < TOK; ++q) {
      const uint4* hr = reinterpret_cast<const uint4*>(hidden + (size_t)min(t0 + q, M - 1) * H);
#pragma unroll
      for (int j = 0; j < NJ; ++j) hq[q][j] = hr[min(tid + j * kT, nv - 1)];
    }
    double acc[TOK];
#pragma unroll
    for (int q = 0; q < TOK; ++q) acc[q] = 0.0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (tid + j * kT < nv) {
        double wf[8];
        unpack8(wq[j], wf);
#pragma unroll
        for (int q = 0; q < TOK; ++q) {
          double hf[8];
          unpack8(hq[q][j], hf);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[q] = fma(hf[i], wf[i], acc[q]);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < TOK; ++q) {
      const double s = wave_sum(acc[q]);
      if (lane == 0) part[q][wv] = s;
    }
    __syncthreads();
    if (tid < TOK && t0 + tid < M) {
      double s = 0.0;
#pragma unroll
      for (int q = 0; q < kGateWaves; ++q) s += part[tid][q];
      logits[(size_t)(t0 + tid) * E + e] = (float)s;
    }
    __syncthreads();  // part is reused by the next pass
  }
}

// Longer rows (more than 8 vectors per thread): one vector at a time.
__global__ __launch_bounds__(kGateWaves * 64) void k_gate_long(const uint16_t* __restrict__ hidden,
                                                               const uint16_t* __restrict__ w, float* logits,
                                                               int M, int E, int H) {
  constexpr int kT = kGateWaves * 64;
  __shared__ double part[kGateTok][kGateWaves];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int e = blockIdx.x;
  const int nv = H / 8;
  const uint4* wr = reinterpret_cast<const uint4*>(w + (size_t)e * H);
  for (int t0 = 0; t0 < M; t0 += kGateTok) {
    double acc[kGateTok];
#pragma unroll
    for (int j = 0; j < kGateTok; ++j) acc[j] = 0.0;
    for (int c = tid; c < nv; c += kT) {
      double wf[8];
      unpack8(wr[c], wf);
#pragma unroll
      for (int j = 0; j < kGateTok; ++j) {
        if (t0 + j < M) {
          double hf[8];
          unpack8(reinterpret_cast<const uint4*>(hidden + (size_t)(t0 + j) * H)[c], hf);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[j] = fma(hf[i], wf[i], acc[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kGateTok; ++j) {
      const double s = wave_sum(acc[j]);
      if (lane == 0) part[j][wv] = s;
    }
    __syncthreads();
    if (tid < kGateTok && t0 + tid < M) {
      double s = 0.0;
#pragma unroll
      for (int q = 0; q < kGateWaves; ++q) s += part[tid][q];
      logits[(size_t)(t0 + tid) * E + e] = (float)s;
    }
    __syncthreads();
  }
}

template <int TOK>
const void* gate_kernel_tok(int nj) {
  switch (nj) {
    case 1: return reinterpret_cast<const void*>(k_gate<1, TOK>);
    case 2: return reinterpret_cast<const void*>(k_gate<2, TOK>);
    case 3:
    case 4: return reinterpret_cast<const void*>(k_gate<4, TOK>);
    default: return reinterpret_cast<const void*>(k_gate<8, TOK>);
  }
}
// vectors per thread rounded up to 1, 2, 4 or 8; one token per pass at M = 1
const void* gate_kernel(int M, int H) {
  const int nj = (H / 8 + kGateWaves * 64 - 1) / (kGateWaves * 64);
  if (nj > 8) return reinterpret_cast<const void*>(k_gate_long);
  return M == 1 ? gate_kernel_tok<1>(nj) : gate_kernel_tok<kGateTok>(nj);
}
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int moe_gate_route_sort(const void* hidden, const void* w_gate, const float* bias, int M, int E, int H,
                                   int k, int n_group, int topk_group, int block, float* out_logits,
                                   int32_t* out_ids, float* out_w, int32_t* sorted_ids,
                                   int32_t* expert_of_block, int32_t* num_post_pad, void* stream) {
  if (M < 0 || M > kGateMaxM || H < 8 || H % 8 != 0) return MRS_ERR_INVALID_ARG;
  int rc = mrs_check_route_args(out_logits, bias, M, E, k, n_group, topk_group, block, out_ids, out_w,
                                sorted_ids, expert_of_block, num_post_pad, MRS_DTYPE_F32);
  if (rc != MRS_OK) return rc;
  if (moe_route_sort_max_rows(M, E, k, block) < 0) return MRS_ERR_OVERFLOW;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (M > 0) {
    if (!hidden || !w_gate) return MRS_ERR_NULL_POINTER;
    if (!aligned16(hidden) || !aligned16(w_gate)) return MRS_ERR_MISALIGNED;
    const uint16_t* h16 = static_cast<const uint16_t*>(hidden);
    const uint16_t* w16 = static_cast<const uint16_t*>(w_gate);
    void* params[] = {&h16, &w16, &out_logits, &M, &E, &H};
    const dim3 grid((unsigned)E);
    if (hipLaunchKernel(gate_kernel(M, H), grid, dim3(kGateWaves * 64), params, 0, st) != hipSuccess)
      return MRS_ERR_LAUNCH;
  }
  // M <= 64: the route-sort runs in one workgroup (asked for explicitly), so it
  // needs no workspace
  return moe_route_sort_ex(out_logits, bias, M, E, k, n_group, topk_group, block, out_ids, out_w, sorted_ids,
                           expert_of_block, num_post_pad, MRS_DTYPE_F32, nullptr, 0, stream,
                           MRS_FLAG_FORCE_SINGLE_WG, nullptr);
}
