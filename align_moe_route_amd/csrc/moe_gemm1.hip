// Grouped GEMM1 over the route-sort metadata, MI355X (gfx950, CDNA4, wave64).
//
// The route-sort output is prepared for the first grouped GEMM and read by it
// directly (page "Kimi-K3 B1 route-sort + prepared-MoE handoff (stack)",
// Summary).  Definition and argument contract: include/moe_gemm1.h.
//
// A workgroup (4 or 8 waves) computes a BM x BN tile of y (BN = 128 or 256).
// BM divides the padding block, so the tile's rows all belong to one expert:
// expert_of_block gives the weight matrix, sorted_ids gives the token of each
// row (a padding row stores zeros into LDS and so produces zeros).  The K loop
// steps by 32 or 64 (k_gemm1): every thread fetches its 16-byte chunks of the next x and W
// tiles into registers while the waves run v_mfma_f32_32x32x16_bf16 on the
// current LDS tiles, then stores them into the other LDS buffer (one barrier
// per step).  LDS rows are XOR-swizzled by
// 16-byte chunk (swz below).  Each XCD takes runs of 8 consecutive row tiles
// (mostly one expert's) and, within a run, the row tiles of one column tile
// one after another (tile_of below), so the workgroups running together on
// an XCD share that expert's weight column tile in its L2.  num_post_pad is
// read on the device: tiles past it exit.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_gemm1.h"
#include "moe_route_sort.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kKAlign = 64;  // K is a multiple of this (every tile's K step divides it)

struct GArgs {
  const uint16_t* x;
  const uint16_t* w;
  const int32_t* sid;
  const int32_t* eob;
  const int32_t* npp;
  uint16_t* y;
  int M, k, E, K, N, block;
  int row_limit;  // rows the metadata can hold: (max_rows / block) * block
  int nrt;        // row tiles: row_limit / BM
};

// LDS slot of chunk c of tile row r (rows are 128 bytes): the chunk index is
// XORed with r mod 8 and, for the second eight rows of every sixteen, with 1
// as well.  Any eight rows starting at a multiple of 8 then read one logical
// chunk from eight distinct 16-byte positions of a 128-byte bank line, and
// any sixteen starting at a multiple of 16 from sixteen distinct positions of
// a 256-byte line, so the MFMA operand reads (32 rows at one chunk) are free
// of bank conflicts whether the LDS serves 128 or 256 bytes per cycle.
//
// With 64-byte rows (K steps of 32: four chunks) the chunk index is XORed
// with (r ^ (r >> 2)) mod 4, which moves a chunk to a different 16-byte
// position in each of four consecutive rows and in each of rows r, r + 4,
// r + 8, r + 12.  rocprofv3 counts no LDS bank-conflict cycles for this
// kernel with it; XOR with ((r >> 1) ^ (r >> 3)) mod 4 gave 36 % conflict
// cycles and rows padded to 80 bytes 30 %, both 1-2 % slower.
template <int CH>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (CH == 8) return r * CH + (c ^ (r & 7) ^ ((r >> 3) & 1));
  else return r * CH + (c ^ ((r ^ (r >> 2)) & 3));
}

// MI355X dispatches workgroup h to XCD h mod 8.  XCD x's j-th workgroup
// (h = 8 j + x) takes, in run m = j / (R ntn), column tile (j / R) mod ntn of
// row tile (8 m + x) R + j mod R: runs of R = kRunRows consecutive row tiles
// go to the XCDs in turn, and inside a run the R row tiles of a column tile
// are dispatched together.  On the 8192 x 896 prefill metadata this cut the
// bytes fetched past the L2 from 5.8 to 4.1 GB per call (row tiles dealt
// one by one to the XCDs: every XCD fetched every expert's weights) and the
// time by 2-3 %.  The grid covers whole runs; workgroups past the last row
// tile return false.
constexpr int kXcds = 8;
constexpr int kRunRows = 8;
__device__ __forceinline__ bool tile_of(int h, int ntn, int nrt, int& rt, int& ct) {
  const int x = h % kXcds, j = h / kXcds;
  const int m = j / (kRunRows * ntn), c = (j / kRunRows) % ntn, r = j % kRunRows;
  rt = (m * kXcds + x) * kRunRows + r;
  ct = c;
  return rt < nrt;
}

// FP32 to BF16, round to nearest even (the inputs are finite).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// A BM x BN tile per workgroup of BN / 32 waves (each wave 64 x 64 when
// BM >= 64): the 256-column tile halves the x traffic per MFMA.  The K step
// is 32 when every thread still has an x chunk to fetch (BM * 4 >= threads):
// the two LDS buffers then take 48 KiB for the 128 x 256 tile, so two
// workgroups share a compute unit (on the 8192 x 896 prefill metadata, 3-4 %
// faster than K steps of 64 with one workgroup per compute unit).
template <int BM, int BN>
__global__ __launch_bounds__(BN * 2) void k_gemm1(GArgs g) {
  constexpr int kThreads = BN * 2;
  constexpr int kBK = BM * 4 >= kThreads ? 32 : 64;  // K per pipeline step
  constexpr int kChunks = kBK / 8;                    // 16-byte chunks per tile row
  static_assert(kKAlign % kBK == 0, "K step");
  constexpr int NW = kThreads / 64;
  constexpr int WGM = BM >= 64 ? 2 : 1;   // waves along the rows
  constexpr int WGN = NW / WGM;           // waves along the columns
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;  // 32x32 MFMA tiles per wave
  constexpr int AP = BM * kChunks / kThreads;  // x chunks per thread per step
  constexpr int BP = BN * kChunks / kThreads;  // W chunks per thread per step
  static_assert(AP >= 1 && BP >= 1 && FM >= 1 && FN >= 1, "tile too small for the workgroup");
  __shared__ u32x4 As[2][BM * kChunks];
  __shared__ u32x4 Bs[2][BN * kChunks];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  int rt, ct;
  if (!tile_of((int)blockIdx.x, g.N / BN, g.nrt, rt, ct)) return;
  const int r0 = rt * BM;
  const int n0 = ct * BN;
  const int npp = min(*g.npp, g.row_limit);
  if (r0 + BM > npp) return;  // npp is a multiple of block and BM divides block
  const int e = g.eob[r0 / g.block];
  if (e < 0 || e >= g.E) return;

  // sources of this thread's chunks: rows of x through sorted_ids, rows of W[e]
  // (a padding row reads token 0's row and stores zeros instead, so every
  // load is unconditional)
  const u32x4* xa[AP];
  bool av[AP];
  const int routes = g.M * g.k;
#pragma unroll
  for (int p = 0; p < AP; ++p) {
    const int idx = tid + p * kThreads;
    const int r = idx / kChunks, c = idx % kChunks;
    const int s = g.sid[r0 + r];
    av[p] = s >= 0 && s < routes;
    const int t = av[p] ? s / g.k : 0;
    xa[p] = reinterpret_cast<const u32x4*>(g.x + (size_t)t * g.K) + c;
  }
  const u32x4* wb[BP];
#pragma unroll
  for (int p = 0; p < BP; ++p) {
    const int idx = tid + p * kThreads;
    const int n = idx / kChunks, c = idx % kChunks;
    wb[p] = reinterpret_cast<const u32x4*>(g.w + ((size_t)e * g.N + n0 + n) * g.K) + c;
  }

  u32x4 ra[AP], rb[BP];
  auto gload = [&](int kt) {
#pragma unroll
    for (int p = 0; p < AP; ++p) ra[p] = xa[p][kt * kChunks];
#pragma unroll
    for (int p = 0; p < BP; ++p) rb[p] = wb[p][kt * kChunks];
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < AP; ++p) {
      const int idx = tid + p * kThreads;
      As[buf][swz<kChunks>(idx / kChunks, idx % kChunks)] = av[p] ? ra[p] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int p = 0; p < BP; ++p) {
      const int idx = tid + p * kThreads;
      Bs[buf][swz<kChunks>(idx / kChunks, idx % kChunks)] = rb[p];
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

  const int wm = wv / WGN, wn = wv % WGN;
  const int lr = lane & 31, lh = lane >> 5;
  const int nk = g.K / kBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      // lanes 0-31 supply k [16kk, 16kk+8) of their row, lanes 32-63 the next 8
      const int c = kk * 2 + lh;
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = __builtin_bit_cast(bf16x8, As[cur][swz<kChunks>(wm * WTM + i * 32 + lr, c)]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8, Bs[cur][swz<kChunks>(wn * WTN + j * 32 + lr, c)]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // 32x32 accumulator layout: lane column lr; register q holds row
  // 8*(q/4) + 4*lh + q%4 of the 32-row tile
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = r0 + wm * WTM + i * 32 + 8 * (q / 4) + 4 * lh + (q % 4);
        const int col = n0 + wn * WTN + j * 32 + lr;
        g.y[(size_t)row * g.N + col] = f2bf(acc[i][j][q]);
      }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int gemm1_impl(const void* x, const void* w, const int32_t* sorted_ids, const int32_t* expert_of_block,
               const int32_t* num_post_pad, int M, int k, int E, int K, int N, int block, void* y,
               hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (M < 0 || k < 1 || k > 64 || E < 1 || E > 4096 || K <= 0 || K % kKAlign != 0 || N <= 0 ||
      N % 128 != 0 || block < 32 || block % 32 != 0)
    return MRS_ERR_INVALID_ARG;
  if (!x || !w || !sorted_ids || !expert_of_block || !num_post_pad || !y) return MRS_ERR_NULL_POINTER;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return MRS_ERR_MISALIGNED;
  const int64_t max_rows = moe_route_sort_max_rows(M, E, k, block);
  if (max_rows < 0) return MRS_ERR_OVERFLOW;
  const int64_t row_limit = max_rows / block * block;
  if (row_limit == 0) return MRS_OK;  // no token: nothing to write
  const int bm = block % 128 == 0 ? 128 : (block % 64 == 0 ? 64 : 32);
  const int bn = (bm >= 64 && N % 256 == 0) ? 256 : 128;
  const int64_t nrt = row_limit / bm, ntn = N / bn;
  // whole runs of kRunRows row tiles on every XCD (tile_of)
  const int64_t groups = ((nrt + kXcds * kRunRows - 1) / (kXcds * kRunRows)) * kRunRows;
  if (groups * kXcds * ntn > INT32_MAX) return MRS_ERR_OVERFLOW;
  GArgs g{static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), sorted_ids, expert_of_block,
          num_post_pad, static_cast<uint16_t*>(y), M, k, E, K, N, block, (int)row_limit, (int)nrt};
  const void* fn = bm == 128 ? (bn == 256 ? reinterpret_cast<const void*>(k_gemm1<128, 256>)
                                          : reinterpret_cast<const void*>(k_gemm1<128, 128>))
                   : bm == 64 ? (bn == 256 ? reinterpret_cast<const void*>(k_gemm1<64, 256>)
                                           : reinterpret_cast<const void*>(k_gemm1<64, 128>))
                              : reinterpret_cast<const void*>(k_gemm1<32, 128>);
  const dim3 grid((unsigned)(groups * kXcds * ntn));
  void* params[] = {&g};
  hipError_t err;
  if (ev0 && ev1)
    err = hipExtLaunchKernel(fn, grid, dim3(bn * 2), params, 0, stream, ev0, ev1, 0);
  else
    err = hipLaunchKernel(fn, grid, dim3(bn * 2), params, 0, stream);
  return err == hipSuccess ? MRS_OK : MRS_ERR_LAUNCH;
}

}  // namespace

extern "C" int moe_grouped_gemm1(const void* x, const void* w, const int32_t* sorted_ids,
                                 const int32_t* expert_of_block, const int32_t* num_post_pad, int M,
                                 int k, int E, int K, int N, int block, void* y, hipStream_t stream) {
  return gemm1_impl(x, w, sorted_ids, expert_of_block, num_post_pad, M, k, E, K, N, block, y, stream,
                    nullptr, nullptr);
}

extern "C" int moe_grouped_gemm1_profiled(const void* x, const void* w, const int32_t* sorted_ids,
                                          const int32_t* expert_of_block, const int32_t* num_post_pad,
                                          int M, int k, int E, int K, int N, int block, void* y,
                                          hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (!start || !stop) return MRS_ERR_NULL_POINTER;
  return gemm1_impl(x, w, sorted_ids, expert_of_block, num_post_pad, M, k, E, K, N, block, y, stream,
                    start, stop);
}
