// MoE route-sort for MI355X (gfx950, CDNA4, wave64): kernels and C ABI.
//
// The path (page "Kimi-K3 B1 route-sort + prepared-MoE handoff (stack)",
// Summary): FP32 conversion of router logits, per-expert correction bias,
// grouped top-k, then the two sort phases that produce expert-sorted,
// block-padded dispatch metadata for a grouped GEMM.  Exact definitions of
// every output are in include/moe_route_sort.h.
//
// Structure
//   selection   one wave64 per token.  Keys are ranked with a fast sigmoid
//               (v_exp_f32 + v_rcp_f32) whose error is bounded; a token whose
//               k-th/(k+1)-th key gap or group-boundary gap is wider than that
//               bound is decided exactly by the fast ranking ("certified").
//               Every other token -- and every token of a shape the wave
//               layout does not cover -- is re-decided by the whole workgroup
//               from correctly rounded keys.  Weights always use the correctly
//               rounded sigmoid.
//   histogram   per-workgroup LDS bitsets: bit tl of word e is set when the
//               workgroup's token tl picked expert e.  The popcount is the
//               workgroup's histogram (replacing one contended global atomic
//               per route, as on the page "gfx1250 ordinary-TP route
//               optimization", Summary), and the popcount of the bits below tl
//               is the slot's stable rank inside the workgroup.
//   prefix      column scan of the workgroup histograms in workgroup order,
//               then an exclusive scan of the padded per-expert totals.
//   scatter     slot -> off[e] + (routes to e in earlier workgroups) +
//               (earlier tokens of this workgroup with e): a stable counting
//               sort, so the order never depends on scheduling.
// Small calls (M <= 64) run everything in one workgroup and one launch.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_route_sort.h"

namespace {

constexpr int kWave = 64;
constexpr int kWG = 256;                 // threads per workgroup, all kernels
constexpr int kNWaves = kWG / kWave;
constexpr int kTwMax = 64;               // tokens per workgroup: one bit each in a 64-bit word
constexpr int kEMax = 4096;              // 16 KiB of 32-bit counters, the pages' LDS bound
constexpr int kEptMax = kEMax / kWG;     // experts per thread in the exact selection
constexpr int kSmallSlotsMax = 2048;     // M*k bound of the single-workgroup path
constexpr size_t kLdsLimit = 64 * 1024;
constexpr size_t kWsHeader = 256;

enum { KIND_SMALL = 0, KIND_SELECT = 1, KIND_SCATTER = 2 };

struct Args {
  const void* logits;
  const float* bias;
  int M, E, k, n_group, topk_group, block;
  int G;       // experts per group
  int tw;      // tokens per workgroup
  int nwg;     // workgroups of the multi-workgroup path
  int fast;    // the wave layout covers this shape
  int gstage;  // the group stage changes the result (1 < topk_group < n_group, G > 1)
  int32_t* out_ids;
  float* out_w;
  int32_t* sorted_ids;
  int32_t* eob;
  int32_t* npp;
  int32_t* ws_cnt;   // [E]
  int32_t* ws_pad;   // [E]
  int32_t* ws_hist;  // [nwg][E]
  int32_t* stats;
};

// ----------------------------------------------------------------------------
// LDS plan shared by host (size) and device (carving).
// ----------------------------------------------------------------------------
struct LdsPlan {
  size_t bits, redd, off, ids, cand_a, cand_i, esc, grp, misc, red, scan, total;
};

__host__ __device__ inline LdsPlan lds_plan(int kind, int E, int n_group, int gstage, int tw, int k) {
  LdsPlan p{};
  size_t o = 0;
  p.bits = o; o += (size_t)E * 8;
  p.redd = o; o += (size_t)kNWaves * 8;
  if (kind != KIND_SELECT) { p.off = o; o += (size_t)E * 4; }
  if (kind == KIND_SMALL) { p.ids = o; o += (size_t)tw * k * 4; }
  if (kind != KIND_SCATTER) {
    p.cand_a = o; o += (size_t)kNWaves * kWave * 4;
    p.cand_i = o; o += (size_t)kNWaves * kWave * 4;
    p.esc = o; o += (size_t)kTwMax * 4;
    p.grp = o; o += gstage ? (size_t)3 * n_group * 4 : 0;
  }
  p.misc = o; o += 16 * 4;
  p.red = o; o += (size_t)2 * kNWaves * 4;
  p.scan = o; o += (size_t)kNWaves * 4;
  p.total = (o + 15) & ~(size_t)15;
  return p;
}

struct Lds {
  unsigned long long* bits;
  double* redd;
  int* off;
  int* ids;
  float* cand_a;
  int* cand_i;
  int* esc;
  unsigned* grp;
  int* misc;
  int* red;
  int* scan;
};

extern __shared__ __align__(16) unsigned char g_lds[];

__device__ inline Lds carve(int kind, const Args& a) {
  const LdsPlan p = lds_plan(kind, a.E, a.n_group, a.gstage, a.tw, a.k);
  Lds L;
  L.bits = reinterpret_cast<unsigned long long*>(g_lds + p.bits);
  L.redd = reinterpret_cast<double*>(g_lds + p.redd);
  L.off = reinterpret_cast<int*>(g_lds + p.off);
  L.ids = reinterpret_cast<int*>(g_lds + p.ids);
  L.cand_a = reinterpret_cast<float*>(g_lds + p.cand_a);
  L.cand_i = reinterpret_cast<int*>(g_lds + p.cand_i);
  L.esc = reinterpret_cast<int*>(g_lds + p.esc);
  L.grp = reinterpret_cast<unsigned*>(g_lds + p.grp);
  L.misc = reinterpret_cast<int*>(g_lds + p.misc);
  L.red = reinterpret_cast<int*>(g_lds + p.red);
  L.scan = reinterpret_cast<int*>(g_lds + p.scan);
  return L;
}

// ----------------------------------------------------------------------------
// Scalar helpers.
// ----------------------------------------------------------------------------
// Order-preserving map of FP32 onto uint32 (larger float -> larger integer).
__device__ __forceinline__ uint32_t f2s(float f) {
  const uint32_t u = __float_as_uint(f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float s2f(uint32_t s) {
  return __uint_as_float((s & 0x80000000u) ? (s ^ 0x80000000u) : ~s);
}
__device__ __forceinline__ float next_down(float f) {
  uint32_t u = __float_as_uint(f);
  if (f > 0.0f) u -= 1u;
  else if (f < 0.0f) u += 1u;
  else u = 0x80000001u;
  return __uint_as_float(u);
}
__device__ __forceinline__ int pad_up(int c, int block) {
  return c == 0 ? 0 : ((c - 1) / block + 1) * block;
}

template <bool BF16>
__device__ __forceinline__ float load_logit(const void* base, size_t i) {
  if constexpr (BF16) {
    const uint16_t h = reinterpret_cast<const uint16_t*>(base)[i];
    return __uint_as_float((uint32_t)h << 16);  // BF16 is the top half of FP32
  } else {
    return reinterpret_cast<const float*>(base)[i];
  }
}

// Fast sigmoid for ranking: 1 / (1 + 2^(-x*log2(e))) with the hardware
// exp2 and reciprocal.  Its distance to the correctly rounded sigmoid is below
// 2^-21 for every FP32 x (about 2.6e-7 from the error terms: argument rounding,
// 1-ulp exp2, rounding of 1+e, 1-ulp reciprocal); the certification margins
// below are built on 2^-21.
__device__ __forceinline__ float sigmoid_fast(float x) {
  const float e = __builtin_amdgcn_exp2f(x * -1.44269504088896341f);
  return __builtin_amdgcn_rcpf(1.0f + e);
}

// Correctly rounded FP32 sigmoid.  For |x| < 2^-10 the float64 quotient can
// land exactly on an FP32 rounding midpoint (0.5 + x/4 is one for many BF16
// x) while the cubic term, below float64 resolution at 0.5, decides the side;
// there the series 1/2 + x/4 - x^3/48 + x^5/480 is split into an exact head
// and a small tail and the rounding side is read off their sum.  Elsewhere
// RN32 of the float64 value 1 / (1 + exp(-x)).
__device__ __noinline__ float sigmoid_exact(float x) {
  const double xd = (double)x;
  if (fabs(xd) < 0x1p-10) {
    const double hi = 0.5 + 0.25 * xd;  // exact for |x| >= 2^-29; else far from a midpoint
    const double x2 = xd * xd;
    const double lo = xd * x2 * (-1.0 / 48.0 + x2 * (1.0 / 480.0));
    const float f = (float)hi;
    const double fb = (double)f;
    if (fb == hi) return f;
    const uint32_t fu = __float_as_uint(f);
    const float g = __uint_as_float(fb > hi ? fu - 1u : fu + 1u);  // other neighbour of hi
    const double gb = (double)g;
    const double mid = 0.5 * (fb + gb);
    const double d = (hi - mid) + lo;  // side of the midpoint the exact value lies on
    const float up = fb > gb ? f : g;
    const float dn = fb > gb ? g : f;
    if (d > 0.0) return up;
    if (d < 0.0) return dn;
    return (__float_as_uint(up) & 1u) ? dn : up;
  }
  const double e = exp(-xd);
  return (float)(1.0 / (1.0 + e));
}

// ----------------------------------------------------------------------------
// Wave-level helpers (wave64).
// ----------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// m-th largest of the per-lane values v (lanes that do not take part pass 0;
// at least m lanes take part).  Bitwise bisection: one compare + ballot per bit.
__device__ __forceinline__ uint32_t wave_kth(uint32_t v, int m) {
  uint32_t T = 0;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = T | (1u << b);
    if (__popcll(__ballot(v >= c)) >= m) T = c;
  }
  return T;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d));
  return v;
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(v, d);
    if (l >= d) v += y;
  }
  return v;
}

// ----------------------------------------------------------------------------
// Workgroup-level helpers (all kWG threads must call them).
// ----------------------------------------------------------------------------
__device__ int wg_excl_scan(const Lds& L, int v) {
  const int w = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane_id() == kWave - 1) L.scan[w] = x;
  __syncthreads();
  int pre = 0;
  for (int q = 0; q < w; ++q) pre += L.scan[q];
  __syncthreads();
  return pre + x - v;
}

__device__ double wg_sum_d(const Lds& L, double v) {
  const int w = threadIdx.x >> 6;
  v = wave_sum_d(v);
  if (lane_id() == 0) L.redd[w] = v;
  __syncthreads();
  double s = 0.0;
  for (int q = 0; q < kNWaves; ++q) s += L.redd[q];
  __syncthreads();
  return s;
}

__device__ float wg_max_f(const Lds& L, float v) {
  const int w = threadIdx.x >> 6;
  v = wave_max_f(v);
  if (lane_id() == 0) L.red[w] = __float_as_int(v);
  __syncthreads();
  float m = v;
  for (int q = 0; q < kNWaves; ++q) m = fmaxf(m, __int_as_float(L.red[q]));
  __syncthreads();
  return m;
}

// Number of (mask-selected) values >= c over the workgroup.  `parity` picks
// one of two LDS buffers so consecutive calls need a single barrier each.
__device__ __forceinline__ int wg_count_ge(const Lds& L, const uint32_t* u, uint32_t mask, uint32_t c,
                                           int parity) {
  int n = 0;
#pragma unroll
  for (int i = 0; i < kEptMax; ++i) n += __popcll(__ballot(((mask >> i) & 1u) && u[i] >= c));
  const int w = threadIdx.x >> 6;
  if (lane_id() == 0) L.red[parity * kNWaves + w] = n;
  __syncthreads();
  int s = 0;
  for (int q = 0; q < kNWaves; ++q) s += L.red[parity * kNWaves + q];
  return s;
}

// Select the m largest values (ties to the lower index) among the mask-
// selected entries; thread r holds entries [r*n, (r+1)*n) in index order.
// Returns this thread's selection bits.
__device__ uint32_t wg_select(const Lds& L, const uint32_t* u, uint32_t mask, int m) {
  uint32_t T = 0;
  int parity = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = T | (1u << b);
    if (wg_count_ge(L, u, mask, c, parity) >= m) T = c;
    parity ^= 1;
  }
  const int gt = (T == 0xFFFFFFFFu) ? 0 : wg_count_ge(L, u, mask, T + 1u, parity);
  const int r = m - gt;  // equal values to take, lowest index first
  uint32_t sel = 0, tie = 0;
#pragma unroll
  for (int i = 0; i < kEptMax; ++i) {
    if ((mask >> i) & 1u) {
      if (u[i] > T) sel |= 1u << i;
      else if (u[i] == T) tie |= 1u << i;
    }
  }
  int rank = wg_excl_scan(L, __popc(tie));
#pragma unroll
  for (int i = 0; i < kEptMax; ++i) {
    if ((tie >> i) & 1u) {
      if (rank < r) sel |= 1u << i;
      ++rank;
    }
  }
  return sel;
}

// ----------------------------------------------------------------------------
// Exact selection of one token by the whole workgroup (correctly rounded keys).
// Thread r owns experts [r*ept, (r+1)*ept).
// ----------------------------------------------------------------------------
template <bool BF16>
__device__ void exact_token(const Args& a, const Lds& L, int t, int tl, int* ids_cache) {
  const int tid = threadIdx.x;
  const int E = a.E, G = a.G;
  const int ept = (E + kWG - 1) / kWG;
  const int e0 = tid * ept;
  const size_t row = (size_t)t * E;
  uint32_t u[kEptMax];
  uint32_t valid = 0;
#pragma unroll
  for (int i = 0; i < kEptMax; ++i) {
    u[i] = 0;
    const int e = e0 + i;
    if (i < ept && e < E) {
      const float s = sigmoid_exact(load_logit<BF16>(a.logits, row + e));
      u[i] = f2s(s + a.bias[e]);
      valid |= 1u << i;
    }
  }
  uint32_t allow = valid;
  if (a.gstage) {
    unsigned* gmax = L.grp;
    unsigned* gsc = L.grp + a.n_group;   // count of the maximum, then the group score
    unsigned* gsec = L.grp + 2 * a.n_group;  // largest value below the maximum, then the flags
    for (int g = tid; g < a.n_group; g += kWG) { gmax[g] = 0u; gsc[g] = 0u; gsec[g] = 0u; }
    __syncthreads();
    {  // group maxima
      int cg = -1;
      uint32_t cm = 0;
#pragma unroll
      for (int i = 0; i < kEptMax; ++i) {
        if ((valid >> i) & 1u) {
          const int g = (e0 + i) / G;
          if (g != cg) {
            if (cg >= 0) atomicMax(&gmax[cg], cm);
            cg = g;
            cm = 0;
          }
          cm = u[i] > cm ? u[i] : cm;
        }
      }
      if (cg >= 0) atomicMax(&gmax[cg], cm);
    }
    __syncthreads();
    {  // how often the maximum occurs, and the largest value below it
      int cg = -1;
      uint32_t gm = 0, c = 0, m2 = 0;
#pragma unroll
      for (int i = 0; i < kEptMax; ++i) {
        if ((valid >> i) & 1u) {
          const int g = (e0 + i) / G;
          if (g != cg) {
            if (cg >= 0) {
              if (c) atomicAdd(&gsc[cg], c);
              if (m2) atomicMax(&gsec[cg], m2);
            }
            cg = g;
            gm = gmax[g];
            c = 0;
            m2 = 0;
          }
          if (u[i] == gm) ++c;
          else m2 = u[i] > m2 ? u[i] : m2;
        }
      }
      if (cg >= 0) {
        if (c) atomicAdd(&gsc[cg], c);
        if (m2) atomicMax(&gsec[cg], m2);
      }
    }
    __syncthreads();
    for (int g = tid; g < a.n_group; g += kWG) {  // group score = top1 + top2 (FP32)
      const float t1 = s2f(gmax[g]);
      const float t2 = gsc[g] >= 2u ? t1 : s2f(gsec[g]);
      gsc[g] = f2s(t1 + t2);
    }
    __syncthreads();
    const int gpt = (a.n_group + kWG - 1) / kWG;
    const int g0 = tid * gpt;
    uint32_t gu[kEptMax];
    uint32_t gval = 0;
#pragma unroll
    for (int i = 0; i < kEptMax; ++i) {
      gu[i] = 0;
      if (i < gpt && g0 + i < a.n_group) {
        gu[i] = gsc[g0 + i];
        gval |= 1u << i;
      }
    }
    const uint32_t gsel = wg_select(L, gu, gval, a.topk_group);
#pragma unroll
    for (int i = 0; i < kEptMax; ++i)
      if ((gval >> i) & 1u) gsec[g0 + i] = (gsel >> i) & 1u;
    __syncthreads();
    allow = 0;
#pragma unroll
    for (int i = 0; i < kEptMax; ++i)
      if (((valid >> i) & 1u) && gsec[(e0 + i) / G]) allow |= 1u << i;
    __syncthreads();
  }
  const uint32_t sel = wg_select(L, u, allow, a.k);
  double part = 0.0;
#pragma unroll
  for (int i = 0; i < kEptMax; ++i)
    if ((sel >> i) & 1u) part += (double)sigmoid_exact(load_logit<BF16>(a.logits, row + e0 + i));
  const double ssum = wg_sum_d(L, part);
  int pos = wg_excl_scan(L, __popc(sel));
#pragma unroll
  for (int i = 0; i < kEptMax; ++i) {
    if ((sel >> i) & 1u) {
      const int e = e0 + i;
      const double s = (double)sigmoid_exact(load_logit<BF16>(a.logits, row + e));
      a.out_ids[(size_t)t * a.k + pos] = e;
      a.out_w[(size_t)t * a.k + pos] = (float)(s / ssum);
      atomicOr(&L.bits[e], 1ull << tl);
      if (ids_cache) ids_cache[tl * a.k + pos] = e;
      ++pos;
    }
  }
}

// ----------------------------------------------------------------------------
// Fast certified selection of one token by one wave.  Layout: E % 64 == 0 and
// n_group divides 64; lane l owns the contiguous experts [l*epl, (l+1)*epl),
// so group g is owned by the 64/n_group consecutive lanes starting at
// g*64/n_group.  Returns false when the token must be decided exactly.
// ----------------------------------------------------------------------------
template <int EPLM, bool BF16>
__device__ bool fast_token(const Args& a, const Lds& L, int t, int tl, double delta, double epsg,
                           int* ids_cache) {
  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  const int epl = a.E >> 6;
  const int lpg = kWave / a.n_group;
  const int e0 = lane * epl;
  const size_t row = (size_t)t * a.E;

  // keys from the fast sigmoid; lane-local top-2
  float av[EPLM];
  float lm = -INFINITY, l2 = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPLM; ++i) {
    av[i] = -INFINITY;
    if (i < epl) {
      const float x = load_logit<BF16>(a.logits, row + e0 + i);
      const float key = sigmoid_fast(x) + a.bias[e0 + i];
      av[i] = key;
      l2 = fmaxf(l2, fminf(lm, key));
      lm = fmaxf(lm, key);
    }
  }

  bool allowed = true;
  if (a.gstage) {
    // group top-2 over the lpg lanes of the group, then group score
    float g1 = lm, g2 = l2;
    for (int d = 1; d < lpg; d <<= 1) {
      const float p1 = __shfl_xor(g1, d);
      const float p2 = __shfl_xor(g2, d);
      const float n2 = fmaxf(fminf(g1, p1), fmaxf(g2, p2));
      g1 = fmaxf(g1, p1);
      g2 = n2;
    }
    const float gs = g1 + g2;
    const bool leader = (lane % lpg) == 0;
    const uint32_t gsu = leader ? f2s(gs) : 0u;
    const uint32_t aG = wave_kth(gsu, a.topk_group);
    const uint32_t bG = wave_kth(gsu, a.topk_group + 1);
    const double gap = (double)s2f(aG) - (double)s2f(bG);
    if (!(gap > 2.0 * epsg)) return false;  // group boundary not certified
    allowed = f2s(gs) >= aG;
  }

  // candidate threshold: the k-th largest lane maximum among allowed lanes is
  // a lower bound of the k-th largest key (k distinct lanes reach it)
  if (__popcll(__ballot(allowed)) < a.k) return false;
  const uint32_t tau0 = wave_kth(allowed ? f2s(lm) : 0u, a.k);
  const float thr = next_down((float)((double)s2f(tau0) - 2.0 * delta));
  unsigned long long cflags = 0;
  int mine = 0;
#pragma unroll
  for (int i = 0; i < EPLM; ++i) {
    if (i < epl && allowed && av[i] >= thr) {
      cflags |= 1ull << i;
      ++mine;
    }
  }
  const int total = wave_sum_i(mine);
  if (total > kWave) return false;
  int slot = wave_incl_scan(mine) - mine;
  float* ca_buf = L.cand_a + w * kWave;
  int* ci_buf = L.cand_i + w * kWave;
#pragma unroll
  for (int i = 0; i < EPLM; ++i) {
    if ((cflags >> i) & 1ull) {
      ca_buf[slot] = av[i];
      ci_buf[slot] = e0 + i;
      ++slot;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  // one candidate per lane, in expert order
  const bool has = lane < total;
  const float ca = has ? ca_buf[lane] : -INFINITY;
  const int ci = has ? ci_buf[lane] : 0;
  __builtin_amdgcn_wave_barrier();
  const uint32_t cu = has ? f2s(ca) : 0u;
  const uint32_t kth = wave_kth(cu, a.k);
  if (__popcll(__ballot(has && cu >= kth)) != a.k) return false;  // tie at the k-th key
  if (total > a.k) {
    const float nxt = wave_max_f((has && cu < kth) ? ca : -INFINITY);
    const double gap = (double)s2f(kth) - (double)nxt;
    if (!(gap > 2.0 * delta)) return false;  // k-th / (k+1)-th boundary not certified
  }
  // certified: the k lanes with key >= kth are the exact picks
  const bool sel = has && cu >= kth;
  const unsigned long long selm = __ballot(sel);
  const int pos = __popcll(selm & ((1ull << lane) - 1ull));
  double s = 0.0;
  if (sel) s = (double)sigmoid_exact(load_logit<BF16>(a.logits, row + ci));
  const double ssum = wave_sum_d(s);
  if (sel) {
    a.out_ids[(size_t)t * a.k + pos] = ci;
    a.out_w[(size_t)t * a.k + pos] = (float)(s / ssum);
    atomicOr(&L.bits[ci], 1ull << tl);
    if (ids_cache) ids_cache[tl * a.k + pos] = ci;
  }
  return true;
}

// Selection of tokens [t0, t0+nt) by one workgroup, with the histogram bitsets.
template <int EPLM, bool BF16>
__device__ void select_tokens(const Args& a, const Lds& L, int t0, int nt, int* ids_cache) {
  const int tid = threadIdx.x;
  for (int e = tid; e < a.E; e += kWG) L.bits[e] = 0ull;
  if (tid == 0) L.misc[0] = 0;
  float bm = 0.0f;
  for (int e = tid; e < a.E; e += kWG) bm = fmaxf(bm, fabsf(a.bias[e]));
  bm = wg_max_f(L, bm);  // contains barriers
  // |fast key - exact key| <= 2^-21 + (rounding of both sums) <= delta;
  // |fast group score - exact group score| <= 2*delta + rounding <= epsg
  const double B = 1.0 + (double)bm + 0x1p-20;  // bound on |key|
  const double delta = 0x1p-21 + (B + 1.0) * 0x1p-23;
  const double epsg = 2.0 * delta + (2.0 * B + 1.0) * 0x1p-23;
  if (a.fast) {
    const int w = tid >> 6;
    for (int tl = w; tl < nt; tl += kNWaves) {
      const bool ok = fast_token<EPLM, BF16>(a, L, t0 + tl, tl, delta, epsg, ids_cache);
      if (!ok && lane_id() == 0) {
        const int q = atomicAdd(&L.misc[0], 1);
        L.esc[q] = tl;
      }
    }
  } else {
    for (int tl = tid; tl < nt; tl += kWG) L.esc[tl] = tl;
    if (tid == 0) L.misc[0] = nt;
  }
  __syncthreads();
  const int nesc = L.misc[0];
  for (int q = 0; q < nesc; ++q) {
    const int tl = L.esc[q];
    exact_token<BF16>(a, L, t0 + tl, tl, ids_cache);
  }
  if (tid == 0 && a.stats) {
    atomicAdd(&a.stats[0], nesc);
    atomicAdd(&a.stats[1], nt - nesc);
  }
  __syncthreads();
}

// Exclusive scan of padded counts over all experts into L.off; returns the
// total (valid in every thread).  `padded(e)` gives expert e's padded count.
template <typename F>
__device__ int expert_offsets(const Args& a, const Lds& L, F padded) {
  const int tid = threadIdx.x;
  const int ept = (a.E + kWG - 1) / kWG;
  const int e0 = tid * ept;
  int local = 0;
  for (int i = 0; i < ept; ++i) {
    const int e = e0 + i;
    if (e < a.E) {
      const int p = padded(e);
      L.off[e] = p;
      local += p;
    }
  }
  int pre = wg_excl_scan(L, local);
  for (int i = 0; i < ept; ++i) {
    const int e = e0 + i;
    if (e < a.E) {
      const int p = L.off[e];
      L.off[e] = pre;
      pre += p;
    }
  }
  if (tid == kWG - 1) L.misc[1] = pre;
  __syncthreads();
  return L.misc[1];
}

// ----------------------------------------------------------------------------
// Kernels.
// ----------------------------------------------------------------------------
// Everything in one workgroup (M <= 64): one launch per call.
template <int EPLM, bool BF16>
__global__ __launch_bounds__(kWG) void k_small(Args a) {
  const Lds L = carve(KIND_SMALL, a);
  select_tokens<EPLM, BF16>(a, L, 0, a.M, L.ids);
  const int tid = threadIdx.x;
  const int total = expert_offsets(a, L, [&](int e) { return pad_up(__popcll(L.bits[e]), a.block); });
  if (tid == 0) *a.npp = total;
  const int sentinel = a.M * a.k;
  for (int e = tid; e < a.E; e += kWG) {
    const int c = __popcll(L.bits[e]);
    const int p = pad_up(c, a.block);
    const int o = L.off[e];
    for (int r = c; r < p; ++r) a.sorted_ids[o + r] = sentinel;
    for (int b = o / a.block; b < (o + p) / a.block; ++b) a.eob[b] = e;
  }
  for (int q = tid; q < sentinel; q += kWG) {
    const int tl = q / a.k;
    const int e = L.ids[q];
    const int rank = __popcll(L.bits[e] & ((1ull << tl) - 1ull));
    a.sorted_ids[L.off[e] + rank] = q;
  }
}

// Multi-workgroup path, launch 1: selection and per-workgroup histograms.
template <int EPLM, bool BF16>
__global__ __launch_bounds__(kWG) void k_select(Args a) {
  const Lds L = carve(KIND_SELECT, a);
  const int w = blockIdx.x;
  const int t0 = w * a.tw;
  const int nt = min(a.tw, a.M - t0);
  select_tokens<EPLM, BF16>(a, L, t0, nt, nullptr);
  for (int e = threadIdx.x; e < a.E; e += kWG)
    a.ws_hist[(size_t)w * a.E + e] = __popcll(L.bits[e]);
}

// Launch 2: per expert, exclusive scan of the histogram column in workgroup
// order (in place) and the padded total.  64 experts x 4 row ranges per block.
__global__ __launch_bounds__(kWG) void k_colscan(Args a) {
  __shared__ int part[kNWaves][kWave];
  const int ex = threadIdx.x & (kWave - 1);
  const int pt = threadIdx.x >> 6;
  const int e = blockIdx.x * kWave + ex;
  const int chunk = (a.nwg + kNWaves - 1) / kNWaves;
  const int w0 = pt * chunk;
  const int w1 = min(a.nwg, w0 + chunk);
  int s = 0;
  if (e < a.E)
    for (int w = w0; w < w1; ++w) s += a.ws_hist[(size_t)w * a.E + e];
  part[pt][ex] = s;
  __syncthreads();
  int pre = 0, total = 0;
  for (int q = 0; q < kNWaves; ++q) {
    if (q < pt) pre += part[q][ex];
    total += part[q][ex];
  }
  if (e < a.E) {
    int run = pre;
    for (int w = w0; w < w1; ++w) {
      const size_t i = (size_t)w * a.E + e;
      const int v = a.ws_hist[i];
      a.ws_hist[i] = run;
      run += v;
    }
    if (pt == 0) {
      a.ws_cnt[e] = total;
      a.ws_pad[e] = pad_up(total, a.block);
    }
  }
}

// Launch 3: expert offsets, padding, expert_of_block and the stable scatter.
__global__ __launch_bounds__(kWG) void k_scatter(Args a) {
  const Lds L = carve(KIND_SCATTER, a);
  const int tid = threadIdx.x;
  const int w = blockIdx.x;
  const int t0 = w * a.tw;
  const int nt = min(a.tw, a.M - t0);
  for (int e = tid; e < a.E; e += kWG) L.bits[e] = 0ull;
  const int total = expert_offsets(a, L, [&](int e) { return a.ws_pad[e]; });
  if (w == 0 && tid == 0) *a.npp = total;
  const int sentinel = a.M * a.k;
  const int es0 = (int)((int64_t)w * a.E / a.nwg);
  const int es1 = (int)((int64_t)(w + 1) * a.E / a.nwg);
  for (int e = es0; e < es1; ++e) {
    const int c = a.ws_cnt[e];
    const int p = a.ws_pad[e];
    const int o = L.off[e];
    for (int r = c + tid; r < p; r += kWG) a.sorted_ids[o + r] = sentinel;
    for (int b = tid; b < p / a.block; b += kWG) a.eob[o / a.block + b] = e;
  }
  const int ns = nt * a.k;
  const int32_t* ids = a.out_ids + (size_t)t0 * a.k;
  for (int q = tid; q < ns; q += kWG) atomicOr(&L.bits[ids[q]], 1ull << (q / a.k));
  __syncthreads();
  const int32_t* colpre = a.ws_hist + (size_t)w * a.E;
  for (int q = tid; q < ns; q += kWG) {
    const int tl = q / a.k;
    const int e = ids[q];
    const int rank = colpre[e] + __popcll(L.bits[e] & ((1ull << tl) - 1ull));
    a.sorted_ids[L.off[e] + rank] = t0 * a.k + q;
  }
}

__global__ void k_zero_npp(int32_t* npp) { *npp = 0; }

__global__ __launch_bounds__(kWG) void k_sigmoid_probe(const float* x, int n, float* f, float* e) {
  const int i = blockIdx.x * kWG + threadIdx.x;
  if (i < n) {
    f[i] = sigmoid_fast(x[i]);
    e[i] = sigmoid_exact(x[i]);
  }
}

// ----------------------------------------------------------------------------
// Host side.
// ----------------------------------------------------------------------------
int choose_tw(int M) {
  int tw = (M + 511) / 512;
  if (tw < 4) tw = 4;
  if (tw > kTwMax) tw = kTwMax;
  return tw;
}

bool valid_sizes(int M, int E, int k, int block) {
  return M >= 0 && E >= 1 && E <= kEMax && k >= 1 && k <= 64 && block >= 1;
}

int64_t max_rows_of(int M, int E, int k, int block) {
  const int64_t routes = (int64_t)M * k;
  const int64_t r = routes + (routes < E ? routes : (int64_t)E) * (int64_t)(block - 1);
  return r;
}

size_t workspace_of(int M, int E) {
  if (M == 0) return 0;
  const int tw = choose_tw(M);
  const int64_t nwg = ((int64_t)M + tw - 1) / tw;
  return kWsHeader + (size_t)2 * E * 4 + (size_t)nwg * E * 4;
}

int eplm_bucket(int epl) {
  int b = 1;
  while (b < epl) b <<= 1;
  return b;
}

typedef void (*KernelFn)(Args);

#define MRS_PICK(KER)                                                                 \
  KernelFn pick_##KER(int eplm, bool bf16) {                                          \
    switch (eplm) {                                                                   \
      case 1: return bf16 ? KER<1, true> : KER<1, false>;                             \
      case 2: return bf16 ? KER<2, true> : KER<2, false>;                             \
      case 4: return bf16 ? KER<4, true> : KER<4, false>;                             \
      case 8: return bf16 ? KER<8, true> : KER<8, false>;                             \
      case 16: return bf16 ? KER<16, true> : KER<16, false>;                          \
      case 32: return bf16 ? KER<32, true> : KER<32, false>;                          \
      default: return bf16 ? KER<64, true> : KER<64, false>;                          \
    }                                                                                 \
  }
MRS_PICK(k_small)
MRS_PICK(k_select)
#undef MRS_PICK

int launch(KernelFn fn, int grid, size_t lds, hipStream_t stream, Args* a) {
  void* params[] = {a};
  const hipError_t err =
      hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(kWG), params, lds, stream);
  return err == hipSuccess ? MRS_OK : MRS_ERR_LAUNCH;
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

}  // namespace

// ----------------------------------------------------------------------------
// C ABI.
// ----------------------------------------------------------------------------
extern "C" {

const char* moe_route_sort_strerror(int code) {
  switch (code) {
    case MRS_OK: return "ok";
    case MRS_ERR_INVALID_ARG: return "invalid argument (size, mode or flag outside the contract)";
    case MRS_ERR_NULL_POINTER: return "required pointer is NULL";
    case MRS_ERR_MISALIGNED: return "misaligned pointer (logits need 16 bytes, other arrays 4)";
    case MRS_ERR_WORKSPACE: return "workspace missing or too small";
    case MRS_ERR_OVERFLOW: return "M*k or the sorted-row capacity does not fit int32";
    case MRS_ERR_LAUNCH: return "HIP kernel launch failed";
    default: return "unknown error code";
  }
}

int64_t moe_route_sort_max_rows(int M, int E, int k, int block) {
  if (!valid_sizes(M, E, k, block)) return -1;
  const int64_t r = max_rows_of(M, E, k, block);
  return r > INT32_MAX ? -1 : r;
}

int64_t moe_route_sort_max_blocks(int M, int E, int k, int block) {
  const int64_t r = moe_route_sort_max_rows(M, E, k, block);
  return r < 0 ? -1 : r / block;
}

size_t moe_route_sort_workspace_bytes(int M, int E, int k, int block) {
  if (!valid_sizes(M, E, k, block)) return (size_t)-1;
  return workspace_of(M, E);
}

int moe_route_sort_ex(const void* logits, const float* bias, int M, int E, int k, int n_group,
                      int topk_group, int block, int32_t* out_ids, float* out_w,
                      int32_t* sorted_ids, int32_t* expert_of_block, int32_t* num_post_pad,
                      int logits_dtype, void* workspace, size_t workspace_bytes, void* stream,
                      unsigned flags, int32_t* stats) {
  const unsigned known = MRS_FLAG_FORCE_SINGLE_WG | MRS_FLAG_FORCE_MULTI_WG | MRS_FLAG_FORCE_EXACT;
  if ((flags & ~known) != 0u) return MRS_ERR_INVALID_ARG;
  if ((flags & MRS_FLAG_FORCE_SINGLE_WG) && (flags & MRS_FLAG_FORCE_MULTI_WG)) return MRS_ERR_INVALID_ARG;
  if (!valid_sizes(M, E, k, block) || n_group < 1 || E % n_group != 0 || topk_group < 1 ||
      topk_group > n_group || (int64_t)k > (int64_t)topk_group * (E / n_group) ||
      (logits_dtype != MRS_DTYPE_F32 && logits_dtype != MRS_DTYPE_BF16))
    return MRS_ERR_INVALID_ARG;
  if ((int64_t)M * k > INT32_MAX || max_rows_of(M, E, k, block) > INT32_MAX) return MRS_ERR_OVERFLOW;
  if (num_post_pad == nullptr) return MRS_ERR_NULL_POINTER;
  if (!aligned(num_post_pad, 4)) return MRS_ERR_MISALIGNED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (M == 0) {
    void* params[] = {&num_post_pad};
    const hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(k_zero_npp), dim3(1), dim3(1),
                                           params, 0, st);
    return err == hipSuccess ? MRS_OK : MRS_ERR_LAUNCH;
  }
  if (!logits || !bias || !out_ids || !out_w || !sorted_ids || !expert_of_block)
    return MRS_ERR_NULL_POINTER;
  if (!aligned(logits, 16) || !aligned(bias, 4) || !aligned(out_ids, 4) || !aligned(out_w, 4) ||
      !aligned(sorted_ids, 4) || !aligned(expert_of_block, 4) || (stats && !aligned(stats, 4)))
    return MRS_ERR_MISALIGNED;

  Args a{};
  a.logits = logits;
  a.bias = bias;
  a.M = M;
  a.E = E;
  a.k = k;
  a.n_group = n_group;
  a.topk_group = topk_group;
  a.block = block;
  a.G = E / n_group;
  a.gstage = (n_group > 1 && topk_group < n_group && a.G > 1) ? 1 : 0;
  a.fast = (E % kWave == 0 && kWave % n_group == 0 && !(flags & MRS_FLAG_FORCE_EXACT)) ? 1 : 0;
  a.out_ids = out_ids;
  a.out_w = out_w;
  a.sorted_ids = sorted_ids;
  a.eob = expert_of_block;
  a.npp = num_post_pad;
  a.stats = stats;
  const bool bf16 = logits_dtype == MRS_DTYPE_BF16;
  const int eplm = a.fast ? eplm_bucket(E / kWave) : 1;

  const bool small_fits = M <= kTwMax && (int64_t)M * k <= kSmallSlotsMax &&
                          lds_plan(KIND_SMALL, E, n_group, a.gstage, M, k).total <= kLdsLimit;
  bool small = small_fits && !(flags & MRS_FLAG_FORCE_MULTI_WG);
  if ((flags & MRS_FLAG_FORCE_SINGLE_WG) && !small_fits) return MRS_ERR_INVALID_ARG;
  if (small) {
    a.tw = M;
    a.nwg = 1;
    const size_t lds = lds_plan(KIND_SMALL, E, n_group, a.gstage, a.tw, k).total;
    return launch(pick_k_small(eplm, bf16), 1, lds, st, &a);
  }

  a.tw = choose_tw(M);
  a.nwg = (M + a.tw - 1) / a.tw;
  const size_t need = workspace_of(M, E);
  if (workspace == nullptr || workspace_bytes < need) return MRS_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return MRS_ERR_MISALIGNED;
  int32_t* ws = reinterpret_cast<int32_t*>(reinterpret_cast<unsigned char*>(workspace) + kWsHeader);
  a.ws_cnt = ws;
  a.ws_pad = ws + E;
  a.ws_hist = ws + 2 * E;
  const size_t lds_sel = lds_plan(KIND_SELECT, E, n_group, a.gstage, a.tw, k).total;
  const size_t lds_sct = lds_plan(KIND_SCATTER, E, n_group, a.gstage, a.tw, k).total;
  if (lds_sel > kLdsLimit || lds_sct > kLdsLimit) return MRS_ERR_INVALID_ARG;
  int rc = launch(pick_k_select(eplm, bf16), a.nwg, lds_sel, st, &a);
  if (rc == MRS_OK) rc = launch(k_colscan, (E + kWave - 1) / kWave, 0, st, &a);
  if (rc == MRS_OK) rc = launch(k_scatter, a.nwg, lds_sct, st, &a);
  return rc;
}

int moe_route_sort(const void* logits, const float* bias, int M, int E, int k, int n_group,
                   int topk_group, int block, int32_t* out_ids, float* out_w,
                   int32_t* sorted_ids, int32_t* expert_of_block, int32_t* num_post_pad,
                   int logits_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return moe_route_sort_ex(logits, bias, M, E, k, n_group, topk_group, block, out_ids, out_w,
                           sorted_ids, expert_of_block, num_post_pad, logits_dtype, workspace,
                           workspace_bytes, stream, 0u, nullptr);
}

int moe_route_sort_sigmoid_probe(const float* x, int n, float* fast_out, float* exact_out,
                                 void* stream) {
  if (n < 0) return MRS_ERR_INVALID_ARG;
  if (n == 0) return MRS_OK;
  if (!x || !fast_out || !exact_out) return MRS_ERR_NULL_POINTER;
  if (!aligned(x, 4) || !aligned(fast_out, 4) || !aligned(exact_out, 4)) return MRS_ERR_MISALIGNED;
  void* params[] = {&x, &n, &fast_out, &exact_out};
  const hipError_t err =
      hipLaunchKernel(reinterpret_cast<const void*>(k_sigmoid_probe), dim3((n + kWG - 1) / kWG),
                      dim3(kWG), params, 0, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? MRS_OK : MRS_ERR_LAUNCH;
}

}  // extern "C"
