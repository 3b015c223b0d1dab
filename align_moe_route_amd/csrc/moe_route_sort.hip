// MoE route-sort for MI355X (gfx950, CDNA4, wave64): kernels and C ABI.
//
// The path (page "Kimi-K3 B1 route-sort + prepared-MoE handoff (stack)",
// Summary): FP32 conversion of router logits, per-expert correction bias,
// grouped top-k, then the two sort phases that produce expert-sorted,
// block-padded dispatch metadata for a grouped GEMM.  Exact definitions of
// every output are in include/moe_route_sort.h.
//
// Workgroups of 1024 threads (16 waves) take tw = ceil(M / 256) consecutive
// tokens each (one workgroup per compute unit at the 8192-token shape); the
// rows are copied into LDS with global_load_lds (wave by wave, so a wave's
// compute overlaps the others' copies) or read as 16-byte vectors.  Long FP32
// rows read as vectors go straight into the key registers, and a wave
// requests the first half of its next token's row as soon as the current
// token's keys are no longer needed (see lean_token).  Small batches (one
// token per wave, at most kKeysPreMax keys) have the whole workgroup compute
// every exact key into LDS first (LOAD_KEYS).
//
// Selection, one token per wave segment of 32 or 64 lanes; lane l owns
// experts [l*epl, (l+1)*epl), or, for FP32 rows read as 16-byte vectors with
// one token per wave, interleaved vectors of its group (see Ownership):
//   1. keys = sigmoid(x) + b and each lane's two largest keys.  BF16 logits
//      look their sigmoid up in an LDS table that is correctly rounded for
//      every BF16 value, so the keys are exact.  FP32 logits use sigmoid_fast
//      (|key error| <= delta) to find candidates only;
//   2. group stage: each group's top two merged across its lanes with DPP,
//      group score, rank of every group by (score desc, index asc) by counting
//      in LDS.  With fast keys the kept set is accepted only if it beats the
//      dropped groups by more than the fast scores' error; otherwise the wave
//      computes correctly rounded keys for the few experts that can be among
//      their group's top two, which makes the group scores exact;
//   3. threshold: a lower bound of the k-th largest of the kept lanes' top-two
//      keys (at least k keys reach it), by ballot-count bisection over the
//      highest differing bits; with fast keys it is lowered by 2*delta;
//   4. the candidates above it (about 16-20) are compacted in expert order;
//      their exact keys are ranked by (key desc, index asc), which picks the k
//      experts exactly, with no tie exemption;
//   5. weights from the same exact sigmoid values, normalised in float64.
//   A token with more candidates than lanes (heavy exact ties) and every token
//   of a shape outside this layout is decided by the whole workgroup from
//   exact keys held in LDS.
// Histogram and ranks: per-workgroup LDS bitsets, bit tl of word e set when
//   token tl of the workgroup picked expert e.  Popcount = the workgroup's
//   count for e (no global atomic per route; compare the workgroup histograms
//   of the page "gfx1250 ordinary-TP route optimization", Summary); popcount
//   of the bits below tl = the slot's stable rank inside the workgroup.
// Large M: three launches -- select (+ histogram row, slot records), column
//   scan of the histograms in workgroup order, scatter.  Exchanging those rows
//   between workgroups inside one launch needs agent-scope (cross-XCD) memory
//   round trips of about 2 us each on MI355X; the two kernel boundaries cost
//   less than the two device-wide waits that would replace them.
// M <= 64 (while faster): everything in one workgroup and one launch; at
//   most 192 tokens: two launches (the scatter folds the column scan in).

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <unordered_map>
#include <type_traits>

#include "moe_route_sort.h"
#include "route_internal.h"
#include "sigmoid_rn.h"

namespace {

constexpr int kWave = 64;
constexpr int kNW = 16;                  // waves per workgroup
constexpr int kWG = kNW * kWave;         // threads per workgroup, all kernels
constexpr int kTwMax = 64;               // tokens per workgroup: one bit each in a 64-bit word
constexpr int kEMax = 4096;              // 16 KiB of 32-bit counters, the pages' LDS bound
constexpr int kKeysPreMax = 2048;        // small batches with at most this many keys precompute them
constexpr int kBiasRegMax = 32;          // lanes keep their biases in registers up to this many experts
// Correctly rounded sigmoid of every BF16 value, 8192 FP32 entries: entry
// 4096 s + t is the value at the BF16 pattern (0x3300 + t) | s << 15.  Below
// the window (|x| < 2^-25) the sigmoid rounds to 0.5, above it (|x| >= 128)
// to 1 or 0, so clamping t into [0, 4095] gives the exact value for every
// BF16 x.  In LDS the negative half starts at byte 32768, so that the sign
// bit of a pattern is already the sign bit of its entry's byte offset
// (4 t + 32768 s): 48 KiB, of which bytes [16384, 32768) hold no entry.
constexpr int kSigEntries = 8192;
constexpr int kSigBytes = kSigEntries * 4;     // the table in global memory
constexpr int kSigLdsBytes = 3 * kSigBytes / 2;  // its LDS image
constexpr uint32_t kSigBase = 0x3300;
constexpr size_t kLdsLimit = 160 * 1024;
constexpr size_t kWsHeader = 256;
constexpr int kMaxDevices = 64;          // devices whose per-device host state is kept

enum { KIND_SMALL = 0, KIND_SELECT = 1, KIND_SCATTER = 2 };
// LOAD_KEYS: the whole workgroup computes every exact key (and score) of the
// batch into LDS first; the waves then select from them (small batches)
enum { LOAD_VEC = 0, LOAD_STAGE = 1, LOAD_KEYS = 2 };
enum { TOK_DONE = 0, TOK_ESCALATE = 1 };

struct Args {
  const void* logits;
  const float* bias;
  int M, E, k, n_group, topk_group, block;
  uint32_t blk_sh;        // n / block == (n * blk_mul) >> blk_sh for 0 <= n < 2^31
  unsigned long long blk_mul;
  uint32_t k_mul;         // q / k == (q * k_mul) >> 18 for 0 <= q < 4096
  int G;       // experts per group
  int seg;    // lanes per token in the wave path (32 or 64)
  int lg_lpg;  // log2 of the lanes per group in the wave path (seg / n_group)
  int epl;     // experts per lane in the wave path (E / seg)
  int ilw;     // FP32 vector loads, 64-lane segments: lanes of a block of ilw lanes interleave
               // their 16-byte vectors (1: every lane owns a contiguous run)
  int nbuf;    // LDS row buffers per segment (2 when a wave takes several rounds)
  int stage_bytes;  // bytes of one staged logits row (0: rows are read straight from HBM)
  int tw;      // tokens per workgroup
  int nwg;     // workgroups of the multi-workgroup path
  int fast;    // the wave layout covers this shape
  int tbl;     // BF16 logits: keys from the sigmoid table in LDS (exact)
  const float* sigtab;  // the table in device memory (copied into LDS by every workgroup)
  int bias_dma;  // bias is copied into LDS by DMA (16-byte aligned, E % 4 == 0)
  int rows_first;  // issue the row copies before the shared data (latency-bound calls)
  int gstage;  // the group stage changes the result (1 < topk_group < n_group, G > 1)
  int keys_pre;  // LOAD_KEYS: token tl's keys at stage + tl*stage_bytes, its scores E floats later
  int32_t* out_ids;
  float* out_w;
  int32_t* sorted_ids;
  int32_t* eob;
  int32_t* npp;
  int32_t* ws_tot;   // [E] routes per expert
  int32_t* ws_pad;   // [E] padded routes per expert
  int32_t* ws_hist;  // [nwg][E] per-workgroup counts, then exclusive column prefixes
  int32_t* ws_slot;  // [M*k] expert | (rank inside the workgroup << 16)
  int fold;          // at most kFoldRows workgroups: the scatter sums the raw histogram rows
                     // itself and the column-scan launch is skipped
  int32_t* stats;
  const int32_t* in_ids;  // sort-only entry: caller's expert ids [M, k]
  int e_lo, EL;  // experts [e_lo, e_lo + EL) get metadata (all E unless a local range is asked for)
  // sort-only entry with caller counters: counters[e] rows already head expert
  // e's segment; ws_c0 is the workspace copy the kernels read; cap is the
  // caller's row capacity.  counters == nullptr: no counters.
  int32_t* counters;
  int32_t* ws_c0;
  int cap;
};

// ----------------------------------------------------------------------------
// LDS plan shared by host (size) and device (carving).
// ----------------------------------------------------------------------------
struct LdsPlan {
  size_t sig, bits, redd, off, cpre, ids, bias, biasT, cand_i, cand_c, gcomp, u, stage, ukey, grp, esc, misc, red, scan, total;
};

__host__ __device__ inline size_t stage_total(int fast, int seg, int nbuf, int stage_bytes, int key_rows = 0) {
  if (key_rows > 0) return (size_t)key_rows * stage_bytes;  // LOAD_KEYS: one row per token
  return fast ? (size_t)kNW * nbuf * (kWave / seg) * stage_bytes : 0;
}

__host__ __device__ inline LdsPlan lds_plan(int kind, int E, int n_group, int gstage, size_t stage,
                                            int tw, int k, int tbl) {
  LdsPlan p{};
  size_t o = 0;
  auto take = [&](size_t n) { size_t r = o; o = (o + n + 15) & ~(size_t)15; return r; };
  if (kind != KIND_SCATTER && tbl) p.sig = take(kSigLdsBytes);  // at LDS offset 0
  if (kind != KIND_SCATTER) p.bits = take((size_t)E * 8);
  p.redd = take((size_t)kNW * 8);
  if (kind != KIND_SELECT) p.off = take((size_t)E * 4);
  if (kind == KIND_SCATTER) p.cpre = take((size_t)E * 12);  // column prefixes, counts, initial counters
  if (kind != KIND_SCATTER) {
    p.ids = take((size_t)tw * k * 4);
    p.bias = take((size_t)E * 4);
    p.biasT = take((size_t)E * 4);
    p.cand_i = take((size_t)kNW * kWave * 4);
    p.cand_c = take((size_t)kNW * kWave * 8);
    p.gcomp = p.cand_c;  // group composites (step 2) and candidate keys (step 5) of a wave never overlap
    if (o < 1024) o = 1024;  // staging buffers start past 1 KiB (see stage_rows_async)
    // union: wave staging buffers (wave loop) / exact keys + group arrays (after it)
    const size_t ex = (size_t)E * 4 + (gstage ? (size_t)3 * n_group * 4 + 16 : 0);
    const size_t un = stage > ex ? stage : ex;
    p.u = take(un);
    p.stage = p.u;
    p.ukey = p.u;
    p.grp = p.u + (((size_t)E * 4 + 15) & ~(size_t)15);
    p.esc = take((size_t)kTwMax * 4);
  }
  p.misc = take(16 * 4);
  p.red = take((size_t)2 * kNW * 4);
  p.scan = take((size_t)kNW * 4);
  p.total = o;
  return p;
}

struct Lds {
  unsigned long long* bits;
  double* redd;
  int* off;
  int* cpre;
  int* ids;
  float* bias;
  float* biasT;  // bias[lane run i of lane l] at i * seg + l: conflict-free lane reads
  int* cand_i;
  unsigned long long* cand_c;
  unsigned long long* gcomp;
  unsigned char* stage;
  uint32_t* ukey;
  unsigned* grp;
  int* esc;
  int* misc;
  int* red;
  int* scan;
};

extern __shared__ __align__(16) unsigned char g_lds[];

__device__ inline Lds carve(int kind, const Args& a) {
  const LdsPlan p = lds_plan(kind, a.E, a.n_group, a.gstage,
                             stage_total(a.fast, a.seg, a.nbuf, a.stage_bytes, a.keys_pre ? a.tw : 0),
                             a.tw, a.k, a.tbl);
  Lds L;
  L.bits = reinterpret_cast<unsigned long long*>(g_lds + p.bits);
  L.redd = reinterpret_cast<double*>(g_lds + p.redd);
  L.off = reinterpret_cast<int*>(g_lds + p.off);
  L.cpre = reinterpret_cast<int*>(g_lds + p.cpre);
  L.ids = reinterpret_cast<int*>(g_lds + p.ids);
  L.bias = reinterpret_cast<float*>(g_lds + p.bias);
  L.biasT = reinterpret_cast<float*>(g_lds + p.biasT);
  L.cand_i = reinterpret_cast<int*>(g_lds + p.cand_i);
  L.cand_c = reinterpret_cast<unsigned long long*>(g_lds + p.cand_c);
  L.gcomp = reinterpret_cast<unsigned long long*>(g_lds + p.gcomp);
  L.stage = g_lds + p.stage;
  L.ukey = reinterpret_cast<uint32_t*>(g_lds + p.ukey);
  L.grp = reinterpret_cast<unsigned*>(g_lds + p.grp);
  L.esc = reinterpret_cast<int*>(g_lds + p.esc);
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
// n / block for 0 <= n < 2^31 by multiply and shift: with l = ceil(log2 block),
// mul = ceil(2^(31+l) / block) makes the error of n*mul/2^(31+l) below
// n / 2^(31+l) < 1/block, so the floor is exact.
__device__ __forceinline__ int div_block(int n, const Args& a) {
  return (int)(((unsigned long long)(uint32_t)n * a.blk_mul) >> a.blk_sh);
}
// q / k for a slot index q of at most kTwMax tokens (q < 4096, k <= 64):
// k_mul = ceil(2^18 / k) = (2^18 + e) / k with e < k adds q*e/(k*2^18) to
// q/k, less than 1/k because q*(k-1) < 2^18, so the floor is exact.
__device__ __forceinline__ int div_k(int q, const Args& a) { return (int)(((uint32_t)q * a.k_mul) >> 18); }
__device__ __forceinline__ int pad_block(int c, const Args& a) {
  return (c == 0) ? 0 : (div_block(c - 1, a) + 1) * a.block;
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
// 2^-21 for every FP32 x (error terms: argument rounding, 1-ulp exp2,
// rounding of 1+e, 1-ulp reciprocal: about 2.6e-7; measured on MI355X below
// 1.2e-7); the margins of the selection are built on 2^-21.
__device__ __forceinline__ float sigmoid_fast(float x) {
  const float e = __builtin_amdgcn_exp2f(x * -1.44269504088896341f);
  return __builtin_amdgcn_rcpf(1.0f + e);
}

// Correctly rounded FP32 sigmoid (sigmoid_rn.h: float64 quotient, with the
// rare inputs near an FP32 rounding midpoint settled in double-double).
__device__ __forceinline__ float sigmoid_exact(float x) { return sigrn::sigmoid_rn32(x); }
// The double-double settlement as a call (reached about once in 2^19
// evaluations), for code that keeps many registers live around it.
__device__ __attribute__((noinline)) float sigmoid_settle(float x, float dn, float up) {
  return sigrn::rn32_resolve((double)x, dn, up);
}

// The sigmoid table, generated at build time (gen_sig_table.cpp runs
// sigmoid_rn32 on the host for every entry) and held in kSigCopies identical
// copies, one per XCD: workgroups are dealt to the eight XCDs in turn, so
// workgroup w copies copy w mod 8 into LDS offset 0 and each XCD's L2 fetches
// one 32 KiB copy per call.  (On the 8192 x 896 workload: 15.2 MB fetched by
// the selection kernel per call; 32 copies spread over every XCD, 23.3 MB at
// the same speed.)
#include "sig_table.inc"
constexpr int kSigCopies = 8;
#define SIG_ROW {SIG_TABLE_BITS}
#define SIG_ROW4 SIG_ROW, SIG_ROW, SIG_ROW, SIG_ROW
// Not const: an internal const array that no device code names would be
// dropped from the code object, and the host looks it up by name.
__device__ __align__(16) uint32_t g_sig_table[kSigCopies][kSigEntries] = {SIG_ROW4, SIG_ROW4};
#undef SIG_ROW4
#undef SIG_ROW
__device__ __forceinline__ const float* sig_table_copy(const float* base, int wg) {
  return base + (size_t)(wg & (kSigCopies - 1)) * kSigEntries;
}


// LDS byte offset of a BF16 pattern's entry: 4 * clamp(|h| - base, 0, 4095)
// + 32768 * sign (the pattern's own sign bit, in place).
__device__ __forceinline__ uint32_t sig_off1(uint32_t h) {
  const int t = (int)(h & 0x7FFFu) - (int)kSigBase;
  const uint32_t c = (uint32_t)min(max(t, 0), 4095);
  return (c << 2) | (h & 0x8000u);
}
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
// Both entries of a pair of BF16 patterns packed in one word (low half first),
// with packed 16-bit integer arithmetic; the sign bits stay where they are.
__device__ __forceinline__ void sig_off2(uint32_t d, uint32_t& o0, uint32_t& o1) {
  u16x2 m = __builtin_bit_cast(u16x2, d & 0x7FFF7FFFu);
  m = __builtin_elementwise_sub_sat(m, (u16x2){(unsigned short)kSigBase, (unsigned short)kSigBase});
  m = __builtin_elementwise_min(m, (u16x2){4095, 4095});
  m = m << (u16x2){2, 2};
  const uint32_t v = __builtin_bit_cast(uint32_t, m) | (d & 0x80008000u);  // one v_and_or_b32
  o0 = __builtin_amdgcn_perm(0u, v, 0x0C0C0100u);  // bytes 0-1 of v (a byte permute keeps the and-or whole)
  o1 = v >> 16;
}
// LDS float index of table entry j (the negative half starts at byte 32768)
__host__ __device__ constexpr int sig_lds_index(int j) { return (j & 4095) + (j >> 12) * 8192; }
// The table sits at LDS address 0 (the kernels that use it have no static
// LDS, so their dynamic LDS starts there; the host checks this), which lets
// the byte offset serve directly as the LDS address.
typedef __attribute__((address_space(3))) const float* lds_cfloat_ptr;
__device__ __forceinline__ float sig_lds(uint32_t off) { return *reinterpret_cast<lds_cfloat_ptr>((size_t)off); }

// ----------------------------------------------------------------------------
// Wave-level helpers (wave64, DPP row shifts and broadcasts).
// ----------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }
// The wave's index in its workgroup, in a scalar register (addresses derived
// from it then need no vector registers).
__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); }

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kRowHalfMirror = 0x141, kRowMirror = 0x140;

__device__ __forceinline__ uint32_t readlane(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// Inclusive prefix sum over the wave (row shifts 1,2,4,8 then row broadcasts).
__device__ __forceinline__ int wave_incl_scan(int v) {
  uint32_t u = (uint32_t)v;
  u += dpp<kRowShr1>(0u, u);
  u += dpp<kRowShr2>(0u, u);
  u += dpp<kRowShr4>(0u, u);
  u += dpp<kRowShr8>(0u, u);
  u += dpp<kRowBcast15, 0xA>(0u, u);
  u += dpp<kRowBcast31, 0xC>(0u, u);
  return (int)u;
}
__device__ __forceinline__ int wave_sum_i(int v) { return (int)readlane((uint32_t)wave_incl_scan(v), 63); }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t u) {
  u = max(u, dpp<kRowShr1>(0u, u));
  u = max(u, dpp<kRowShr2>(0u, u));
  u = max(u, dpp<kRowShr4>(0u, u));
  u = max(u, dpp<kRowShr8>(0u, u));
  u = max(u, dpp<kRowBcast15, 0xA>(0u, u));
  u = max(u, dpp<kRowBcast31, 0xC>(0u, u));
  return readlane(u, 63);
}
__device__ __forceinline__ double wave_sum_d(double v) {
  auto step = [](double x, auto sh) {
    const uint64_t b = __double_as_longlong(x);
    const uint32_t lo = sh((uint32_t)b), hi = sh((uint32_t)(b >> 32));
    return x + __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
  };
  v = step(v, [](uint32_t u) { return dpp<kRowShr1>(0u, u); });
  v = step(v, [](uint32_t u) { return dpp<kRowShr2>(0u, u); });
  v = step(v, [](uint32_t u) { return dpp<kRowShr4>(0u, u); });
  v = step(v, [](uint32_t u) { return dpp<kRowShr8>(0u, u); });
  v = step(v, [](uint32_t u) { return dpp<kRowBcast15, 0xA>(0u, u); });
  v = step(v, [](uint32_t u) { return dpp<kRowBcast31, 0xC>(0u, u); });
  const uint64_t b = __double_as_longlong(v);
  const uint32_t lo = readlane((uint32_t)b, 63), hi = readlane((uint32_t)(b >> 32), 63);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Partner for level `lev` of a butterfly over aligned blocks of 2^(lev+1)
// lanes: lanes of the two halves of each block meet pairwise.
__device__ __forceinline__ float butterfly_partner(float v, int lev) {
  const uint32_t u = __float_as_uint(v);
  switch (lev) {
    case 0: return __uint_as_float(dpp<kQuadXor1>(u, u));
    case 1: return __uint_as_float(dpp<kQuadXor2>(u, u));
    case 2: return __uint_as_float(dpp<kRowHalfMirror>(u, u));
    case 3: return __uint_as_float(dpp<kRowMirror>(u, u));
    default: return __uint_as_float((uint32_t)__builtin_amdgcn_ds_swizzle((int)u, 0x401F));  // xor 16
  }
}

// ----------------------------------------------------------------------------
// Workgroup-level helpers (all kWG threads must call them).
// ----------------------------------------------------------------------------
// REUSE = false: the caller writes L.scan no more before its next barrier, so
// the barrier that protects the wave totals from a later scan is left out.
template <bool REUSE = true>
__device__ int wg_excl_scan(const Lds& L, int v) {
  const int w = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane_id() == kWave - 1) L.scan[w] = x;
  __syncthreads();
  int pre = 0;
  for (int q = 0; q < w; ++q) pre += L.scan[q];
  if (REUSE) __syncthreads();
  return pre + x - v;
}

__device__ double wg_sum_d(const Lds& L, double v) {
  const int w = threadIdx.x >> 6;
  v = wave_sum_d(v);
  if (lane_id() == 0) L.redd[w] = v;
  __syncthreads();
  double s = 0.0;
  for (int q = 0; q < kNW; ++q) s += L.redd[q];
  __syncthreads();
  return s;
}

// Number of selected entries >= c among arr[i0 + i] (i < n, bit i of mask).
__device__ __forceinline__ int wg_count_ge(const Lds& L, const uint32_t* arr, int i0, int n, uint32_t mask,
                                           uint32_t c, int parity) {
  int cnt = 0;
  for (int i = 0; i < n; ++i) cnt += (((mask >> i) & 1u) && arr[i0 + i] >= c) ? 1 : 0;
  const int s = wave_sum_i(cnt);
  const int w = threadIdx.x >> 6;
  if (lane_id() == 0) L.red[parity * kNW + w] = s;
  __syncthreads();
  int t = 0;
  for (int q = 0; q < kNW; ++q) t += L.red[parity * kNW + q];
  return t;
}

// Select the m largest of the mask-selected entries (ties to the lower index);
// thread r holds entries [i0, i0+n) of arr in index order.  Returns this
// thread's selection bits.
__device__ uint32_t wg_select(const Lds& L, const uint32_t* arr, int i0, int n, uint32_t mask, int m) {
  uint32_t T = 0;
  int parity = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = T | (1u << b);
    if (wg_count_ge(L, arr, i0, n, mask, c, parity) >= m) T = c;
    parity ^= 1;
  }
  const int gt = (T == 0xFFFFFFFFu) ? 0 : wg_count_ge(L, arr, i0, n, mask, T + 1u, parity);
  const int r = m - gt;  // equal values to take, lowest index first
  uint32_t sel = 0, tie = 0;
  for (int i = 0; i < n; ++i) {
    if ((mask >> i) & 1u) {
      const uint32_t v = arr[i0 + i];
      if (v > T) sel |= 1u << i;
      else if (v == T) tie |= 1u << i;
    }
  }
  int rank = wg_excl_scan(L, __popc(tie));
  for (int i = 0; i < n; ++i) {
    if ((tie >> i) & 1u) {
      if (rank < r) sel |= 1u << i;
      ++rank;
    }
  }
  return sel;
}

// ----------------------------------------------------------------------------
// Exact selection of one token by the whole workgroup (correctly rounded keys
// in LDS).  Thread r owns experts [r*ept, (r+1)*ept).
// ----------------------------------------------------------------------------
template <bool BF16>
__device__ void exact_token_wg(const Args& a, const Lds& L, int t, int tl, int* ids_cache) {
  const int tid = threadIdx.x;
  const int E = a.E, G = a.G;
  const size_t row = (size_t)t * E;
  uint32_t* uk = L.ukey;
  for (int e = tid; e < E; e += kWG) {
    const float s = sigmoid_exact(load_logit<BF16>(a.logits, row + e));
    uk[e] = f2s(s + a.bias[e]);
  }
  const int ept = (E + kWG - 1) / kWG;
  const int e0 = min(E, tid * ept);
  const int n = min(ept, E - e0);
  const uint32_t valid = n >= 32 ? 0xFFFFFFFFu : ((1u << n) - 1u);
  __syncthreads();
  uint32_t allow = valid;
  if (a.gstage) {
    unsigned* gmax = L.grp;
    unsigned* gsc = L.grp + a.n_group;       // count of the maximum, then the group score
    unsigned* gsec = L.grp + 2 * a.n_group;  // largest value below the maximum, then the flags
    for (int g = tid; g < a.n_group; g += kWG) { gmax[g] = 0u; gsc[g] = 0u; gsec[g] = 0u; }
    __syncthreads();
    {  // group maxima
      int cg = -1;
      uint32_t cm = 0;
      for (int i = 0; i < n; ++i) {
        const int g = (e0 + i) / G;
        if (g != cg) {
          if (cg >= 0) atomicMax(&gmax[cg], cm);
          cg = g;
          cm = 0;
        }
        cm = max(cm, uk[e0 + i]);
      }
      if (cg >= 0) atomicMax(&gmax[cg], cm);
    }
    __syncthreads();
    {  // how often the maximum occurs, and the largest value below it
      int cg = -1;
      uint32_t gm = 0, c = 0, m2 = 0;
      for (int i = 0; i < n; ++i) {
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
        const uint32_t v = uk[e0 + i];
        if (v == gm) ++c;
        else m2 = max(m2, v);
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
    const int g0 = min(a.n_group, tid * gpt);
    const int gn = min(gpt, a.n_group - g0);
    const uint32_t gval = gn >= 32 ? 0xFFFFFFFFu : ((1u << gn) - 1u);
    const uint32_t gsel = wg_select(L, gsc, g0, gn, gval, a.topk_group);
    for (int i = 0; i < gn; ++i) gsec[g0 + i] = (gsel >> i) & 1u;
    __syncthreads();
    allow = 0;
    for (int i = 0; i < n; ++i)
      if (gsec[(e0 + i) / G]) allow |= 1u << i;
    __syncthreads();
  }
  const uint32_t sel = wg_select(L, uk, e0, n, allow, a.k);
  double part = 0.0;
  for (int i = 0; i < n; ++i)
    if ((sel >> i) & 1u) part += (double)sigmoid_exact(load_logit<BF16>(a.logits, row + e0 + i));
  const double ssum = wg_sum_d(L, part);
  int pos = wg_excl_scan(L, __popc(sel));
  for (int i = 0; i < n; ++i) {
    if ((sel >> i) & 1u) {
      const int e = e0 + i;
      const double s = (double)sigmoid_exact(load_logit<BF16>(a.logits, row + e));
      a.out_ids[(size_t)t * a.k + pos] = e;
      a.out_w[(size_t)t * a.k + pos] = (float)(s / ssum);
      atomicOr(&L.bits[e], 1ull << tl);
      ids_cache[tl * a.k + pos] = e;
      ++pos;
    }
  }
  __syncthreads();
}

// ----------------------------------------------------------------------------
// Selection by wave segments (see the header comment).  A wave works on
// NSEG = 64 / SEG tokens at once, one per segment of SEG consecutive lanes;
// every per-token step (reductions, scans, ballot counts, rank counts) stays
// inside its segment, so a wave pays the per-token control work once for
// NSEG tokens.  Layout: E % SEG == 0, n_group divides SEG, lane l of a segment
// owns experts [l*epl, (l+1)*epl) with epl = E / SEG.  EPL > 0 fixes epl at
// compile time; EPL == 0 reads it from the arguments (up to 64).
// ----------------------------------------------------------------------------
// Which experts a lane of a wave-path segment holds in its register slots.
// Contiguous runs (w = 1): slot i of lane l holds expert l*epl + i.
// Interleaved (w > 1; FP32 vector loads, one token per wave): the w lanes of a
// block (a group, or the whole wave when no group stage runs) hold the
// block's w*epl experts as interleaved 16-byte vectors, lane j of the block
// holding vectors j, j + w, j + 2w, ..., so one load instruction reads w*16
// contiguous bytes per block instead of 16 bytes from each of 64 separate
// lines.  Every lane still holds experts of one group only.
struct Ownership {
  int w, e_slot0;  // block width in lanes, expert of slot 0
  __device__ __forceinline__ Ownership(int ls, int epl, int w_) : w(w_) {
    const int j = ls & (w - 1);
    e_slot0 = (ls - j) * epl + 4 * j;
  }
  __device__ __forceinline__ int expert(int i) const {
    return w == 1 ? e_slot0 + i : e_slot0 + 4 * w * (i >> 2) + (i & 3);  // w is a constant 1 but for FP32 vectors
  }
  // slot and lane of expert e: the inverse of expert()
  __device__ static void place(int e, int epl, int w, int& slot, int& lane) {
    const int r = e % (w * epl), v = r >> 2;
    slot = 4 * (v / w) + (r & 3);
    lane = (e - r) / epl + v % w;
  }
};

// Largest and second largest correctly rounded key over the register slots
// in rm of a lane (slot i holds expert own.expert(i)); x = the token's row.
__device__ __forceinline__ float2 exact_top2(const float* x, const float* bias, unsigned long long rm,
                                                       Ownership own) {
  float e1 = -INFINITY, e2 = -INFINITY;
  while (rm) {
    const int e = own.expert((int)__builtin_ctzll(rm));
    rm &= rm - 1;
    bool amb;
    float up;
    float s = sigrn::sigmoid_rn32_try(x[e], amb, up);
    if (amb) s = sigmoid_settle(x[e], s, up);
    const float key = s + bias[e];
    e2 = __builtin_amdgcn_fmed3f(e1, e2, key);
    e1 = __builtin_amdgcn_fmed3f(e1, key, INFINITY);
  }
  return make_float2(e1, e2);
}

// s_waitcnt vmcnt(0) with the other counters left free (gfx9 encoding)
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N), N < 64
template <int N>
__device__ __forceinline__ void wait_vmem_upto() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Copy the rows of the tokens of a wave (one per segment, token < 0 = none:
// row 0 is copied in its place, so every call issues the same instructions)
// from HBM into per-segment LDS buffers with gfx950's global_load_lds_dwordx4
// (no VGPRs in flight).  Lane l writes LDS at base + 16*l, so the base for a
// segment's instruction is shifted back by its first lane.  With EPL known the
// wave issues exactly row_dma_count<SEG, EPL, SZ>() instructions.
template <int SEG, int EPL, int SZ>
constexpr int row_dma_count() {
  return (kWave / SEG) * ((EPL * SZ + 15) / 16);
}
template <int SEG, int EPL>
__device__ __forceinline__ void stage_rows_async(const Args& a, unsigned char* buf, int stage_bytes, int tok,
                                                 int sz) {
  constexpr int NSEG = kWave / SEG;
  const int lane = lane_id();
  const int seg = lane / SEG;
  const int ls = lane % SEG;
  const int chunks = (a.E * sz) >> 4;
  const int jn = EPL > 0 ? (EPL * sz + 15) / 16 : (chunks + SEG - 1) / SEG;  // instructions per segment
  const unsigned char* src = reinterpret_cast<const unsigned char*>(a.logits) + (size_t)(tok < 0 ? 0 : tok) * a.E * sz;
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    unsigned char* dst = buf + (size_t)s * stage_bytes - (size_t)s * SEG * 16;  // >= 0: buffers start past 1 KiB
#pragma unroll
    for (int j = 0; j < (EPL > 0 ? (EPL * 4 + 15) / 16 : 64); ++j) {
      if (j >= jn) break;
      const int c = j * SEG + ls;
      if (seg == s && c < chunks)
        __builtin_amdgcn_global_load_lds(src + (size_t)c * 16,
                                         (__attribute__((address_space(3))) void*)(dst + j * SEG * 16), 16, 0, 0);
    }
  }
}

// Segment-local reductions and scans: DPP row shifts inside 16-lane rows,
// then row broadcasts that join rows 0-1 and 2-3 (and, for 64-lane segments,
// the two halves).  The result of a reduction is returned in every lane.
template <int SEG>
__device__ __forceinline__ uint32_t seg_bcast(uint32_t u) {
  if constexpr (SEG == 64) return readlane(u, 63);
  const uint32_t lo = readlane(u, 31), hi = readlane(u, 63);
  return lane_id() < 32 ? lo : hi;
}
// The segment's maximum (minimum) in its last lane only (lane SEG - 1 of the
// segment); for a value that only one lane reads afterwards.
template <int SEG>
__device__ __forceinline__ uint32_t seg_max_last(uint32_t u) {
  u = max(u, dpp<kRowShr1>(0u, u));
  u = max(u, dpp<kRowShr2>(0u, u));
  u = max(u, dpp<kRowShr4>(0u, u));
  u = max(u, dpp<kRowShr8>(0u, u));
  u = max(u, dpp<kRowBcast15, 0xA>(0u, u));
  if constexpr (SEG == 64) u = max(u, dpp<kRowBcast31, 0xC>(0u, u));
  return u;
}
template <int SEG>
__device__ __forceinline__ uint32_t seg_min_last(uint32_t u) {
  u = min(u, dpp<kRowShr1>(0xFFFFFFFFu, u));
  u = min(u, dpp<kRowShr2>(0xFFFFFFFFu, u));
  u = min(u, dpp<kRowShr4>(0xFFFFFFFFu, u));
  u = min(u, dpp<kRowShr8>(0xFFFFFFFFu, u));
  u = min(u, dpp<kRowBcast15, 0xA>(0xFFFFFFFFu, u));
  if constexpr (SEG == 64) u = min(u, dpp<kRowBcast31, 0xC>(0xFFFFFFFFu, u));
  return u;
}
template <int SEG>
__device__ __forceinline__ uint32_t seg_max_u32(uint32_t u) {
  return seg_bcast<SEG>(seg_max_last<SEG>(u));
}
template <int SEG>
__device__ __forceinline__ uint32_t seg_min_u32(uint32_t u) {
  return seg_bcast<SEG>(seg_min_last<SEG>(u));
}
// Row shift with every row enabled: lanes shifted in from outside the row
// read 0 (bound_ctrl), so the add can take the shifted operand directly.
template <int CTRL>
__device__ __forceinline__ uint32_t shr0(uint32_t u) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)u, CTRL, 0xF, 0xF, true);
}
template <int SEG>
__device__ __forceinline__ int seg_incl_scan(int v) {
  uint32_t u = (uint32_t)v;
  u += shr0<kRowShr1>(u);
  u += shr0<kRowShr2>(u);
  u += shr0<kRowShr4>(u);
  u += shr0<kRowShr8>(u);
  u += dpp<kRowBcast15, 0xA>(0u, u);
  if constexpr (SEG == 64) u += dpp<kRowBcast31, 0xC>(0u, u);
  return (int)u;
}
template <int SEG>
__device__ __forceinline__ double seg_sum_d(double v) {
  auto step = [](double x, auto sh) {
    const uint64_t b = __double_as_longlong(x);
    const uint32_t lo = sh((uint32_t)b), hi = sh((uint32_t)(b >> 32));
    return x + __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
  };
  // row shifts with every row enabled: lanes shifted in from outside the row
  // read 0 (bound_ctrl), so no zeroed destination is needed
  auto shr = [](uint32_t u, auto ctrl) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)u, decltype(ctrl)::value, 0xF, 0xF, true);
  };
  v = step(v, [&](uint32_t u) { return shr(u, std::integral_constant<int, kRowShr1>{}); });
  v = step(v, [&](uint32_t u) { return shr(u, std::integral_constant<int, kRowShr2>{}); });
  v = step(v, [&](uint32_t u) { return shr(u, std::integral_constant<int, kRowShr4>{}); });
  v = step(v, [&](uint32_t u) { return shr(u, std::integral_constant<int, kRowShr8>{}); });
  v = step(v, [](uint32_t u) { return dpp<kRowBcast15, 0xA>(0u, u); });
  if constexpr (SEG == 64) v = step(v, [](uint32_t u) { return dpp<kRowBcast31, 0xC>(0u, u); });
  const uint64_t b = __double_as_longlong(v);
  const uint32_t lo = seg_bcast<SEG>((uint32_t)b), hi = seg_bcast<SEG>((uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// Bits of a ballot that belong to segment s, shifted down to bit 0.
template <int SEG>
__device__ __forceinline__ unsigned long long seg_bits(unsigned long long bal, int s) {
  if constexpr (SEG == 64) return bal;
  return (bal >> (s * SEG)) & 0xFFFFFFFFull;
}

// One token per segment (see the header comment).  BF16 logits take their
// correctly rounded sigmoid from the LDS table, so every key is exact and one
// pass decides the token.  FP32 logits rank with sigmoid_fast: the group
// boundary is certified against the error of the fast scores (else the group
// scores are made exact in place) and the candidate line is lowered by twice
// the key error.  Written for a short instruction stream: compile-time layout,
// table offsets with packed 16-bit arithmetic, straight-line group and
// threshold stages.  LPG > 0 fixes the lanes per group at compile time (the
// group stage then has no run-time branches or loop bounds); LPG == 0 reads
// it from the arguments.  Maxima use v_med3 with +inf, which, unlike fmaxf,
// needs no NaN-canonicalising copy of its operands (no key is NaN).
//
// Long FP32 rows read as vectors (more than 32 experts per lane, 64-lane
// segments) are loaded straight into the key registers `av`, and each key
// replaces its logit there, so no staging registers are needed.  Once the
// candidates are known the keys are dead: the wave then requests the first
// half of its next token's row (`next_t`) into `av`, after the candidates'
// own logits, so that the transfer overlaps the ranking and output steps and
// the next token starts on data already in flight (`have_row`; it requests
// the second half itself).
template <int SEG, int EPL, bool BF16, int MODE>
constexpr bool row_in_keys() {
  return !BF16 && MODE == LOAD_VEC && SEG == 64 && (EPL == 0 || EPL > 32);
}

// Requests vectors [Q0, Q1) of the lane's run of row `row` into v: slot 4q+j
// holds expert own.expert(4q+j) (a load past the lane's run repeats its last
// vector).
template <int EPLM, int Q0, int Q1>
__device__ __forceinline__ void load_row_vec(const Args& a, size_t row, int e_slot0, int vs, int nq,
                                             float (&v)[EPLM]) {
  const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.logits) + row + e_slot0);
#pragma unroll
  for (int q = Q0; q < Q1; ++q) {
    const float4 x = src[(size_t)min(q, nq - 1) * vs];
    v[4 * q + 0] = x.x;
    v[4 * q + 1] = x.y;
    v[4 * q + 2] = x.z;
    v[4 * q + 3] = x.w;
  }
}

template <int SEG, int EPL, bool BF16, int MODE, int LPG = 0>
__device__ __forceinline__ int lean_token(const Args& a, const Lds& L, bool act, int t, int tl,
                                          const unsigned char* stage, const float* bv, float d2, float e2,
                                          float (&av)[EPL > 0 ? EPL : 64], bool have_row,
                                          int next_t) {
  // BF16 keys (from the table) and precomputed keys are exact; FP32 logits
  // give fast keys, within delta of the exact ones (d2 >= 2 delta and e2 >= 2
  // epsg are those bounds as floats, rounded up)
  constexpr bool exact = BF16 || MODE == LOAD_KEYS;
  constexpr int NSEG = kWave / SEG;
  constexpr int EPLM = EPL > 0 ? EPL : 64;
  constexpr bool RIK = row_in_keys<SEG, EPL, BF16, MODE>();
  using MaskT = typename std::conditional<(EPLM > 32), unsigned long long, uint32_t>::type;
  const int lane = lane_id();
  const int w = wave_index();
  const int seg = NSEG == 1 ? 0 : (lane >> 5);
  const int ls = lane & (SEG - 1);
  const int epl = EPL > 0 ? EPL : a.epl;
  const int e0 = ls * epl;
  const size_t row = (size_t)(act ? t : 0) * a.E;
  // register slot i of the lane holds expert own.expert(i) (see Ownership)
  constexpr bool IL = SEG == 64 && !BF16 && MODE == LOAD_VEC;
  const int ilw = IL ? a.ilw : 1;
  const Ownership own(ls, epl, ilw);
  // lanes of segment 1 (32-lane segments): the upper half of the wave
  const unsigned long long seg1 = NSEG == 1 ? 0ull : 0xFFFFFFFF00000000ull;

  // ---- 1. keys and lane top-2 ----
  float lm = -INFINITY, l2 = -INFINITY;
  auto bias_of = [&](int i) { return (EPLM <= kBiasRegMax) ? bv[i] : L.biasT[i * SEG + ls]; };
  auto put_key = [&](int i, float key) {
    av[i] = key;
    l2 = __builtin_amdgcn_fmed3f(lm, l2, key);  // second largest of {lm >= l2, key}
    lm = __builtin_amdgcn_fmed3f(lm, key, INFINITY);
  };
  auto put_pair = [&](int i, uint32_t d) {  // BF16 logits of experts i, i+1 packed in d
    uint32_t o0, o1;
    sig_off2(d, o0, o1);
    put_key(i, sig_lds(o0) + bias_of(i));
    put_key(i + 1, sig_lds(o1) + bias_of(i + 1));
  };
  auto put = [&](int i, float x) { put_key(i, sigmoid_fast(x) + bias_of(i)); };  // FP32 logit of expert i
  if (EPL == 0 && !RIK) {  // slots past epl stay defined (their candidate bits are masked off)
#pragma unroll
    for (int i = 0; i < EPLM; ++i) av[i] = 0.0f;
  }
  if constexpr (MODE == LOAD_KEYS) {  // exact keys of this token, in expert order
    const float* kr = reinterpret_cast<const float*>(stage) + e0;
#pragma unroll
    for (int i = 0; i < EPLM; ++i)
      if (EPL > 0 || i < epl) put_key(i, kr[i]);
  } else if constexpr (RIK) {
    // slots past epl hold a copy of the last vector; their bits are masked off
    // the first half of the run may already be in flight (requested during
    // the previous token); the second half is requested here
    if (!have_row) load_row_vec<EPLM, 0, EPLM / 8>(a, row, own.e_slot0, ilw, epl / 4, av);
    load_row_vec<EPLM, EPLM / 8, EPLM / 4>(a, row, own.e_slot0, ilw, epl / 4, av);
    __builtin_amdgcn_sched_barrier(0);  // every request is out before the first key waits
#pragma unroll
    for (int q = 0; q < EPLM / 4; ++q) {
      if (EPL > 0 || 4 * q < epl) {  // wave-uniform
        put(4 * q + 0, av[4 * q + 0]);
        put(4 * q + 1, av[4 * q + 1]);
        put(4 * q + 2, av[4 * q + 2]);
        put(4 * q + 3, av[4 * q + 3]);
      }
    }
  } else {  // an idle segment's buffer holds a valid row too (row 0), so no branch here
    if constexpr (MODE == LOAD_STAGE && !BF16) {
      const float* s32 = reinterpret_cast<const float*>(stage) + e0;
#pragma unroll
      for (int i = 0; i < EPLM; ++i)
        if (i < epl) put(i, s32[i]);
    } else if constexpr (MODE == LOAD_STAGE && EPL > 0 && EPL % 4 == 0) {
      // the lane run is 8-byte aligned: read all of it, then request every
      // table entry, then form the keys, so a wave waits for LDS twice rather
      // than once per pair of logits
      const uint2* s64 = reinterpret_cast<const uint2*>(stage + e0 * 2);
      uint2 raw[EPL / 4];
#pragma unroll
      for (int j = 0; j < EPL / 4; ++j) raw[j] = s64[j];
      uint32_t off[EPL];
#pragma unroll
      for (int j = 0; j < EPL / 4; ++j) {
        sig_off2(raw[j].x, off[4 * j], off[4 * j + 1]);
        sig_off2(raw[j].y, off[4 * j + 2], off[4 * j + 3]);
      }
#pragma unroll
      for (int i = 0; i < EPL; ++i) av[i] = sig_lds(off[i]);
#pragma unroll
      for (int i = 0; i < EPL; ++i) put_key(i, av[i] + bias_of(i));
    } else if constexpr (MODE == LOAD_STAGE) {
      if (EPL > 0 ? (EPL % 2 == 0) : (epl % 2 == 0)) {  // the lane run is 4-byte aligned
        const uint32_t* s32 = reinterpret_cast<const uint32_t*>(stage + e0 * 2);
#pragma unroll
        for (int j = 0; j < EPLM / 2; ++j)
          if (2 * j < epl) put_pair(2 * j, s32[j]);
      } else {
        const uint16_t* s16 = reinterpret_cast<const uint16_t*>(stage) + e0;
#pragma unroll
        for (int i = 0; i < EPLM; ++i)
          if (i < epl) put_key(i, sig_lds(sig_off1(s16[i])) + bias_of(i));
      }
    } else {  // lane run is a whole number of 16-byte vectors
      constexpr int PER = BF16 ? 8 : 4;  // logits per vector
      static_assert(EPLM < PER || EPLM % PER == 0, "vector width");
      const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const unsigned char*>(a.logits) +
                                                       (row + own.e_slot0) * (BF16 ? 2 : 4));
      const int vs = IL ? ilw : 1;  // vectors between a lane's consecutive vectors
      // every load of the lane run is issued before the first use (a load past
      // the run repeats the last vector, which stays inside the row)
      constexpr int NQ = EPLM >= PER ? EPLM / PER : 0;
      // runs of more than 32 FP32 logits arrive in two batches, so the raw
      // vectors and the keys do not need registers for the whole run at once
      constexpr int NB = (!BF16 && NQ > 8) ? 2 : 1;
      constexpr int QB = NQ > 0 ? NQ / NB : 1;
      const int nq = epl / PER;
      uint4 raw[QB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int q = 0; q < QB; ++q) raw[q] = src[(size_t)min(b * QB + q, nq - 1) * vs];
#pragma unroll
        for (int qq = 0; qq < QB; ++qq) {
          const int q = b * QB + qq;
          if (q < nq) {
            if constexpr (BF16) {
              put_pair(q * 8 + 0, raw[qq].x);
              put_pair(q * 8 + 2, raw[qq].y);
              put_pair(q * 8 + 4, raw[qq].z);
              put_pair(q * 8 + 6, raw[qq].w);
            } else {
              put(q * 4 + 0, __uint_as_float(raw[qq].x));
              put(q * 4 + 1, __uint_as_float(raw[qq].y));
              put(q * 4 + 2, __uint_as_float(raw[qq].z));
              put(q * 4 + 3, __uint_as_float(raw[qq].w));
            }
          }
        }
        if (NB > 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- 2. group stage ----
  bool allowed = act;
  if (a.gstage) {
    constexpr int LG = LPG == 1 ? 0 : LPG == 2 ? 1 : LPG == 4 ? 2 : LPG == 8 ? 3 : LPG == 16 ? 4 : LPG == 32 ? 5 : -1;
    static_assert(LPG == 0 || LG >= 0, "lanes per group: a power of two up to 32");
    const int lg_lpg = LPG ? LG : a.lg_lpg;
    const int ngs = LPG ? SEG / LPG : a.n_group;  // groups in a segment (n_group)
    const int g = ls >> lg_lpg;
    unsigned long long* gc = L.gcomp + w * kWave + seg * SEG;
    // (largest, second largest) of the group in every lane of the group
    auto merge = [&](float& g1, float& g2) {
#pragma unroll
      for (int lev = 0; lev < (SEG == 64 ? 5 : 4); ++lev) {
        if (lev < lg_lpg) {  // wave-uniform
          // merge two (largest, second largest) pairs: the new second largest is
          // the median of both largest values and the larger second value
          const float p1 = butterfly_partner(g1, lev);
          const float p2 = butterfly_partner(g2, lev);
          g2 = __builtin_amdgcn_fmed3f(g1, p1, __builtin_amdgcn_fmed3f(g2, p2, INFINITY));
          g1 = __builtin_amdgcn_fmed3f(g1, p1, INFINITY);
        }
      }
    };
    // rank of the lane's group by (score desc, index asc), counted over the
    // (score, ~group) composites of the segment
    auto rank_of = [&](uint32_t gsu) {
      const unsigned long long cg = ((unsigned long long)gsu << 32) | (uint32_t)(0xFFFFu - g);
      if ((ls & ((1 << lg_lpg) - 1)) == 0) gc[g] = cg;
      wave_sync_lds();
      int rank = 0;
      if constexpr (LPG > 0) {
#pragma unroll
        for (int h = 0; h < SEG / LPG; ++h) rank += (gc[h] > cg ? 1 : 0);
      } else {
        for (int h = 0; h < ngs; h += 2) {  // n_group is even here
          const unsigned long long c0 = gc[h], c1 = gc[h + 1];
          rank += (c0 > cg ? 1 : 0) + (c1 > cg ? 1 : 0);
        }
      }
      return rank;
    };
    float g1 = lm, g2 = l2;
    merge(g1, g2);
    uint32_t gsu = f2s(g1 + g2);
    int rank = rank_of(gsu);
    if (!exact) {
      // The kept groups' lowest score must beat the others' highest by more
      // than the error of two fast group scores.  Otherwise the group scores
      // are made exact: an expert whose fast key is below its group's fast
      // second largest minus 2 delta has an exact key below the group's exact
      // second largest (at least two experts reach the fast second largest
      // minus delta exactly), so only the experts at or above that bound
      // -- typically the group's top two -- need a correctly rounded key.
      const bool keep0 = rank < a.topk_group;
      const uint32_t kept_min = seg_min_u32<SEG>(keep0 ? gsu : 0xFFFFFFFFu);
      const uint32_t drop_max = seg_max_u32<SEG>(keep0 ? 0u : gsu);
      // next_down of the rounded difference is at most the exact one
      const float gap = next_down(s2f(kept_min) - s2f(drop_max));
      const bool need = act && !(gap > e2);  // uniform in the segment
      if (__ballot(need)) {  // wave-uniform
        const float c2 = next_down(g2 - d2);
        MaskT rm = 0;
#pragma unroll
        for (int i = 0; i < EPLM; ++i)
          if ((EPL > 0 || i < epl) && av[i] >= c2) rm |= (MaskT)1 << i;
        if (!need) rm = 0;
        const float2 et = exact_top2(reinterpret_cast<const float*>(a.logits) + row, L.bias, rm, own);
        float e1 = et.x, e2 = et.y;
        merge(e1, e2);
        if (need) gsu = f2s(e1 + e2);
        wave_sync_lds();  // every lane has read the fast composites
        rank = rank_of(gsu);
        if (a.stats && need && ls == 0) atomicAdd(&L.misc[3], 1);
      }
    }
    allowed = act && rank < a.topk_group;
    wave_sync_lds();  // every lane has read the composites before step 5 reuses the space
  }

  // ---- 3. threshold: k-th largest of the kept lanes' two largest keys ----
  // At least k keys reach it, so every key of the exact top k does (with fast
  // keys: every exact top-k key has a fast key >= it - 2 delta).
  const bool two = EPLM >= 2 && (EPL > 0 || epl >= 2);
  const uint32_t u1 = allowed ? f2s(lm) : 0u;
  const uint32_t u2 = (allowed && two) ? f2s(l2) : 0u;
  const unsigned long long ab = __ballot(allowed);
  // segment extremes, read from each segment's last lane
  const uint32_t vmax = seg_max_last<SEG>(u1);
  const uint32_t vmin = seg_min_last<SEG>(allowed ? (two ? u2 : u1) : 0xFFFFFFFFu);
  // lower end of the search: the smallest kept lane maximum when there are at
  // least k kept lanes (every lane maximum reaches it), else the smallest value
  const uint32_t vmin1 = seg_min_last<SEG>(allowed ? u1 : 0xFFFFFFFFu);
  uint32_t Ts[NSEG], bs[NSEG];
  int okseg[NSEG];
#pragma unroll
  for (int q = 0; q < NSEG; ++q) {
    const int nal = (int)__popcll(seg_bits<SEG>(ab, q));
    const uint32_t hi = readlane(vmax, q * SEG + SEG - 1);
    const uint32_t lo = nal >= a.k ? readlane(vmin1, q * SEG + SEG - 1) : readlane(vmin, q * SEG + SEG - 1);
    const int nval = nal * (two ? 2 : 1);
    okseg[q] = nval >= a.k;
    const int top = (lo >= hi) ? -1 : 31 - __builtin_clz(hi ^ lo);
    Ts[q] = top < 0 ? min(hi, lo) : (hi & ~((2u << top) - 1u));  // every value counted is >= Ts
    bs[q] = top < 0 ? 0u : (1u << top);
  }
  constexpr int kSteps = 9;  // resolve the 9 highest differing bits
#pragma unroll
  for (int j = 0; j < kSteps; ++j) {
#pragma unroll
    for (int q = 0; q < NSEG; ++q) {
      const uint32_t c = Ts[q] | bs[q];
      const int n = (int)(__popcll(seg_bits<SEG>(__ballot(u1 >= c), q)) + __popcll(seg_bits<SEG>(__ballot(u2 >= c), q)));
      Ts[q] = n >= a.k ? c : Ts[q];
      bs[q] >>= 1;
    }
  }
  const uint32_t T = (NSEG == 1 || seg == 0) ? Ts[0] : Ts[NSEG - 1];
  float thr = s2f(T);
  if (!exact) thr = next_down(thr - d2);
  const bool ok = (NSEG == 1 || seg == 0) ? okseg[0] : okseg[NSEG - 1];
  int status = (act && ok) ? TOK_DONE : TOK_ESCALATE;

  // ---- 4. candidates (keys >= thr), compacted in expert order ----
  // The sign of key - thr is 1 exactly when key < thr (keys are never -0 and a
  // nonzero difference never rounds to zero); alignbit shifts it into the mask.
  uint32_t below_lo = 0, below_hi = 0;
#pragma unroll
  for (int i = EPLM - 1; i >= 0; --i) {
    const uint32_t d = __float_as_uint(av[i] - thr);
    if (i >= 32) below_hi = __builtin_amdgcn_alignbit(below_hi, d, 31);
    else below_lo = __builtin_amdgcn_alignbit(below_lo, d, 31);
  }
  MaskT cm;
  if constexpr (EPLM > 32)
    cm = ~(((unsigned long long)below_hi << 32) | below_lo) & (epl >= 64 ? ~0ull : ((1ull << epl) - 1ull));
  else
    cm = ~below_lo & (EPLM == 32 ? 0xFFFFFFFFu : ((1u << (EPL > 0 ? EPL : epl)) - 1u));
  if (!allowed || status != TOK_DONE) cm = 0;
  const int mine = (int)__popcll((unsigned long long)cm);
  const int incl = seg_incl_scan<SEG>(mine);
  const int total = (int)seg_bcast<SEG>((uint32_t)incl);
  if (status == TOK_DONE && total > SEG) status = TOK_ESCALATE;
  int* ci = L.cand_i + w * kWave + seg * SEG;
  if (status == TOK_DONE) {
    int slot = incl - mine;
    while (cm) {
      const int i = (int)__builtin_ctzll((unsigned long long)cm);
      ci[slot++] = own.expert(i);
      cm &= cm - 1;
    }
  }
  wave_sync_lds();

  // ---- 5. ranks of the candidates by (key desc, index asc) ----
  const bool has = status == TOK_DONE && ls < total;
  const int ce = has ? ci[ls] : 0;
  float sf = 0.0f;
  unsigned long long mykey = 0ull;  // below every real key
  if constexpr (MODE == LOAD_KEYS) {
    if (has) {
      const float* kr = reinterpret_cast<const float*>(stage);
      sf = kr[a.E + ce];
      mykey = ((unsigned long long)f2s(kr[ce]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)ce);
    }
  } else if constexpr (RIK) {
    // The candidate's score is settled before the next row is requested, and
    // the request is made on every path (a wave with no next row reads one
    // 16-byte vector 16 times), so the compiler's in-order load accounting
    // never makes a later wait cover that row.
    const float x = reinterpret_cast<const float*>(a.logits)[row + (has ? ce : 0)];
    bool amb;
    float up;
    sf = sigrn::sigmoid_rn32_try(x, amb, up);
    if (__ballot(has && amb)) {
      if (has && amb) sf = sigmoid_settle(x, sf, up);
    }
    const bool pf = next_t >= 0;  // wave-uniform
    __builtin_amdgcn_sched_barrier(0);
    load_row_vec<EPLM, 0, EPLM / 8>(a, pf ? (size_t)next_t * a.E : row, pf ? own.e_slot0 : 0, pf ? ilw : 0, epl / 4,
                                    av);
    __builtin_amdgcn_sched_barrier(0);
    if (has) mykey = ((unsigned long long)f2s(sf + L.bias[ce]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)ce);
    else sf = 0.0f;
  } else if (has) {
    if constexpr (BF16) {
      uint32_t h;
      if constexpr (MODE == LOAD_STAGE) h = reinterpret_cast<const uint16_t*>(stage)[ce];
      else h = reinterpret_cast<const uint16_t*>(a.logits)[row + ce];
      sf = sig_lds(sig_off1(h));
    } else {
      float x;
      if constexpr (MODE == LOAD_STAGE) x = reinterpret_cast<const float*>(stage)[ce];
      else x = reinterpret_cast<const float*>(a.logits)[row + ce];
      sf = sigmoid_exact(x);
    }
    mykey = ((unsigned long long)f2s(sf + L.bias[ce]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)ce);
  }
  unsigned long long* cc = L.cand_c + w * kWave + seg * SEG;
  cc[ls] = mykey;
  wave_sync_lds();
  const int tot_ok = status == TOK_DONE ? total : 0;
  int tmax = (int)readlane((uint32_t)tot_ok, 0);
  if (NSEG == 2) tmax = max(tmax, (int)readlane((uint32_t)tot_ok, SEG));
  int rank = 0;
  for (int j = 0; j < tmax; j += 4) {  // entries past total hold 0 (below every key)
    const unsigned long long c0 = cc[j], c1 = cc[j + 1], c2 = cc[j + 2], c3 = cc[j + 3];
    rank += (c0 > mykey ? 1 : 0) + (c1 > mykey ? 1 : 0) + (c2 > mykey ? 1 : 0) + (c3 > mykey ? 1 : 0);
  }
  const bool sel = has && rank < a.k;

  // ---- 6. outputs in expert order; weights s / sum(s), the sum in float64 ----
  const unsigned long long sb = __ballot(sel) & (NSEG == 1 ? ~0ull : (seg ? seg1 : ~seg1));
  // picks in lower lanes (mbcnt: no lane mask held in registers)
  int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(sb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)sb, 0u));
  if (IL && ilw > 1) {
    // candidates were compacted in lane order, which is not expert order here:
    // a pick's position is the number of picks with a smaller expert id
    int* sv = reinterpret_cast<int*>(cc);
    wave_sync_lds();  // every lane has finished reading the composites
    sv[ls] = sel ? ce : 0x7FFFFFFF;
    wave_sync_lds();
    pos = 0;
    for (int j = 0; j < tmax; ++j) pos += sv[j] < ce ? 1 : 0;
  }
  const double ssum = seg_sum_d<SEG>(sel ? (double)sf : 0.0);
  // |error| <= 2^-24 (sum to FP32) + 2^-23 (rcp) + 2^-24 (product), relative
  const float rs = __builtin_amdgcn_rcpf((float)ssum);
  if (sel) {
    a.out_ids[(size_t)t * a.k + pos] = ce;
    a.out_w[(size_t)t * a.k + pos] = sf * rs;
    atomicOr(&L.bits[ce], 1ull << tl);
    L.ids[tl * a.k + pos] = ce;
  }
  wave_sync_lds();
  return status;
}

// Selection of tokens [t0, t0+nt) by one workgroup, with the histogram bitsets
// and the per-token expert lists in LDS.  Wave w, round it takes tokens
// (it*kNW + w)*NSEG + segment.
// One token over all experts: its k picks are distinct and ascending, so pick
// j owns rows [j*block, (j+1)*block) -- its slot j, then sentinels (M*k = k)
// -- and block j; no scan over the experts is needed, and only the blocks'
// experts (expert_of_block) depend on the selection.  Threads i0, i0+stride,
// ... write the rows and num_post_pad.
__device__ void one_token_rows(const Args& a, int i0, int stride) {
  const int rows = a.k * a.block;
  for (int r = i0; r < rows; r += stride) {
    const int j = div_block(r, a);
    a.sorted_ids[r] = r == j * a.block ? j : a.k;
  }
  if (i0 == 0) *a.npp = rows;
}

template <int SEG, int EPL, bool BF16, int MODE, int LPG = 0>
__device__ void select_tokens(const Args& a, const Lds& L, int t0, int nt) {
  constexpr int NSEG = kWave / SEG;
  constexpr int EPLM = EPL > 0 ? EPL : 64;
  const int tid = threadIdx.x;
  const int w = wave_index();
  const int seg = lane_id() / SEG;
  const int ls = lane_id() % SEG;
  const int sb = a.stage_bytes;
  unsigned char* stg = L.stage + (size_t)w * a.nbuf * NSEG * sb;
  auto tok_of = [&](int it) { const int tl = (it * kNW + w) * NSEG + seg; return tl < nt ? tl : -1; };
  // DMA into LDS: the sigmoid table (at LDS address 0) and the bias first, then
  // this wave's first rows, so that a wave can wait for the shared data while
  // its own rows are still in flight
  const int wbase = w * kWave * 16;  // LDS bytes of the lanes before this wave in one pass
  if (a.rows_first && a.fast && MODE == LOAD_STAGE) {
    const int tl = tok_of(0);
    stage_rows_async<SEG, EPL>(a, stg, sb, tl < 0 ? -1 : t0 + tl, BF16 ? 2 : 4);
  }
  if (a.tbl) {
    const unsigned char* src = reinterpret_cast<const unsigned char*>(sig_table_copy(a.sigtab, blockIdx.x));
    // 16 KiB per pass: the positive half to LDS byte 0, the negative half to 32768
    static_assert(kWG * 16 * 2 == kSigBytes, "two passes over the table");
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_global_load_lds(src + (size_t)(j * kWG + tid) * 16,
                                       (__attribute__((address_space(3))) void*)(size_t)(j * 32768 + wbase), 16,
                                       0, 0);
  }
  if (MODE != LOAD_KEYS && a.bias_dma) {  // precomputed keys already hold the bias
    const unsigned char* src = reinterpret_cast<const unsigned char*>(a.bias);
    unsigned char* dst = reinterpret_cast<unsigned char*>(L.bias);
    const int chunks = a.E / 4;
    for (int j = 0; j * kWG < chunks; ++j)
      if (j * kWG + tid < chunks)
        __builtin_amdgcn_global_load_lds(src + (size_t)(j * kWG + tid) * 16,
                                         (__attribute__((address_space(3))) void*)(dst + j * kWG * 16 + wbase), 16,
                                         0, 0);
  }
  // With one round per wave, only the first wave of each SIMD requests its
  // rows together with the shared data; the others request theirs after the
  // shared data has arrived, so the first rows land sooner and their compute
  // overlaps the others' transfer (measured on the 8192 x 896 workload: 4
  // early waves 20.2-20.4 us per call, 8 early 20.5, 2 early 20.5-20.6, none 20.9).
  const bool late = !a.rows_first && a.nbuf == 1 && w >= kNW / 4;
  if (!a.rows_first && !late && a.fast && MODE == LOAD_STAGE) {
    const int tl = tok_of(0);
    stage_rows_async<SEG, EPL>(a, stg, sb, tl < 0 ? -1 : t0 + tl, BF16 ? 2 : 4);
  }
  for (int e = tid; e < a.E; e += kWG) {
    L.bits[e] = 0ull;
    if (MODE != LOAD_KEYS && !a.bias_dma) L.bias[e] = a.bias[e];
  }
  if (tid == 0) {
    L.misc[0] = 0;  // tokens for the workgroup-wide exact selection
    L.misc[3] = 0;  // tokens whose group scores were made exact by their wave (statistics)
    L.misc[4] = kNW * NSEG;  // next token to claim (row-in-registers loop)
  }
  if constexpr (MODE == LOAD_KEYS) {
    // every exact key and score of the batch, one (token, expert) per thread
    // and pass: RN32 sigmoid (float64 quotient, double-double when it lies
    // near a rounding midpoint) plus the bias
    // Pair i = tl * E + e goes to thread i mod kWG, so the pairs of a batch
    // spread over every wave; both of a thread's logits are requested before
    // the first sigmoid.
    static_assert(kKeysPreMax <= 2 * kWG, "at most two (token, expert) pairs per thread");
    const int row_f = a.stage_bytes / 4;  // floats per token: E keys, then E scores
    float* kf = reinterpret_cast<float*>(L.stage);
    const int np = nt * a.E;
    const int npass = np > kWG ? 2 : 1;  // wave-uniform
    float xv[2], bv2[2];
    int tlv[2], ev[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (j < npass) {
        const int i = tid + j * kWG;
        const int ii = i < np ? i : 0;  // past the last pair: a valid dummy read
        tlv[j] = ii / a.E;
        ev[j] = ii - tlv[j] * a.E;
        bv2[j] = a.bias[ev[j]];
        xv[j] = load_logit<BF16>(a.logits, (size_t)(t0 + tlv[j]) * a.E + ev[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (j < npass && tid + j * kWG < np) {
        bool amb;
        float up;
        float sc = sigrn::sigmoid_rn32_try(xv[j], amb, up);
        if (amb) sc = sigmoid_settle(xv[j], sc, up);
        kf[tlv[j] * row_f + ev[j]] = sc + bv2[j];
        kf[tlv[j] * row_f + a.E + ev[j]] = sc;
      }
    }
  }
  if (MODE != LOAD_KEYS && (a.tbl || a.bias_dma)) {
    // loads complete in order: with R row copies issued after the shared
    // data, vmcnt <= R means the table and bias copies of this wave are done
    constexpr int R = EPL > 0 ? row_dma_count<SEG, EPL, BF16 ? 2 : 4>() : 0;
    if (!a.rows_first && !late && a.fast && MODE == LOAD_STAGE && R > 0) wait_vmem_upto<R>();
    else wait_vmem_all();
  }
  __syncthreads();
  if constexpr (MODE == LOAD_KEYS) {
    // one token over all experts: the waves without a token write the sorted
    // rows, which do not depend on the selection, while wave 0 selects (and
    // their store counts never reach wave 0's waits)
    if (a.M == 1 && a.e_lo == 0 && a.EL == a.E && w > 0) one_token_rows(a, tid - kWave, kWG - kWave);
  }
  if (late && a.fast && MODE == LOAD_STAGE) {
    const int tl = tok_of(0);
    stage_rows_async<SEG, EPL>(a, stg, sb, tl < 0 ? -1 : t0 + tl, BF16 ? 2 : 4);
  }
  if (a.fast) {
    const int epl = EPL > 0 ? EPL : a.epl;
    // the experts of the lane's register slots, as lean_token holds them
    constexpr bool IL = SEG == 64 && !BF16 && MODE == LOAD_VEC;
    const int ilw = IL ? a.ilw : 1;
    const Ownership own(ls, epl, ilw);
    constexpr bool RIK = row_in_keys<SEG, EPL, BF16, MODE>();
    float av[EPLM];  // keys of the wave's token (with RIK also its row, in flight)
    if (RIK && w * NSEG < nt) {
      // the first row overlaps the bias set-up below (its wait comes with the first key)
      const int tl = tok_of(0);
      load_row_vec<EPLM, 0, EPLM / 8>(a, (size_t)(t0 + tl) * a.E, own.e_slot0, ilw, epl / 4, av);
    }
    float bv[EPLM <= kBiasRegMax ? EPLM : 1] = {};
    float bmax = 0.0f;
    if constexpr (MODE == LOAD_KEYS) {
      // the keys are complete and exact: no biases or error bounds are needed
    } else if constexpr (EPLM <= kBiasRegMax) {
#pragma unroll
      for (int i = 0; i < EPLM; ++i) {
        bv[i] = i < epl ? L.bias[own.expert(i)] : 0.0f;
        bmax = fmaxf(bmax, fabsf(bv[i]));
      }
    } else {
      // lanes read their biases from a transposed copy: lane runs of 64
      // experts would put every lane of a wave on the same LDS bank
      for (int e = tid; e < a.E; e += kWG) {
        int slot, ln;
        Ownership::place(e, epl, ilw, slot, ln);
        L.biasT[slot * SEG + ln] = L.bias[e];
      }
      __syncthreads();
      for (int i = 0; i < epl; ++i) bmax = fmaxf(bmax, fabsf(L.biasT[i * SEG + ls]));
    }
    // Every segment covers all experts, so this is max |bias|.
    // |fast key - exact key| <= 2^-21 + rounding of both sums <= delta;
    // |fast group score - exact group score| <= 2*delta + rounding <= epsg
    const double B = 1.0 + (double)__uint_as_float(wave_max_u32(__float_as_uint(bmax))) + 0x1p-20;
    const double delta = 0x1p-21 + (B + 1.0) * 0x1p-23;
    const double epsg = 2.0 * delta + (2.0 * B + 1.0) * 0x1p-23;
    auto up_f = [](double x) {  // the least float >= x > 0, in a scalar register
      const float f = (float)x;
      const uint32_t u = __float_as_uint(f) + ((double)f < x ? 1u : 0u);
      return __uint_as_float(__builtin_amdgcn_readfirstlane(u));
    };
    const float d2 = up_f(2.0 * delta), e2 = up_f(2.0 * epsg);
    if constexpr (RIK) {
      // One token per wave at a time, taken from a workgroup counter: a wave
      // that the SIMD's issue order favours takes more tokens, so the waves of
      // a workgroup finish together (with four tokens each, the last wave of a
      // workgroup ended 12-17 us after the first on the 16384 x 4096
      // workload).  The first token is w (its first half-row was requested
      // above); the next is claimed before the current one starts, so that
      // its first half-row can be prefetched.
      int tl = w;
      while (tl < nt) {  // wave-uniform
        int nx = 0;
        if (ls == 0) nx = atomicAdd(&L.misc[4], 1);
        nx = __builtin_amdgcn_readfirstlane(nx);
        const int st =
            lean_token<SEG, EPL, BF16, MODE, LPG>(a, L, true, t0 + tl, tl, stg, bv, d2, e2, av, true,
                                                  nx < nt ? t0 + nx : -1);
        if (st == TOK_ESCALATE && ls == 0) {
          const int q = atomicAdd(&L.misc[0], 1);
          L.esc[q] = tl;
        }
        tl = nx;
      }
    } else {
      for (int it = 0; (it * kNW + w) * NSEG < nt; ++it) {
        const int tl = tok_of(it);
        const int tn = ((it + 1) * kNW + w) * NSEG < nt ? t0 + tok_of(it + 1) : -1;
        const int cb = a.nbuf > 1 ? (it & 1) : 0;
        const unsigned char* cur = stg + (size_t)(cb * NSEG + seg) * sb;
        if (MODE == LOAD_STAGE) {
          wait_vmem_all();  // this round's rows have landed in LDS
          // the host gives two buffers whenever a wave has a next round
          if (a.nbuf > 1 && ((it + 1) * kNW + w) * NSEG < nt) {
            const int tn = tok_of(it + 1);
            stage_rows_async<SEG, EPL>(a, stg + (size_t)(cb ^ 1) * NSEG * sb, sb, tn < 0 ? -1 : t0 + tn,
                                       BF16 ? 2 : 4);
          }
        }
        const bool act = tl >= 0;
        const int st = lean_token<SEG, EPL, BF16, MODE, LPG>(a, L, act, t0 + tl, tl, cur, bv, d2, e2, av, false, tn);
        if (act && st == TOK_ESCALATE && ls == 0) {
          const int q = atomicAdd(&L.misc[0], 1);
          L.esc[q] = tl;
        }
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
    exact_token_wg<BF16>(a, L, t0 + tl, tl, L.ids);
  }
  if (tid == 0 && a.stats) {
    atomicAdd(&a.stats[0], nesc);
    atomicAdd(&a.stats[1], nt - nesc);
    atomicAdd(&a.stats[2], L.misc[3]);
  }
  // no barrier here: the bitsets and expert lists were complete at the one
  // above, and exact_token_wg ends with its own
}

// Exclusive scan of padded counts over all experts into L.off; returns the
// total (in every thread).  `padded(e)` gives expert e's padded count.
template <typename F>
__device__ int expert_offsets(const Args& a, const Lds& L, int n, F padded) {
  const int tid = threadIdx.x;
  const int ept = (n + kWG - 1) / kWG;
  const int e0 = tid * ept;
  int local = 0;
  for (int i = 0; i < ept; ++i) {
    const int e = e0 + i;
    if (e < n) {
      const int p = padded(e);
      L.off[e] = p;
      local += p;
    }
  }
  int pre = wg_excl_scan<false>(L, local);
  for (int i = 0; i < ept; ++i) {
    const int e = e0 + i;
    if (e < n) {
      const int p = L.off[e];
      L.off[e] = pre;
      pre += p;
    }
  }
  if (tid == kWG - 1) L.misc[1] = pre;
  __syncthreads();
  return L.misc[1];
}

// Single-workgroup kernels: the sentinel rows after each expert's routes and
// its expert_of_block entries, for experts [0, n) with counts cnt(e) and
// offsets off[e] (multiples of the block).  A wave whose experts have short
// runs of sentinel rows lets every lane write its own expert's rows (one store
// per row of the longest run); when the longest run is more than four times
// the number of its experts with routes (a step of the walk costs about four
// such stores), the wave walks those experts and its 64 lanes write one
// expert's rows together.
template <typename F>
__device__ void write_padding(const Args& a, int n, const int* off, F cnt) {
  const int lane = lane_id();
  const int sentinel = a.M * a.k;
  for (int eb = (int)threadIdx.x - lane; eb < n; eb += kWG) {  // wave-uniform base
    const int e = eb + lane;
    int c = 0, p = 0, o = 0;
    if (e < n) {
      c = cnt(e);
      p = pad_block(c, a);
      o = off[e];
    }
    unsigned long long m = __ballot(p > 0);
    if (!m) continue;
    if ((int)wave_max_u32((uint32_t)(p - c)) <= 4 * (int)__popcll(m)) {
      if (p > 0) {
        for (int r = c; r < p; ++r) a.sorted_ids[o + r] = sentinel;
        for (int b = div_block(o, a); b < div_block(o + p, a); ++b) a.eob[b] = e;
      }
      continue;
    }
    while (m) {
      const int l = (int)__builtin_ctzll(m);
      m &= m - 1;
      const int cl = (int)readlane((uint32_t)c, l), pl = (int)readlane((uint32_t)p, l);
      const int ol = (int)readlane((uint32_t)o, l);
      for (int r = cl + lane; r < pl; r += kWave) a.sorted_ids[ol + r] = sentinel;
      const int b0 = div_block(ol, a), nb = div_block(pl, a);
      for (int b = lane; b < nb; b += kWave) a.eob[b0 + b] = eb + l;
    }
  }
}

// ----------------------------------------------------------------------------
// Kernels.
// ----------------------------------------------------------------------------
// Everything in one workgroup (M <= 64): one launch per call.
template <int SEG, int EPL, bool BF16, int MODE, int LPG = 0>
__global__ __launch_bounds__(kWG) void k_small(Args a) {
  const Lds L = carve(KIND_SMALL, a);
  const int tid = threadIdx.x;
  const bool one = a.M == 1 && a.e_lo == 0 && a.EL == a.E;
  select_tokens<SEG, EPL, BF16, MODE, LPG>(a, L, 0, a.M);
  if (one) {
    // (precomputed keys: the rows were written during the selection)
    if constexpr (MODE != LOAD_KEYS) one_token_rows(a, tid, kWG);
    for (int j = tid; j < a.k; j += kWG) a.eob[j] = L.ids[j];
    return;
  }
  // metadata of experts [e_lo, e_lo + EL), numbered from 0
  const unsigned long long* bits = L.bits + a.e_lo;
  const int sentinel = a.M * a.k;
  if (a.EL <= kWave && sentinel <= 4 * kWave) {
    // one expert per lane and a few routes: wave 0 writes all of the metadata
    // (offsets by a wave scan, no workgroup barrier)
    if (tid >= kWave) return;
    const int c = tid < a.EL ? __popcll(bits[tid]) : 0;
    const int p = pad_block(c, a);
    const int incl = wave_incl_scan(p);
    if (tid < a.EL) L.off[tid] = incl - p;
    if (tid == 0) *a.npp = (int)readlane((uint32_t)incl, kWave - 1);
    wave_sync_lds();
    write_padding(a, a.EL, L.off, [&](int e) { return __popcll(bits[e]); });
    for (int q = tid; q < sentinel; q += kWave) {
      const int e = L.ids[q] - a.e_lo;
      if ((unsigned)e < (unsigned)a.EL)
        a.sorted_ids[L.off[e] + __popcll(bits[e] & ((1ull << div_k(q, a)) - 1ull))] = q;
    }
    return;
  }
  const int total = expert_offsets(a, L, a.EL, [&](int e) { return pad_block(__popcll(bits[e]), a); });
  if (tid == 0) *a.npp = total;
  write_padding(a, a.EL, L.off, [&](int e) { return __popcll(bits[e]); });
  for (int q = tid; q < sentinel; q += kWG) {
    const int tl = div_k(q, a);
    const int e = L.ids[q] - a.e_lo;
    if ((unsigned)e < (unsigned)a.EL) {
      const int rank = __popcll(bits[e] & ((1ull << tl) - 1ull));
      a.sorted_ids[L.off[e] + rank] = q;
    }
  }
}

// Multi-workgroup path, launch 1: selection, per-workgroup histogram row and
// one record (expert, rank inside the workgroup) per slot.
template <int SEG, int EPL, bool BF16, int MODE, int LPG = 0>
__global__ __launch_bounds__(kWG) void k_select(Args a) {
  const Lds L = carve(KIND_SELECT, a);
  const int w = blockIdx.x;
  const int t0 = w * a.tw;
  const int nt = min(a.tw, a.M - t0);
  select_tokens<SEG, EPL, BF16, MODE, LPG>(a, L, t0, nt);
  // histogram row and slot records over experts [e_lo, e_lo + EL), numbered
  // from 0; a pick outside that range is recorded as a dropped route (-1)
  const unsigned long long* bits = L.bits + a.e_lo;
  for (int e = threadIdx.x; e < a.EL; e += kWG)
    a.ws_hist[(size_t)w * a.EL + e] = __popcll(bits[e]);
  const int ns = nt * a.k;
  int32_t* rec = a.ws_slot + (size_t)t0 * a.k;
  for (int q = threadIdx.x; q < ns; q += kWG) {
    const int tl = div_k(q, a);
    const int e = L.ids[q] - a.e_lo;
    rec[q] = (unsigned)e < (unsigned)a.EL ? (e | (__popcll(bits[e] & ((1ull << tl) - 1ull)) << 16)) : -1;
  }
}

// Launch 2: per expert, exclusive scan of its histogram column in workgroup
// order (in place), the expert's total and its padded total.  A block covers
// 64 experts with lane = expert, so every row access is one coalesced 256-byte
// wave load; wave w owns a contiguous range of rows, kept in registers when
// it has at most kColRegRows of them.
constexpr int kColRegRows = 16;

__global__ __launch_bounds__(kWG) void k_colscan(Args a) {
  __shared__ int part[kNW][kWave];
  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  const int e = blockIdx.x * kWave + lane;
  const bool ok = e < a.E;
  const int rpw = (a.nwg + kNW - 1) / kNW;
  const int r0 = min(a.nwg, w * rpw);
  const int r1 = min(a.nwg, r0 + rpw);
  int32_t* col = a.ws_hist + (ok ? e : 0);
  const size_t stride = (size_t)a.E;
  const bool inreg = rpw <= kColRegRows;
  int v[kColRegRows];
  int s = 0;
  if (inreg) {
#pragma unroll
    for (int r = 0; r < kColRegRows; ++r) {
      v[r] = (ok && r0 + r < r1) ? col[(size_t)(r0 + r) * stride] : 0;
      s += v[r];
    }
  } else if (ok) {
    for (int r = r0; r < r1; ++r) s += col[(size_t)r * stride];
  }
  part[w][lane] = s;
  __syncthreads();
  int pre = 0, total = 0;
#pragma unroll
  for (int q = 0; q < kNW; ++q) {
    const int x = part[q][lane];
    pre += q < w ? x : 0;
    total += x;
  }
  if (!ok) return;
  if (inreg) {
#pragma unroll
    for (int r = 0; r < kColRegRows; ++r) {
      if (r0 + r < r1) {
        col[(size_t)(r0 + r) * stride] = pre;
        pre += v[r];
      }
    }
  } else {
    for (int r = r0; r < r1; ++r) {
      const int x = col[(size_t)r * stride];
      col[(size_t)r * stride] = pre;
      pre += x;
    }
  }
  if (w == 0) {
    a.ws_tot[e] = total;
    if (a.counters) {  // -1 marks a negative counter or a segment past the capacity
      const int c0 = a.ws_c0[e];
      const long long t = (long long)total + c0;
      a.ws_pad[e] = (c0 < 0 || t > a.cap) ? -1 : pad_block((int)t, a);
    } else {
      a.ws_pad[e] = pad_block(total, a);
    }
  }
}

// Last launch: expert offsets, padding, expert_of_block and the stable
// scatter.  Everything the block reads from the workspace (its slot records,
// the padded totals, its row of column prefixes, the counts of the experts
// whose padding it writes -- or, folded, the raw histogram rows) is requested
// up front, so the block waits for one round trip.
constexpr int kRecPerThread = (kTwMax * 64 + kWG - 1) / kWG;
constexpr int kEPerThread = kEMax / kWG;
// With this many workgroups or fewer, each scatter block reads every raw
// histogram row itself (one load per row and expert, all in flight together)
// instead of waiting for a column-scan launch.
constexpr int kFoldRows = 16;

__global__ __launch_bounds__(kWG) void k_scatter(Args a) {
  const Lds L = carve(KIND_SCATTER, a);
  const int tid = threadIdx.x;
  const int w = blockIdx.x;
  const int t0 = w * a.tw;
  const int nt = min(a.tw, a.M - t0);
  const int ns = nt * a.k;
  const int32_t* rec = a.ws_slot + (size_t)t0 * a.k;
  const int32_t* colpre = a.ws_hist + (size_t)w * a.E;
  const int ept = (a.E + kWG - 1) / kWG;  // experts per thread in the offset scan (contiguous)
  const int es0 = (int)((int64_t)w * a.E / a.nwg);
  const int es1 = (int)((int64_t)(w + 1) * a.E / a.nwg);
  int rv[kRecPerThread], pv[kEPerThread];
#pragma unroll
  for (int j = 0; j < kRecPerThread; ++j) {
    const int q = tid + j * kWG;
    rv[j] = q < ns ? rec[q] : 0;
  }
  // cnt: counts of the experts this block pads (at e - es0), or, folded, of
  // every expert (at e); c0s: the caller's initial counters (sort-only entry)
  int* cnt = L.cpre + a.E;
  int* c0s = L.cpre + 2 * a.E;
  if (a.counters)
    for (int e = tid; e < a.E; e += kWG) c0s[e] = a.ws_c0[e];
  // padded size of a segment holding t routes after c0 caller rows; -1 when c0
  // is negative or the segment alone passes the caller's capacity
  auto padc = [&](int t, int c0) {
    const long long n = (long long)t + c0;
    return (c0 < 0 || n > a.cap) ? -1 : pad_block((int)n, a);
  };
  if (a.fold) {
    // the column prefix of this block (rows before it) and every expert's
    // total, from the raw histogram rows
#pragma unroll 1
    for (int i = 0; i < kEPerThread; ++i) {
      const int e2 = tid + i * kWG;
      if (e2 >= a.E) break;
      int hv[kFoldRows];
#pragma unroll
      for (int r = 0; r < kFoldRows; ++r) hv[r] = r < a.nwg ? a.ws_hist[(size_t)r * a.E + e2] : 0;
      int tot = 0, pre = 0;
#pragma unroll
      for (int r = 0; r < kFoldRows; ++r) {
        tot += hv[r];
        pre += r < w ? hv[r] : 0;
      }
      L.cpre[e2] = pre;
      cnt[e2] = tot;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kEPerThread; ++i) {
      const int e = tid * ept + i;
      pv[i] = (i < ept && e < a.E) ? (a.counters ? padc(cnt[e], c0s[e]) : pad_block(cnt[e], a)) : 0;
    }
  } else {
    int cv[kEPerThread], tv[kEPerThread];
#pragma unroll
    for (int i = 0; i < kEPerThread; ++i) {
      const int e = tid * ept + i;
      pv[i] = (i < ept && e < a.E) ? a.ws_pad[e] : 0;
      const int e2 = tid + i * kWG;
      cv[i] = e2 < a.E ? colpre[e2] : 0;
      tv[i] = es0 + e2 < es1 ? a.ws_tot[es0 + e2] : 0;
    }
#pragma unroll
    for (int i = 0; i < kEPerThread; ++i) {
      const int e2 = tid + i * kWG;
      if (e2 < a.E) L.cpre[e2] = cv[i];
      if (es0 + e2 < es1) cnt[e2] = tv[i];
    }
  }
  if (a.counters) {
    // every block reaches the same verdict; on a negative counter or a total
    // past the capacity nothing is written but num_post_pad = -1
    double part = 0.0;
#pragma unroll
    for (int i = 0; i < kEPerThread; ++i) part += pv[i] < 0 ? 1e18 : (double)pv[i];
    if (wg_sum_d(L, part) > (double)a.cap) {
      if (w == 0 && tid == 0) *a.npp = -1;
      return;
    }
  }
  // exclusive scan of the padded totals over all experts
  int local = 0;
#pragma unroll
  for (int i = 0; i < kEPerThread; ++i) local += pv[i];
  int pre = wg_excl_scan<false>(L, local);
#pragma unroll
  for (int i = 0; i < kEPerThread; ++i) {
    const int e = tid * ept + i;
    if (i < ept && e < a.E) {
      L.off[e] = pre;
      pre += pv[i];
    }
  }
  if (tid == kWG - 1) L.misc[1] = pre;
  __syncthreads();
  const int total = L.misc[1];
  if (w == 0 && tid == 0) *a.npp = total;
  const int sentinel = a.M * a.k;
  // one wave per expert of this block's share: padding rows, expert_of_block
  const int lane = lane_id();
  for (int e = es0 + (tid >> 6); e < es1; e += kNW) {
    const int c = cnt[a.fold ? e : e - es0] + (a.counters ? c0s[e] : 0);
    const int o = L.off[e];
    const int p = (e + 1 < a.E ? L.off[e + 1] : total) - o;
    for (int r = c + lane; r < p; r += kWave) a.sorted_ids[o + r] = sentinel;
    const int b0 = div_block(o, a), nb = div_block(p, a);
    for (int b = lane; b < nb; b += kWave) a.eob[b0 + b] = e;
  }
#pragma unroll
  for (int j = 0; j < kRecPerThread; ++j) {
    const int q = tid + j * kWG;
    if (q < ns && rv[j] >= 0) {  // a negative record is a dropped route (sort-only entry)
      const int e = rv[j] & 0xFFFF;
      a.sorted_ids[L.off[e] + (a.counters ? c0s[e] : 0) + L.cpre[e] + (rv[j] >> 16)] = t0 * a.k + q;
    }
  }
  if (a.counters && w == 0)  // every block read the initial values from the workspace copy
    for (int e = tid; e < a.E; e += kWG) a.counters[e] = c0s[e] + (a.fold ? cnt[e] : a.ws_tot[e]);
}

// ----------------------------------------------------------------------------
// Sort-only entry: the two sort phases from expert ids given by the caller.
// An id outside [0, E) is a dropped route: it claims no row (page "gfx1250
// ordinary-TP route optimization", Dispatch and contracts).
// ----------------------------------------------------------------------------
struct IdsLds {
  unsigned long long* bits;  // [E] bit tl: token tl of the workgroup routes to e
  int* cnt;                  // [E] routes of the workgroup per expert
  int* rec;                  // [tw*k] expert | rank << 16, or -1 for a dropped route
  int* off;                  // [E] expert offsets (single-workgroup kernel)
  int* c0;                   // [E] the caller's initial counters (single-workgroup kernel)
  double* redd;              // [kNW] partial sums
  int* misc;
  int* scan;
};
struct IdsPlan {
  size_t cnt, rec, off, c0, redd, misc, scan, total;
};
__host__ __device__ inline IdsPlan ids_lds_plan(int E, int tw, int k) {
  IdsPlan p{};
  size_t o = 0;
  auto take = [&](size_t n) { size_t r = o; o = (o + n + 15) & ~(size_t)15; return r; };
  take((size_t)E * 8);
  p.cnt = take((size_t)E * 4);
  p.rec = take((size_t)tw * k * 4);
  p.off = take((size_t)E * 4);
  p.c0 = take((size_t)E * 4);
  p.redd = take((size_t)kNW * 8);
  p.misc = take(16 * 4);
  p.scan = take((size_t)kNW * 4);
  p.total = o;
  return p;
}
__device__ inline IdsLds ids_carve(const Args& a) {
  const IdsPlan p = ids_lds_plan(a.E, a.tw, a.k);
  IdsLds L;
  L.bits = reinterpret_cast<unsigned long long*>(g_lds);
  L.cnt = reinterpret_cast<int*>(g_lds + p.cnt);
  L.rec = reinterpret_cast<int*>(g_lds + p.rec);
  L.off = reinterpret_cast<int*>(g_lds + p.off);
  L.c0 = reinterpret_cast<int*>(g_lds + p.c0);
  L.redd = reinterpret_cast<double*>(g_lds + p.redd);
  L.misc = reinterpret_cast<int*>(g_lds + p.misc);
  L.scan = reinterpret_cast<int*>(g_lds + p.scan);
  return L;
}

// Counts and stable ranks of the slots of tokens [t0, t0+nt).  With distinct
// ids in every row the rank of slot (tl, j) is the number of earlier tokens of
// the workgroup routed to the same expert (a popcount of the bitset); when a
// row repeats an expert, one thread ranks the slots in slot order instead.
__device__ void ids_local(const Args& a, const IdsLds& L, int t0, int nt) {
  const int tid = threadIdx.x;
  const int ns = nt * a.k;
  const int32_t* src = a.in_ids + (size_t)t0 * a.k;
  for (int e = tid; e < a.E; e += kWG) L.bits[e] = 0ull;
  if (tid == 0) L.misc[0] = 0;
  int iv[kRecPerThread];
#pragma unroll
  for (int j = 0; j < kRecPerThread; ++j) {
    const int q = tid + j * kWG;
    iv[j] = q < ns ? src[q] : -1;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kRecPerThread; ++j) {
    const int q = tid + j * kWG;
    const int e = iv[j];
    if (q < ns && e >= 0 && e < a.E) {
      const unsigned long long bit = 1ull << div_k(q, a);
      if (atomicOr(&L.bits[e], bit) & bit) L.misc[0] = 1;  // this token already routes to e
    }
  }
  __syncthreads();
  if (L.misc[0] == 0) {
    for (int e = tid; e < a.E; e += kWG) L.cnt[e] = __popcll(L.bits[e]);
#pragma unroll
    for (int j = 0; j < kRecPerThread; ++j) {
      const int q = tid + j * kWG;
      const int e = iv[j];
      if (q < ns) {
        const int tl = div_k(q, a);
        L.rec[q] = (e >= 0 && e < a.E) ? (e | (__popcll(L.bits[e] & ((1ull << tl) - 1ull)) << 16)) : -1;
      }
    }
  } else {
    for (int e = tid; e < a.E; e += kWG) L.cnt[e] = 0;
    __syncthreads();
    if (tid == 0) {
      for (int q = 0; q < ns; ++q) {
        const int e = src[q];
        L.rec[q] = (e >= 0 && e < a.E) ? (e | (L.cnt[e]++ << 16)) : -1;
      }
    }
  }
  __syncthreads();
}

// Multi-workgroup path, launch 1: per-workgroup histogram row and slot records.
__global__ __launch_bounds__(kWG) void k_ids_hist(Args a) {
  const IdsLds L = ids_carve(a);
  const int w = blockIdx.x;
  if (a.counters && w == 0)  // the later launches read this copy; the last one advances the counters
    for (int e = threadIdx.x; e < a.E; e += kWG) a.ws_c0[e] = a.counters[e];
  const int t0 = w * a.tw;
  const int nt = min(a.tw, a.M - t0);
  ids_local(a, L, t0, nt);
  for (int e = threadIdx.x; e < a.E; e += kWG) a.ws_hist[(size_t)w * a.E + e] = L.cnt[e];
  const int ns = nt * a.k;
  int32_t* rec = a.ws_slot + (size_t)t0 * a.k;
  for (int q = threadIdx.x; q < ns; q += kWG) rec[q] = L.rec[q];
}

// M <= 64: the whole sort in one workgroup.  With caller counters, expert e's
// segment holds counters[e] caller rows first (not written), the counters are
// read before anything is written and advanced at the end; a negative counter
// or a total past the capacity writes num_post_pad = -1 and nothing else.
__global__ __launch_bounds__(kWG) void k_ids_small(Args a) {
  const IdsLds L = ids_carve(a);
  const int tid = threadIdx.x;
  if (a.counters)
    for (int e = tid; e < a.E; e += kWG) L.c0[e] = a.counters[e];
  ids_local(a, L, 0, a.M);  // ends with a barrier
  auto c0_of = [&](int e) { return a.counters ? L.c0[e] : 0; };
  // padded size of expert e's segment; -1 for a negative counter or a
  // segment past the capacity
  auto padded = [&](int e) {
    if (!a.counters) return pad_block(L.cnt[e], a);
    const int c0 = L.c0[e];
    const long long n = (long long)L.cnt[e] + c0;
    return (c0 < 0 || n > a.cap) ? -1 : pad_block((int)n, a);
  };
  const int ept = (a.E + kWG - 1) / kWG;
  const int e0 = tid * ept;
  if (a.counters) {
    double part = 0.0;
    for (int i = 0; i < ept; ++i)
      if (e0 + i < a.E) {
        const int p = padded(e0 + i);
        part += p < 0 ? 1e18 : (double)p;
      }
    const int w = tid >> 6;
    part = wave_sum_d(part);
    if (lane_id() == 0) L.redd[w] = part;
    __syncthreads();
    double sum = 0.0;
    for (int q = 0; q < kNW; ++q) sum += L.redd[q];
    if (sum > (double)a.cap) {
      if (tid == 0) *a.npp = -1;
      return;
    }
  }
  int local = 0;
  for (int i = 0; i < ept; ++i)
    if (e0 + i < a.E) local += padded(e0 + i);
  int pre = 0;
  {  // exclusive scan of the padded counts (wave scan, then across waves)
    const int w = tid >> 6;
    const int x = wave_incl_scan(local);
    if (lane_id() == kWave - 1) L.scan[w] = x;
    __syncthreads();
    for (int q = 0; q < w; ++q) pre += L.scan[q];
    pre += x - local;
  }
  for (int i = 0; i < ept; ++i) {
    const int e = e0 + i;
    if (e < a.E) {
      L.off[e] = pre;
      pre += padded(e);
    }
  }
  if (tid == kWG - 1) *a.npp = pre;
  __syncthreads();
  const int sentinel = a.M * a.k;
  write_padding(a, a.E, L.off, [&](int e) { return c0_of(e) + L.cnt[e]; });
  for (int q = tid; q < sentinel; q += kWG) {
    const int r = L.rec[q];
    if (r >= 0) a.sorted_ids[L.off[r & 0xFFFF] + c0_of(r & 0xFFFF) + (r >> 16)] = q;
  }
  if (a.counters)
    for (int e = tid; e < a.E; e += kWG) a.counters[e] = L.c0[e] + L.cnt[e];
}

__global__ void k_zero_npp(int32_t* npp) { *npp = 0; }

__global__ __launch_bounds__(256) void k_sigmoid_probe(const float* x, int n, float* f, float* e) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    f[i] = sigmoid_fast(x[i]);
    e[i] = sigmoid_exact(x[i]);
  }
}

// Sigmoid of BF16 patterns through the LDS table, by the single-value (o1)
// and the packed-pair (o2, pairing element i with i ^ 1) address forms.
__global__ __launch_bounds__(256) void k_sigmoid_table_probe(const float* table, const uint16_t* h, int n, float* o1,
                                                             float* o2) {
  float* tab = reinterpret_cast<float*>(g_lds);
  const float* src = sig_table_copy(table, blockIdx.x);
  for (int j = threadIdx.x; j < kSigEntries; j += 256) tab[sig_lds_index(j)] = src[j];
  __syncthreads();
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    o1[i] = sig_lds(sig_off1(h[i]));
    const int p = i & ~1;
    const uint32_t d = (uint32_t)h[p] | ((p + 1 < n ? (uint32_t)h[p + 1] : 0u) << 16);
    uint32_t a0, a1;
    sig_off2(d, a0, a1);
    o2[i] = sig_lds((i & 1) ? a1 : a0);
  }
}

// ----------------------------------------------------------------------------
// Host side.
// ----------------------------------------------------------------------------
// One workgroup for the whole call (one launch) while that is faster than
// the three-launch path: its time grows with M and E while the other stays
// near 12-25 us.  Measured crossovers (one workgroup faster below them): 56
// tokens at E = 64 (FP32), 28 at E = 896 (BF16), 20 at E = 4096 (FP32), which
// M^4 * E = 6.3e8 follows; up to 16 tokens (one per wave) it was faster at
// every E measured.
bool single_wg_faster(int M, int E) {
  const double m = M;
  return M <= 16 || m * m * m * m * E <= 6.3e8;
}

int choose_tw(int M) {
  int tw = (M + 255) / 256;  // one workgroup per compute unit
  // at least 4 tokens per workgroup: below that, the per-workgroup copies of
  // the shared data and the histogram rows cost more than the extra compute
  // units save (512 x 896 workload: 14.2 us per call at 2 tokens, 13.3 at 4
  // or 8, 14.3 at 16)
  if (tw < 4) tw = 4;
  // up to 192 tokens: at most kFoldRows workgroups (at most 12 tokens each),
  // so the column scan folds into the scatter (896 experts, top-16: 96 and 128
  // tokens 12.8 us per call against 13.7, 192 tokens 13.35 against 13.75; at
  // 256 tokens, 16 per workgroup, it was 2 % slower)
  if (M <= 12 * kFoldRows && tw < (M + kFoldRows - 1) / kFoldRows) tw = (M + kFoldRows - 1) / kFoldRows;
  if (tw > kTwMax) tw = kTwMax;
  return tw;
}

bool valid_sizes(int M, int E, int k, int block) {
  return M >= 0 && E >= 1 && E <= kEMax && k >= 1 && k <= 64 && block >= 1;
}

int64_t max_rows_of(int M, int E, int k, int block) {
  const int64_t routes = (int64_t)M * k;
  return routes + (routes < E ? routes : (int64_t)E) * (int64_t)(block - 1);
}

size_t align16(size_t n) { return (n + 15) & ~(size_t)15; }

size_t workspace_of(int M, int E, int k) {
  if (M == 0) return 0;
  const int tw = choose_tw(M);
  const int64_t nwg = ((int64_t)M + tw - 1) / tw;
  return kWsHeader + align16((size_t)3 * E * 4) + align16((size_t)nwg * E * 4) +
         align16((size_t)M * k * 4);
}

typedef void (*KernelFn)(Args);

// Experts per lane compiled as constants (straight-line code).  With 64-lane
// segments any other value runs the variant that reads it at run time; 32-lane
// segments are used only for the listed values.  FP32 rows with 64 experts per
// lane also take the run-time variant: the constant one issues fewer
// instructions but measured slower on the 16384 x 4096 workload (k_select
// 72.5 against 68.9 us).  A lane run that is a whole number of 16-byte vectors
// loads straight from HBM (LOAD_VEC), otherwise the rows go through the wave's
// LDS staging buffers (LOAD_STAGE).
constexpr bool vec_mode(int epl, bool bf16) { return (epl * (bf16 ? 2 : 4)) % 16 == 0; }
bool seg32_epl(int epl) {
  return epl == 2 || epl == 4 || epl == 8 || epl == 16 || epl == 28 || epl == 32;
}

#define MRS_PICK(KER)                                                                              \
  template <int SEG, int EPL, bool BF16>                                                           \
  KernelFn fix_##KER() { return KER<SEG, EPL, BF16, vec_mode(EPL, BF16) ? LOAD_VEC : LOAD_STAGE>; } \
  template <bool BF16>                                                                             \
  KernelFn pick1_##KER(int seg, int epl, int mode) {                                               \
    if (seg == 32) {                                                                               \
      switch (epl) {                                                                               \
        case 2: return fix_##KER<32, 2, BF16>();                                                   \
        case 4: return fix_##KER<32, 4, BF16>();                                                   \
        case 8: return fix_##KER<32, 8, BF16>();                                                   \
        case 16: return fix_##KER<32, 16, BF16>();                                                 \
        case 28: return fix_##KER<32, 28, BF16>();                                                 \
        case 32: return fix_##KER<32, 32, BF16>();                                                 \
        default: return nullptr;                                                                   \
      }                                                                                            \
    }                                                                                              \
    switch (epl) {                                                                                 \
      case 1: return fix_##KER<64, 1, BF16>();                                                     \
      case 2: return fix_##KER<64, 2, BF16>();                                                     \
      case 4: return fix_##KER<64, 4, BF16>();                                                     \
      case 8: return fix_##KER<64, 8, BF16>();                                                     \
      case 14: return fix_##KER<64, 14, BF16>();                                                   \
      case 16: return fix_##KER<64, 16, BF16>();                                                   \
      case 32: return fix_##KER<64, 32, BF16>();                                                   \
      case 64:                                                                                     \
        if constexpr (BF16) return fix_##KER<64, 64, BF16>();                                      \
        [[fallthrough]];                                                                           \
      default: return mode == LOAD_VEC ? KER<64, 0, BF16, LOAD_VEC> : KER<64, 0, BF16, LOAD_STAGE>; \
    }                                                                                              \
  }                                                                                                \
  KernelFn pick_##KER(int seg, int epl, bool bf16, int mode) {                                     \
    return bf16 ? pick1_##KER<true>(seg, epl, mode) : pick1_##KER<false>(seg, epl, mode);         \
  }
MRS_PICK(k_small)
MRS_PICK(k_select)
#undef MRS_PICK

// Layouts compiled with the lanes per group fixed (group stage without run-time
// branches): BF16 rows of 896 experts in 8 groups, as 32-lane segments of 28
// experts per lane (batches) and as 64-lane segments of 14 (a few tokens).
KernelFn pick_fixed_group(bool small, int seg, int epl, bool bf16, int mode, int lpg) {
  if (!bf16 || mode != LOAD_STAGE) return nullptr;
  if (seg == 32 && epl == 28 && lpg == 4)
    return small ? k_small<32, 28, true, LOAD_STAGE, 4> : k_select<32, 28, true, LOAD_STAGE, 4>;
  if (seg == 64 && epl == 14 && lpg == 8)
    return small ? k_small<64, 14, true, LOAD_STAGE, 8> : k_select<64, 14, true, LOAD_STAGE, 8>;
  return nullptr;
}

// Precomputed keys (LOAD_KEYS), 64-lane segments: the usual experts per lane
// compiled as constants, BF16 rows of 896 experts in 8 groups also with the
// lanes per group (8) fixed; other layouts read both at run time.
template <bool BF16>
KernelFn pick1_keys_small(int epl) {
  switch (epl) {
    case 1: return k_small<64, 1, BF16, LOAD_KEYS>;
    case 2: return k_small<64, 2, BF16, LOAD_KEYS>;
    case 4: return k_small<64, 4, BF16, LOAD_KEYS>;
    case 8: return k_small<64, 8, BF16, LOAD_KEYS>;
    case 14: return k_small<64, 14, BF16, LOAD_KEYS>;
    case 16: return k_small<64, 16, BF16, LOAD_KEYS>;
    default: return k_small<64, 0, BF16, LOAD_KEYS>;
  }
}
KernelFn pick_keys_small(int epl, bool bf16, int lpg) {
  // eight lanes per group: the 896-expert shape (BF16 decode, FP32 gate
  // output) and 64 experts in 8 groups
  if (epl == 14 && lpg == 8) return bf16 ? k_small<64, 14, true, LOAD_KEYS, 8> : k_small<64, 14, false, LOAD_KEYS, 8>;
  if (epl == 1 && lpg == 8) return bf16 ? k_small<64, 1, true, LOAD_KEYS, 8> : k_small<64, 1, false, LOAD_KEYS, 8>;
  return bf16 ? pick1_keys_small<true>(epl) : pick1_keys_small<false>(epl);
}

// Optional HIP events of one call (diagnostics): launch i is made with
// hipExtLaunchKernel, which stamps ev[2i] and ev[2i+1] with the start and end
// of that kernel's own execution.
constexpr int kMaxLaunches = 3;
struct Timing {
  hipEvent_t ev[2 * kMaxLaunches];
  int n;  // launches so far
};

// Raises a kernel's dynamic-LDS limit when a launch needs more than 64 KiB;
// the largest value set so far per (kernel, device) is remembered, so the
// runtime is asked once per kernel and device rather than on every launch.
bool ensure_lds_limit(const void* fn, size_t lds) {
  if (lds <= 64 * 1024) return true;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  static std::mutex mu;
  static std::unordered_map<const void*, size_t> set[kMaxDevices];
  if (dev < 0 || dev >= kMaxDevices) return false;
  std::lock_guard<std::mutex> lock(mu);
  size_t& cur = set[dev][fn];
  if (cur >= lds) return true;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) return false;
  cur = lds;
  return true;
}

int launch(const void* fn, int grid, int block, size_t lds, hipStream_t stream, void** params, Timing* tm) {
  if (!ensure_lds_limit(fn, lds)) return MRS_ERR_LAUNCH;
  hipError_t err;
  if (tm) {
    if (tm->n >= kMaxLaunches) return MRS_ERR_LAUNCH;
    err = hipExtLaunchKernel(fn, dim3(grid), dim3(block), params, lds, stream, tm->ev[2 * tm->n],
                             tm->ev[2 * tm->n + 1], 0);
    ++tm->n;
  } else {
    err = hipLaunchKernel(fn, dim3(grid), dim3(block), params, lds, stream);
  }
  return err == hipSuccess ? MRS_OK : MRS_ERR_LAUNCH;
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Kernels that read the sigmoid table address it at LDS address 0, which
// holds when they have no static LDS (their dynamic LDS then starts at 0).
bool no_static_lds(const void* fn) {
  static std::mutex mu;
  static std::unordered_map<const void*, bool> known;
  std::lock_guard<std::mutex> lock(mu);
  auto it = known.find(fn);
  if (it != known.end()) return it->second;
  hipFuncAttributes attr{};
  const bool ok = hipFuncGetAttributes(&attr, fn) == hipSuccess && attr.sharedSizeBytes == 0;
  known.emplace(fn, ok);
  return ok;
}

// Scratch of moe_route_sort_static: the workspace of a call held in the
// library's own device memory, one copy per GPU for the life of the process.
// Host code never uses the array's name as an address: scratch_address()
// asks the runtime for the current device's address once per device
// (hipGetSymbolAddress) and every launch gets that pointer.  No call reads a
// scratch word that it did not write earlier in the same call, so the array
// needs no clearing; calls that overlap in time on one GPU share it and race.
constexpr size_t kStaticScratchBytes = (size_t)8 << 20;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MRS_ERR_LAUNCH;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MRS_ERR_LAUNCH;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MRS_OK;
}

// The device address of the sigmoid table (looked up once per device; no
// launch, no wait).
std::atomic<const float*> g_table_addr[kMaxDevices];
std::mutex g_table_mu;

int sig_table_address(const float** table) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MRS_ERR_LAUNCH;
  const float* t = g_table_addr[dev].load(std::memory_order_acquire);
  if (!t) {
    std::lock_guard<std::mutex> lock(g_table_mu);
    t = g_table_addr[dev].load(std::memory_order_relaxed);
    if (!t) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_sig_table)) != hipSuccess || p == nullptr) return MRS_ERR_LAUNCH;
      t = reinterpret_cast<const float*>(p);
      g_table_addr[dev].store(t, std::memory_order_release);
    }
  }
  *table = t;
  return MRS_OK;
}

}  // namespace

int mrs_check_route_args(const void* logits, const float* bias, int M, int E, int k, int n_group,
                         int topk_group, int block, const int32_t* out_ids, const float* out_w,
                         const int32_t* sorted_ids, const int32_t* expert_of_block,
                         const int32_t* num_post_pad, int logits_dtype) {
  if (!valid_sizes(M, E, k, block) || n_group < 1 || E % n_group != 0 || topk_group < 1 ||
      topk_group > n_group || (int64_t)k > (int64_t)topk_group * (E / n_group) ||
      (logits_dtype != MRS_DTYPE_F32 && logits_dtype != MRS_DTYPE_BF16))
    return MRS_ERR_INVALID_ARG;
  if ((int64_t)M * k > INT32_MAX) return MRS_ERR_OVERFLOW;
  if (num_post_pad == nullptr) return MRS_ERR_NULL_POINTER;
  if (!aligned(num_post_pad, 4)) return MRS_ERR_MISALIGNED;
  if (M == 0) return MRS_OK;  // only num_post_pad is written
  if (!logits || !bias || !out_ids || !out_w || !sorted_ids || !expert_of_block) return MRS_ERR_NULL_POINTER;
  if (!aligned(logits, 16) || !aligned(bias, 4) || !aligned(out_ids, 4) || !aligned(out_w, 4) ||
      !aligned(sorted_ids, 4) || !aligned(expert_of_block, 4))
    return MRS_ERR_MISALIGNED;
  return MRS_OK;
}

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
    case MRS_ERR_SCRATCH: return "the call needs more scratch than moe_route_sort_static's 8 MiB";
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
  return workspace_of(M, E, k);
}

static int route_sort_impl(const void* logits, const float* bias, int M, int E, int k, int n_group,
                           int topk_group, int block, int e_lo, int EL, int32_t* out_ids, float* out_w,
                           int32_t* sorted_ids, int32_t* expert_of_block, int32_t* num_post_pad,
                           int logits_dtype, void* workspace, size_t workspace_bytes, void* stream,
                           unsigned flags, int32_t* stats, Timing* tm) {
  const unsigned known = MRS_FLAG_FORCE_SINGLE_WG | MRS_FLAG_FORCE_MULTI_WG | MRS_FLAG_FORCE_EXACT;
  if ((flags & ~known) != 0u) return MRS_ERR_INVALID_ARG;
  if ((flags & MRS_FLAG_FORCE_SINGLE_WG) && (flags & MRS_FLAG_FORCE_MULTI_WG)) return MRS_ERR_INVALID_ARG;
  if (e_lo < 0 || EL < 1 || e_lo > E - EL) return MRS_ERR_INVALID_ARG;
  {
    const int rc = mrs_check_route_args(logits, bias, M, E, k, n_group, topk_group, block, out_ids, out_w,
                                        sorted_ids, expert_of_block, num_post_pad, logits_dtype);
    if (rc != MRS_OK) return rc;
  }
  if (max_rows_of(M, EL, k, block) > INT32_MAX) return MRS_ERR_OVERFLOW;
  if (stats && !aligned(stats, 4)) return MRS_ERR_MISALIGNED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (M == 0) {
    void* params[] = {&num_post_pad};
    return launch(reinterpret_cast<const void*>(k_zero_npp), 1, 1, 0, st, params, tm);
  }

  Args a{};
  a.logits = logits;
  a.bias = bias;
  a.M = M;
  a.E = E;
  a.e_lo = e_lo;
  a.EL = EL;
  a.k = k;
  a.n_group = n_group;
  a.topk_group = topk_group;
  a.block = block;
  {
    uint32_t l = 0;
    while ((1ull << l) < (unsigned long long)block) ++l;
    a.blk_sh = 31 + l;
    a.blk_mul = ((1ull << (31 + l)) + (unsigned long long)block - 1) / (unsigned long long)block;
  }
  a.k_mul = ((1u << 18) + (uint32_t)k - 1u) / (uint32_t)k;
  a.G = E / n_group;
  a.gstage = (n_group > 1 && topk_group < n_group && a.G > 1) ? 1 : 0;
  a.out_ids = out_ids;
  a.out_w = out_w;
  a.sorted_ids = sorted_ids;
  a.eob = expert_of_block;
  a.npp = num_post_pad;
  a.stats = stats;
  const bool bf16 = logits_dtype == MRS_DTYPE_BF16;
  const int sz = bf16 ? 2 : 4;
  const bool want_small = M <= kTwMax && !(flags & MRS_FLAG_FORCE_MULTI_WG) &&
                          ((flags & MRS_FLAG_FORCE_SINGLE_WG) || single_wg_faster(M, E));
  const int tw = want_small ? M : choose_tw(M);

  // Wave layout: 32-lane segments (two tokens per wave) when the shape allows
  // and more than one token per wave is available, else 64-lane segments,
  // else the workgroup-wide exact path for every token.
  auto seg_ok = [&](int seg) {
    return E % seg == 0 && seg % n_group == 0 && E / seg <= 64 && (seg == 64 || seg32_epl(E / seg));
  };
  a.fast = 0;
  a.seg = kWave;
  if (!(flags & MRS_FLAG_FORCE_EXACT)) {
    const int order[2] = {tw > kNW ? 32 : 64, tw > kNW ? 64 : 32};
    for (int q = 0; q < 2 && !a.fast; ++q) {
      const int seg = order[q];
      if (!seg_ok(seg)) continue;
      const int epl = E / seg;
      const int sb = vec_mode(epl, bf16) ? 0 : E * sz;
      const int nbuf = tw > kNW * (kWave / seg) ? 2 : 1;
      const LdsPlan pl = lds_plan(want_small ? KIND_SMALL : KIND_SELECT, E, n_group, a.gstage,
                                  stage_total(1, seg, nbuf, sb), tw, k, bf16 ? 1 : 0);
      if (pl.total > kLdsLimit) continue;
      a.fast = 1;
      a.seg = seg;
      a.lg_lpg = 31 - __builtin_clz((unsigned)(seg / n_group));
      a.epl = epl;
      // FP32 vector loads with one token per wave: interleave the vectors of
      // a group's lanes (of the whole wave when no group stage runs)
      a.ilw = (seg == 64 && !bf16 && vec_mode(epl, false)) ? (a.gstage ? (1 << a.lg_lpg) : 64) : 1;
      a.stage_bytes = sb;
      a.nbuf = nbuf;
    }
  }
  if (!a.fast) {
    a.epl = 1;
    a.ilw = 1;
    a.stage_bytes = 0;
    a.nbuf = 1;
  }
  // Small batches (one token per wave, at most kKeysPreMax keys): the
  // workgroup computes every exact key into LDS up front, about one per
  // thread, instead of copying the 32 KiB table and reading rows per wave.
  a.keys_pre = 0;
  if (want_small && a.fast && a.seg == kWave && M <= kNW && (int64_t)M * E <= kKeysPreMax) {
    a.keys_pre = 1;
    a.stage_bytes = 8 * E;  // E keys then E scores per token
    a.nbuf = 1;
  }
  a.tbl = (a.fast && bf16 && !a.keys_pre) ? 1 : 0;
  a.bias_dma = (aligned(bias, 16) && E % 4 == 0) ? 1 : 0;
  const int mode = a.keys_pre ? LOAD_KEYS : (a.stage_bytes ? LOAD_STAGE : LOAD_VEC);
  const size_t stg = stage_total(a.fast, a.seg, a.nbuf, a.stage_bytes, a.keys_pre ? M : 0);

  const bool small_fits =
      M <= kTwMax && lds_plan(KIND_SMALL, E, n_group, a.gstage, stg, M, k, a.tbl).total <= kLdsLimit;
  if ((flags & MRS_FLAG_FORCE_SINGLE_WG) && !small_fits) return MRS_ERR_INVALID_ARG;
  if (want_small && !small_fits) return MRS_ERR_INVALID_ARG;  // cannot happen: the plan above fits
  if (a.tbl) {
    const int rc = sig_table_address(&a.sigtab);
    if (rc != MRS_OK) return rc;
  }
  if (want_small) {
    a.tw = M;
    a.nwg = 1;
    a.rows_first = 1;
    const size_t lds = lds_plan(KIND_SMALL, E, n_group, a.gstage, stg, a.tw, k, a.tbl).total;
    void* params[] = {&a};
    KernelFn kf = nullptr;
    if (a.keys_pre) kf = pick_keys_small(a.epl, bf16, a.gstage ? a.seg / n_group : 0);
    else if (a.gstage) kf = pick_fixed_group(true, a.seg, a.epl, bf16, mode, a.seg / n_group);
    if (!kf) kf = pick_k_small(a.seg, a.epl, bf16, mode);
    const void* fn = reinterpret_cast<const void*>(kf);
    if (a.tbl && !no_static_lds(fn)) return MRS_ERR_LAUNCH;
    return launch(fn, 1, kWG, lds, st, params, tm);
  }
  a.tw = choose_tw(M);
  a.nwg = (M + a.tw - 1) / a.tw;
  const size_t need = workspace_of(M, E, k);
  if (workspace == nullptr || workspace_bytes < need) return MRS_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return MRS_ERR_MISALIGNED;
  unsigned char* ws = reinterpret_cast<unsigned char*>(workspace) + kWsHeader;
  a.ws_tot = reinterpret_cast<int32_t*>(ws);
  a.ws_pad = a.ws_tot + E;
  ws += align16((size_t)3 * E * 4);
  a.ws_hist = reinterpret_cast<int32_t*>(ws);
  ws += align16((size_t)a.nwg * E * 4);
  a.ws_slot = reinterpret_cast<int32_t*>(ws);
  a.fold = a.nwg <= kFoldRows ? 1 : 0;
  const size_t lds_sel = lds_plan(KIND_SELECT, E, n_group, a.gstage, stg, a.tw, k, a.tbl).total;
  const size_t lds_sct = lds_plan(KIND_SCATTER, E, n_group, a.gstage, 0, a.tw, k, 0).total;
  if (lds_sel > kLdsLimit || lds_sct > kLdsLimit) return MRS_ERR_INVALID_ARG;
  void* p_one[] = {&a};
  KernelFn ks = a.gstage ? pick_fixed_group(false, a.seg, a.epl, bf16, mode, a.seg / n_group) : nullptr;
  if (!ks) ks = pick_k_select(a.seg, a.epl, bf16, mode);
  const void* fsel = reinterpret_cast<const void*>(ks);
  if (a.tbl && !no_static_lds(fsel)) return MRS_ERR_LAUNCH;
  int rc = launch(fsel, a.nwg, kWG, lds_sel, st, p_one, tm);
  // the sort phases see only the experts that get metadata
  Args as = a;
  as.E = EL;
  void* p_sort[] = {&as};
  if (rc == MRS_OK && !as.fold)
    rc = launch(reinterpret_cast<const void*>(k_colscan), (EL + kWave - 1) / kWave, kWG, 0, st, p_sort, tm);
  if (rc == MRS_OK) rc = launch(reinterpret_cast<const void*>(k_scatter), a.nwg, kWG, lds_sct, st, p_sort, tm);
  return rc;
}

int moe_route_sort_ex(const void* logits, const float* bias, int M, int E, int k, int n_group,
                      int topk_group, int block, int32_t* out_ids, float* out_w,
                      int32_t* sorted_ids, int32_t* expert_of_block, int32_t* num_post_pad,
                      int logits_dtype, void* workspace, size_t workspace_bytes, void* stream,
                      unsigned flags, int32_t* stats) {
  return route_sort_impl(logits, bias, M, E, k, n_group, topk_group, block, 0, E, out_ids, out_w, sorted_ids,
                         expert_of_block, num_post_pad, logits_dtype, workspace, workspace_bytes, stream, flags,
                         stats, nullptr);
}

int moe_route_sort_profiled(const void* logits, const float* bias, int M, int E, int k, int n_group,
                            int topk_group, int block, int32_t* out_ids, float* out_w,
                            int32_t* sorted_ids, int32_t* expert_of_block, int32_t* num_post_pad,
                            int logits_dtype, void* workspace, size_t workspace_bytes, void* stream,
                            unsigned flags, int32_t* stats, void* const* events, int* n_launches) {
  if (!events || !n_launches) return MRS_ERR_NULL_POINTER;
  Timing tm{};
  for (int i = 0; i < 2 * kMaxLaunches; ++i) {
    if (!events[i]) return MRS_ERR_NULL_POINTER;
    tm.ev[i] = reinterpret_cast<hipEvent_t>(events[i]);
  }
  const int rc = route_sort_impl(logits, bias, M, E, k, n_group, topk_group, block, 0, E, out_ids, out_w,
                                 sorted_ids, expert_of_block, num_post_pad, logits_dtype, workspace,
                                 workspace_bytes, stream, flags, stats, &tm);
  *n_launches = tm.n;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  for (int i = 2 * tm.n; rc == MRS_OK && i < 2 * kMaxLaunches; ++i)
    if (hipEventRecord(tm.ev[i], st) != hipSuccess) return MRS_ERR_LAUNCH;
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

int moe_route_sort_static(const void* logits, const float* bias, int M, int E, int k, int n_group,
                          int topk_group, int block, int32_t* out_ids, float* out_w, int32_t* sorted_ids,
                          int32_t* expert_of_block, int32_t* num_post_pad, int logits_dtype, void* stream) {
  const int rc = mrs_check_route_args(logits, bias, M, E, k, n_group, topk_group, block, out_ids, out_w,
                                      sorted_ids, expert_of_block, num_post_pad, logits_dtype);
  if (rc != MRS_OK) return rc;
  if (max_rows_of(M, E, k, block) > INT32_MAX) return MRS_ERR_OVERFLOW;
  if (workspace_of(M, E, k) > kStaticScratchBytes) return MRS_ERR_SCRATCH;
  void* ws = nullptr;
  if (workspace_of(M, E, k) > 0) {
    const int rs = scratch_address(&ws);
    if (rs != MRS_OK) return rs;
  }
  return route_sort_impl(logits, bias, M, E, k, n_group, topk_group, block, 0, E, out_ids, out_w, sorted_ids,
                         expert_of_block, num_post_pad, logits_dtype, ws, ws ? kStaticScratchBytes : 0, stream,
                         0u, nullptr, nullptr);
}

int moe_route_sort_local(const void* logits, const float* bias, int M, int E, int k, int n_group,
                         int topk_group, int block, int local_begin, int local_count, int32_t* out_ids,
                         float* out_w, int32_t* sorted_ids, int32_t* expert_of_block, int32_t* num_post_pad,
                         int logits_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return route_sort_impl(logits, bias, M, E, k, n_group, topk_group, block, local_begin, local_count, out_ids,
                         out_w, sorted_ids, expert_of_block, num_post_pad, logits_dtype, workspace,
                         workspace_bytes, stream, 0u, nullptr, nullptr);
}

static int sort_from_ids_impl(const int32_t* ids, int M, int E, int k, int block, int32_t* counters,
                              int64_t rows_capacity, int32_t* sorted_ids, int32_t* expert_of_block,
                              int32_t* num_post_pad, void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_sizes(M, E, k, block)) return MRS_ERR_INVALID_ARG;
  if (counters && (rows_capacity < 0 || rows_capacity > (int64_t)INT32_MAX - (block - 1)))
    return MRS_ERR_INVALID_ARG;
  if ((int64_t)M * k > INT32_MAX || (!counters && max_rows_of(M, E, k, block) > INT32_MAX))
    return MRS_ERR_OVERFLOW;
  if (num_post_pad == nullptr) return MRS_ERR_NULL_POINTER;
  if (!aligned(num_post_pad, 4)) return MRS_ERR_MISALIGNED;
  if (counters && !aligned(counters, 4)) return MRS_ERR_MISALIGNED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (M == 0 && !counters) {
    void* params[] = {&num_post_pad};
    return launch(reinterpret_cast<const void*>(k_zero_npp), 1, 1, 0, st, params, nullptr);
  }
  if ((M > 0 && !ids) || !sorted_ids || !expert_of_block) return MRS_ERR_NULL_POINTER;
  if (!aligned(ids, 4) || !aligned(sorted_ids, 4) || !aligned(expert_of_block, 4)) return MRS_ERR_MISALIGNED;
  Args a{};
  a.M = M;
  a.E = E;
  a.k = k;
  a.block = block;
  {
    uint32_t l = 0;
    while ((1ull << l) < (unsigned long long)block) ++l;
    a.blk_sh = 31 + l;
    a.blk_mul = ((1ull << (31 + l)) + (unsigned long long)block - 1) / (unsigned long long)block;
  }
  a.k_mul = ((1u << 18) + (uint32_t)k - 1u) / (uint32_t)k;
  a.in_ids = ids;
  a.sorted_ids = sorted_ids;
  a.eob = expert_of_block;
  a.npp = num_post_pad;
  a.counters = counters;
  a.cap = (int)(counters ? rows_capacity : 0);
  void* p_one[] = {&a};
  if (M <= kTwMax) {
    a.tw = M;
    a.nwg = 1;
    const size_t lds = ids_lds_plan(E, M, k).total;
    if (lds > kLdsLimit) return MRS_ERR_INVALID_ARG;
    return launch(reinterpret_cast<const void*>(k_ids_small), 1, kWG, lds, st, p_one, nullptr);
  }
  a.tw = choose_tw(M);
  a.nwg = (M + a.tw - 1) / a.tw;
  const size_t need = workspace_of(M, E, k);
  if (workspace == nullptr || workspace_bytes < need) return MRS_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return MRS_ERR_MISALIGNED;
  unsigned char* ws = reinterpret_cast<unsigned char*>(workspace) + kWsHeader;
  a.ws_tot = reinterpret_cast<int32_t*>(ws);
  a.ws_pad = a.ws_tot + E;
  a.ws_c0 = a.ws_tot + 2 * E;
  ws += align16((size_t)3 * E * 4);
  a.ws_hist = reinterpret_cast<int32_t*>(ws);
  ws += align16((size_t)a.nwg * E * 4);
  a.ws_slot = reinterpret_cast<int32_t*>(ws);
  a.fold = a.nwg <= kFoldRows ? 1 : 0;
  const size_t lds_h = ids_lds_plan(E, a.tw, k).total;
  const size_t lds_sct = lds_plan(KIND_SCATTER, E, 1, 0, 0, a.tw, k, 0).total;
  if (lds_h > kLdsLimit || lds_sct > kLdsLimit) return MRS_ERR_INVALID_ARG;
  int rc = launch(reinterpret_cast<const void*>(k_ids_hist), a.nwg, kWG, lds_h, st, p_one, nullptr);
  if (rc == MRS_OK && !a.fold)
    rc = launch(reinterpret_cast<const void*>(k_colscan), (E + kWave - 1) / kWave, kWG, 0, st, p_one, nullptr);
  if (rc == MRS_OK) rc = launch(reinterpret_cast<const void*>(k_scatter), a.nwg, kWG, lds_sct, st, p_one, nullptr);
  return rc;
}

int moe_sort_from_ids(const int32_t* ids, int M, int E, int k, int block, int32_t* sorted_ids,
                      int32_t* expert_of_block, int32_t* num_post_pad, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return sort_from_ids_impl(ids, M, E, k, block, nullptr, 0, sorted_ids, expert_of_block, num_post_pad, workspace,
                            workspace_bytes, stream);
}

int moe_sort_from_ids_counters(const int32_t* ids, int M, int E, int k, int block, int32_t* counters,
                               int64_t rows_capacity, int32_t* sorted_ids, int32_t* expert_of_block,
                               int32_t* num_post_pad, void* workspace, size_t workspace_bytes, void* stream) {
  if (!counters) return MRS_ERR_NULL_POINTER;
  return sort_from_ids_impl(ids, M, E, k, block, counters, rows_capacity, sorted_ids, expert_of_block,
                            num_post_pad, workspace, workspace_bytes, stream);
}

int moe_route_sort_sigmoid_table_probe(const uint16_t* bf16_bits, int n, float* out_single,
                                       float* out_pair, void* stream) {
  if (n < 0) return MRS_ERR_INVALID_ARG;
  if (n == 0) return MRS_OK;
  if (!bf16_bits || !out_single || !out_pair) return MRS_ERR_NULL_POINTER;
  if (!aligned(bf16_bits, 2) || !aligned(out_single, 4) || !aligned(out_pair, 4)) return MRS_ERR_MISALIGNED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const float* table = nullptr;
  const int rc = sig_table_address(&table);
  if (rc != MRS_OK) return rc;
  void* params[] = {&table, &bf16_bits, &n, &out_single, &out_pair};
  const hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(k_sigmoid_table_probe), dim3((n + 255) / 256),
                                         dim3(256), params, kSigLdsBytes, st);
  return err == hipSuccess ? MRS_OK : MRS_ERR_LAUNCH;
}

int moe_route_sort_sigmoid_probe(const float* x, int n, float* fast_out, float* exact_out,
                                 void* stream) {
  if (n < 0) return MRS_ERR_INVALID_ARG;
  if (n == 0) return MRS_OK;
  if (!x || !fast_out || !exact_out) return MRS_ERR_NULL_POINTER;
  if (!aligned(x, 4) || !aligned(fast_out, 4) || !aligned(exact_out, 4)) return MRS_ERR_MISALIGNED;
  void* params[] = {&x, &n, &fast_out, &exact_out};
  const hipError_t err =
      hipLaunchKernel(reinterpret_cast<const void*>(k_sigmoid_probe), dim3((n + 255) / 256), dim3(256),
                      params, 0, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? MRS_OK : MRS_ERR_LAUNCH;
}

}  // extern "C"
