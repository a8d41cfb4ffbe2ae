// Device helpers of the verify step for gfx950 (wave64): logit loads, the
// penalized key, the orderable key, fixed-point masses, Philox4x32-10 and
// block reductions.  Included by sd_verify.hip only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <limits.h>
#include <math.h>

#include "sd_verify.h"

namespace sdv {

constexpr int WAVE = 64;
constexpr int VEC = 8;                 // logits per 16-byte bf16 load
constexpr uint32_t KEEP_ALL = 0u;      // orderable cut key meaning "no top-p cut"
constexpr int NONFINITE = 1;           // RowStat.flags bit

// Arguments as the kernels see them (copied by value into every launch).
struct Args {
  const void* tgt;
  const void* drf;
  int64_t ldt, ldd;
  int dtype, B, K_max, V;
  const int32_t* ids;
  const int32_t* kpr;
  const float* temp;
  float top_p, rep, D;
  const int32_t* prior;
  const int32_t* poff;
  uint64_t seed, offset;
  uint32_t flags;
  int fp_shift;       // fixed-point scale exponent of masses (see e_fixed)
  const float* tpr;   // per-request top-p, or null (top_p)
  const float* dpr;   // per-request TV budget, or null (D)
  int Vd;             // draft rows hold ids 0..Vd-1 (Vd <= V); ids Vd..V-1 have q = 0
};

// Per processed row (target j or draft j of request r).
struct RowStat {
  float M;        // largest processed key (penalized logit, before 1/T)
  float c;        // log2(e) / T
  double Zk;      // sum over kept tokens of exp2((key - M) * c)
  uint32_t kord;  // top-p cut: tokens with orderable key >= kord are kept (KEEP_ALL: none)
  int32_t idcut;  // unused (kept for layout)
  uint32_t flags; // NONFINITE
  float kx;       // processed key of the draft token x_j (rows j < K_r)
};
static_assert(sizeof(RowStat) == 32, "RowStat layout");

__device__ __forceinline__ int request_k(const Args& a, int r) {
  return a.kpr ? a.kpr[r] : a.K_max;
}

__device__ __forceinline__ float request_top_p(const Args& a, int r) {
  return a.tpr ? a.tpr[r] : a.top_p;
}

__device__ __forceinline__ float request_D(const Args& a, int r) {
  return a.dpr ? a.dpr[r] : a.D;
}

// A request's top-p and TV budget are usable: top-p in (0, 1], D >= 0.
__device__ __forceinline__ bool params_ok(float tp, float D) {
  return tp > 0.0f && tp <= 1.0f && D >= 0.0f;
}

__device__ __forceinline__ float request_t(const Args& a, int r) {
  return a.temp ? a.temp[r] : 1.0f;
}

__device__ __forceinline__ const char* target_row(const Args& a, int r, int j) {
  const int es = a.dtype == SD_BF16 ? 2 : 4;
  return static_cast<const char*>(a.tgt) +
         ((int64_t)r * (a.K_max + 1) + j) * a.ldt * es;
}

__device__ __forceinline__ const char* draft_row(const Args& a, int r, int j) {
  const int es = a.dtype == SD_BF16 ? 2 : 4;
  return static_cast<const char*>(a.drf) +
         ((int64_t)r * a.K_max + j) * a.ldd * es;
}

// Load logits [8k, 8k+8) of a row as fp32.  Elements >= V become -inf (they
// are also excluded explicitly by callers that look at ids).  Reads never
// pass the row's 16-byte-aligned extent: a bf16 row holds a multiple of 8
// elements per stride; an fp32 row a multiple of 4.
template <int DT>
__device__ __forceinline__ void load8(const char* row, int k, int V, float (&z)[VEC]) {
  const int i0 = k * VEC;
  const uint4* p = reinterpret_cast<const uint4*>(row);
  if constexpr (DT == SD_BF16) {
    uint4 w = p[k];
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      z[2 * e] = __uint_as_float(u[e] << 16);
      z[2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
    }
  } else {
    uint4 w0 = p[2 * k];
    uint4 w1 = (i0 + 4 < V) ? p[2 * k + 1] : make_uint4(0, 0, 0, 0);
    z[0] = __uint_as_float(w0.x); z[1] = __uint_as_float(w0.y);
    z[2] = __uint_as_float(w0.z); z[3] = __uint_as_float(w0.w);
    z[4] = __uint_as_float(w1.x); z[5] = __uint_as_float(w1.y);
    z[6] = __uint_as_float(w1.z); z[7] = __uint_as_float(w1.w);
  }
  if (i0 + VEC > V) {
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      if (i0 + e >= V) z[e] = -INFINITY;
  }
}

// load8 over a row that holds only Vr logits, inside a vocabulary of V >= Vr
// ids: vectors past the row read as -inf without a memory access.
template <int DT>
__device__ __forceinline__ void load8_row(const char* row, int k, int Vr, float (&z)[VEC]) {
  if (k * VEC < Vr) {
    load8<DT>(row, k, Vr, z);
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) z[e] = -INFINITY;
  }
}

// Raw words of one 8-logit vector: one 16-byte word (bf16) or two (fp32).
template <int DT>
struct RawVec {
  uint4 w[DT == SD_BF16 ? 1 : 2];
};

// A row of Vr logits as a buffer resource over the 16-byte words that hold
// them (ceil(Vr / 8) for bf16, ceil(Vr / 4) for fp32): loads past those
// words return zeros and touch no memory.  row must be the same for every
// lane of the workgroup.
template <int DT>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const char* row, int Vr) {
  const int words = DT == SD_BF16 ? (Vr + 7) / 8 : (Vr + 3) / 4;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(row), (short)0, words * 16, 0x00020000);
}

// Issues the loads of vector k of a row (its resource from raw_rsrc) and
// returns their destination registers without waiting; a vector past the
// row end, or any vector when !in, reads zero words (which unpack turns
// into -inf) without a memory access.  The loads are issued whatever k and
// in are, so a wait for them counts exactly the loads issued after them.
template <int DT>
__device__ __forceinline__ RawVec<DT> load_raw(__amdgpu_buffer_rsrc_t rs, int k, bool in) {
  RawVec<DT> r;
  const uint32_t off = in ? (uint32_t)k * (DT == SD_BF16 ? 16u : 32u) : 0x80000000u;
  const auto v0 = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
  r.w[0] = make_uint4(v0[0], v0[1], v0[2], v0[3]);
  if constexpr (DT != SD_BF16) {
    const auto v1 = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u, 0, 0);
    r.w[1] = make_uint4(v1[0], v1[1], v1[2], v1[3]);
  }
  return r;
}

// The logits of a loaded vector k of a row of Vr logits (-inf past its end).
template <int DT>
__device__ __forceinline__ void unpack(const RawVec<DT>& r, int k, int Vr, float (&z)[VEC]) {
  if constexpr (DT == SD_BF16) {
    const uint32_t u[4] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      z[2 * e] = __uint_as_float(u[e] << 16);
      z[2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
    }
  } else {
    z[0] = __uint_as_float(r.w[0].x); z[1] = __uint_as_float(r.w[0].y);
    z[2] = __uint_as_float(r.w[0].z); z[3] = __uint_as_float(r.w[0].w);
    z[4] = __uint_as_float(r.w[1].x); z[5] = __uint_as_float(r.w[1].y);
    z[6] = __uint_as_float(r.w[1].z); z[7] = __uint_as_float(r.w[1].w);
  }
  const int i0 = k * VEC;
  if (i0 + VEC > Vr) {
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      if (i0 + e >= Vr) z[e] = -INFINITY;
  }
}

template <int DT>
__device__ __forceinline__ float load1(const char* row, int i) {
  if constexpr (DT == SD_BF16) {
    uint16_t b = reinterpret_cast<const uint16_t*>(row)[i];
    return __uint_as_float((uint32_t)b << 16);
  } else {
    return reinterpret_cast<const float*>(row)[i];
  }
}

// Repetition penalty on one logit ("What I Gave Up...", section "A knob for
// accepting more draft tokens", names the penalty; the formula is a reading:
// positive logits are divided by r, the others multiplied by r; one IEEE
// fp32 operation each, built with correctly rounded division).
__device__ __forceinline__ float penalize(float z, float r) {
  return z > 0.0f ? z / r : z * r;
}

// Monotone map of a (non-NaN) float to uint32: larger float -> larger key;
// -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t ord_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ bool nonfinite(float z) {
  return z != z || z == INFINITY;
}

// exp2 on the hardware unit (v_exp_f32): results below 2^-126 flush to 0,
// which only drops tokens whose mass is below 2^-126 of the row max.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2((key - M) * c): the unnormalized probability relative to the row max.
__device__ __forceinline__ float e_rel(float key, float M, float c) {
  return fast_exp2((key - M) * c);
}

// Fixed-point mass (truncated): deterministic, order-independent sums.
__device__ __forceinline__ uint64_t e_fixed(float e, int shift) {
  return (uint64_t)(e * __uint_as_float((uint32_t)(127 + shift) << 23));
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64 multiplies with key bumps by the Weyl constants.
__device__ __forceinline__ uint4 philox(uint4 c, uint2 k) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    if (i) {
      k.x += 0x9E3779B9u;
      k.y += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c.x), lo0 = 0xD2511F53u * c.x;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c.z), lo1 = 0xCD9E8D57u * c.z;
    c = make_uint4(hi1 ^ c.y ^ k.x, lo1, hi0 ^ c.w ^ k.y, lo0);
  }
  return c;
}

// Uniforms of (row r, position j): word 0 -> u, word 1 -> v, (w >> 8) * 2^-24.
__device__ __forceinline__ void uniforms(uint64_t seed, uint64_t off, int r, int j,
                                         float& u, float& v) {
  const uint4 b = philox(make_uint4((uint32_t)j, (uint32_t)r, (uint32_t)off,
                                    (uint32_t)(off >> 32)),
                         make_uint2((uint32_t)seed, (uint32_t)(seed >> 32)));
  u = (float)(b.x >> 8) * 0x1p-24f;
  v = (float)(b.y >> 8) * 0x1p-24f;
}

// ---- wave and block reductions (deterministic: fixed lane order) ----
//
// Cross-lane steps use DPP moves (quad permutes, row mirrors, row shifts and
// broadcasts within the 64-lane wave), which run in the vector ALU with no
// LDS round trip; the four 16-lane rows are combined through readlane.
// Every lane of the wave must be active.

enum : int {
  DPP_XOR1 = 0xB1,          // quad_perm [1, 0, 3, 2]
  DPP_XOR2 = 0x4E,          // quad_perm [2, 3, 0, 1]
  DPP_ROW_SHR1 = 0x111,
  DPP_ROW_SHR2 = 0x112,
  DPP_ROW_SHR4 = 0x114,
  DPP_ROW_SHR8 = 0x118,
  DPP_ROW_MIRROR = 0x140,   // lane i of a row reads lane 15 - i
  DPP_ROW_HALF_MIRROR = 0x141,   // lane i of a half row reads lane 7 - i
  DPP_ROW_BCAST15 = 0x142,  // lane 15 of each row to the next row
  DPP_ROW_BCAST31 = 0x143,  // lane 31 to rows 2 and 3
};

// x of the lane that DPP control CTRL names; 0 where the source lane is out
// of its row or the destination row is masked off.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i32(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xF, true);
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(dpp_i32<CTRL, ROW_MASK>(__float_as_int(x)));
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)dpp_i32<CTRL, ROW_MASK>((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)dpp_i32<CTRL, ROW_MASK>((int)(uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Value of x in lane `lane` (uniform across the wave).
__device__ __forceinline__ int lane_read(int x, int lane) {
  return __builtin_amdgcn_readlane(x, lane);
}
__device__ __forceinline__ float lane_read(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}
__device__ __forceinline__ double lane_read(double x, int lane) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ double wave_sum(double x) {
  x += dpp_f64<DPP_XOR1>(x);
  x += dpp_f64<DPP_XOR2>(x);
  x += dpp_f64<DPP_ROW_HALF_MIRROR>(x);
  x += dpp_f64<DPP_ROW_MIRROR>(x);   // every lane: its row's total
  return (lane_read(x, 0) + lane_read(x, 16)) + (lane_read(x, 32) + lane_read(x, 48));
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t x) {
#pragma unroll
  for (int o = WAVE / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f32<DPP_XOR1>(x));
  x = fmaxf(x, dpp_f32<DPP_XOR2>(x));
  x = fmaxf(x, dpp_f32<DPP_ROW_HALF_MIRROR>(x));
  x = fmaxf(x, dpp_f32<DPP_ROW_MIRROR>(x));
  return fmaxf(fmaxf(lane_read(x, 0), lane_read(x, 16)), fmaxf(lane_read(x, 32), lane_read(x, 48)));
}

// Sum across the block; every thread gets the result.  scratch: >= NT/64 doubles.
template <int NT>
__device__ __forceinline__ double block_sum(double x, double* scratch) {
  x = wave_sum(x);
  const int w = threadIdx.x / WAVE, l = threadIdx.x % WAVE;
  __syncthreads();
  if (l == 0) scratch[w] = x;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < NT / WAVE; ++i) s += scratch[i];
  return s;
}

template <int NT>
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t x, uint64_t* scratch) {
  x = wave_sum_u64(x);
  const int w = threadIdx.x / WAVE, l = threadIdx.x % WAVE;
  __syncthreads();
  if (l == 0) scratch[w] = x;
  __syncthreads();
  uint64_t s = 0;
#pragma unroll
  for (int i = 0; i < NT / WAVE; ++i) s += scratch[i];
  return s;
}

template <int NT>
__device__ __forceinline__ float block_max(float x, float* scratch) {
  x = wave_max(x);
  const int w = threadIdx.x / WAVE, l = threadIdx.x % WAVE;
  __syncthreads();
  if (l == 0) scratch[w] = x;
  __syncthreads();
  float s = -INFINITY;
#pragma unroll
  for (int i = 0; i < NT / WAVE; ++i) s = fmaxf(s, scratch[i]);
  return s;
}

template <int NT>
__device__ __forceinline__ int block_or(int x, int* scratch) {
  const int w = threadIdx.x / WAVE;
  x = __any(x) ? 1 : 0;
  __syncthreads();
  if (threadIdx.x % WAVE == 0) scratch[w] = x;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int i = 0; i < NT / WAVE; ++i) s |= scratch[i];
  return s;
}

// Wave-level inclusive scans: shifts within each 16-lane row, then the row
// totals carried to the rows above (fixed order).
__device__ __forceinline__ double wave_incl_scan(double x) {
  x += dpp_f64<DPP_ROW_SHR1>(x);
  x += dpp_f64<DPP_ROW_SHR2>(x);
  x += dpp_f64<DPP_ROW_SHR4>(x);
  x += dpp_f64<DPP_ROW_SHR8>(x);
  x += dpp_f64<DPP_ROW_BCAST15, 0xA>(x);
  x += dpp_f64<DPP_ROW_BCAST31, 0xC>(x);
  return x;
}

__device__ __forceinline__ int wave_incl_scan_int(int x) {
  x += dpp_i32<DPP_ROW_SHR1>(x);
  x += dpp_i32<DPP_ROW_SHR2>(x);
  x += dpp_i32<DPP_ROW_SHR4>(x);
  x += dpp_i32<DPP_ROW_SHR8>(x);
  x += dpp_i32<DPP_ROW_BCAST15, 0xA>(x);
  x += dpp_i32<DPP_ROW_BCAST31, 0xC>(x);
  return x;
}

// Block inclusive scan: wave scans, then the wave totals in order.
// wtot: NT / WAVE doubles.  Deterministic.
template <int NT>
__device__ __forceinline__ double block_incl_scan_fast(double x, double* wtot) {
  const int w = threadIdx.x / WAVE, l = threadIdx.x % WAVE;
  x = wave_incl_scan(x);
  __syncthreads();
  if (l == WAVE - 1) wtot[w] = x;
  __syncthreads();
  double off = 0.0;
  for (int i = 0; i < w; ++i) off += wtot[i];
  return x + off;
}

// Block exclusive scan of ints; *total receives the block total.
template <int NT>
__device__ __forceinline__ int block_excl_scan_int(int x, int* wtot, int* total) {
  const int w = threadIdx.x / WAVE, l = threadIdx.x % WAVE;
  const int incl = wave_incl_scan_int(x);
  __syncthreads();
  if (l == WAVE - 1) wtot[w] = incl;
  __syncthreads();
  int off = 0, tot = 0;
  for (int i = 0; i < NT / WAVE; ++i) {
    if (i < w) off += wtot[i];
    tot += wtot[i];
  }
  *total = tot;
  return off + incl - x;
}

// Inclusive scan of one double per thread across the block (Hillis-Steele in
// LDS, fixed order).  buf: NT doubles.  Returns the inclusive prefix.
template <int NT>
__device__ __forceinline__ double block_incl_scan(double x, double* buf) {
  __syncthreads();
  buf[threadIdx.x] = x;
  __syncthreads();
#pragma unroll
  for (int o = 1; o < NT; o <<= 1) {
    const double y = threadIdx.x >= (unsigned)o ? buf[threadIdx.x - o] : 0.0;
    __syncthreads();
    x += y;
    buf[threadIdx.x] = x;
    __syncthreads();
  }
  return x;
}

// ---- penalty set as a bitmap in LDS ----
// Bits [lo, lo + nbits) of the vocabulary; bit i - lo set iff token i is in
// prior_r (valid ids) or in the draft prefix x_0..x_{j-1} (unless
// PENALTY_PRIOR_ONLY).  Returns whether any bit can be set (block-uniform),
// i.e. whether the penalty is active for this row.
template <int NT>
__device__ __forceinline__ bool build_penalty_bitmap(const Args& a, int r, int j, int lo, int nbits,
                                     uint32_t* bm) {
  if (a.rep == 1.0f) return false;
  int p0 = 0, p1 = 0;
  if (a.prior && a.poff) {
    p0 = a.poff[r];
    p1 = a.poff[r + 1];
    if (p1 < p0) p1 = p0;
  }
  const int npre = (a.flags & SD_PENALTY_PRIOR_ONLY) ? 0 : j;
  if (p1 == p0 && npre == 0) return false;
  const int nw = (nbits + 31) / 32;
  for (int w = threadIdx.x; w < nw; w += NT) bm[w] = 0u;
  __syncthreads();
  for (int t = p0 + threadIdx.x; t < p1; t += NT) {
    const int id = a.prior[t];
    if (id >= lo && id < lo + nbits && id < a.V) atomicOr(&bm[(id - lo) >> 5], 1u << ((id - lo) & 31));
  }
  for (int t = threadIdx.x; t < npre; t += NT) {
    const int id = a.ids[(int64_t)r * a.K_max + t];
    if (id >= lo && id < lo + nbits && id < a.V) atomicOr(&bm[(id - lo) >> 5], 1u << ((id - lo) & 31));
  }
  __syncthreads();
  return true;
}

// Penalize the 8 logits of vector k (ids 8k..8k+7) whose bits are set.  The
// bitmap covers ids from lo (a multiple of 8).
__device__ __forceinline__ void apply_penalty8(const uint32_t* bm, int k, int lo, float r,
                                               float (&z)[VEC]) {
  const int b = k * VEC - lo;
  const uint32_t bits = (bm[b >> 5] >> (b & 31)) & 0xFFu;
  if (bits) {
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      if (bits & (1u << e)) z[e] = penalize(z[e], r);
  }
}

}  // namespace sdv
