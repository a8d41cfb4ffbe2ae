// Exact row-level building blocks of the verify step, written for one
// workgroup of NT threads that streams rows from global memory.  They serve
// the general multi-pass path (any dtype, any V up to 2^19, top-p on or off)
// and the exact route of the single-pass kernel.  Every result is
// returned to all threads of the block.  Included by sd_verify.hip only.
#pragma once
#include "sdv_device.h"

namespace sdv {

constexpr int HBINS = 4096;   // radix histogram bins (12 key bits)

// LDS the exact routines use (carved by the caller).
struct ExactLds {
  uint64_t* hmass;   // HBINS
  uint32_t* hcnt;    // HBINS
  uint64_t* su;      // NT   (uint64 scan buffer)
  double* sd;        // NT   (double scan buffer / reduction scratch)
  float* sf;         // NT / WAVE
  int* si;           // NT / WAVE + 4
  double* ctot;      // ceil(nvec / NT) chunk totals of a draw
};

// Top-p membership: every token whose key is at least the cut key is kept
// (tokens tied with the boundary token included).
__device__ __forceinline__ bool kept(const RowStat& s, uint32_t o) {
  return s.kord == KEEP_ALL || o >= s.kord;
}

// Processed probability of token x from its row statistics, in fp64.
__device__ __forceinline__ double prob_at(const RowStat& s, float kx, double T) {
  if (!kept(s, ord_key(kx))) return 0.0;
  return exp(((double)kx - (double)s.M) / T) / s.Zk;
}

template <int NT>
__device__ uint64_t block_incl_scan_u64(uint64_t x, uint64_t* buf) {
  __syncthreads();
  buf[threadIdx.x] = x;
  __syncthreads();
  for (int o = 1; o < NT; o <<= 1) {
    const uint64_t y = threadIdx.x >= (unsigned)o ? buf[threadIdx.x - o] : 0;
    __syncthreads();
    x += y;
    buf[threadIdx.x] = x;
    __syncthreads();
  }
  return x;
}

// Descending scan of histogram bins for the top-p crossing.
// beta = first non-empty bin (from the top) with above + mass >= TP, or the
// last non-empty bin if the masses never reach TP.  above_out = above0 +
// mass of all bins above beta.  nbins is a multiple of NT or <= NT.
template <int NT>
__device__ __forceinline__ void find_crossing(const uint64_t* hm, const uint32_t* hc, int nbins,
                              uint64_t above0, double TP, int& beta_out,
                              uint64_t& above_out, uint64_t* sbuf, int* sint) {
  const int per = nbins >= NT ? nbins / NT : 1;
  const int t = threadIdx.x;
  const bool active = t * per < nbins;
  uint64_t own = 0;
  if (active)
    for (int q = 0; q < per; ++q) own += hm[nbins - 1 - (t * per + q)];
  if (t == 0) { sint[0] = INT_MAX; sint[1] = -1; }
  const uint64_t incl = block_incl_scan_u64<NT>(own, sbuf);
  const uint64_t excl = incl - own;
  int first = INT_MAX, lastne = -1;
  if (active) {
    uint64_t run = above0 + excl;
    for (int q = 0; q < per; ++q) {
      const int pos = t * per + q, b = nbins - 1 - pos;
      if (hc[b] == 0) continue;
      lastne = pos;
      if (first == INT_MAX && (double)(run + hm[b]) >= TP) first = pos;
      run += hm[b];
    }
  }
  __syncthreads();
  if (first != INT_MAX) atomicMin(&sint[0], first);
  if (lastne >= 0) atomicMax(&sint[1], lastne);
  __syncthreads();
  const int pos = sint[0] != INT_MAX ? sint[0] : sint[1];
  if (active && pos >= t * per && pos < (t + 1) * per) {
    uint64_t run = above0 + excl;
    for (int q = t * per; q < pos; ++q) run += hm[nbins - 1 - q];
    sbuf[0] = run;   // the scan's reads of sbuf are complete
  }
  __syncthreads();
  beta_out = nbins - 1 - pos;
  above_out = sbuf[0];
  __syncthreads();
}

// Vectors per thread and step of the row passes below: RU over one row, RU2
// over two rows side by side.  A step's loads go out while the step before
// it computes (two register sets), so 2 RU (or 2 x 2 RU2) loads per thread
// are in flight.
constexpr int RU = 4;
constexpr int RU2 = 2;

// Streams one row (TWO: two rows, r2 beside r1) in steps of RUX vectors per
// thread: kv(base, u) is the vector a thread takes as the u-th of the step
// at base (steps at base = 0, RUX NT, ... while base < nvec; every thread
// runs every step); step(base, z1, z2) gets the step's logits unpacked
// (-inf past a row's end, which holds V1 or V2 logits; vectors k >= nvec
// read nothing).  The next step's loads are in flight while a step runs.
template <int DT, int NT, int RUX, bool TWO, class KV, class STEP>
__device__ __forceinline__ void stream_steps(const char* r1, int V1, const char* r2, int V2, int nvec,
                                             KV&& kv, STEP&& step) {
  RawVec<DT> a1[RUX], a2[RUX], b1[RUX], b2[RUX];
  const __amdgpu_buffer_rsrc_t rs1 = raw_rsrc<DT>(r1, V1);
  const __amdgpu_buffer_rsrc_t rs2 = raw_rsrc<DT>(r2, TWO ? V2 : 0);
  auto issue = [&](int base, RawVec<DT> (&x1)[RUX], RawVec<DT> (&x2)[RUX]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < RUX; ++u) {
      const int k = kv(base, u);
      const bool in = base < nvec && k < nvec;
      x1[u] = load_raw<DT>(rs1, k, in);
      if constexpr (TWO) x2[u] = load_raw<DT>(rs2, k, in);
    }
  };
  auto run = [&](int base, const RawVec<DT> (&x1)[RUX], const RawVec<DT> (&x2)[RUX]) __attribute__((always_inline)) {
    float z1[RUX][VEC], z2[RUX][VEC];
#pragma unroll
    for (int u = 0; u < RUX; ++u) {
      const int k = kv(base, u);
      unpack<DT>(x1[u], k, k < nvec ? V1 : 0, z1[u]);
      if constexpr (TWO) unpack<DT>(x2[u], k, k < nvec ? V2 : 0, z2[u]);
    }
    step(base, z1, z2);
  };
  constexpr int SV = RUX * NT;
  issue(0, a1, a2);
  for (int base = 0; base < nvec; base += 2 * SV) {
    issue(base + SV, b1, b2);
    run(base, a1, a2);
    if (base + SV >= nvec) break;
    issue(base + 2 * SV, a1, a2);
    run(base + SV, b1, b2);
  }
}

// One pass over vectors k = threadIdx.x + i NT (i = 0, 1, ...) of a row of V
// logits (nvec vectors of the pass; vectors past the row read as -inf):
// f(k, z) for each, in ascending i per thread.
template <int DT, int NT, class F>
__device__ __forceinline__ void row_pass(const char* row, int V, int nvec, F&& f) {
  const int tid = threadIdx.x;
  stream_steps<DT, NT, RU, false>(
      row, V, row, V, nvec,
      [&](int base, int u) __attribute__((always_inline)) { return base + u * NT + tid; },
      [&](int base, float (&z)[RU][VEC], float (&)[RU][VEC]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < RU; ++u)
          if (base + u * NT + tid < nvec) f(base + u * NT + tid, z[u]);
      });
}

// A row's pointer advanced to vector k0 (the rows of a pass over vectors
// [k0, ...))
template <int DT>
__device__ __forceinline__ const char* row_from(const char* row, int k0) {
  return row + (size_t)k0 * VEC * (DT == SD_BF16 ? 2 : 4);
}

// Max and normalizer of vectors [k0, k1) of a processed row of V logits
// (bm covers ids from bmlo): M the block max, Z = sum exp2((key - M) c)
// (0 when M is -inf), bad whether a NaN was met while every logit before it
// was -inf (otherwise a NaN makes Z NaN).  RU vectors per step (the next
// step's loads in flight), one max update (and fp64 rescale of Z) per step,
// the step's terms summed in fp32.
template <int DT, int NT>
__device__ __forceinline__ void row_max_z(const Args& a, const char* row, int V, float c, bool pen,
                                          const uint32_t* bm, int bmlo, const ExactLds& L, int k0, int k1,
                                          float& Mout, double& Zout, int& badout) {
  float m = -INFINITY;
  double Z = 0.0;
  int bad = 0;
  const int tid = threadIdx.x;
  const int nv = k1 - k0;
  stream_steps<DT, NT, RU, false>(
      row_from<DT>(row, k0), max(V - k0 * VEC, 0), row_from<DT>(row, k0), max(V - k0 * VEC, 0), nv,
      [&](int base, int u) __attribute__((always_inline)) { return base + u * NT + tid; },
      [&](int base, float (&z)[RU][VEC], float (&)[RU][VEC]) __attribute__((always_inline)) {
        float vm = -INFINITY;
#pragma unroll
        for (int u = 0; u < RU; ++u) {
          if (pen && base + u * NT + tid < nv) apply_penalty8(bm, k0 + base + u * NT + tid, bmlo, a.rep, z[u]);
#pragma unroll
          for (int e = 0; e < VEC; ++e) vm = fmaxf(vm, z[u][e]);
        }
        if (vm > m) {
          if (m > -INFINITY) Z *= exp2(((double)m - (double)vm) * (double)c);
          m = vm;
        }
        // Non-finite logits need no test per element: +inf becomes the max
        // (caught by the caller), and a NaN turns its term, hence Z, into
        // NaN once the running max is finite; only a NaN met while every
        // logit so far is -inf is looked for explicitly.
        if (m > -INFINITY) {
          float su = 0.0f;
#pragma unroll
          for (int u = 0; u < RU; ++u) {
            float sv[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) sv[e] = e_rel(z[u][e], m, c);
            su += ((sv[0] + sv[1]) + (sv[2] + sv[3])) + ((sv[4] + sv[5]) + (sv[6] + sv[7]));
          }
          Z += (double)su;
        } else {
#pragma unroll
          for (int u = 0; u < RU; ++u)
#pragma unroll
            for (int e = 0; e < VEC; ++e) bad |= z[u][e] != z[u][e];
        }
      });
  const float M = block_max<NT>(m, L.sf);
  Z = (m > -INFINITY) ? Z * exp2(((double)m - (double)M) * (double)c) : 0.0;
  Zout = block_sum<NT>(Z, L.sd);
  badout = block_or<NT>(bad, L.si);
  Mout = M;
}

// Statistics and top-p cut of one processed row, streaming it from global
// memory: pass 0 gives the max M and Z = sum exp2((key - M) c) (online per
// thread, fp64 totals); with top-p, three histogram passes over 12 + 12 + 8
// bits of the orderable key with fixed-point masses find the cut key.  The
// row holds V logits (a.V for a target row, a.Vd for a draft row: ids past
// a draft row have q = 0 and take no part).
template <int DT, int NT>
__device__ __forceinline__ RowStat row_stats_dev(const Args& a, const char* row, int V, float c,
                                 bool pen, const uint32_t* bm, const ExactLds& L, float top_p) {
  const int nvec = (V + VEC - 1) / VEC;
  float M;
  double Zall;
  int bad;
  row_max_z<DT, NT>(a, row, V, c, pen, bm, 0, L, 0, nvec, M, Zall, bad);
  if (!(M > -INFINITY) || !(M < INFINITY) || Zall != Zall) bad = 1;

  RowStat out;
  out.M = M;
  out.c = c;
  out.Zk = Zall;
  out.kord = KEEP_ALL;
  out.idcut = INT_MAX;
  out.flags = bad ? NONFINITE : 0;
  out.kx = 0.0f;
  if (bad || !(top_p < 1.0f) || V <= 1) return out;

  const int sh = a.fp_shift;
  const double tp = (double)top_p;
  // Tokens whose key is below L hold at most (1 - top_p)/2 of the mass
  // together, so the cut lies at or above L; level-1 bins below L's bin are
  // not histogrammed (they are either fully in or fully out).
  const double lg = log2((1.0 - tp) * Zall / (2.0 * (double)V));
  const float Lk = (float)((double)M + lg / (double)c);
  const uint32_t binL = (Lk > -INFINITY) ? (ord_key(Lk) >> 20) : 0u;

  // Level 1: ord bits [31:20].
  for (int b = threadIdx.x; b < HBINS; b += NT) { L.hmass[b] = 0; L.hcnt[b] = 0; }
  __syncthreads();
  uint64_t zfp = 0;
  row_pass<DT, NT>(row, V, nvec, [&](int k, float (&z)[VEC]) {
    if (pen) apply_penalty8(bm, k, 0, a.rep, z);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if (k * VEC + e >= V) continue;
      const uint64_t ef = e_fixed(e_rel(z[e], M, c), sh);
      zfp += ef;
      const uint32_t b = ord_key(z[e]) >> 20;
      if (b >= binL) {
        atomicAdd(&L.hcnt[b], 1u);
        if (ef) atomicAdd(reinterpret_cast<unsigned long long*>(&L.hmass[b]), (unsigned long long)ef);
      }
    }
  });
  const uint64_t Zfp = block_sum_u64<NT>(zfp, L.su);
  const double TP = tp * (double)Zfp;
  int b1;
  uint64_t above;
  find_crossing<NT>(L.hmass, L.hcnt, HBINS, 0, TP, b1, above, L.su, L.si);

  // Level 2: ord bits [19:8] among tokens of bin b1.
  for (int b = threadIdx.x; b < HBINS; b += NT) { L.hmass[b] = 0; L.hcnt[b] = 0; }
  __syncthreads();
  row_pass<DT, NT>(row, V, nvec, [&](int k, float (&z)[VEC]) {
    if (pen) apply_penalty8(bm, k, 0, a.rep, z);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if (k * VEC + e >= V) continue;
      const uint32_t o = ord_key(z[e]);
      if ((int)(o >> 20) != b1) continue;
      const uint32_t b = (o >> 8) & 0xFFFu;
      atomicAdd(&L.hcnt[b], 1u);
      const uint64_t ef = e_fixed(e_rel(z[e], M, c), sh);
      if (ef) atomicAdd(reinterpret_cast<unsigned long long*>(&L.hmass[b]), (unsigned long long)ef);
    }
  });
  __syncthreads();
  int b2;
  find_crossing<NT>(L.hmass, L.hcnt, HBINS, above, TP, b2, above, L.su, L.si);
  const uint32_t pre24 = ((uint32_t)b1 << 12) | (uint32_t)b2;
  if (DT == SD_BF16 && !pen) {
    // bf16 keys have zero low 16 bits: the 24-bit prefix is the whole key
    // (a penalized key is an fp32 quotient or product, so not with a penalty)
    out.kord = pre24 << 8;
    out.Zk = (double)(above + L.hmass[b2]) * exp2(-(double)sh);
    __syncthreads();
    return out;
  }

  // Level 3: ord bits [7:0] among tokens with the 24-bit prefix.
  for (int b = threadIdx.x; b < 256; b += NT) { L.hmass[b] = 0; L.hcnt[b] = 0; }
  __syncthreads();
  row_pass<DT, NT>(row, V, nvec, [&](int k, float (&z)[VEC]) {
    if (pen) apply_penalty8(bm, k, 0, a.rep, z);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if (k * VEC + e >= V) continue;
      const uint32_t o = ord_key(z[e]);
      if ((o >> 8) != pre24) continue;
      atomicAdd(&L.hcnt[o & 0xFFu], 1u);
      const uint64_t ef = e_fixed(e_rel(z[e], M, c), sh);
      if (ef) atomicAdd(reinterpret_cast<unsigned long long*>(&L.hmass[o & 0xFFu]), (unsigned long long)ef);
    }
  });
  __syncthreads();
  int b3;
  find_crossing<NT>(L.hmass, L.hcnt, 256, above, TP, b3, above, L.su, L.si);
  // The cut key's group (all tokens tied at it) is kept whole.
  out.kord = (pre24 << 8) | (uint32_t)b3;
  out.Zk = (double)(above + L.hmass[b3]) * exp2(-(double)sh);
  __syncthreads();
  return out;
}

// sum |p - q| over vectors [k0, k1) of the processed, truncated rows (the
// block's total; bm covers ids from bmlo).  TV(p, q) is half the sum over
// the whole row.  ALLK: neither row is truncated (no cut comparison).
template <int DT, int NT, bool ALLK = false>
__device__ __forceinline__ double pair_tv_range(const Args& a, const char* trow, const char* drow,
                                                const RowStat& P, const RowStat& Q, bool pen,
                                                const uint32_t* bm, int bmlo, const ExactLds& L, int k0,
                                                int k1) {
  const int V = a.V;
  const float ip = (float)(1.0 / P.Zk), iq = (float)(1.0 / Q.Zk);
  double acc = 0.0;
  const int tid = threadIdx.x;
  const int nv = k1 - k0;
  stream_steps<DT, NT, RU2, true>(
      row_from<DT>(trow, k0), max(V - k0 * VEC, 0), row_from<DT>(drow, k0), max(a.Vd - k0 * VEC, 0), nv,
      [&](int base, int u) __attribute__((always_inline)) { return base + u * NT + tid; },
      [&](int base, float (&zp)[RU2][VEC], float (&zq)[RU2][VEC]) __attribute__((always_inline)) {
        float s = 0.0f;
#pragma unroll
        for (int u = 0; u < RU2; ++u) {
          const int kr = base + u * NT + tid;
          if (kr >= nv) continue;
          const int k = k0 + kr;
          if (pen) {
            apply_penalty8(bm, k, bmlo, a.rep, zp[u]);
            apply_penalty8(bm, k, bmlo, a.rep, zq[u]);
          }
          bool kp[VEC], kq[VEC];
          bool any = false;
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const int id = k * VEC + e;
            kp[e] = id < V && (ALLK || kept(P, ord_key(zp[u][e])));
            kq[e] = id < a.Vd && (ALLK || kept(Q, ord_key(zq[u][e])));
            any |= kp[e] | kq[e];
          }
          // (vectors of the wave outside both nuclei add zeros: skipped)
          if (!__any(any)) continue;
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const float p = kp[e] ? e_rel(zp[u][e], P.M, P.c) * ip : 0.0f;
            const float q = kq[e] ? e_rel(zq[u][e], Q.M, Q.c) * iq : 0.0f;
            s += fabsf(p - q);
          }
        }
        acc += (double)s;
      });
  return block_sum<NT>(acc, L.sd);
}

// d = TV(p, q) = 1/2 sum |p - q| over the processed, truncated rows.
template <int DT, int NT>
__device__ __forceinline__ double pair_tv_dev(const Args& a, const char* trow, const char* drow,
                              const RowStat& P, const RowStat& Q, bool pen,
                              const uint32_t* bm, const ExactLds& L) {
  const int nvec = (a.V + VEC - 1) / VEC;
  return fmin(0.5 * pair_tv_range<DT, NT>(a, trow, drow, P, Q, pen, bm, 0, L, 0, nvec), 1.0);
}

struct Drawn {
  int y;
  double S;
  int resid_zero;
};

// Inverse-CDF draw over ascending token ids: mode 0 draws from
// max(p - q, 0) (falling back to p when that has no mass), mode 1 from p.
// A chunk is one wave's share of one step of a pass over the rows (mode 0:
// both rows, side by side): RU2 blocks of 64 consecutive vectors in
// ascending order, CHV = 128 consecutive vectors, so a step takes one wave
// reduction, not one per vector.  One pass writes every chunk's total; a
// block scan over the totals finds the chunk that holds t = v S; wave 0
// reads that chunk again and scans it block by block, lane by lane; the
// crossing lane walks its 8 tokens.  A vector's weights are summed in fp32
// in token order, the same running sum the walk compares, and every sum
// above that is fp64 in a fixed order.  The pass may be split over
// workgroups by chunk ranges (draw_totals) with the same totals.
constexpr int CHV = RU2 * WAVE;   // vectors per chunk

// Draw weights of vector k (0 past the row) and their fp32 sum in token
// order; sp: the sum of p alone (mode 1's weights), in the same order.  bm
// covers ids from bmlo.  ALLK: neither row is truncated (top-p off), so no
// key is compared with a cut.
template <int DT, bool ALLK = false>
__device__ __forceinline__ float draw_vec_w(const Args& a, const RowStat& P, const RowStat& Q, float ip,
                                            float iq, int k, int md, bool pen, const uint32_t* bm,
                                            int bmlo, float (&zp)[VEC], float (&zq)[VEC], float (&w)[VEC],
                                            float& sp) {
  const int V = a.V, nvec = (V + VEC - 1) / VEC;
  float s = 0.0f;
  sp = 0.0f;
  if (k >= nvec) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) w[e] = 0.0f;
    return s;
  }
  if (pen) apply_penalty8(bm, k, bmlo, a.rep, zp);
  if (md == 0 && pen) apply_penalty8(bm, k, bmlo, a.rep, zq);
  bool kp[VEC];
  bool any = false;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    kp[e] = k * VEC + e < V && (ALLK || kept(P, ord_key(zp[e])));
    any |= kp[e];
  }
  // (a weight is zero outside p's nucleus: vectors of the wave with none
  // of its tokens skip the exponentials)
  if (!__any(any)) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) w[e] = 0.0f;
    return s;
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    const int id = k * VEC + e;
    float p = kp[e] ? e_rel(zp[e], P.M, P.c) * ip : 0.0f;
    sp += p;
    if (md == 0) {
      const float q = (id < a.Vd && (ALLK || kept(Q, ord_key(zq[e])))) ? e_rel(zq[e], Q.M, Q.c) * iq : 0.0f;
      p = fmaxf(p - q, 0.0f);
    }
    w[e] = p;
    s += p;
  }
  return s;
}

// Totals of chunks [ch0, ch1) to ctot[ch] (BOTH, with md 0: the totals of
// mode 1's weights too, to ctot1[ch]).  Every thread takes part.
template <int DT, int NT, bool BOTH, bool ALLK = false>
__device__ __forceinline__ void draw_totals(const Args& a, const char* trow, const char* drow,
                                            const RowStat& P, const RowStat& Q, int md, bool pen,
                                            const uint32_t* bm, int bmlo, int ch0, int ch1, double* ctot,
                                            double* ctot1) {
  const int V = a.V, nvec = (V + VEC - 1) / VEC;
  const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
  const float ip = (float)(1.0 / P.Zk), iq = (float)(1.0 / Q.Zk);
  const int k0 = ch0 * CHV;
  const int nv = min(nvec, ch1 * CHV) - k0;
  stream_steps<DT, NT, RU2, true>(
      row_from<DT>(trow, k0), max(V - k0 * VEC, 0), row_from<DT>(drow, k0),
      md == 0 ? max(a.Vd - k0 * VEC, 0) : 0, nv,
      [&](int base, int u) __attribute__((always_inline)) { return base + wv * CHV + u * WAVE + lane; },
      [&](int base, float (&zp)[RU2][VEC], float (&zq)[RU2][VEC]) __attribute__((always_inline)) {
        const int kr0 = base + wv * CHV;   // this wave's chunk
        double ls = 0.0, ls1 = 0.0;
#pragma unroll
        for (int u = 0; u < RU2; ++u) {
          float w[VEC];
          float sp;
          ls += (double)draw_vec_w<DT, ALLK>(a, P, Q, ip, iq, k0 + kr0 + u * WAVE + lane, md, pen, bm, bmlo,
                                             zp[u], zq[u], w, sp);
          if (BOTH) ls1 += (double)sp;
        }
        const double cs = wave_sum(ls);
        const int ch = ch0 + kr0 / CHV;
        if (lane == 0 && ch < ch1) ctot[ch] = cs;
        if (BOTH) {
          const double cs1 = wave_sum(ls1);
          if (lane == 0 && ch < ch1) ctot1[ch] = cs1;
        }
      });
}

// Block scan over the nch chunk totals: S, t = v S, and the crossing
// chunk (returned; -1 when S is not positive), the mass before it in
// ctot[nch].  Every thread takes part.
template <int NT>
__device__ __forceinline__ int draw_scan(double* ctot, int nch, float v, const ExactLds& L, double& S,
                                         double& t) {
  // (thread t owns chunks t per ..)
  const int per = (nch + NT - 1) / NT;
  const int c0 = min((int)threadIdx.x * per, nch), c1 = min(c0 + per, nch);
  double own = 0.0;
  for (int ch = c0; ch < c1; ++ch) own += ctot[ch];
  const double incl = block_incl_scan_fast<NT>(own, L.sd);
  __syncthreads();   // the scan's reads of its wave totals are done
  L.sd[threadIdx.x] = incl;
  if (threadIdx.x == 0) { L.si[0] = -1; L.si[1] = -1; }
  __syncthreads();
  // the previous thread's inclusive total is this thread's exclusive one,
  // exactly: the crossing thread below is unique and exists when S > 0
  const double excl = threadIdx.x ? L.sd[threadIdx.x - 1] : 0.0;
  S = L.sd[NT - 1];
  t = (double)v * S;
  if (S > 0.0 && incl > t && excl <= t) {
    double R = excl;
    int cs = c1 - 1;
    for (int ch = c0; ch < c1; ++ch) {
      if (R + ctot[ch] > t) { cs = ch; break; }
      R += ctot[ch];
    }
    L.si[0] = cs;
    ctot[nch] = R;
  }
  __syncthreads();
  const int cs = L.si[0];
  __syncthreads();
  return cs;
}

// The token of crossing chunk cs (t and the mass before the chunk, R): wave
// 0 reads the chunk again and walks it; returned to every thread.  bm
// covers the chunk's ids, from bmlo.
template <int DT, int NT, bool ALLK = false>
__device__ __forceinline__ int draw_resolve(const Args& a, const char* trow, const char* drow,
                                            const RowStat& P, const RowStat& Q, int mode, bool pen,
                                            const uint32_t* bm, int bmlo, int cs, double t, double R0,
                                            const ExactLds& L) {
  const int V = a.V, nvec = (V + VEC - 1) / VEC;
  const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
  const float ip = (float)(1.0 / P.Zk), iq = (float)(1.0 / Q.Zk);
  if (wv == 0 && cs >= 0) {
    // the crossing chunk's RU2 blocks of 64 vectors, in ascending order
    float zp[RU2][VEC], zq[RU2][VEC];
#pragma unroll
    for (int u = 0; u < RU2; ++u) {
      const int k = cs * CHV + u * WAVE + lane;
      load8_row<DT>(trow, k, k < nvec ? V : 0, zp[u]);
      if (mode == 0) load8_row<DT>(drow, k, k < nvec ? a.Vd : 0, zq[u]);
    }
    double R = R0;
    int found = 0, y = -1, lastpos = -1;
#pragma unroll
    for (int u = 0; u < RU2; ++u) {
      const int k = cs * CHV + u * WAVE + lane;
      float w[VEC];
      float sp;
      const double ls = (double)draw_vec_w<DT, ALLK>(a, P, Q, ip, iq, k, mode, pen, bm, bmlo, zp[u], zq[u], w, sp);
      const double li = wave_incl_scan(ls);
      // the last token with weight so far (rounding fallback)
      const uint64_t pos = __ballot(ls > 0.0);
      if (pos) {
        const int lp = 63 - __builtin_clzll(pos);
        int e_last = -1;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          if (w[e] > 0.0f) e_last = e;
        const int cand = __shfl(k * VEC + e_last, lp);
        lastpos = cand;
      }
      if (!found) {
        // the first lane whose inclusive total exceeds t walks its tokens
        const uint64_t hit = __ballot(R + li > t);
        if (hit) {
          const int src = __builtin_ctzll(hit);
          int yy = -1;
          if (lane == src) {
            const double C0 = R + li - ls;
            float c = 0.0f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
              c += w[e];
              if (yy < 0 && C0 + (double)c > t) yy = k * VEC + e;
            }
          }
          y = __shfl(yy, src);
          found = 1;
        }
        R += __shfl(li, WAVE - 1);
      }
    }
    if (lane == 0) L.si[1] = (found && y >= 0) ? y : lastpos;
  }
  __syncthreads();
  const int y = L.si[1];
  __syncthreads();
  return y;
}

// The whole draw in one workgroup (L.ctot holds nch + 1 doubles).
template <int DT, int NT, bool ALLK = false>
__device__ __forceinline__ Drawn draw_dev(const Args& a, const char* trow, const char* drow, const RowStat& P,
                          const RowStat& Q, int mode, float v, bool pen, const uint32_t* bm,
                          const ExactLds& L) {
  const int nvec = (a.V + VEC - 1) / VEC;
  const int nch = (nvec + CHV - 1) / CHV;
  Drawn out;
  out.resid_zero = 0;
  double S = 0.0, t = 0.0;
  int cs = -1;
  for (int pass = 0; pass < 2; ++pass) {
    draw_totals<DT, NT, false, ALLK>(a, trow, drow, P, Q, mode, pen, bm, 0, 0, nch, L.ctot, nullptr);
    __syncthreads();
    cs = draw_scan<NT>(L.ctot, nch, v, L, S, t);
    if (!(S > 0.0) && mode == 0) {   // zero residual: draw from p
      mode = 1;
      out.resid_zero = 1;
      continue;
    }
    break;
  }
  out.S = S;
  out.y = draw_resolve<DT, NT, ALLK>(a, trow, drow, P, Q, mode, pen, bm, 0, cs, t, L.ctot[nch], L);
  return out;
}

// theta, pi(x), the acceptance test of one position (one thread).
struct Decision {
  double px, qx, th, pix;
  bool accept;
};

// The decision from p(x) and q(x) already computed.
__device__ __forceinline__ Decision decide_from(double px, double qx, double D, bool tv_valid,
                                                double d, float u) {
  Decision o;
  o.px = px;
  o.qx = qx;
  if (tv_valid) o.th = (d <= D) ? 1.0 : D / d;
  else o.th = (D >= 1.0) ? 1.0 : 0.0;   // D = 0: theta only matters when p = q
  o.pix = (1.0 - o.th) * o.px + o.th * o.qx;
  o.accept = (double)u * o.qx < o.pix;
  return o;
}

__device__ __forceinline__ Decision decide(const RowStat& P, const RowStat& Q, float kxp,
                                           float kxq, double T, double D, bool tv_valid,
                                           double d, float u) {
  return decide_from(prob_at(P, kxp, T), prob_at(Q, kxq, T), D, tv_valid, d, u);
}

}  // namespace sdv
