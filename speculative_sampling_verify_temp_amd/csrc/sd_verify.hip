// Speculative-sampling verify step on gfx950: kernels and the C ABI.
//
// Sampling path, three launches on the caller's stream:
//   k_row_prepare  one workgroup per processed row (target j <= K_r, draft
//                  j < K_r): penalty -> max M and normalizer Z of
//                  exp2((key - M) log2e / T); for top-p, an exact radix
//                  select of the cut key over fixed-point masses (tokens
//                  tied with the boundary token are kept).
//   k_pair_tv      one workgroup per position j < K_r: TV(p_j, q_j) over the
//                  processed, truncated rows (skipped when theta cannot
//                  depend on d and no statistics are requested).
//   k_finalize     one workgroup per request: theta, pi, Philox uniforms,
//                  acceptance, first rejection, then the inverse-CDF draw of
//                  the correction or bonus token by a block prefix scan.
// Greedy path, two launches: k_greedy_partial (argmax of slices of the
// target rows) and k_greedy_final (reduce, first mismatch, outputs).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <limits.h>
#include <math.h>
#include <string.h>

#include "sd_verify.h"
#include "sdv_device.h"

using namespace sdv;

namespace {

constexpr int NT_ROW = 512;                  // row kernels
constexpr int CHUNK = NT_ROW * VEC;          // logits per block step
constexpr int HBINS = 4096;                  // radix histogram bins (12 bits)
constexpr int NT_G = 256;                    // greedy partial kernel
constexpr int G_SLICE = 8192;                // logits per greedy workgroup
constexpr int MAX_V = 1 << 19;

__device__ __forceinline__ int row_index(const Args& a, int r, bool target, int j) {
  return r * (2 * a.K_max + 1) + (target ? j : a.K_max + 1 + j);
}

// Top-p membership: every token whose key is at least the cut key is kept
// (tokens tied at the boundary included).
__device__ __forceinline__ bool kept(const RowStat& s, uint32_t o, int id) {
  (void)id;
  return s.kord == KEEP_ALL || o >= s.kord;
}

// Block-wide inclusive scan of one uint64 per thread (fixed order).
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
// last non-empty bin if the masses never reach TP.  above_beta = above0 +
// mass of all bins above beta.  nbins is a multiple of NT or <= NT.
template <int NT>
__device__ void find_crossing(const uint64_t* hm, const uint32_t* hc, int nbins,
                              uint64_t above0, double TP, int& beta_out,
                              uint64_t& above_out, uint64_t* sbuf, int* sint) {
  const int per = nbins >= NT ? nbins / NT : 1;
  const int t = threadIdx.x;
  const bool active = t * per < nbins;
  // thread t owns positions [t*per, (t+1)*per) in descending bin order
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
  int pos = sint[0] != INT_MAX ? sint[0] : sint[1];
  __syncthreads();
  // mass above pos: recompute on thread 0 from the owner's exclusive prefix
  if (t == 0) sint[2] = pos;
  __syncthreads();
  pos = sint[2];
  if (active && pos >= t * per && pos < (t + 1) * per) {
    uint64_t run = above0 + excl;
    for (int q = t * per; q < pos; ++q) run += hm[nbins - 1 - q];
    sbuf[0] = run;   // sbuf is free again after the scan (all reads done)
  }
  __syncthreads();
  beta_out = nbins - 1 - pos;
  above_out = sbuf[0];
  __syncthreads();
}

// ---------------------------------------------------------------------------
// k_row_prepare: statistics and top-p cut of one processed row.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(NT_ROW) void k_row_prepare(Args a, RowStat* rs, int bm_words) {
  constexpr int NT = NT_ROW;
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* bm = reinterpret_cast<uint32_t*>(smem);
  uint64_t* hmass = reinterpret_cast<uint64_t*>(smem + ((bm_words * 4 + 15) & ~15));
  uint32_t* hcnt = reinterpret_cast<uint32_t*>(hmass + HBINS);
  __shared__ double sd[NT / WAVE];
  __shared__ float sf[NT / WAVE];
  __shared__ int si[NT / WAVE + 4];
  __shared__ uint64_t su[NT];

  const int nrows = 2 * a.K_max + 1;
  const int r = blockIdx.x / nrows, rho = blockIdx.x % nrows;
  const int K = request_k(a, r);
  if (K < 0 || K > a.K_max) return;
  const bool is_t = rho <= a.K_max;
  const int j = is_t ? rho : rho - a.K_max - 1;
  if (is_t ? (j > K) : (j >= K)) return;
  const float T = request_t(a, r);
  if (!(T > 0.0f) || !(T < INFINITY)) return;
  const char* row = is_t ? target_row(a, r, j) : draft_row(a, r, j);
  const float c = 1.4426950408889634f / T;
  const int V = a.V, nvec = (V + VEC - 1) / VEC;
  const bool pen = build_penalty_bitmap<NT>(a, r, j, 0, V, bm);

  // Pass 0: max and normalizer (per-thread online rescaling, fp64 totals).
  float m = -INFINITY;
  double Z = 0.0;
  int bad = 0;
  for (int k = threadIdx.x; k < nvec; k += NT) {
    float z[VEC];
    load8<DT>(row, k, V, z);
    if (pen) apply_penalty8(bm, k, 0, a.rep, z);
    float vm = -INFINITY;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      bad |= nonfinite(z[e]);
      vm = fmaxf(vm, z[e]);
    }
    if (vm > m) {
      if (m > -INFINITY) Z *= exp2(((double)m - (double)vm) * (double)c);
      m = vm;
    }
    if (m > -INFINITY) {
      float s[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) s[e] = e_rel(z[e], m, c);
      Z += (double)(((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7])));
    }
  }
  const float M = block_max<NT>(m, sf);
  Z = (m > -INFINITY) ? Z * exp2(((double)m - (double)M) * (double)c) : 0.0;
  const double Zall = block_sum<NT>(Z, sd);
  bad = block_or<NT>(bad, si);
  if (!(M > -INFINITY)) bad = 1;

  RowStat out;
  out.M = M;
  out.c = c;
  out.Zk = Zall;
  out.kord = KEEP_ALL;
  out.idcut = INT_MAX;
  out.flags = bad ? NONFINITE : 0;
  out.kx = 0.0f;

  if (!bad && a.top_p < 1.0f && V > 1) {
    const int sh = a.fp_shift;
    const double tp = (double)a.top_p;
    // Tokens whose key is below L hold at most (1 - top_p)/2 of the mass
    // together, so the cut lies at or above L; level-1 bins below L's bin are
    // not histogrammed (they are either fully in or fully out).
    const double lg = log2((1.0 - tp) * Zall / (2.0 * (double)V));
    const float L = (float)((double)M + lg / (double)c);
    const uint32_t binL = (L > -INFINITY) ? (ord_key(L) >> 20) : 0u;

    // Level 1: ord bits [31:20].
    for (int b = threadIdx.x; b < HBINS; b += NT) { hmass[b] = 0; hcnt[b] = 0; }
    __syncthreads();
    uint64_t zfp = 0;
    for (int k = threadIdx.x; k < nvec; k += NT) {
      float z[VEC];
      load8<DT>(row, k, V, z);
      if (pen) apply_penalty8(bm, k, 0, a.rep, z);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        if (k * VEC + e >= V) continue;
        const uint64_t ef = e_fixed(e_rel(z[e], M, c), sh);
        zfp += ef;
        const uint32_t b = ord_key(z[e]) >> 20;
        if (b >= binL) {
          atomicAdd(&hcnt[b], 1u);
          if (ef) atomicAdd(reinterpret_cast<unsigned long long*>(&hmass[b]), (unsigned long long)ef);
        }
      }
    }
    const uint64_t Zfp = block_sum_u64<NT>(zfp, su);
    const double TP = tp * (double)Zfp;
    int b1;
    uint64_t above;
    find_crossing<NT>(hmass, hcnt, HBINS, 0, TP, b1, above, su, si);

    // Level 2: ord bits [19:8] among tokens of bin b1.
    for (int b = threadIdx.x; b < HBINS; b += NT) { hmass[b] = 0; hcnt[b] = 0; }
    __syncthreads();
    for (int k = threadIdx.x; k < nvec; k += NT) {
      float z[VEC];
      load8<DT>(row, k, V, z);
      if (pen) apply_penalty8(bm, k, 0, a.rep, z);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        if (k * VEC + e >= V) continue;
        const uint32_t o = ord_key(z[e]);
        if ((int)(o >> 20) != b1) continue;
        const uint32_t b = (o >> 8) & 0xFFFu;
        atomicAdd(&hcnt[b], 1u);
        const uint64_t ef = e_fixed(e_rel(z[e], M, c), sh);
        if (ef) atomicAdd(reinterpret_cast<unsigned long long*>(&hmass[b]), (unsigned long long)ef);
      }
    }
    __syncthreads();
    int b2;
    find_crossing<NT>(hmass, hcnt, HBINS, above, TP, b2, above, su, si);
    const uint32_t pre24 = ((uint32_t)b1 << 12) | (uint32_t)b2;

    // Level 3: ord bits [7:0] among tokens with the 24-bit prefix.
    for (int b = threadIdx.x; b < 256; b += NT) { hmass[b] = 0; hcnt[b] = 0; }
    __syncthreads();
    for (int k = threadIdx.x; k < nvec; k += NT) {
      float z[VEC];
      load8<DT>(row, k, V, z);
      if (pen) apply_penalty8(bm, k, 0, a.rep, z);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        if (k * VEC + e >= V) continue;
        const uint32_t o = ord_key(z[e]);
        if ((o >> 8) != pre24) continue;
        atomicAdd(&hcnt[o & 0xFFu], 1u);
        const uint64_t ef = e_fixed(e_rel(z[e], M, c), sh);
        if (ef) atomicAdd(reinterpret_cast<unsigned long long*>(&hmass[o & 0xFFu]), (unsigned long long)ef);
      }
    }
    __syncthreads();
    int b3;
    find_crossing<NT>(hmass, hcnt, 256, above, TP, b3, above, su, si);
    // The cut key's group (all tokens tied at it) is kept whole.
    const uint32_t kord = (pre24 << 8) | (uint32_t)b3;
    out.kord = kord;
    out.idcut = INT_MAX;
    out.Zk = (double)(above + hmass[b3]) * exp2(-(double)sh);
    __syncthreads();
  }

  if (threadIdx.x == 0) {
    if (j < K) {
      const int x = a.ids[(int64_t)r * a.K_max + j];
      if (x >= 0 && x < V) {
        float z = load1<DT>(row, x);
        if (pen && ((bm[x >> 5] >> (x & 31)) & 1u)) z = penalize(z, a.rep);
        out.kx = z;
      }
    }
    rs[row_index(a, r, is_t, j)] = out;
  }
}

// ---------------------------------------------------------------------------
// k_pair_tv: d_j = TV(p_j, q_j) over the processed, truncated rows.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(NT_ROW) void k_pair_tv(Args a, const RowStat* rs, double* dout,
                                                   int bm_words) {
  constexpr int NT = NT_ROW;
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* bm = reinterpret_cast<uint32_t*>(smem);
  __shared__ double sd[NT / WAVE];
  if (a.K_max == 0) return;
  const int r = blockIdx.x / a.K_max, j = blockIdx.x % a.K_max;
  const int K = request_k(a, r);
  if (K < 0 || K > a.K_max || j >= K) return;
  const float T = request_t(a, r);
  if (!(T > 0.0f) || !(T < INFINITY)) return;
  const RowStat P = rs[row_index(a, r, true, j)], Q = rs[row_index(a, r, false, j)];
  if ((P.flags | Q.flags) & NONFINITE) {
    if (threadIdx.x == 0) dout[(int64_t)r * a.K_max + j] = 0.0;
    return;
  }
  const char* trow = target_row(a, r, j);
  const char* drow = draft_row(a, r, j);
  const int V = a.V, nvec = (V + VEC - 1) / VEC;
  const bool pen = build_penalty_bitmap<NT>(a, r, j, 0, V, bm);
  const float ip = (float)(1.0 / P.Zk), iq = (float)(1.0 / Q.Zk);
  double acc = 0.0;
  for (int k = threadIdx.x; k < nvec; k += NT) {
    float zp[VEC], zq[VEC];
    load8<DT>(trow, k, V, zp);
    load8<DT>(drow, k, V, zq);
    if (pen) {
      apply_penalty8(bm, k, 0, a.rep, zp);
      apply_penalty8(bm, k, 0, a.rep, zq);
    }
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int id = k * VEC + e;
      const float p = (id < V && kept(P, ord_key(zp[e]), id)) ? e_rel(zp[e], P.M, P.c) * ip : 0.0f;
      const float q = (id < V && kept(Q, ord_key(zq[e]), id)) ? e_rel(zq[e], Q.M, Q.c) * iq : 0.0f;
      s += fabsf(p - q);
    }
    acc += (double)s;
  }
  const double tot = block_sum<NT>(acc, sd);
  if (threadIdx.x == 0) dout[(int64_t)r * a.K_max + j] = fmin(0.5 * tot, 1.0);
}

// Processed probability of token x from its row statistics, in fp64.
__device__ __forceinline__ double prob_at(const RowStat& s, float kx, int x, double T) {
  if (!kept(s, ord_key(kx), x)) return 0.0;
  return exp(((double)kx - (double)s.M) / T) / s.Zk;
}

// ---------------------------------------------------------------------------
// k_finalize: decisions and the correction / bonus draw of one request.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(NT_ROW) void k_finalize(Args a, const RowStat* rs, const double* dtv,
                                                    int tv_valid, int bm_words,
                                                    int32_t* out_acc, int32_t* out_tok,
                                                    uint32_t* out_status, float* out_stats) {
  constexpr int NT = NT_ROW;
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* bm = reinterpret_cast<uint32_t*>(smem);
  double* ctot = reinterpret_cast<double*>(smem + ((bm_words * 4 + 15) & ~15));
  __shared__ double scan_buf[NT];
  __shared__ int si[NT / WAVE + 4];
  __shared__ int sh_n;
  __shared__ int sh_mode;     // 0: residual, 1: bonus / fallback from p_n, 2: none
  __shared__ double sh_S, sh_t, sh_R;
  __shared__ int sh_ch;
  __shared__ int sh_y;
  __shared__ uint32_t sh_st;
  __shared__ float sh_stat[(SD_MAX_K + 1) * SD_NSTAT];

  const int r = blockIdx.x;
  const int V = a.V, K1 = a.K_max + 1;
  const int K = request_k(a, r);
  const float T = request_t(a, r);

  // ---- status ----
  uint32_t st = 0;
  if (K < 0 || K > a.K_max) st |= SD_ST_BAD_K;
  if (!(T > 0.0f) || !(T < INFINITY)) st |= SD_ST_BAD_TEMP;
  int badid = 0, badprior = 0, nonfin = 0;
  if (!(st & SD_ST_BAD_K))
    for (int t = threadIdx.x; t < K; t += NT) {
      const int x = a.ids[(int64_t)r * a.K_max + t];
      badid |= (x < 0 || x >= V);
    }
  if (a.prior && a.poff) {
    const int p0 = a.poff[r], p1 = a.poff[r + 1];
    for (int t = p0 + threadIdx.x; t < p1; t += NT) {
      const int id = a.prior[t];
      badprior |= (id < 0 || id >= V);
    }
  }
  if (!(st & (SD_ST_BAD_K | SD_ST_BAD_TEMP)))
    for (int t = threadIdx.x; t < 2 * K + 1; t += NT) {
      const bool tg = t <= K;
      const int jj = tg ? t : t - K - 1;
      nonfin |= (rs[row_index(a, r, tg, jj)].flags & NONFINITE) ? 1 : 0;
    }
  if (block_or<NT>(badid, si)) st |= SD_ST_BAD_DRAFT_ID;
  if (block_or<NT>(badprior, si)) st |= SD_ST_BAD_PRIOR;
  if (block_or<NT>(nonfin, si)) st |= SD_ST_NONFINITE;

  if (st & SD_ST_INVALID_MASK) {
    for (int t = threadIdx.x; t < K1; t += NT) out_tok[(int64_t)r * K1 + t] = -1;
    if (out_stats)
      for (int t = threadIdx.x; t < K1 * SD_NSTAT; t += NT) out_stats[(int64_t)r * K1 * SD_NSTAT + t] = 0.0f;
    if (threadIdx.x == 0) {
      out_acc[r] = -1;
      if (out_status) out_status[r] = st;
    }
    return;
  }

  // ---- decisions (one thread; K <= SD_MAX_K positions) ----
  if (threadIdx.x == 0) {
    const double Td = (double)T;
    const double D = (double)a.D;
    int n = K;
    for (int jj = 0; jj <= K; ++jj) {
      float u, v;
      uniforms(a.seed, a.offset, r, jj, u, v);
      float* sv = &sh_stat[jj * SD_NSTAT];
      for (int s = 0; s < SD_NSTAT; ++s) sv[s] = 0.0f;
      sv[SD_STAT_U] = u;
      sv[SD_STAT_V] = v;
      if (jj == K) break;
      const int x = a.ids[(int64_t)r * a.K_max + jj];
      const RowStat P = rs[row_index(a, r, true, jj)], Q = rs[row_index(a, r, false, jj)];
      const double px = prob_at(P, P.kx, x, Td), qx = prob_at(Q, Q.kx, x, Td);
      double th;
      double d = 0.0;
      if (tv_valid) {
        d = dtv[(int64_t)r * a.K_max + jj];
        th = (d <= D) ? 1.0 : D / d;
      } else {
        th = (D >= 1.0) ? 1.0 : 0.0;   // D = 0: theta only matters when p = q
      }
      const double pix = (1.0 - th) * px + th * qx;
      if (qx == 0.0) st |= SD_ST_Q_ZERO;
      sv[SD_STAT_D] = (float)d;
      sv[SD_STAT_THETA] = (float)th;
      sv[SD_STAT_PX] = (float)px;
      sv[SD_STAT_QX] = (float)qx;
      sv[SD_STAT_PIX] = (float)pix;
      if (n == K && !((double)u * qx < pix)) n = jj;
    }
    sh_n = n;
    sh_mode = (n < K) ? 0 : ((a.flags & SD_NO_BONUS) ? 2 : 1);
    sh_st = st;
  }
  __syncthreads();
  const int n = sh_n;
  int mode = sh_mode;

  // ---- draw: inverse CDF over ascending ids, fp64 block prefix sums ----
  if (mode != 2) {
    const bool pen = build_penalty_bitmap<NT>(a, r, n, 0, V, bm);
    const RowStat P = rs[row_index(a, r, true, n)];
    RowStat Q = P;
    if (n < K) Q = rs[row_index(a, r, false, n)];
    const char* trow = target_row(a, r, n);
    const char* drow = (n < K) ? draft_row(a, r, n) : trow;
    const float ip = (float)(1.0 / P.Zk), iq = (float)(1.0 / Q.Zk);
    const int nvec = (V + VEC - 1) / VEC;
    const int nch = (nvec + NT - 1) / NT;
    const float vn = sh_stat[n * SD_NSTAT + SD_STAT_V];

    auto own_sum = [&](int k, int md, float (&w)[VEC]) -> double {
      double s = 0.0;
      if (k < nvec) {
        float zp[VEC], zq[VEC];
        load8<DT>(trow, k, V, zp);
        if (pen) apply_penalty8(bm, k, 0, a.rep, zp);
        if (md == 0) {
          load8<DT>(drow, k, V, zq);
          if (pen) apply_penalty8(bm, k, 0, a.rep, zq);
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const int id = k * VEC + e;
          float p = (id < V && kept(P, ord_key(zp[e]), id)) ? e_rel(zp[e], P.M, P.c) * ip : 0.0f;
          if (md == 0) {
            const float q = (id < V && kept(Q, ord_key(zq[e]), id)) ? e_rel(zq[e], Q.M, Q.c) * iq : 0.0f;
            p = fmaxf(p - q, 0.0f);
          }
          w[e] = p;
          s += (double)p;
        }
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) w[e] = 0.0f;
      }
      return s;
    };

    for (int pass = 0; pass < 2; ++pass) {
      for (int ch = 0; ch < nch; ++ch) {
        float w[VEC];
        const double own = own_sum(ch * NT + threadIdx.x, mode, w);
        const double incl = block_incl_scan<NT>(own, scan_buf);
        if (threadIdx.x == NT - 1) ctot[ch] = incl;
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        double S = 0.0;
        for (int ch = 0; ch < nch; ++ch) S += ctot[ch];
        sh_S = S;
        const double t = (double)vn * S;
        double R = 0.0;
        int chs = -1, lastpos = -1;
        double Rlast = 0.0, Racc = 0.0;
        for (int ch = 0; ch < nch; ++ch) {
          if (ctot[ch] > 0.0) { lastpos = ch; Rlast = Racc; }
          if (chs < 0 && Racc + ctot[ch] > t) { chs = ch; R = Racc; }
          Racc += ctot[ch];
        }
        if (chs < 0) { chs = lastpos; R = Rlast; }
        sh_t = t;
        sh_R = R;
        sh_ch = chs;
      }
      __syncthreads();
      if (!(sh_S > 0.0) && mode == 0) {   // zero residual: draw from p_n
        mode = 1;
        if (threadIdx.x == 0) sh_st |= SD_ST_RESID_ZERO;
        __syncthreads();
        continue;
      }
      break;
    }

    if (threadIdx.x == 0) sh_y = -1;
    if (sh_ch >= 0) {
      float w[VEC];
      const int k = sh_ch * NT + threadIdx.x;
      const double own = own_sum(k, mode, w);
      const double incl = block_incl_scan<NT>(own, scan_buf);
      const double prev = threadIdx.x ? scan_buf[threadIdx.x - 1] : 0.0;
      const double R = sh_R, t = sh_t;
      __syncthreads();
      if (threadIdx.x == 0) si[0] = INT_MAX;
      __syncthreads();
      if (R + incl > t) atomicMin(&si[0], (int)threadIdx.x);
      __syncthreads();
      if ((int)threadIdx.x == si[0]) {
        double C = R + prev;
        int y = -1, lastpos = -1;
        for (int e = 0; e < VEC; ++e) {
          if (w[e] > 0.0f) lastpos = k * VEC + e;
          C += (double)w[e];
          if (C > t) { y = k * VEC + e; break; }
        }
        sh_y = (y >= 0) ? y : lastpos;
      }
      __syncthreads();
    }
    if (threadIdx.x == 0) sh_stat[n * SD_NSTAT + SD_STAT_S] = (float)sh_S;
  }
  __syncthreads();

  // ---- outputs ----
  for (int t = threadIdx.x; t < K1; t += NT) {
    int v = -1;
    if (t < n) v = a.ids[(int64_t)r * a.K_max + t];
    else if (t == n && mode != 2) v = sh_y;
    out_tok[(int64_t)r * K1 + t] = v;
  }
  if (out_stats)
    for (int t = threadIdx.x; t < K1 * SD_NSTAT; t += NT)
      out_stats[(int64_t)r * K1 * SD_NSTAT + t] = (t < (K + 1) * SD_NSTAT) ? sh_stat[t] : 0.0f;
  if (threadIdx.x == 0) {
    out_acc[r] = n;
    if (out_status) out_status[r] = sh_st;
  }
}

// ---------------------------------------------------------------------------
// Debug export of processed rows.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(NT_ROW) void k_debug_rows(Args a, const RowStat* rs, int bm_words,
                                                      float* out_p, float* out_q) {
  constexpr int NT = NT_ROW;
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* bm = reinterpret_cast<uint32_t*>(smem);
  const int nrows = 2 * a.K_max + 1;
  const int r = blockIdx.x / nrows, rho = blockIdx.x % nrows;
  const int K = request_k(a, r);
  if (K < 0 || K > a.K_max) return;
  const bool is_t = rho <= a.K_max;
  const int j = is_t ? rho : rho - a.K_max - 1;
  if (is_t ? (j > K) : (j >= K)) return;
  const float T = request_t(a, r);
  if (!(T > 0.0f) || !(T < INFINITY)) return;
  const RowStat S = rs[row_index(a, r, is_t, j)];
  if (S.flags & NONFINITE) return;
  const char* row = is_t ? target_row(a, r, j) : draft_row(a, r, j);
  float* out = is_t ? out_p + ((int64_t)r * (a.K_max + 1) + j) * a.V
                    : out_q + ((int64_t)r * a.K_max + j) * a.V;
  const int V = a.V, nvec = (V + VEC - 1) / VEC;
  const bool pen = build_penalty_bitmap<NT>(a, r, j, 0, V, bm);
  const float ip = (float)(1.0 / S.Zk);
  for (int k = threadIdx.x; k < nvec; k += NT) {
    float z[VEC];
    load8<DT>(row, k, V, z);
    if (pen) apply_penalty8(bm, k, 0, a.rep, z);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int id = k * VEC + e;
      if (id < V) out[id] = kept(S, ord_key(z[e]), id) ? e_rel(z[e], S.M, S.c) * ip : 0.0f;
    }
  }
}

__global__ void k_debug_uniforms(uint64_t seed, uint64_t off, int B, int npos, float* ou, float* ov) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)B * npos) return;
  float u, v;
  uniforms(seed, off, (int)(i / npos), (int)(i % npos), u, v);
  ou[i] = u;
  ov[i] = v;
}

// ---------------------------------------------------------------------------
// Greedy verify.
// ---------------------------------------------------------------------------
struct GPart {
  uint32_t ord;
  int32_t id;
  uint32_t nan;
  uint32_t pad;
};

__device__ __forceinline__ bool better(uint32_t o1, int i1, uint32_t o2, int i2) {
  return o1 > o2 || (o1 == o2 && i1 < i2);
}

template <int DT>
__global__ __launch_bounds__(NT_G) void k_greedy_partial(Args a, GPart* parts, int ns) {
  constexpr int NT = NT_G;
  __shared__ uint32_t bm[G_SLICE / 32];
  __shared__ uint32_t so[NT / WAVE];
  __shared__ int sidx[NT / WAVE];
  __shared__ int snan[NT / WAVE];
  const int s = blockIdx.x % ns;
  const int rj = blockIdx.x / ns;
  const int j = rj % (a.K_max + 1), r = rj / (a.K_max + 1);
  const int K = request_k(a, r);
  if (K < 0 || K > a.K_max || j > K) return;
  const int V = a.V, lo = s * G_SLICE, hi = min(V, lo + G_SLICE);
  const char* row = target_row(a, r, j);
  const bool pen = build_penalty_bitmap<NT>(a, r, j, lo, G_SLICE, bm);
  uint32_t bo = 0;
  int bi = INT_MAX, nan = 0;
  const int k0 = lo / VEC, k1 = (hi + VEC - 1) / VEC;
  for (int k = k0 + threadIdx.x; k < k1; k += NT) {
    float z[VEC];
    load8<DT>(row, k, V, z);
    if (pen) apply_penalty8(bm, k, lo, a.rep, z);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int id = k * VEC + e;
      if (id >= V) continue;
      if (z[e] != z[e]) { nan = 1; continue; }
      const uint32_t o = ord_key(z[e]);
      if (better(o, id, bo, bi)) { bo = o; bi = id; }
    }
  }
#pragma unroll
  for (int off = WAVE / 2; off > 0; off >>= 1) {
    const uint32_t o2 = __shfl_xor(bo, off);
    const int i2 = __shfl_xor(bi, off);
    if (better(o2, i2, bo, bi)) { bo = o2; bi = i2; }
    nan |= __shfl_xor(nan, off);
  }
  const int w = threadIdx.x / WAVE;
  if (threadIdx.x % WAVE == 0) { so[w] = bo; sidx[w] = bi; snan[w] = nan; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int q = 1; q < NT / WAVE; ++q) {
      if (better(so[q], sidx[q], bo, bi)) { bo = so[q]; bi = sidx[q]; }
      nan |= snan[q];
    }
    GPart g;
    g.ord = bo; g.id = bi; g.nan = (uint32_t)nan; g.pad = 0;
    parts[blockIdx.x] = g;
  }
}

__global__ __launch_bounds__(64) void k_greedy_final(Args a, const GPart* parts, int ns,
                                                     int32_t* out_acc, int32_t* out_tok,
                                                     uint32_t* out_status, int32_t* out_argmax) {
  __shared__ int g[SD_MAX_K + 1];
  __shared__ int anynan;
  const int r = blockIdx.x;
  const int K1 = a.K_max + 1, V = a.V;
  const int K = request_k(a, r);
  uint32_t st = 0;
  if (K < 0 || K > a.K_max) st |= SD_ST_BAD_K;
  int badid = 0, badprior = 0;
  if (!st)
    for (int t = threadIdx.x; t < K; t += 64) {
      const int x = a.ids[(int64_t)r * a.K_max + t];
      badid |= (x < 0 || x >= V);
    }
  if (a.prior && a.poff) {
    const int p0 = a.poff[r], p1 = a.poff[r + 1];
    for (int t = p0 + threadIdx.x; t < p1; t += 64) {
      const int id = a.prior[t];
      badprior |= (id < 0 || id >= V);
    }
  }
  if (threadIdx.x == 0) anynan = 0;
  __syncthreads();
  if (!st && (int)threadIdx.x <= K) {
    const int jj = threadIdx.x;
    uint32_t bo = 0;
    int bi = INT_MAX, nan = 0;
    for (int s = 0; s < ns; ++s) {
      const GPart p = parts[((int64_t)r * K1 + jj) * ns + s];
      nan |= (int)p.nan;
      if (better(p.ord, p.id, bo, bi)) { bo = p.ord; bi = p.id; }
    }
    g[jj] = bi;
    if (nan) atomicOr(&anynan, 1);
  }
  if (__any(badid)) st |= SD_ST_BAD_DRAFT_ID;
  if (__any(badprior)) st |= SD_ST_BAD_PRIOR;
  __syncthreads();
  if (anynan && !(st & SD_ST_BAD_K)) st |= SD_ST_NONFINITE;
  if (threadIdx.x != 0) return;
  int64_t base = (int64_t)r * K1;
  if (st & SD_ST_INVALID_MASK) {
    for (int t = 0; t < K1; ++t) {
      out_tok[base + t] = -1;
      if (out_argmax) out_argmax[base + t] = -1;
    }
    out_acc[r] = -1;
    if (out_status) out_status[r] = st;
    return;
  }
  int n = K;
  for (int jj = 0; jj < K; ++jj)
    if (a.ids[(int64_t)r * a.K_max + jj] != g[jj]) { n = jj; break; }
  for (int t = 0; t < K1; ++t) {
    int v = -1;
    if (t < n) v = a.ids[(int64_t)r * a.K_max + t];
    else if (t == n && !(n == K && (a.flags & SD_NO_BONUS))) v = g[n];
    out_tok[base + t] = v;
    if (out_argmax) out_argmax[base + t] = (t <= K) ? g[t] : -1;
  }
  out_acc[r] = n;
  if (out_status) out_status[r] = st;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Layout {
  size_t rs, dtv, gp, total;
  int ns;
};

Layout layout(const sd_verify_args_t* a) {
  Layout L;
  const size_t B = (size_t)a->B, K = (size_t)a->K_max;
  L.ns = (a->V + G_SLICE - 1) / G_SLICE;
  size_t off = 0;
  L.rs = off;  off = align_up(off + B * (2 * K + 1) * sizeof(RowStat), 256);
  L.dtv = off; off = align_up(off + B * K * sizeof(double), 256);
  L.gp = off;  off = align_up(off + B * (K + 1) * (size_t)L.ns * sizeof(GPart), 256);
  L.total = off;
  return L;
}

int ceil_log2(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

int check_common(const sd_verify_args_t* a, bool sample) {
  if (!a) return SD_EINVAL;
  if (a->dtype != SD_F32 && a->dtype != SD_BF16) return SD_EINVAL;
  if (a->B < 1 || a->K_max < 0 || a->V < 1) return SD_EINVAL;
  if (a->K_max > SD_MAX_K || a->V > MAX_V) return SD_EUNSUPPORTED;
  if ((int64_t)a->B * (2 * a->K_max + 1) > INT_MAX / 2) return SD_EUNSUPPORTED;
  const int es = a->dtype == SD_BF16 ? 2 : 4;
  if (!a->target_logits || a->ld_target < a->V || (a->ld_target * es) % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(a->target_logits) & 15u))
    return SD_EINVAL;
  if (a->K_max > 0 && !a->draft_ids) return SD_EINVAL;
  if (sample && a->K_max > 0 &&
      (!a->draft_logits || a->ld_draft < a->V || (a->ld_draft * es) % 16 != 0 ||
       (reinterpret_cast<uintptr_t>(a->draft_logits) & 15u)))
    return SD_EINVAL;
  if (!(a->rep_penalty > 0.0f) || !(a->rep_penalty < INFINITY)) return SD_EINVAL;
  if (sample) {
    if (!(a->top_p > 0.0f) || !(a->top_p <= 1.0f)) return SD_EINVAL;
    if (!(a->tv_budget >= 0.0f)) return SD_EINVAL;
  }
  if ((a->prior_ids == nullptr) != (a->prior_offsets == nullptr)) return SD_EINVAL;
  if (a->flags & ~(SD_NO_BONUS | SD_PENALTY_PRIOR_ONLY)) return SD_EINVAL;
  return SD_OK;
}

Args make_args(const sd_verify_args_t* s) {
  Args a;
  a.tgt = s->target_logits;
  a.drf = s->draft_logits;
  a.ldt = s->ld_target;
  a.ldd = s->ld_draft;
  a.dtype = s->dtype;
  a.B = s->B;
  a.K_max = s->K_max;
  a.V = s->V;
  a.ids = s->draft_ids;
  a.kpr = s->k_per_row;
  a.temp = s->temperature;
  a.top_p = s->top_p;
  a.rep = s->rep_penalty;
  a.D = s->tv_budget;
  a.prior = s->prior_ids;
  a.poff = s->prior_offsets;
  a.seed = s->seed;
  a.offset = s->offset;
  a.flags = s->flags;
  a.fp_shift = 62 - ceil_log2(s->V);
  return a;
}

int bitmap_words(int V) { return (V + 31) / 32; }

size_t row_lds(int V) { return align_up((size_t)bitmap_words(V) * 4, 16) + HBINS * 12; }

size_t fin_lds(int V) {
  const int nch = ((V + VEC - 1) / VEC + NT_ROW - 1) / NT_ROW;
  return align_up((size_t)bitmap_words(V) * 4, 16) + (size_t)nch * 8;
}

int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SD_OK : SD_EHIP;
}

template <int DT>
int run_prepare(const Args& a, const Layout& L, char* ws, hipStream_t st) {
  const int grid = a.B * (2 * a.K_max + 1);
  hipLaunchKernelGGL(k_row_prepare<DT>, dim3(grid), dim3(NT_ROW), row_lds(a.V), st, a,
                     reinterpret_cast<RowStat*>(ws + L.rs), bitmap_words(a.V));
  return launch_status();
}

bool needs_tv(const Args& a, const float* stats) {
  return stats != nullptr || (a.D > 0.0f && a.D < 1.0f);
}

// One phase of the sampling path (0: rows, 1: TV, 2: finalize).
template <int DT>
int run_phase(const Args& a, const Layout& L, char* ws, int phase, int32_t* acc, int32_t* tok,
              uint32_t* status, float* stats, hipStream_t st) {
  const bool need_tv = needs_tv(a, stats);
  if (phase == 0) return run_prepare<DT>(a, L, ws, st);
  if (phase == 1) {
    if (!need_tv || a.K_max == 0) return SD_OK;
    hipLaunchKernelGGL(k_pair_tv<DT>, dim3(a.B * a.K_max), dim3(NT_ROW),
                       align_up((size_t)bitmap_words(a.V) * 4, 16), st, a,
                       reinterpret_cast<const RowStat*>(ws + L.rs),
                       reinterpret_cast<double*>(ws + L.dtv), bitmap_words(a.V));
    return launch_status();
  }
  hipLaunchKernelGGL(k_finalize<DT>, dim3(a.B), dim3(NT_ROW), fin_lds(a.V), st, a,
                     reinterpret_cast<const RowStat*>(ws + L.rs),
                     reinterpret_cast<const double*>(ws + L.dtv), need_tv ? 1 : 0,
                     bitmap_words(a.V), acc, tok, status, stats);
  return launch_status();
}

template <int DT>
int run_sample(const Args& a, const Layout& L, char* ws, int32_t* acc, int32_t* tok,
               uint32_t* status, float* stats, hipStream_t st) {
  for (int ph = 0; ph < 3; ++ph) {
    const int rc = run_phase<DT>(a, L, ws, ph, acc, tok, status, stats, st);
    if (rc) return rc;
  }
  return SD_OK;
}

template <int DT>
int run_greedy(const Args& a, const Layout& L, char* ws, int32_t* acc, int32_t* tok,
               uint32_t* status, int32_t* amax, hipStream_t st) {
  const int64_t grid = (int64_t)a.B * (a.K_max + 1) * L.ns;
  if (grid > INT_MAX) return SD_EUNSUPPORTED;
  GPart* parts = reinterpret_cast<GPart*>(ws + L.gp);
  hipLaunchKernelGGL(k_greedy_partial<DT>, dim3((unsigned)grid), dim3(NT_G), 0, st, a, parts, L.ns);
  int rc = launch_status();
  if (rc) return rc;
  hipLaunchKernelGGL(k_greedy_final, dim3(a.B), dim3(64), 0, st, a, parts, L.ns, acc, tok, status, amax);
  return launch_status();
}

}  // namespace

extern "C" {

int sd_verify_workspace_bytes(const sd_verify_args_t* args, size_t* bytes) {
  if (!args || !bytes) return SD_EINVAL;
  if (args->B < 1 || args->K_max < 0 || args->V < 1) return SD_EINVAL;
  if (args->K_max > SD_MAX_K || args->V > MAX_V) return SD_EUNSUPPORTED;
  *bytes = layout(args).total;
  return SD_OK;
}

int sd_verify_sample(const sd_verify_args_t* args, void* workspace, size_t workspace_bytes,
                     int32_t* out_accepted, int32_t* out_tokens, uint32_t* out_status,
                     float* out_stats, void* stream) {
  int rc = check_common(args, true);
  if (rc) return rc;
  if (!out_accepted || !out_tokens) return SD_EINVAL;
  const Layout L = layout(args);
  if (!workspace || workspace_bytes < L.total) return SD_EWORKSPACE;
  const Args a = make_args(args);
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return a.dtype == SD_BF16 ? run_sample<SD_BF16>(a, L, ws, out_accepted, out_tokens, out_status, out_stats, st)
                            : run_sample<SD_F32>(a, L, ws, out_accepted, out_tokens, out_status, out_stats, st);
}

int sd_verify_greedy(const sd_verify_args_t* args, void* workspace, size_t workspace_bytes,
                     int32_t* out_accepted, int32_t* out_tokens, uint32_t* out_status,
                     int32_t* out_argmax, void* stream) {
  int rc = check_common(args, false);
  if (rc) return rc;
  if (!out_accepted || !out_tokens) return SD_EINVAL;
  const Layout L = layout(args);
  if (!workspace || workspace_bytes < L.total) return SD_EWORKSPACE;
  const Args a = make_args(args);
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return a.dtype == SD_BF16 ? run_greedy<SD_BF16>(a, L, ws, out_accepted, out_tokens, out_status, out_argmax, st)
                            : run_greedy<SD_F32>(a, L, ws, out_accepted, out_tokens, out_status, out_argmax, st);
}

const char* sd_strerror(int code) {
  switch (code) {
    case SD_OK: return "ok";
    case SD_EINVAL: return "invalid argument";
    case SD_EWORKSPACE: return "workspace missing or too small";
    case SD_EHIP: return "HIP runtime error";
    case SD_EUNSUPPORTED: return "unsupported size (K_max or V beyond this build's limits)";
    default: return "unknown error code";
  }
}

int sd_debug_process_rows(const sd_verify_args_t* args, void* workspace, size_t workspace_bytes,
                          float* out_p, float* out_q, void* stream) {
  int rc = check_common(args, true);
  if (rc) return rc;
  if (!out_p || (args->K_max > 0 && !out_q)) return SD_EINVAL;
  const Layout L = layout(args);
  if (!workspace || workspace_bytes < L.total) return SD_EWORKSPACE;
  const Args a = make_args(args);
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = a.dtype == SD_BF16 ? run_prepare<SD_BF16>(a, L, ws, st) : run_prepare<SD_F32>(a, L, ws, st);
  if (rc) return rc;
  const int grid = a.B * (2 * a.K_max + 1);
  const size_t lds = align_up((size_t)bitmap_words(a.V) * 4, 16);
  if (a.dtype == SD_BF16)
    hipLaunchKernelGGL(k_debug_rows<SD_BF16>, dim3(grid), dim3(NT_ROW), lds, st, a,
                       reinterpret_cast<const RowStat*>(ws + L.rs), bitmap_words(a.V), out_p, out_q);
  else
    hipLaunchKernelGGL(k_debug_rows<SD_F32>, dim3(grid), dim3(NT_ROW), lds, st, a,
                       reinterpret_cast<const RowStat*>(ws + L.rs), bitmap_words(a.V), out_p, out_q);
  return launch_status();
}

int sd_debug_run_phase(const sd_verify_args_t* args, void* workspace, size_t workspace_bytes,
                       int phase, int32_t* out_accepted, int32_t* out_tokens, uint32_t* out_status,
                       float* out_stats, void* stream) {
  int rc = check_common(args, true);
  if (rc) return rc;
  if (phase < 0 || phase > 2) return SD_EINVAL;
  if (phase == 2 && (!out_accepted || !out_tokens)) return SD_EINVAL;
  const Layout L = layout(args);
  if (!workspace || workspace_bytes < L.total) return SD_EWORKSPACE;
  const Args a = make_args(args);
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return a.dtype == SD_BF16
             ? run_phase<SD_BF16>(a, L, ws, phase, out_accepted, out_tokens, out_status, out_stats, st)
             : run_phase<SD_F32>(a, L, ws, phase, out_accepted, out_tokens, out_status, out_stats, st);
}

int sd_debug_uniforms(uint64_t seed, uint64_t offset, int32_t B, int32_t npos, float* out_u,
                      float* out_v, void* stream) {
  if (B < 1 || npos < 1 || !out_u || !out_v) return SD_EINVAL;
  const int64_t n = (int64_t)B * npos;
  if (n > (int64_t)INT_MAX) return SD_EUNSUPPORTED;
  hipLaunchKernelGGL(k_debug_uniforms, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), seed, offset, B, npos, out_u, out_v);
  return launch_status();
}

}  // extern "C"
