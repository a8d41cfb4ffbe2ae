// Speculative-sampling verify step on gfx950: kernels and the C ABI.
//
// Single-pass sampling path (bf16 logits, top-p on, V <= 155648), two
// launches on the caller's stream:
//   k_pair_fast      one 1024-thread workgroup per position pair (target j,
//                    draft j) and one per bonus row.  The target row is held
//                    in registers (19 x 16 bytes per thread); its max,
//                    normalizer and exact top-p cut come from a histogram of
//                    bf16 keys.  The draft row streams past it once, building
//                    its own histogram and saving the draft key of every
//                    target-nucleus token in LDS.  TV, p(x), q(x), theta,
//                    pi and the acceptance of position j follow; a rejected
//                    position draws its correction from the register-held
//                    data.  Every logit is read from HBM once.  Pairs the
//                    on-chip path cannot cover (a cut outside the histogram
//                    window, a huge nucleus, penalized tokens at the cut)
//                    take the exact multi-pass routines inside the same
//                    workgroup.
//   k_fast_finalize  one wave per request: first rejection, emitted tokens,
//                    status and statistics.
// General path (fp32, top-p off, larger V), three launches:
//   k_row_prepare / k_pair_tv / k_finalize built on the same exact routines.
// Greedy path, two launches: k_greedy_partial (argmax of slices of the
// target rows) and k_greedy_final (reduce, first mismatch, outputs).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <limits.h>
#include <math.h>
#include <string.h>
#include <stddef.h>
#include <mutex>
#include <utility>
#include <vector>

#include "sd_verify.h"
#include "sdv_device.h"
#include "sdv_exact.h"

using namespace sdv;

namespace {

constexpr int NT_ROW = 512;                  // general-path row kernels
constexpr int NT_G = 256;                    // greedy partial kernel
constexpr int G_SLICE = 8192;                // logits per greedy workgroup
static_assert(G_SLICE % (8 * NT_G) == 0, "greedy slice geometry");
constexpr int MAX_V = 1 << 19;

__device__ __forceinline__ int row_index(const Args& a, int r, bool target, int j) {
  return r * (2 * a.K_max + 1) + (target ? j : a.K_max + 1 + j);
}

__host__ __device__ constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// General path kernels.
// ---------------------------------------------------------------------------

// LDS of the exact routines after the bitmap: histograms then chunk totals.
__device__ ExactLds carve_exact(unsigned char* p, double* sd, float* sf, int* si, uint64_t* su) {
  ExactLds L;
  L.hmass = reinterpret_cast<uint64_t*>(p);
  L.hcnt = reinterpret_cast<uint32_t*>(p + HBINS * 8);
  L.ctot = reinterpret_cast<double*>(p + HBINS * 12);
  L.su = su;
  L.sd = sd;
  L.sf = sf;
  L.si = si;
  return L;
}

size_t exact_lds(int V, int NT) {
  const int nch = ((V + VEC - 1) / VEC + NT - 1) / NT;
  return (size_t)HBINS * 12 + (size_t)nch * 8;
}

template <int DT>
__global__ __launch_bounds__(NT_ROW) void k_row_prepare(Args a, RowStat* rs, int bm_words) {
  constexpr int NT = NT_ROW;
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* bm = reinterpret_cast<uint32_t*>(smem);
  __shared__ double sd[NT];
  __shared__ float sf[NT / WAVE];
  __shared__ int si[NT / WAVE + 4];
  __shared__ uint64_t su[NT];
  const ExactLds L = carve_exact(smem + align_up(bm_words * 4, 16), sd, sf, si, su);

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
  const bool pen = build_penalty_bitmap<NT>(a, r, j, 0, a.V, bm);
  RowStat out = row_stats_dev<DT, NT>(a, row, is_t ? a.V : a.Vd, c, pen, bm, L, request_top_p(a, r));
  if (threadIdx.x == 0) {
    if (j < K) {
      const int x = a.ids[(int64_t)r * a.K_max + j];
      if (x >= 0 && x < a.V) {
        float z = (is_t || x < a.Vd) ? load1<DT>(row, x) : -INFINITY;
        if (pen && ((bm[x >> 5] >> (x & 31)) & 1u)) z = penalize(z, a.rep);
        out.kx = z;
      }
    }
    rs[row_index(a, r, is_t, j)] = out;
  }
}

// Slices of the general path's TV and draw passes at small batch sizes:
// each (pair) or (request) task is split over workgroups by vector ranges
// so that a call fills the device's 256 compute units with one workgroup
// each; from 128 tasks on a task keeps one workgroup.  Slices hold
// TV_SLICE_MIN vectors, or DRAW_SLICE_CH draw chunks, at least.
constexpr int SLICE_TASKS = 256;
constexpr int TV_SLICE_MIN = 512;
constexpr int DRAW_SLICE_CH = 2;

__host__ __device__ inline int slices_for(int tasks, int smax) {
  if (tasks <= 0 || 2 * tasks > SLICE_TASKS) return 1;
  return max(1, min(smax, SLICE_TASKS / tasks));
}

__host__ __device__ inline int tv_slices(int B, int K, int V) {
  return slices_for(B * K, max(1, (V + VEC - 1) / VEC / TV_SLICE_MIN));
}

__host__ __device__ inline int draw_chunks(int V) { return ((V + VEC - 1) / VEC + CHV - 1) / CHV; }

__host__ __device__ inline int draw_slices(int B, int V) {
  return slices_for(B, max(1, draw_chunks(V) / DRAW_SLICE_CH));
}

// |p - q| sums of the pairs' rows: workgroup b takes slice b % S of pair
// b / S (vectors [s len, s len + len) with len = ceil(nvec / S)) and writes
// its sum to dpart[b]; d = min(sum over the pair's slices / 2, 1).
// Rows without top-p at small batch sizes: each row's max and normalizer
// pass is split over workgroups by vector ranges (ROW_SLICE_MIN vectors at
// least), and k_row_combine merges the slices.  (Rows with top-p keep one
// workgroup: their cut's histogram passes need the whole row.)
constexpr int ROW_SLICE_MIN = 512;

__host__ __device__ inline int row_slices(int B, int K, int V, bool topp) {
  if (topp) return 1;
  return slices_for(B * (2 * K + 1), min(WAVE, max(1, (V + VEC - 1) / VEC / ROW_SLICE_MIN)));
}

struct RowPart {
  float M;       // the slice's max (-inf: none)
  int bad;       // a NaN met while the slice's logits so far were -inf
  double Z;      // sum exp2((key - M) c) over the slice
};
static_assert(sizeof(RowPart) == 16, "RowPart layout");

// The row's decode: row u = r (2 K_max + 1) + rho of the prepared rows, and
// whether k_row_prepare would skip it (request or position not valid).
__device__ __forceinline__ bool row_task(const Args& a, int u, int& r, bool& is_t, int& j, int& K, float& c) {
  const int nrows = 2 * a.K_max + 1;
  r = u / nrows;
  const int rho = u % nrows;
  K = request_k(a, r);
  if (K < 0 || K > a.K_max) return false;
  is_t = rho <= a.K_max;
  j = is_t ? rho : rho - a.K_max - 1;
  if (is_t ? (j > K) : (j >= K)) return false;
  const float T = request_t(a, r);
  if (!(T > 0.0f) || !(T < INFINITY)) return false;
  c = 1.4426950408889634f / T;
  return true;
}

// Slice b % S of prepared row b / S: vectors [s len, s len + len) with
// len = ceil(nvec / S) of the row's own length.
template <int DT>
__global__ __launch_bounds__(NT_ROW) void k_row_part(Args a, RowPart* parts, int S) {
  constexpr int NT = NT_ROW;
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* bm = reinterpret_cast<uint32_t*>(smem);
  __shared__ double sd[NT];
  __shared__ float sf[NT / WAVE];
  __shared__ int si[NT / WAVE + 4];
  const int u = blockIdx.x / S, sl = blockIdx.x % S;
  int r, j, K;
  bool is_t;
  float c;
  if (!row_task(a, u, r, is_t, j, K, c)) return;
  const int Vr = is_t ? a.V : a.Vd;
  const int nvec = (Vr + VEC - 1) / VEC, len = (nvec + S - 1) / S;
  const int k0 = min(nvec, sl * len), k1 = min(nvec, k0 + len);
  const bool pen = build_penalty_bitmap<NT>(a, r, j, k0 * VEC, (k1 - k0) * VEC, bm);
  ExactLds L{};
  L.sd = sd;
  L.sf = sf;
  L.si = si;
  RowPart o;
  row_max_z<DT, NT>(a, is_t ? target_row(a, r, j) : draft_row(a, r, j), Vr, c, pen, bm, k0 * VEC, L, k0, k1,
                    o.M, o.Z, o.bad);
  if (threadIdx.x == 0) parts[blockIdx.x] = o;
}

// One wave per prepared row: the slices merged into the row's statistics
// (no top-p: every token kept), with the draft token's key (penalized when
// it is in the position's penalty set: prior ids and, unless
// PENALTY_PRIOR_ONLY, the draft prefix).
template <int DT>
__global__ __launch_bounds__(WAVE) void k_row_combine(Args a, const RowPart* parts, RowStat* rs, int S) {
  const int u = blockIdx.x, lane = threadIdx.x;
  int r, j, K;
  bool is_t;
  float c;
  if (!row_task(a, u, r, is_t, j, K, c)) return;
  const RowPart* pp = parts + (int64_t)u * S;
  // (S <= WAVE slices: one per lane)
  const RowPart q = lane < S ? pp[lane] : RowPart{-INFINITY, 0, 0.0};
  const float M = wave_max(q.M);
  const int bad0 = __any(q.bad != 0) ? 1 : 0;
  const double Z = wave_sum(q.M > -INFINITY ? q.Z * exp2(((double)q.M - (double)M) * (double)c) : 0.0);
  int x = -1;
  if (j < K) x = a.ids[(int64_t)r * a.K_max + j];
  int hit = 0;
  if (x >= 0 && x < a.V && a.rep != 1.0f) {
    if (a.prior && a.poff)
      for (int t = a.poff[r] + lane; t < a.poff[r + 1]; t += WAVE) hit |= a.prior[t] == x;
    if (!(a.flags & SD_PENALTY_PRIOR_ONLY))
      for (int t = lane; t < j; t += WAVE) hit |= a.ids[(int64_t)r * a.K_max + t] == x;
  }
  const bool pen_x = __any(hit);
  if (lane == 0) {
    const int bad = bad0 || !(M > -INFINITY) || !(M < INFINITY) || Z != Z;
    RowStat out;
    out.M = M;
    out.c = c;
    out.Zk = Z;
    out.kord = KEEP_ALL;
    out.idcut = INT_MAX;
    out.flags = bad ? NONFINITE : 0;
    out.kx = 0.0f;
    if (x >= 0 && x < a.V) {
      float z = (is_t || x < a.Vd) ? load1<DT>(is_t ? target_row(a, r, j) : draft_row(a, r, j), x) : -INFINITY;
      if (pen_x) z = penalize(z, a.rep);
      out.kx = z;
    }
    rs[u] = out;
  }
}

template <int DT>
__global__ __launch_bounds__(NT_ROW) void k_pair_tv(Args a, const RowStat* rs, double* dpart, int S) {
  constexpr int NT = NT_ROW;
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* bm = reinterpret_cast<uint32_t*>(smem);
  __shared__ double sd[NT];
  __shared__ float sf[NT / WAVE];
  __shared__ int si[NT / WAVE + 4];
  if (a.K_max == 0) return;
  const int task = blockIdx.x / S, sl = blockIdx.x % S;
  const int r = task / a.K_max, j = task % a.K_max;
  const int K = request_k(a, r);
  if (K < 0 || K > a.K_max || j >= K) return;
  const float T = request_t(a, r);
  if (!(T > 0.0f) || !(T < INFINITY)) return;
  const RowStat P = rs[row_index(a, r, true, j)], Q = rs[row_index(a, r, false, j)];
  if ((P.flags | Q.flags) & NONFINITE) {
    if (threadIdx.x == 0) dpart[blockIdx.x] = 0.0;
    return;
  }
  const int nvec = (a.V + VEC - 1) / VEC, len = (nvec + S - 1) / S;
  const int k0 = min(nvec, sl * len), k1 = min(nvec, k0 + len);
  const bool pen = build_penalty_bitmap<NT>(a, r, j, k0 * VEC, (k1 - k0) * VEC, bm);
  ExactLds L{};
  L.sd = sd;
  L.sf = sf;
  L.si = si;
  // (rows without top-p compare no key with a cut)
  const double part =
      P.kord == KEEP_ALL && Q.kord == KEEP_ALL
          ? pair_tv_range<DT, NT, true>(a, target_row(a, r, j), draft_row(a, r, j), P, Q, pen, bm, k0 * VEC, L, k0,
                                        k1)
          : pair_tv_range<DT, NT>(a, target_row(a, r, j), draft_row(a, r, j), P, Q, pen, bm, k0 * VEC, L, k0, k1);
  if (threadIdx.x == 0) dpart[blockIdx.x] = part;
}

// Request-level checks shared by the finalize kernels.  Returns status bits.
// One invalidating defect is reported per request, the first found in this
// order: K_r out of range, a draft id out of range, a bad temperature; a bad
// per-request parameter is reported beside any of them, and a bad prior id
// (which is only ignored) always.  The logits of a request with an
// invalidating bit are never scanned, so SD_ST_NONFINITE appears only on a
// request that passed every other check.
template <int NT>
__device__ __forceinline__ uint32_t request_status(const Args& a, int r, int K, float T, bool check_temp,
                                   int* si) {
  const bool kbad = K < 0 || K > a.K_max;
  int badid = 0, badprior = 0;
  if (!kbad)
    for (int t = threadIdx.x; t < K; t += NT) {
      const int x = a.ids[(int64_t)r * a.K_max + t];
      badid |= (x < 0 || x >= a.V);
    }
  if (a.prior && a.poff) {
    const int p0 = a.poff[r], p1 = a.poff[r + 1];
    for (int t = p0 + threadIdx.x; t < p1; t += NT) {
      const int id = a.prior[t];
      badprior |= (id < 0 || id >= a.V);
    }
  }
  const bool idbad = block_or<NT>(badid, si) != 0;
  const bool priorbad = block_or<NT>(badprior, si) != 0;
  uint32_t st = kbad ? SD_ST_BAD_K : idbad ? SD_ST_BAD_DRAFT_ID : 0u;
  if (check_temp && st == 0u && (!(T > 0.0f) || !(T < INFINITY))) st |= SD_ST_BAD_TEMP;
  if (check_temp && !params_ok(request_top_p(a, r), request_D(a, r))) st |= SD_ST_BAD_PARAM;
  if (priorbad) st |= SD_ST_BAD_PRIOR;
  return st;
}

// Decisions, first rejection and outputs of request r; without SPLIT also
// the draw, else the draw's choice goes to drec[r] (n, mode; mode 2: no
// draw) for k_draw_tot / k_draw_pick, which fill in the drawn token.
template <int DT, bool SPLIT>
__global__ __launch_bounds__(NT_ROW) void k_finalize(Args a, const RowStat* rs, const double* dpart,
                                                    int tv_valid, int tvS, int bm_words, int2* drec,
                                                    int32_t* out_acc, int32_t* out_tok,
                                                    uint32_t* out_status, float* out_stats) {
  constexpr int NT = NT_ROW;
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* bm = reinterpret_cast<uint32_t*>(smem);
  double* ctot = reinterpret_cast<double*>(smem + align_up(bm_words * 4, 16));
  __shared__ double sd[NT];
  __shared__ float sf[NT / WAVE];
  __shared__ int si[NT / WAVE + 4];
  __shared__ int sh_n, sh_mode;
  __shared__ uint32_t sh_st;
  __shared__ float sh_stat[(SD_MAX_K + 1) * SD_NSTAT];

  const int r = blockIdx.x;
  const int K1 = a.K_max + 1;
  const int K = request_k(a, r);
  const float T = request_t(a, r);
  uint32_t st = request_status<NT>(a, r, K, T, true, si);
  int nonfin = 0;
  if (!(st & SD_ST_INVALID_MASK))
    for (int t = threadIdx.x; t < 2 * K + 1; t += NT) {
      const bool tg = t <= K;
      nonfin |= (rs[row_index(a, r, tg, tg ? t : t - K - 1)].flags & NONFINITE) ? 1 : 0;
    }
  if (block_or<NT>(nonfin, si)) st |= SD_ST_NONFINITE;

  if (st & SD_ST_INVALID_MASK) {
    if (SPLIT && threadIdx.x == 0) drec[r] = make_int2(0, 2);
    for (int t = threadIdx.x; t < K1; t += NT) out_tok[(int64_t)r * K1 + t] = -1;
    if (out_stats)
      for (int t = threadIdx.x; t < K1 * SD_NSTAT; t += NT) out_stats[(int64_t)r * K1 * SD_NSTAT + t] = 0.0f;
    if (threadIdx.x == 0) {
      out_acc[r] = -1;
      if (out_status) out_status[r] = st;
    }
    return;
  }

  // Every position at once (thread jj): its uniforms, statistics and
  // decision; then thread 0 takes the first rejection.
  __shared__ unsigned char sh_acc[SD_MAX_K + 1], sh_qz[SD_MAX_K + 1];
  if ((int)threadIdx.x <= K) {
    const int jj = threadIdx.x;
    float u, v;
    uniforms(a.seed, a.offset, r, jj, u, v);
    float* sv = &sh_stat[jj * SD_NSTAT];
    for (int s = 0; s < SD_NSTAT; ++s) sv[s] = 0.0f;
    sv[SD_STAT_U] = u;
    sv[SD_STAT_V] = v;
    if (jj < K) {
      const RowStat P = rs[row_index(a, r, true, jj)], Q = rs[row_index(a, r, false, jj)];
      double d = 0.0;
      if (tv_valid) {
        const double* dp = dpart + ((int64_t)r * a.K_max + jj) * tvS;
        for (int s = 0; s < tvS; ++s) d += dp[s];
        d = fmin(0.5 * d, 1.0);
      }
      const Decision dc = decide(P, Q, P.kx, Q.kx, (double)T, (double)request_D(a, r), tv_valid != 0, d, u);
      sh_qz[jj] = dc.qx == 0.0;
      sh_acc[jj] = dc.accept;
      sv[SD_STAT_D] = (float)d;
      sv[SD_STAT_THETA] = (float)dc.th;
      sv[SD_STAT_PX] = (float)dc.px;
      sv[SD_STAT_QX] = (float)dc.qx;
      sv[SD_STAT_PIX] = (float)dc.pix;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = K;
    for (int jj = 0; jj < K; ++jj) {
      if (sh_qz[jj]) st |= SD_ST_Q_ZERO;
      if (n == K && !sh_acc[jj]) n = jj;
    }
    sh_n = n;
    sh_mode = (n < K) ? 0 : ((a.flags & SD_NO_BONUS) ? 2 : 1);
    sh_st = st;
  }
  __syncthreads();
  const int n = sh_n, mode = sh_mode;
  int y = -1;
  if (SPLIT) {
    if (threadIdx.x == 0) drec[r] = make_int2(n, mode);
  } else if (mode != 2) {
    const bool pen = build_penalty_bitmap<NT>(a, r, n, 0, a.V, bm);
    const RowStat P = rs[row_index(a, r, true, n)];
    const RowStat Q = (n < K) ? rs[row_index(a, r, false, n)] : P;
    const char* trow = target_row(a, r, n);
    const char* drow = (n < K) ? draft_row(a, r, n) : trow;
    ExactLds L{};
    L.sd = sd;
    L.sf = sf;
    L.si = si;
    L.ctot = ctot;
    // (rows without top-p compare no key with a cut)
    const float v = sh_stat[n * SD_NSTAT + SD_STAT_V];
    const Drawn dw = P.kord == KEEP_ALL && Q.kord == KEEP_ALL
                         ? draw_dev<DT, NT, true>(a, trow, drow, P, Q, mode, v, pen, bm, L)
                         : draw_dev<DT, NT>(a, trow, drow, P, Q, mode, v, pen, bm, L);
    y = dw.y;
    if (threadIdx.x == 0) {
      sh_stat[n * SD_NSTAT + SD_STAT_S] = (float)dw.S;
      if (dw.resid_zero) sh_st |= SD_ST_RESID_ZERO;
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < K1; t += NT) {
    int v = -1;
    if (t < n) v = a.ids[(int64_t)r * a.K_max + t];
    else if (t == n && mode != 2) v = y;
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

// The draw's chunk totals of request r, slice b % S of its chunks (both
// modes' totals for a residual draw, whose mode 1 is the fallback when the
// residual has no mass), to ctot[r][0 .. nch] and ctot[r][nch + 1 ..].
template <int DT>
__global__ __launch_bounds__(NT_ROW) void k_draw_tot(Args a, const RowStat* rs, const int2* drec,
                                                     double* ctot, int S) {
  constexpr int NT = NT_ROW;
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* bm = reinterpret_cast<uint32_t*>(smem);
  const int r = blockIdx.x / S, sl = blockIdx.x % S;
  const int2 rec = drec[r];
  const int n = rec.x, mode = rec.y;
  if (mode == 2) return;
  const int K = request_k(a, r);
  const int nch = draw_chunks(a.V), len = (nch + S - 1) / S;
  const int ch0 = min(nch, sl * len), ch1 = min(nch, ch0 + len);
  if (ch0 >= ch1) return;
  const bool pen = build_penalty_bitmap<NT>(a, r, n, ch0 * CHV * VEC, (ch1 - ch0) * CHV * VEC, bm);
  const RowStat P = rs[row_index(a, r, true, n)];
  const RowStat Q = (n < K) ? rs[row_index(a, r, false, n)] : P;
  const char* trow = target_row(a, r, n);
  const char* drow = (n < K) ? draft_row(a, r, n) : trow;
  double* c0 = ctot + (int64_t)r * 2 * (nch + 1);
  if (P.kord == KEEP_ALL && Q.kord == KEEP_ALL)   // (rows without top-p compare no key with a cut)
    draw_totals<DT, NT, true, true>(a, trow, drow, P, Q, mode, pen, bm, ch0 * CHV * VEC, ch0, ch1, c0,
                                    c0 + nch + 1);
  else
    draw_totals<DT, NT, true>(a, trow, drow, P, Q, mode, pen, bm, ch0 * CHV * VEC, ch0, ch1, c0, c0 + nch + 1);
}

// The draw of request r from its chunk totals: the same scan and crossing
// chunk walk as the one-workgroup draw, so the same token; writes it, S,
// and the zero-residual bit into the outputs k_finalize<DT, true> wrote.
template <int DT>
__global__ __launch_bounds__(NT_ROW) void k_draw_pick(Args a, const RowStat* rs, const int2* drec,
                                                      double* ctot, int32_t* out_tok, uint32_t* out_status,
                                                      float* out_stats) {
  constexpr int NT = NT_ROW;
  __shared__ uint32_t bm[CHV * VEC / 32];
  __shared__ double sd[NT];
  __shared__ int si[NT / WAVE + 4];
  const int r = blockIdx.x;
  const int2 rec = drec[r];
  const int n = rec.x;
  int mode = rec.y;
  if (mode == 2) return;
  const int K = request_k(a, r);
  const int nch = draw_chunks(a.V);
  float u, v;
  uniforms(a.seed, a.offset, r, n, u, v);
  ExactLds L{};
  L.sd = sd;
  L.si = si;
  double* c0 = ctot + (int64_t)r * 2 * (nch + 1);
  double S = 0.0, t = 0.0;
  int cs = draw_scan<NT>(c0, nch, v, L, S, t);
  int resid_zero = 0;
  if (!(S > 0.0) && mode == 0) {   // zero residual: draw from p
    mode = 1;
    resid_zero = 1;
    c0 += nch + 1;
    cs = draw_scan<NT>(c0, nch, v, L, S, t);
  }
  bool pen = false;
  if (cs >= 0) pen = build_penalty_bitmap<NT>(a, r, n, cs * CHV * VEC, CHV * VEC, bm);
  const RowStat P = rs[row_index(a, r, true, n)];
  const RowStat Q = (n < K) ? rs[row_index(a, r, false, n)] : P;
  const char* trow = target_row(a, r, n);
  const char* drow = (n < K) ? draft_row(a, r, n) : trow;
  const int y = draw_resolve<DT, NT>(a, trow, drow, P, Q, mode, pen, bm, cs * CHV * VEC, cs, t, c0[nch], L);
  if (threadIdx.x == 0) {
    const int K1 = a.K_max + 1;
    out_tok[(int64_t)r * K1 + n] = y;
    if (out_stats) out_stats[((int64_t)r * K1 + n) * SD_NSTAT + SD_STAT_S] = (float)S;
    if (out_status && resid_zero) out_status[r] |= SD_ST_RESID_ZERO;
  }
}

// ---------------------------------------------------------------------------
// Single-pass kernel.
// ---------------------------------------------------------------------------

struct UnitOut {
  float d, th, px, qx, pix, u, v, S;
  int32_t accept, y;
  uint32_t flags, why;   // why: FB_* bits of a UO_FALLBACK unit (diagnostics)
};
static_assert(sizeof(UnitOut) == 48, "UnitOut layout");
enum : uint32_t { UO_NONFINITE = 1, UO_QZERO = 2, UO_RESID_ZERO = 4, UO_SLOW = 8, UO_FALLBACK = 16 };
// Why the single pass handed a unit to its exact route: a row's stream
// state out of range (anchor, normalizer, list capacities), its cut not
// settled by the window, or more nucleus candidates than slots.
enum : uint32_t {
  FB_P_STATE = 1, FB_P_CUT = 2, FB_Q_STATE = 4, FB_Q_CUT = 8, FB_SLOTS = 16,
  FB_WIDE = 32,     // (with FB_P_CUT) the target cut came from its whole histogram
  FB_WIDE_Q = 64    // (with FB_Q_CUT) the draft cut likewise
};

// Compile-time loop: f.template operator()<I>() for I = 0 .. N-1, so that
// register arrays indexed by I stay in registers.
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (f.template operator()<I>(), ...);
  }(std::make_integer_sequence<int, N>{});
}

// Keeps the compiler from sinking a round's arithmetic past later loads
// (which would keep the round's load registers alive and spill them).
#define SDV_PIN(x) asm volatile("" : "+v"(x))

typedef int16_t i16x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2 as_u16x2(uint32_t w) { return __builtin_bit_cast(u16x2, w); }
__device__ __forceinline__ uint32_t as_u32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// bf16 value whose 16-bit orderable key is o.
__device__ __forceinline__ float key_of_ord16(uint32_t o) {
  const uint32_t b = (o & 0x8000u) ? (o & 0x7FFFu) : (~o & 0xFFFFu);
  return __uint_as_float(b << 16);
}

// 16-bit orderable key of a float (top half of the 32-bit orderable key;
// -0 = +0).  A token's bin is this key: bins are ranges of the 32-bit
// order, so every key of a higher bin is larger than every key of a lower.
__device__ __forceinline__ uint32_t ord16f(float z) {
  const uint32_t u = __float_as_uint(z + 0.0f);
  return (u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u)) >> 16;
}

// Orderable keys of the two bf16 values packed in w (-0 keeps its own key,
// one below +0; the cut search merges the two).
__device__ __forceinline__ uint32_t ord16x2(uint32_t w) {
  const i16x2 s = __builtin_bit_cast(i16x2, w) >> (i16x2){15, 15};
  return w ^ (__builtin_bit_cast(uint32_t, s) | 0x80008000u);
}

// Codes of a row against its anchor t1 = (top key of the window) + 1:
// 0 above the window, 1..254 the window (key = t1 - code), 255 below.
__device__ __forceinline__ uint32_t code_of(uint32_t t1x2, uint32_t o2) {
  const u16x2 d = __builtin_elementwise_sub_sat(as_u16x2(t1x2), as_u16x2(o2));
  return as_u32(__builtin_elementwise_min(d, (u16x2){255, 255}));
}

__device__ __forceinline__ uint32_t code1(uint32_t t1, float z) {
  const uint32_t o = ord16f(z);
  return o >= t1 ? 0u : (t1 - o > 255u ? 255u : t1 - o);
}

// Bytes of x that are <= t (t <= 254): the top bit of each such byte,
// exact per byte (no borrow crosses a byte).  LOW: t < 127, when known at
// compile time (-1: decided at run time).
template <int LOW = -1>
__device__ __forceinline__ uint32_t le_mask(uint32_t x, uint32_t t) {
  if (LOW == 1 || (LOW < 0 && t < 127u)) {
    const uint32_t r = (x | 0x80808080u) - (t + 1u) * 0x01010101u;
    return ~(r | x) & 0x80808080u;
  }
  const uint32_t r = ((x & 0x7F7F7F7Fu) | 0x80808080u) - (t - 127u) * 0x01010101u;
  return ~(r & x) & 0x80808080u;
}

__device__ __forceinline__ uint32_t pk_max(uint32_t a, uint32_t b) {
  return as_u32(__builtin_elementwise_max(as_u16x2(a), as_u16x2(b)));
}

// Unit handled by block u: pairs (r, j) first, then one bonus row per request.
struct Unit {
  int r, j;
  bool bonus;
};

__device__ __forceinline__ Unit unit_of(const Args& a, int u) {
  Unit w;
  const int npairs = a.B * a.K_max;
  if (u < npairs) {
    w.r = u / a.K_max;
    w.j = u % a.K_max;
    w.bonus = false;
  } else {
    w.r = u - npairs;
    w.j = 0;
    w.bonus = true;
  }
  return w;
}

// w(i) of one target-nucleus token: mode 0 max(p - q, 0), mode 1 p.
__device__ __forceinline__ float nucleus_w(float zp, float zq, int mode, float Mp, float ip,
                                           float kq_cut, float Mq, float iq, float c) {
  const float pr = e_rel(zp, Mp, c) * ip;
  if (mode == 1) return pr;
  const float q = (zq >= kq_cut) ? e_rel(zq, Mq, c) * iq : 0.0f;
  return fmaxf(pr - q, 0.0f);
}

// Single-pass kernel geometry.
constexpr int NT_F = 1024;                   // threads per workgroup
constexpr int NR = 19;                       // 16-byte loads per thread and row
constexpr int MAXV_FAST = NR * NT_F * VEC;   // 155648 logits
constexpr int NSAMP = 4;                     // rounds whose block max anchors a row's codes
constexpr int NSTG = 5;                      // 16-byte loads in flight per thread
constexpr int UP = 32;                       // window bins above the sample max
constexpr int NBIN = 256;                    // codes 0..255
constexpr int NBINW = 8192;                  // bins of a row's key histogram
constexpr int RUP = 4096;                    // exact bins from the window's top key down
constexpr int RNEG = 4094;                   // exact bins below the lumped band
static_assert(RUP + RNEG + 2 <= NBINW && RUP > NBIN, "histogram geometry");
constexpr int E_CAP = 512;                   // exact-key entries per row
constexpr int R_CAP = 64;                    // exact entries in the crossing bin
constexpr int CAPT = 20;                     // nucleus slots per lane
constexpr int PE_CAP = 256;                  // penalized exact entries per row
constexpr int PL_CAP = 256;                  // distinct penalized ids per unit
constexpr int SHP = 40;                      // fixed-point shift of exact-entry masses
constexpr int SHD = 40;                      // fixed-point shift of draw weights (each <= 1)
static_assert(NSTG >= NSAMP && NSTG < NR, "load ring");

// Exact-key list of one row, in two regions.  The stream region holds the
// logits found above the window while streaming, keyed as read; an entry
// whose id is penalized is stale there.  The penalty region holds every
// penalized logit whose penalized key reaches the window, under that key.
struct ExactList {
  float* key;
  int32_t* id;
  uint16_t* raw;   // the unprocessed logit (bf16 bits)
  int* n;
  float* pkey;     // penalty region
  int32_t* pid;
  uint16_t* praw;
  int* np;
};

// Entry i of an exact list with ns stream entries (then the penalty
// region); false for a stale stream entry.
__device__ __forceinline__ bool ex_entry(const ExactList& ex, int ns, int i, const uint32_t* bm,
                                         bool pen, float& k, int& id) {
  if (i < ns) {
    k = ex.key[i];
    id = ex.id[i];
    return !(pen && ((bm[id >> 5] >> (id & 31)) & 1u));
  }
  k = ex.pkey[i - ns];
  id = ex.pid[i - ns];
  return true;
}

struct Cut {
  int ok;         // 0: the window does not settle the cut
  int code;       // crossing bin (0 = above the window)
  float key;      // boundary key: kept iff key >= this
  double zk;      // kept mass, relative to exp2(M c)
};

// Exact top-p cut of a row from its window histogram and exact list, by
// one wave (the caller's wave 0; no block barriers), in two parts so that
// the first can run before the row's normalizer is summed.  Window bins are
// visited from the top; the first non-empty bin whose cumulative mass
// reaches TP is the crossing bin.  A crossing bin that holds exact entries
// is resolved key by key, ties kept together.
//
// wave_cut_prep (needs the row max M): a bin's count is hist - hneg (the
// row's key histogram, whose bins 1..254 are the window, less the
// penalized logits that left it); ecnt / emass (count and fixed-point mass
// of exact entries per bin) start at zero.  Lane L owns bins 4L .. 4L+3.
// It leaves each bin's count in hneg, its exact-entry count in ecnt, its
// mass (a double) in emass, and lane L's exclusive scan in cx[L].
__device__ __forceinline__ void wave_cut_prep(const uint32_t* hist, uint32_t* hneg, const ExactList& ex,
                                              int ns, int np, const uint32_t* bm, bool pen, uint32_t t1,
                                              float M, float c, uint32_t* ecnt, uint64_t* emass,
                                              double* cx) {
  const int ne = ns + np;
  const int lane = threadIdx.x % WAVE;
  for (int i = lane; i < ne; i += WAVE) {
    float k;
    int id;
    if (!ex_entry(ex, ns, i, bm, pen, k, id)) continue;
    const uint32_t b = code1(t1, k);
    if (b < 255u) {
      atomicAdd(&ecnt[b], 1u);
      atomicAdd(reinterpret_cast<unsigned long long*>(&emass[b]),
                (unsigned long long)e_fixed(e_rel(k, M, c), SHP));
    }
  }
  __builtin_amdgcn_wave_barrier();
  uint32_t cnt[4], ec[4];
  double mass[4];
  double lsum = 0.0;
  const uint4 hs = reinterpret_cast<const uint4*>(hist)[lane];
  const uint4 hn = reinterpret_cast<const uint4*>(hneg)[lane];
  const uint32_t hc[4] = {hs.x - hn.x, hs.y - hn.y, hs.z - hn.z, hs.w - hn.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = 4 * lane + i;
    uint32_t n = hc[i];
    if (b == 0 || b == 255) n = 0u;   // not window bins
    cnt[i] = n;
    ec[i] = b < 255 ? ecnt[b] : 0u;
    double m = n ? (double)n * (double)e_rel(key_of_ord16(t1 - b), M, c) : 0.0;
    if (b < 255) m += (double)emass[b] * 0x1p-40;
    mass[i] = m;
    lsum += m;
  }
  const double excl = wave_incl_scan(lsum) - lsum;
  __builtin_amdgcn_wave_barrier();
  reinterpret_cast<uint4*>(hneg)[lane] = make_uint4(cnt[0], cnt[1], cnt[2], cnt[3]);
  reinterpret_cast<uint4*>(ecnt)[lane] = make_uint4(ec[0], ec[1], ec[2], ec[3]);
#pragma unroll
  for (int i = 0; i < 4; ++i) reinterpret_cast<double*>(emass)[4 * lane + i] = mass[i];
  cx[lane] = excl;
}

// wave_cut_finish: the crossing and the cut from wave_cut_prep's bins and
// the threshold TP (mass relative to exp2(M c)); the exact list, M and t1
// as for the prep.
__device__ __forceinline__ Cut wave_cut_finish(const uint32_t* hcnt, const uint32_t* ecnt,
                                               const uint64_t* emass, const double* cx,
                                               const ExactList& ex, int ns, int np, const uint32_t* bm,
                                               bool pen, uint32_t t1, float M, float c, double TP,
                                               float* rkey, double* rmass, int* rid, int* scnt) {
  const int ne = ns + np;
  const int lane = threadIdx.x % WAVE;
  if (lane == 0) *scnt = 0;
  const uint4 h4 = reinterpret_cast<const uint4*>(hcnt)[lane];
  const uint4 e4 = reinterpret_cast<const uint4*>(ecnt)[lane];
  const uint32_t cnt[4] = {h4.x, h4.y, h4.z, h4.w};
  const uint32_t ec[4] = {e4.x, e4.y, e4.z, e4.w};
  double mass[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) mass[i] = reinterpret_cast<const double*>(emass)[4 * lane + i];
  const double excl = cx[lane];
  __builtin_amdgcn_wave_barrier();
  // first crossing bin of this lane
  double cum = excl, cin = 0.0, cex = 0.0;
  int hit = -1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double nx = cum + mass[i];
    if (hit < 0 && (cnt[i] + ec[i]) > 0u && nx >= TP) {
      hit = i;
      cin = nx;
      cex = cum;
    }
    cum = nx;
  }
  const uint64_t bal = __ballot(hit >= 0);
  Cut out;
  out.ok = bal != 0ull;
  out.code = 0;
  out.key = 0.0f;
  out.zk = 0.0;
  if (!out.ok) return out;
  const int src = __builtin_ctzll(bal);
  const int hb = lane_read(hit, src);
  const int b = 4 * src + hb;
  const double c_incl = lane_read(cin, src), c_excl = lane_read(cex, src);
  const int gcnt = lane_read((int)(hb == 0 ? cnt[0] : hb == 1 ? cnt[1] : hb == 2 ? cnt[2] : cnt[3]), src);
  const int necb = lane_read((int)(hb == 0 ? ec[0] : hb == 1 ? ec[1] : hb == 2 ? ec[2] : ec[3]), src);
  out.code = b;
  out.key = b > 0 ? key_of_ord16(t1 - b) : 0.0f;
  out.zk = c_incl;
  if (b > 0 && b < 254 && __float_as_uint(out.key) == 0u) {
    // A +0 crossing bin with a non-empty bin just below (-0, and negative
    // keys above the largest negative bf16): the two share the key 0.
    // Merged when both hold logits of one key each; else unsettled.
    const int b1 = b + 1, l1 = b1 >> 2, i1 = b1 & 3;
    const int n1 = lane_read((int)(i1 == 0 ? cnt[0] : i1 == 1 ? cnt[1] : i1 == 2 ? cnt[2] : cnt[3]), l1);
    const int e1 = lane_read((int)(i1 == 0 ? ec[0] : i1 == 1 ? ec[1] : i1 == 2 ? ec[2] : ec[3]), l1);
    // cumulative through bin b + 1 = through bin b + its mass
    const double m1 = lane_read(i1 == 0 ? mass[0] : i1 == 1 ? mass[1] : i1 == 2 ? mass[2] : mass[3], l1);
    if (n1 > 0 || e1 > 0) {
      if (e1 > 0 || necb > 0) {
        out.ok = 0;
        return out;
      }
      out.zk = c_incl + m1;
      out.code = b1;
      out.key = -0.0f;
    }
  }
  if (necb == 0) return out;
  // Exact resolution inside the crossing bin: gather its entries (plus the
  // bin's unpenalized group), order them canonically (key descending, id
  // ascending); the cut is the largest key whose cumulative mass, ties
  // included, reaches TP.
  if (necb + 1 > R_CAP) {
    out.ok = 0;
    return out;
  }
  for (int i = lane; i < ne; i += WAVE) {
    float k;
    int id;
    if (!ex_entry(ex, ns, i, bm, pen, k, id)) continue;
    if (code1(t1, k) == (uint32_t)b) {
      const int s = atomicAdd(scnt, 1);
      rkey[s] = k;
      rid[s] = id;
      rmass[s] = (double)e_rel(k, M, c);
    }
  }
  __builtin_amdgcn_wave_barrier();
  int n = necb;
  if (gcnt > 0) {
    if (lane == 0) {
      rkey[n] = out.key;
      rid[n] = -1;
      rmass[n] = (double)gcnt * (double)e_rel(out.key, M, c);
    }
    ++n;
  }
  __builtin_amdgcn_wave_barrier();
  float mk = 0.0f;
  double mm = 0.0;
  int rank = 0;
  if (lane < n) {
    mk = rkey[lane];
    const int mi = rid[lane];
    mm = rmass[lane];
    for (int q = 0; q < n; ++q) {
      const float kq = rkey[q];
      const int iq = rid[q];
      rank += (kq > mk || (kq == mk && iq < mi)) ? 1 : 0;
    }
  }
  __builtin_amdgcn_wave_barrier();
  if (lane < n) {
    rkey[rank] = mk;
    rmass[rank] = mm;
  }
  __builtin_amdgcn_wave_barrier();
  // cumulative through the end of my tie group, in canonical order
  double cm = c_excl;
  const float me = lane < n ? rkey[lane] : 0.0f;
  if (lane < n)
    for (int q = 0; q < n; ++q)
      if (rkey[q] >= me) cm += rmass[q];
  const uint64_t reach = __ballot(lane < n && cm >= TP);
  const int pick = reach ? __builtin_ctzll(reach) : n - 1;
  out.key = lane_read(me, pick);
  out.zk = lane_read(cm, pick);
  return out;
}


// Per-wave partials to LDS and one barrier; every thread gets the result.
// Each call site uses its own buffer (NT / WAVE entries).
template <int NT>
__device__ __forceinline__ float bar_max(float x, float* buf) {
  x = wave_max(x);
  if (threadIdx.x % WAVE == 0) buf[threadIdx.x / WAVE] = x;
  __syncthreads();
  float m = buf[0];
#pragma unroll
  for (int i = 1; i < NT / WAVE; ++i) m = fmaxf(m, buf[i]);
  return m;
}

struct CutRes {
  int ok, code;
  float key, M;
  double zk;
};

// A row's key histogram and lists, for wide_cut.
struct WideLds {
  uint32_t* hist;         // the row's key histogram (its exact bins are consumed)
  uint32_t* ecnt4;        // scratch: RUP words
  uint64_t* emass4;       // scratch: RUP words of 8 bytes
  ExactList ex;           // its stream entries (the first ns)
  int ns;
  const int* plid;        // distinct penalized ids
  const uint32_t* plraw;  // their target | draft logits (bf16 bits; all ones: not loaded)
  int npl;
  float* rkey;            // R_CAP entries each
  double* rmass;
  int* rid;
  int* scnt;
  double* wtot;           // NT_F / WAVE
  double TP;              // mass threshold, relative to exp2(M c)
  uint32_t t1;            // the row's anchor: key of bin d is t1 - d
  CutRes* cut;            // the row's cut record (M read; the result written by the caller)
};

// Exact top-p cut of a row over its whole exact key range (bins 0 .. RUP-1
// of its key histogram; bin 0 holds only exact entries), for a row whose
// crossing lies below the window: block-wide, the same rule as wave_cut.
// Every penalized logit leaves the bin of its raw key (taken off the
// histogram in place) and joins the exact entries under its penalized key,
// with the stream entries of unpenalized ids.  The row is the target's
// (DRAFT false: plraw's low halves) or the draft's (high halves; ids from
// Vrow on hold -inf).  ok = 0 when no bin above RUP - 1 reaches the
// threshold, or the crossing bin holds more exact entries than R_CAP, or
// it is the bin of +0 over a bin below it that is not one plain key.
template <bool DRAFT>
__device__ __forceinline__ Cut wide_cut(const WideLds& L, const char* row, int Vrow, const uint32_t* bm,
                                        bool pen, float rep, float M, float c) {
  constexpr int NT = NT_F;
  static_assert(RUP == 4 * NT && RUP <= NBINW, "wide_cut geometry");
  const int tid = threadIdx.x, lane = tid % WAVE;
  uint32_t* const hist = L.hist;
  uint32_t* const ecnt4 = L.ecnt4;
  uint64_t* const emass4 = L.emass4;
  const ExactList& ex = L.ex;
  const int ns = L.ns, npl = L.npl;
  const int* const plid = L.plid;
  const uint32_t* const plraw = L.plraw;
  float* const rkey = L.rkey;
  double* const rmass = L.rmass;
  int* const rid = L.rid;
  int* const scnt = L.scnt;
  const uint32_t t1 = L.t1;
  const double TP = L.TP;
  __shared__ int s_b;   // the crossing bin
  for (int i = tid; i < RUP; i += NT) {
    ecnt4[i] = 0u;
    emass4[i] = 0ull;
  }
  if (tid == 0) {
    *scnt = 0;
    s_b = INT_MAX;
  }
  // the row's logit of penalized id i, as read (bf16 bits)
  auto pen_raw = [&](int i) __attribute__((always_inline)) {
    const int id = plid[i];
    const uint32_t g = plraw[i];
    if (DRAFT && id >= Vrow) return 0xFF80u;
    if (g == 0xFFFFFFFFu) return (uint32_t)reinterpret_cast<const uint16_t*>(row)[id];
    return DRAFT ? g >> 16 : g & 0xFFFFu;
  };
  auto bin_of = [&](float k) __attribute__((always_inline)) {
    const uint32_t o = ord16f(k);
    return o >= t1 ? 0u : t1 - o;
  };
  auto add_exact = [&](float k) __attribute__((always_inline)) {
    const uint32_t b = bin_of(k);
    if (b < (uint32_t)RUP) {
      atomicAdd(&ecnt4[b], 1u);
      atomicAdd(reinterpret_cast<unsigned long long*>(&emass4[b]),
                (unsigned long long)e_fixed(e_rel(k, M, c), SHP));
    }
  };
  __syncthreads();
  for (int i = tid; i < npl; i += NT) {
    const uint32_t raw = pen_raw(i);
    const uint32_t o = raw ^ ((raw & 0x8000u) ? 0xFFFFu : 0x8000u);   // as the stream keyed it
    if (o < t1 && t1 - o < (uint32_t)RUP) atomicSub(&hist[t1 - o], 1u);
    add_exact(penalize(__uint_as_float(raw << 16), rep));
  }
  for (int i = tid; i < ns; i += NT) {
    const int id = ex.id[i];
    if (pen && ((bm[id >> 5] >> (id & 31)) & 1u)) continue;   // stale: listed above
    add_exact(ex.key[i]);
  }
  __syncthreads();
  // thread t: bins 4t .. 4t + 3
  uint32_t cnt[4], ec[4];
  double mass[4];
  double lsum = 0.0;
  const uint4 h4 = reinterpret_cast<const uint4*>(hist)[tid];
  const uint32_t hv[4] = {h4.x, h4.y, h4.z, h4.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int b = 4 * tid + q;
    const uint32_t n = (b == 0 || b > (int)t1) ? 0u : hv[q];
    cnt[q] = n;
    ec[q] = ecnt4[b];
    double m = n ? (double)n * (double)e_rel(key_of_ord16(t1 - (uint32_t)b), M, c) : 0.0;
    m += (double)emass4[b] * 0x1p-40;
    mass[q] = m;
    lsum += m;
  }
  const double incl_t = block_incl_scan_fast<NT>(lsum, L.wtot);
  double cum = incl_t - lsum;
  int hit = -1;
  double cin = 0.0, cex = 0.0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const double nx = cum + mass[q];
    if (hit < 0 && (cnt[q] + ec[q]) > 0u && nx >= TP) {
      hit = q;
      cin = nx;
      cex = cum;
    }
    cum = nx;
  }
  if (hit >= 0) atomicMin(&s_b, 4 * tid + hit);
  __syncthreads();
  const int bstar = s_b;
  Cut out;
  out.ok = 0;
  out.code = 0;
  out.key = 0.0f;
  out.zk = 0.0;
  if (bstar == INT_MAX || bstar >= RUP - 1) {
    __syncthreads();
    return out;
  }
  // the crossing thread publishes its bin's totals, and those of the bin
  // below (for a +0 crossing bin over a -0 one)
  __shared__ double s_w[3];
  __shared__ int s_wi[4];
  __shared__ float s_k;
  if (hit >= 0 && 4 * tid + hit == bstar) {
    auto pick4 = [&](const auto (&x)[4]) __attribute__((always_inline)) {
      return hit == 0 ? x[0] : hit == 1 ? x[1] : hit == 2 ? x[2] : x[3];
    };
    s_w[0] = cin;
    s_w[1] = cex;
    s_wi[0] = (int)pick4(cnt);
    s_wi[1] = (int)pick4(ec);
    const int b1 = bstar + 1;
    const uint32_t n1 = b1 > (int)t1 ? 0u : hist[b1];
    s_wi[2] = (int)n1;
    s_wi[3] = (int)ecnt4[b1];
    s_w[2] = (n1 ? (double)n1 * (double)e_rel(key_of_ord16(t1 - (uint32_t)b1), M, c) : 0.0) +
             (double)emass4[b1] * 0x1p-40;
  }
  __syncthreads();
  const double c_incl = s_w[0], c_excl = s_w[1];
  const int gcnt = s_wi[0], necb = s_wi[1];
  out.ok = 1;
  out.code = bstar;
  out.key = bstar > 0 ? key_of_ord16(t1 - (uint32_t)bstar) : 0.0f;
  out.zk = c_incl;
  // A +0 crossing bin with a non-empty bin just below (-0, and negative
  // keys above the largest negative bf16): the two share the key 0.  Merged
  // when both hold logits of one key each; the rest is left to the passes.
  // (bin 0, the keys above the window, has no key of its own)
  const bool zero_pair = bstar > 0 && __float_as_uint(out.key) == 0u && (s_wi[2] > 0 || s_wi[3] > 0);
  if (necb == 0) {
    if (zero_pair) {
      if (s_wi[3] > 0) out.ok = 0;
      else {
        out.zk = c_incl + s_w[2];
        out.code = bstar + 1;
        out.key = -0.0f;
      }
    }
    __syncthreads();
    return out;
  }
  if (necb + 1 > R_CAP || zero_pair) {
    out.ok = 0;
    __syncthreads();
    return out;
  }
  // Exact resolution inside the crossing bin: its entries plus the bin's
  // unpenalized group, in canonical order (key descending, id ascending).
  auto take = [&](float k, int id) __attribute__((always_inline)) {
    if (bin_of(k) == (uint32_t)bstar) {
      const int sidx = atomicAdd(scnt, 1);
      rkey[sidx] = k;
      rid[sidx] = id;
      rmass[sidx] = (double)e_rel(k, M, c);
    }
  };
  for (int i = tid; i < npl; i += NT) take(penalize(__uint_as_float(pen_raw(i) << 16), rep), plid[i]);
  for (int i = tid; i < ns; i += NT) {
    const int id = ex.id[i];
    if (pen && ((bm[id >> 5] >> (id & 31)) & 1u)) continue;
    take(ex.key[i], id);
  }
  __syncthreads();
  if (tid < WAVE) {
    int n = necb;
    if (gcnt > 0) {
      if (lane == 0) {
        rkey[n] = out.key;
        rid[n] = -1;
        rmass[n] = (double)gcnt * (double)e_rel(out.key, M, c);
      }
      ++n;
    }
    __builtin_amdgcn_wave_barrier();
    float mk = 0.0f;
    double mm = 0.0;
    int rank = 0;
    if (lane < n) {
      mk = rkey[lane];
      const int mi = rid[lane];
      mm = rmass[lane];
      for (int q = 0; q < n; ++q) {
        const float kq = rkey[q];
        const int iq = rid[q];
        rank += (kq > mk || (kq == mk && iq < mi)) ? 1 : 0;
      }
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < n) {
      rkey[rank] = mk;
      rmass[rank] = mm;
    }
    __builtin_amdgcn_wave_barrier();
    double cm = c_excl;
    const float me = lane < n ? rkey[lane] : 0.0f;
    if (lane < n)
      for (int q = 0; q < n; ++q)
        if (rkey[q] >= me) cm += rmass[q];
    const uint64_t reach = __ballot(lane < n && cm >= TP);
    const int pick = reach ? __builtin_ctzll(reach) : n - 1;
    const double zsel = lane_read(cm, pick);
    const float ksel = lane_read(me, pick);
    if (lane == 0) {
      s_w[0] = zsel;
      s_k = ksel;
    }
  }
  __syncthreads();
  out.zk = s_w[0];
  out.key = s_k;
  __syncthreads();
  return out;
}

__device__ __forceinline__ void exact_push(const ExactList& ex, float key, int id, uint32_t raw) {
  const int ix = atomicAdd(ex.n, 1);
  if (ix < E_CAP) {
    ex.key[ix] = key;
    ex.id[ix] = id;
    ex.raw[ix] = (uint16_t)raw;
  }
}

__device__ __forceinline__ void pen_push(const ExactList& ex, float key, int id, uint32_t raw) {
  const int ix = atomicAdd(ex.np, 1);
  if (ix < PE_CAP) {
    ex.pkey[ix] = key;
    ex.pid[ix] = id;
    ex.praw[ix] = (uint16_t)raw;
  }
}

// Unprocessed bf16 bits of token id from an exact list (either region; both
// store the bits as read), or 0xFFFFFFFF if the list has no entry for it.
__device__ __forceinline__ uint32_t exact_raw(const ExactList& ex, int ns, int np, int id) {
  uint32_t raw = 0xFFFFFFFFu;
  for (int i = 0; i < ns; ++i)
    if (ex.id[i] == id) raw = ex.raw[i];
  for (int i = 0; i < np; ++i)
    if (ex.pid[i] == id) raw = ex.praw[i];
  return raw;
}

// Bit e of an 8-bit mask to bit 4e (the candidate layout).
__device__ __forceinline__ uint32_t spread8(uint32_t b) {
  uint32_t x = b & 0xFFu;
  x = (x | (x << 12)) & 0x000F000Fu;   // elements 4..7 to bits 16..19
  x = (x | (x << 6)) & 0x03030303u;    // two elements per byte
  return (x | (x << 3)) & 0x11111111u;   // one per nibble
}

// One 8-logit vector of a row: keys z as read, packed orderable keys o,
// the raw words.  Elements >= V read as -inf.
struct Vec8 {
  float z[VEC];
  uint32_t o[4];
  uint32_t w[4];
};

// TAIL false: the row holds a multiple of 8 logits and every vector streamed
// lies inside it, so no vector needs masking.  V: logits the row holds (a
// draft row may hold fewer than the vocabulary).
template <bool TAIL = true>
__device__ __forceinline__ void vec8(const uint4& ld, int l, int k, int V, Vec8& v) {
  v.w[0] = ld.x;
  v.w[1] = ld.y;
  v.w[2] = ld.z;
  v.w[3] = ld.w;
  // A vector that reaches past the row's V logits (the row-end vector when V
  // is not a multiple of 8, and every vector of a draft row past a shorter
  // draft vocabulary): its elements from V on read as -inf (bf16 0xFF80).
  if (TAIL && (l + 1) * NT_F * VEC > V && k * VEC + VEC > V) {
    const int keep = max(V - k * VEC, 0) * 16;   // bits of the 128 that stay
    const uint64_t m0 = keep >= 64 ? ~0ull : (1ull << keep) - 1ull;
    const uint64_t m1 = keep <= 64 ? 0ull : (1ull << (keep - 64)) - 1ull;
    const uint64_t inf4 = 0xFF80FF80FF80FF80ull;
    const uint64_t lo = (((uint64_t)v.w[1] << 32 | v.w[0]) & m0) | (inf4 & ~m0);
    const uint64_t hi = (((uint64_t)v.w[3] << 32 | v.w[2]) & m1) | (inf4 & ~m1);
    v.w[0] = (uint32_t)lo;
    v.w[1] = (uint32_t)(lo >> 32);
    v.w[2] = (uint32_t)hi;
    v.w[3] = (uint32_t)(hi >> 32);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v.z[2 * e] = __uint_as_float(v.w[e] << 16);
    v.z[2 * e + 1] = __uint_as_float(v.w[e] & 0xFFFF0000u);
    v.o[e] = ord16x2(v.w[e]);
  }
}

// Penalty bits of the 8 logits of vector k.
__device__ __forceinline__ uint32_t pen_bits8(const uint32_t* bm, int k) {
  const int b = k * VEC;
  return (bm[b >> 5] >> (b & 31)) & 0xFFu;
}

__device__ __forceinline__ float max8(const float (&z)[VEC]) {
  return fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])),
               fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
}

// Per-lane running state of one row's stream.
struct RowAcc {
  uint32_t mo;     // packed 16-bit orderable keys: max of the logits as read
  uint32_t lo;     // and their min (a key below that of -inf is a NaN)
  float mpen;      // max of the penalized keys (after the stream)
  double Z;        // the penalty's changes to the normalizer (sum of exp2(key c - anchor c))
};

typedef __attribute__((address_space(3))) uint32_t lds_u32;

// LDS byte address of a shared array.
__device__ __forceinline__ uint32_t lds_addr(const uint32_t* p) {
  return (uint32_t)(size_t)(const lds_u32*)p;
}

// 4 * (16-bit half of a): the byte offset of a histogram word from its bin.
__device__ __forceinline__ uint32_t bin_addr_lo(uint32_t a) {
  uint32_t d;
  asm("v_mad_u32_u16 %0, %1, 4, 0" : "=v"(d) : "v"(a));
  return d;
}
__device__ __forceinline__ uint32_t bin_addr_hi(uint32_t a) {
  uint32_t d;
  asm("v_mad_u32_u16 %0, %1, 4, 0 op_sel:[1,0,0,0]" : "=v"(d) : "v"(a));
  return d;
}

// The key histogram of a row.  A logit's distance below the window's top,
// d = t1 - (its 16-bit orderable key), picks its bin: d < RUP, bin d (one
// bf16 key each: bins 1..254 are the window's codes, bin 0 the keys above
// it, whose counts are not used); then one lumped bin for the band of keys
// of magnitude below 2^-20 that the upper range does not reach (d in
// [RUP, R2)); then RNEG bins of one key each (d in [R2, R3)); then one
// bin for everything below (d >= R3, -inf included).  The row's normalizer
// is the sum over bins of count x the bin's term, so the stream takes no
// exponential per logit; the two lumped bins carry an error bound that the
// cut checks.
struct Bins {
  uint32_t r3x2, wx2;   // packed R3 and R2 - RUP - 1 (the band's width less one)
  int r2, r3;
};

__device__ __forceinline__ Bins row_bins(uint32_t t1) {
  Bins b;
  const int dneg = (int)t1 - (int)ord16f(-0x1p-20f);   // d of the key -2^-20
  b.r2 = max(RUP + 1, dneg + 1);
  b.r3 = min(b.r2 + RNEG, 0xFFFF);
  b.r3x2 = (uint32_t)b.r3 * 0x00010001u;
  b.wx2 = (uint32_t)(b.r2 - RUP - 1) * 0x00010001u;
  return b;
}

// Bins of two logits from their packed distances d.
__device__ __forceinline__ uint32_t bins_of(uint32_t d, const Bins& b) {
  const u16x2 dv = as_u16x2(d);
  const u16x2 m1 = __builtin_elementwise_min(dv, as_u16x2(b.r3x2));
  const u16x2 m2 = __builtin_elementwise_min(
      __builtin_elementwise_sub_sat(dv, (u16x2){(uint16_t)RUP, (uint16_t)RUP}), as_u16x2(b.wx2));
  return as_u32(m1 - m2);
}

// Distance below the window's top (t1 - key) of bin i, or -1 for the two
// lumped bins and unused bins.
__device__ __forceinline__ int bin_dist(int i, const Bins& b) {
  if (i < RUP) return i;
  if (i == RUP) return -1;
  const int d = b.r2 + (i - RUP - 1);
  return d < b.r3 ? d : -1;
}

// Streaming work of one vector of a row against its window: max, codes,
// key histogram, exact entries for keys above the window.  Every logit is
// streamed as read; pen_fix settles the penalized ones afterwards.
// Returns the two code words: the codes of the even elements 0, 2, 4, 6
// and of the odd ones 1, 3, 5, 7 (one byte each, in that order).
// SAMPLED: the vector is in one of the rounds whose block max set the
// anchor, so no finite key of it is above the window.
template <bool SAMPLED = false>
__device__ __forceinline__ uint2 row_vec(Vec8& v, int k, uint32_t t1, const Bins& bn,
                                         uint32_t* hist, const ExactList& ex, RowAcc& acc) {
  const uint32_t t1x2 = t1 | (t1 << 16);
  typedef __attribute__((address_space(3))) char lds_char;
  lds_char* const hb = (lds_char*)(lds_u32*)hist;
  uint32_t cc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // distance, code and bin of the pair, its two counts out at once (each
    // pair's temporaries die before the next pair's are made)
    const uint32_t dd = as_u32(__builtin_elementwise_sub_sat(as_u16x2(t1x2), as_u16x2(v.o[e])));
    cc[e] = as_u32(__builtin_elementwise_min(as_u16x2(dd), (u16x2){255, 255}));
    const uint32_t bb = bins_of(dd, bn);
    __hip_atomic_fetch_add((lds_u32*)(hb + bin_addr_lo(bb)), 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_fetch_add((lds_u32*)(hb + bin_addr_hi(bb)), 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
    SDV_PIN(cc[e]);
  }
  acc.lo = as_u32(__builtin_elementwise_min(
      as_u16x2(acc.lo),
      __builtin_elementwise_min(__builtin_elementwise_min(as_u16x2(v.o[0]), as_u16x2(v.o[1])),
                                __builtin_elementwise_min(as_u16x2(v.o[2]), as_u16x2(v.o[3])))));
  const uint32_t vo = pk_max(pk_max(v.o[0], v.o[1]), pk_max(v.o[2], v.o[3]));
  acc.mo = pk_max(acc.mo, vo);
  if (!SAMPLED &&
      as_u32(__builtin_elementwise_sub_sat(as_u16x2(vo), as_u16x2(t1x2 - 0x00010001u))) != 0u) {
    // Keys above the window (code 0) become exact entries.  Bit 2h + 16i of
    // am is logit 2h + i (a zero 16-bit code half; codes are at most 255).
    uint32_t am = 0u;
#pragma unroll
    for (int h = 0; h < 4; ++h) am |= ((~(cc[h] + 0x7FFF7FFFu) & 0x80008000u) >> 15) << (2 * h);
    while (am) {
      const int p = __builtin_ctz(am);
      am &= am - 1u;
      const int h = (p & 15) >> 1, i = p >> 4;
      const uint32_t wd = h == 0 ? v.w[0] : h == 1 ? v.w[1] : h == 2 ? v.w[2] : v.w[3];
      const uint32_t raw = (wd >> (16 * i)) & 0xFFFFu;
      exact_push(ex, __uint_as_float(raw << 16), k * VEC + 2 * h + i, raw);
    }
  }
  const uint32_t t01 = (cc[1] << 8) | cc[0];   // bytes: codes 0 2 1 3
  const uint32_t t23 = (cc[3] << 8) | cc[2];   // bytes: codes 4 6 5 7
  return make_uint2(__builtin_amdgcn_perm(t23, t01, 0x05040100u),
                    __builtin_amdgcn_perm(t23, t01, 0x07060302u));
}

// After a stream, for one distinct penalized token (id, raw bits as read):
// it leaves its count bin (it was counted under its raw key: hneg counts
// the departures), and if its
// penalized key reaches the window it becomes an entry of the penalty
// region; the normalizer trades the raw term for the penalized one.
__device__ __forceinline__ void pen_fix(uint32_t raw, int id, uint32_t t1, float rep, float c,
                                        float gc, uint32_t* hneg, const ExactList& ex,
                                        RowAcc& acc) {
  const uint32_t o = raw ^ ((raw & 0x8000u) ? 0xFFFFu : 0x8000u);   // as ord16x2
  const uint32_t cr = o >= t1 ? 0u : (t1 - o > 255u ? 255u : t1 - o);
  if (cr >= 1u && cr <= 254u) atomicAdd(&hneg[cr], 1u);
  const float z = __uint_as_float(raw << 16);
  const float zp = penalize(z, rep);
  if (code1(t1, zp) < 255u) pen_push(ex, zp, id, raw);
  acc.Z += (double)fast_exp2(fmaf(zp, c, -gc)) - (double)fast_exp2(fmaf(z, c, -gc));
  acc.mpen = fmaxf(acc.mpen, zp);
}

// Largest processed key of a lane's stream (+inf when the lane read a NaN
// of either sign, whose orderable keys lie beyond those of +-inf: the
// normalizer check then fails).
__device__ __forceinline__ float row_max(const RowAcc& acc) {
  const uint32_t o = max(acc.mo & 0xFFFFu, acc.mo >> 16);
  const uint32_t lo = min(acc.lo & 0xFFFFu, acc.lo >> 16);
  return (lo < 0x007Fu || o > 0xFF80u) ? INFINITY : fmaxf(key_of_ord16(o), acc.mpen);
}

__device__ __forceinline__ RowAcc row_acc_init() {
  RowAcc r;
  r.mo = 0x007F007Fu;   // orderable key of -inf
  r.lo = 0xFFFFFFFFu;
  r.mpen = -INFINITY;
  r.Z = 0.0;
  return r;
}

// Term of a key: exp2(key c - anchor c) as the stream's normalizer takes it.
__device__ __forceinline__ float key_term(float key, float c, float gc) {
  return fast_exp2(fmaf(key, c, -gc));
}

// Worker wk's share (of nwk workers) of a row's normalizer from its key
// histogram (bin groups 4g .. 4g + 3 for g = wk, wk + nwk, ..., the lumped
// bins excepted) and from the stream's exact entries (keys above the
// window; bin 0's count is not used).
__device__ __forceinline__ double hist_z(const uint32_t* hist, const Bins& bn, uint32_t t1, float c,
                                         float gc, const ExactList& ex, int ns, int wk, int nwk) {
  // (fp32 within a thread: a few terms, each count x term with a relative
  // error of a few ulp, as the stream's own per-round sums were)
  float z = 0.0f;
  // (a loop, not unrolled: the stream's codes and the draft ring are live here)
#pragma unroll 1
  for (int g = wk; g < NBINW / 4; g += nwk) {
    const int i0 = 4 * g;
    const uint4 h4 = reinterpret_cast<const uint4*>(hist)[g];
    const uint32_t hv[4] = {h4.x, h4.y, h4.z, h4.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = bin_dist(i0 + q, bn);
      if (hv[q] != 0u && d > 0 && d <= (int)t1)   // (a wave whose bins are all empty skips)
        z = fmaf((float)hv[q], key_term(key_of_ord16(t1 - (uint32_t)d), c, gc), z);
    }
  }
  double zd = (double)z;
  for (int i = wk; i < min(ns, E_CAP); i += nwk) zd += (double)key_term(ex.key[i], c, gc);
  return zd;
}

// The lumped bins' share of the normalizer: each at the middle of its range
// of terms; *err bounds the error (half that range times the count).
__device__ __forceinline__ double lumped_z(const uint32_t* hist, const Bins& bn, uint32_t t1, float c,
                                           float gc, double* err) {
  const int bottom = RUP + 1 + (bn.r3 - bn.r2);
  const double nb = (double)hist[RUP], nbot = (double)hist[bottom];
  double z = 0.0, e = 0.0;
  if (nb > 0.0) {
    const double th = (double)key_term(key_of_ord16(t1 - (uint32_t)RUP), c, gc);
    const double tl = (double)key_term(key_of_ord16(t1 - (uint32_t)min(bn.r2 - 1, (int)t1)), c, gc);
    z += nb * 0.5 * (th + tl);
    e += nb * 0.5 * fabs(th - tl);
  }
  if (nbot > 0.0) {
    const double tb = bn.r3 <= (int)t1 ? (double)key_term(key_of_ord16(t1 - (uint32_t)bn.r3), c, gc) : 0.0;
    z += nbot * 0.5 * tb;
    e += nbot * 0.5 * tb;
  }
  *err = e;
  return z;
}

// A row as a buffer resource of `bytes` bytes: loads past the end return 0
// and touch no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

// Load G of the ring: target round G (G < NR) or draft round G - NR, at the
// thread's byte offset voff.  Lanes past the row end, and every draft load
// of a bonus unit (an empty resource), read zeros without a memory access.
// The rows are read once: the loads are marked non-temporal.
template <int G>
__device__ __forceinline__ uint4 ring_load(__amdgpu_buffer_rsrc_t rt, __amdgpu_buffer_rsrc_t rd,
                                           uint32_t voff) {
  constexpr bool drf = G >= NR;
  constexpr int round = drf ? G - NR : G;
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(drf ? rd : rt, voff, round * NT_F * 16, 2);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Penalty set of unit (r, j): the prior ids of request r, then the draft
// ids x_0 .. x_{j-1} (entries; an id may repeat, the set is their union).
struct PenSet {
  int p0, nprior, npre;
  bool on;
};

__device__ __forceinline__ PenSet pen_set(const Args& a, int r, int j) {
  PenSet ps;
  ps.p0 = 0;
  ps.nprior = 0;
  ps.npre = 0;
  if (a.rep != 1.0f) {
    if (a.prior && a.poff) {
      ps.p0 = a.poff[r];
      const int p1 = a.poff[r + 1];
      ps.nprior = p1 > ps.p0 ? p1 - ps.p0 : 0;
    }
    ps.npre = (a.flags & SD_PENALTY_PRIOR_ONLY) ? 0 : j;
  }
  ps.on = ps.nprior + ps.npre > 0;
  return ps;
}

// Entry `tid` of the penalty set, loaded in two parts by unconditional
// buffer loads (an entry past either list reads nothing): the caller picks
// with pen_pick once the loads are needed.
struct PenFirst {
  int prior, prefix;
};

__device__ __forceinline__ PenFirst pen_first(const Args& a, const PenSet& ps, int r, int tid) {
  const __amdgpu_buffer_rsrc_t rp = row_rsrc(a.prior ? a.prior + ps.p0 : nullptr, ps.nprior * 4);
  const __amdgpu_buffer_rsrc_t rx = row_rsrc(a.ids + (int64_t)r * a.K_max, ps.npre * 4);
  PenFirst f;
  f.prior = __builtin_amdgcn_raw_buffer_load_b32(rp, (uint32_t)tid * 4u, 0, 0);
  f.prefix = __builtin_amdgcn_raw_buffer_load_b32(rx, (uint32_t)(tid - ps.nprior) * 4u, 0, 0);
  return f;
}

__device__ __forceinline__ int pen_pick(const PenSet& ps, PenFirst f, int tid) {
  return tid < ps.nprior ? f.prior : tid < ps.nprior + ps.npre ? f.prefix : -1;
}

// Marks the set's ids in the bitmap (cleared before a barrier) and lists
// each distinct id once (plid; count *npl, more than PL_CAP overflow).
// Returns the list index of id0 if this thread listed it, else -1; the
// caller loads the logits of that id and stores them at plraw[index].  Ids
// listed from later entries get plraw = 0xFFFFFFFF (logits not loaded).
__device__ __forceinline__ int pen_claim(const Args& a, const PenSet& ps, int r, int V, int id0,
                                         uint32_t* bm, int* plid, uint32_t* plraw, int* npl,
                                         int tid) {
  int x0 = -1;
  auto claim = [&](int id, bool first) {
    if (id < 0 || id >= V) return;
    const uint32_t bit = 1u << (id & 31);
    if (atomicOr(&bm[id >> 5], bit) & bit) return;
    const int x = atomicAdd(npl, 1);
    if (x >= PL_CAP) return;
    plid[x] = id;
    if (first) x0 = x;
    else plraw[x] = 0xFFFFFFFFu;
  };
  claim(id0, true);
  const int n = ps.nprior + ps.npre;
  for (int e = tid + NT_F; e < n; e += NT_F)
    claim(e < ps.nprior ? a.prior[ps.p0 + e] : a.ids[(int64_t)r * a.K_max + (e - ps.nprior)], false);
  return x0;
}

// Files the target-nucleus candidates of round l (code words cw0, cw1 of
// the even and odd logits) in the lane's slots, in ascending logit order,
// one word each: draft logit bits (dv; 0 for a bonus row) in bits 0-15,
// the target code in bits 16-23, 8 l + logit in bits 24-31.  Slot (s, lane)
// is word s * NT_F + lane; past CAPT candidates the last slot is reused
// (the unit is then flagged: nslot > CAPT).
// raise: a penalty is active and below 1 (it raises penalized keys).
// LOW: cut_code < 127 when known at compile time (-1: at run time).
template <int LOW = -1>
__device__ __forceinline__ void file_round(int l, uint32_t cw0, uint32_t cw1, uint4 dv,
                                           bool has_d, uint32_t bits, uint32_t cut_code,
                                           bool raise, uint32_t* slots, int& nslot) {
  const int tid = threadIdx.x;
  // Candidates: code <= cut code (bit 4e <-> logit e).  Whether a
  // candidate is in the nucleus is settled when the slot is read.  The codes
  // are those of the logits as read: a penalty that lowers keys (r > 1)
  // cannot make a non-candidate a member, one that raises them can, so then
  // every penalized logit is a candidate.
  uint32_t m = (le_mask<LOW>(cw0, cut_code) >> 7) | (le_mask<LOW>(cw1, cut_code) >> 3);
  if (raise) m |= spread8(bits);
  if (!has_d) dv = make_uint4(0u, 0u, 0u, 0u);
  const uint64_t dlo = (uint64_t)dv.y << 32 | dv.x, dhi = (uint64_t)dv.w << 32 | dv.z;
  while (m) {
    const int p = __builtin_ctz(m);   // 4e: code byte e >> 1 of cw0 or cw1, draft half e of dv
    m &= m - 1u;
    const uint32_t cd = __builtin_amdgcn_ubfe((p & 4) ? cw1 : cw0, (uint32_t)(p & 24), 8u);
    const uint32_t q = (uint32_t)(((p & 16) ? dhi : dlo) >> ((p & 12) << 2)) & 0xFFFFu;
    slots[min(nslot, CAPT - 1) * NT_F + tid] = q | (cd << 16) | ((uint32_t)(l * VEC + (p >> 2)) << 24);
    ++nslot;
  }
}

// Marker for a slot whose target logit lies above or below the window (code
// 0 or 255): its bits are looked up in the row's exact list.
constexpr uint32_t SLOT_EXACT = 0xFFFFu;

// Target bf16 bits of window code cd (1..254) against anchor t1, or
// SLOT_EXACT for codes 0 and 255.
__device__ __forceinline__ uint32_t slot_praw(uint32_t cd, uint32_t t1) {
  const uint32_t o = t1 - cd;
  return (cd == 0u || cd == 255u) ? SLOT_EXACT : (o & 0x8000u) ? (o & 0x7FFFu) : (~o & 0xFFFFu);
}

// Two zero words that stand in for an absent per-request array, so that a
// block can issue all of its request loads at once.
__device__ int32_t g_zero_words[2];

struct ReqWords {
  uint64_t off;        // two words: the request's prior-id list bounds
  uint32_t k, t, x;    // K, T (bits), the draft token
  uint32_t tp, d;      // the request's top-p and TV budget (bits)
};

// The scalar loads issued back to back and awaited once (the compiler
// would otherwise wait for each before issuing the next): four, and the two
// per-request parameter words when PR.  Every pointer must address
// readable words.
template <bool PR>
__device__ __forceinline__ ReqWords request_words(const int32_t* po, const int32_t* pk,
                                                  const int32_t* pt, const int32_t* px,
                                                  const int32_t* ptp, const int32_t* pd) {
  ReqWords w;
  w.tp = w.d = 0u;
  if constexpr (!PR) {
    asm volatile(
        "s_load_dwordx2 %0, %4, 0x0\n\t"
        "s_load_dword %1, %5, 0x0\n\t"
        "s_load_dword %2, %6, 0x0\n\t"
        "s_load_dword %3, %7, 0x0\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&s"(w.off), "=&s"(w.k), "=&s"(w.t), "=&s"(w.x)
        : "s"(po), "s"(pk), "s"(pt), "s"(px));
    return w;
  }
  asm volatile(
      "s_load_dwordx2 %0, %6, 0x0\n\t"
      "s_load_dword %1, %7, 0x0\n\t"
      "s_load_dword %2, %8, 0x0\n\t"
      "s_load_dword %3, %9, 0x0\n\t"
      "s_load_dword %4, %10, 0x0\n\t"
      "s_load_dword %5, %11, 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(w.off), "=&s"(w.k), "=&s"(w.t), "=&s"(w.x), "=&s"(w.tp), "=&s"(w.d)
      : "s"(po), "s"(pk), "s"(pt), "s"(px), "s"(ptp), "s"(pd));
  return w;
}

// Exact multi-pass processing of a unit that the single pass could not settle
// (its cut lies outside the window, its nucleus overflows the slots, or a
// row is not finite), by the same workgroup right away: it re-reads the
// unit's rows with the general-path routines (row statistics with the
// radix-select cut, TV, decision, draw).  bm holds the unit's penalty
// bitmap when pen; ex is carved from the single pass's histogram and slot
// space, which is free by then.  Writes the unit's record with UO_SLOW |
// UO_FALLBACK and the reasons why.
// cpk / cqk: the single pass's settled cuts of the target / draft row (null:
// recompute), which a unit handed over for a slot overflow carries.
// TV of a bf16 pair from per-key tables (the exact route).  Every logit of
// the pair is a bf16 value, and p (or q) depends on the value alone unless
// the token is penalized, so p is tabulated for the TBL keys from the row
// max down (p_tbl[i] for the key of 16-bit order t1 - i, t1 the order of
// the row max), when the row's cut lies inside that range (every key below
// it is then cut, p = 0).  A penalized token's p is computed directly.
// The table entries are the direct values, so the sum is the direct pass's.
constexpr int TBL = 4096;

__device__ __forceinline__ bool tbl_fits(const RowStat& s) {
  return s.kord != KEEP_ALL && (int)(s.kord >> 16) > (int)ord16f(s.M) - (TBL - 2);
}

template <int NT>
__device__ __forceinline__ void build_tbl(const RowStat& s, float* tbl) {
  const uint32_t t1 = ord16f(s.M);
  const float is = (float)(1.0 / s.Zk);
  for (int i = threadIdx.x; i < TBL; i += NT) {
    const int o = (int)t1 - i;
    float v = 0.0f;
    if (o >= 0x0080 && i < TBL - 1) {   // (orders below -inf's hold no logit; the last entry stays 0)
      const float k = key_of_ord16((uint32_t)o);
      v = kept(s, ord_key(k)) ? e_rel(k, s.M, s.c) * is : 0.0f;
    }
    tbl[i] = v;
  }
}

template <int NT>
__device__ __forceinline__ double pair_tv_tbl(const Args& a, const char* trow, const char* drow,
                                              const RowStat& P, const RowStat& Q, bool pen,
                                              const uint32_t* bm, const ExactLds& L, const float* tp,
                                              const float* tq) {
  const int V = a.V, nvec = (V + VEC - 1) / VEC;
  const float ip = (float)(1.0 / P.Zk), iq = (float)(1.0 / Q.Zk);
  const int t1p = (int)ord16f(P.M), t1q = (int)ord16f(Q.M);
  double acc = 0.0;
  const int tid = threadIdx.x;
  stream_steps<SD_BF16, NT, RU2, true>(
      trow, V, drow, a.Vd, nvec,
      [&](int base, int u) __attribute__((always_inline)) { return base + u * NT + tid; },
      [&](int base, float (&zp)[RU2][VEC], float (&zq)[RU2][VEC]) __attribute__((always_inline)) {
        float s = 0.0f;
#pragma unroll
        for (int u = 0; u < RU2; ++u) {
          const int k = base + u * NT + tid;
          if (k >= nvec) continue;
          const uint32_t bits = pen ? (bm[(k * VEC) >> 5] >> ((k * VEC) & 31)) & 0xFFu : 0u;
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const int id = k * VEC + e;
            float p, q;
            if (bits & (1u << e)) {   // penalized: direct
              const float kp = penalize(zp[u][e], a.rep), kq = penalize(zq[u][e], a.rep);
              p = id < V && kept(P, ord_key(kp)) ? e_rel(kp, P.M, P.c) * ip : 0.0f;
              q = id < a.Vd && kept(Q, ord_key(kq)) ? e_rel(kq, Q.M, Q.c) * iq : 0.0f;
            } else {
              p = tp[min(max(t1p - (int)ord16f(zp[u][e]), 0), TBL - 1)];
              q = tq[min(max(t1q - (int)ord16f(zq[u][e]), 0), TBL - 1)];
            }
            s += fabsf(p - q);
          }
        }
        acc += (double)s;
      });
  return fmin(0.5 * block_sum<NT>(acc, L.sd), 1.0);
}

template <int NT>
__device__ __forceinline__ void exact_unit(const Args& a, UnitOut* uo, int u, const uint32_t* bm,
                                        const ExactLds& ex, uint32_t why, const CutRes* cpk,
                                        const CutRes* cqk, const WideLds& wlp, const WideLds& wlq) {
  const int tid = threadIdx.x;
  __shared__ int s_acc;
  // (the unit's request values are derived again here, so that none of
  // them is held through the single pass for this route's sake)
  const Unit un = unit_of(a, u);
  const int r = un.r;
  const bool bonus = un.bonus;
  const int j = bonus ? request_k(a, r) : un.j;
  const float T = request_t(a, r);
  const PenSet ps = pen_set(a, r, j);
  const bool pen = ps.on;
  float u_j, v_j;
  uniforms(a.seed, a.offset, r, j, u_j, v_j);
  const float c = 1.4426950408889634f / T;
  const char* trow = target_row(a, r, j);
  const char* drow = bonus ? trow : draft_row(a, r, j);
  UnitOut out;
  out.d = out.th = out.px = out.qx = out.pix = out.S = 0.0f;
  out.u = u_j;
  out.v = v_j;
  out.accept = 1;
  out.y = -1;
  out.flags = UO_SLOW | UO_FALLBACK;
  out.why = why;
  const float tpr = request_top_p(a, r);
  auto from_cut = [&](const CutRes& k) {
    RowStat s;
    s.M = k.M;
    s.c = c;
    s.Zk = k.zk;
    s.kord = ord_key(k.key);
    s.idcut = INT_MAX;
    s.flags = 0;
    s.kx = 0.0f;
    return s;
  };
  // Cuts over a row's whole key histogram (their scratch is in the space
  // the exact passes use: they run first), the target's before the draft's.
  if (why & FB_P_CUT) {
    const float M = wlp.cut->M;
    const Cut w = wide_cut<false>(wlp, trow, a.V, bm, pen, a.rep, M, c);
    if (w.ok && tid == 0) *wlp.cut = CutRes{1, w.code, w.key, M, w.zk};
    __syncthreads();
    if (w.ok) {
      cpk = wlp.cut;
      out.why |= FB_WIDE;
    }
  }
  if ((why & FB_Q_CUT) && !bonus) {
    const float M = wlq.cut->M;
    const Cut w = wide_cut<true>(wlq, drow, a.Vd, bm, pen, a.rep, M, c);
    if (w.ok && tid == 0) *wlq.cut = CutRes{1, w.code, w.key, M, w.zk};
    __syncthreads();
    if (w.ok) {
      cqk = wlq.cut;
      out.why |= FB_WIDE_Q;
    }
  }
  const RowStat P = cpk ? from_cut(*cpk) : row_stats_dev<SD_BF16, NT>(a, trow, a.V, c, pen, bm, ex, tpr);
  if (P.flags & NONFINITE) {
    if (tid == 0) {
      out.flags = UO_NONFINITE | UO_FALLBACK;
      out.accept = 0;
      uo[u] = out;
    }
    return;
  }
  if (bonus) {
    const Drawn dw = draw_dev<SD_BF16, NT>(a, trow, trow, P, P, 1, v_j, pen, bm, ex);
    if (tid == 0) {
      out.y = dw.y;
      out.S = (float)dw.S;
      uo[u] = out;
    }
    return;
  }
  const RowStat Q = cqk ? from_cut(*cqk) : row_stats_dev<SD_BF16, NT>(a, drow, a.Vd, c, pen, bm, ex, tpr);
  if (Q.flags & NONFINITE) {
    if (tid == 0) {
      out.flags = UO_NONFINITE | UO_FALLBACK;
      out.accept = 0;
      uo[u] = out;
    }
    return;
  }
  double d;
  if (tbl_fits(P) && tbl_fits(Q)) {
    // (the tables take the radix passes' histogram space, free by now)
    float* tp = reinterpret_cast<float*>(ex.hmass);
    build_tbl<NT>(P, tp);
    build_tbl<NT>(Q, tp + TBL);
    __syncthreads();
    d = pair_tv_tbl<NT>(a, trow, drow, P, Q, pen, bm, ex, tp, tp + TBL);
  } else {
    d = pair_tv_dev<SD_BF16, NT>(a, trow, drow, P, Q, pen, bm, ex);
  }
  if (tid == 0) {
    const int x = a.ids[(int64_t)r * a.K_max + j];
    float kxp = -INFINITY, kxq = -INFINITY;
    if (x >= 0 && x < a.V) {
      kxp = load1<SD_BF16>(trow, x);
      kxq = x < a.Vd ? load1<SD_BF16>(drow, x) : -INFINITY;
      if (pen && ((bm[x >> 5] >> (x & 31)) & 1u)) {
        kxp = penalize(kxp, a.rep);
        kxq = penalize(kxq, a.rep);
      }
    }
    const Decision dc = decide(P, Q, kxp, kxq, (double)T, (double)request_D(a, r), true, d, u_j);
    out.d = (float)d;
    out.th = (float)dc.th;
    out.px = (float)dc.px;
    out.qx = (float)dc.qx;
    out.pix = (float)dc.pix;
    out.accept = dc.accept ? 1 : 0;
    if (dc.qx == 0.0) out.flags |= UO_QZERO;
    s_acc = out.accept;
  }
  __syncthreads();
  if (!s_acc) {
    const Drawn dw = draw_dev<SD_BF16, NT>(a, trow, drow, P, Q, 0, v_j, pen, bm, ex);
    if (tid == 0) {
      out.y = dw.y;
      out.S = (float)dw.S;
      if (dw.resid_zero) out.flags |= UO_RESID_ZERO;
    }
  }
  if (tid == 0) uo[u] = out;
}

// PR: per-request top-p / TV budget arrays are given (else the host-checked
// scalars apply to every request).
template <bool PR>
__global__ __launch_bounds__(NT_F) void k_pair_fast(Args a, UnitOut* uo) {
  constexpr int NT = NT_F;
  __shared__ uint32_t bm[MAXV_FAST / 32];
  // The draft row's key histogram and the nucleus slots.  The target row's
  // histogram lives in the slots' space: it is read for the last time by the
  // target cut, and the slots are filed after it.
  struct HistSlots {
    uint32_t histq[NBINW];
    uint32_t slot_arr[CAPT * NT];   // slot (s, lane) at s * NT + lane (file_round)
  };
  static_assert(CAPT * NT >= NBINW, "the target histogram shares the slots' space");
  __shared__ __align__(16) HistSlots hsl;
  auto& slot_arr = hsl.slot_arr;
  __shared__ float ekey[2][E_CAP];
  __shared__ int32_t eid[2][E_CAP];
  __shared__ uint16_t eraw[2][E_CAP];
  __shared__ uint32_t ecnt[NBIN];
  __shared__ uint64_t emass[NBIN];
  __shared__ __align__(16) uint32_t hneg[NBIN];   // penalized logits that left a bin
  __shared__ double cxs[WAVE];                   // the window cut's per-lane scan
  __shared__ float rkey[R_CAP];
  __shared__ double rmass[R_CAP];
  __shared__ int rid[R_CAP];
  __shared__ double sd[NT / WAVE];
  __shared__ double scanw[NT / WAVE];   // draw: per-wave scan totals
  __shared__ unsigned long long rtf[NR + 1];   // draw: per-round weight totals (fixed point)
  __shared__ float sf[NT / WAVE];
  __shared__ int si[NT / WAVE + 8];
  __shared__ int s_ne[2];
  __shared__ int s_acc;
  __shared__ int s_rcnt;
  __shared__ float red_f[4][NT / WAVE];    // per-wave partials, one row per reduction site
  __shared__ double red_d[3][NT / WAVE];
  __shared__ int red_i[2][NT / WAVE];
  __shared__ CutRes s_cut[2];
  __shared__ double s_tp[2];     // each cut's mass threshold and row anchor (for a wide cut)
  __shared__ uint32_t s_t1[2];
  __shared__ float pkey_arr[2][PE_CAP];
  __shared__ int32_t pid_arr[2][PE_CAP];
  __shared__ uint16_t praw_arr[2][PE_CAP];
  __shared__ int s_np[2];
  __shared__ int plid[PL_CAP];         // distinct penalized ids
  __shared__ uint32_t plraw[PL_CAP];    // their target | draft logits (bf16 bits)
  __shared__ int s_npl;
  __shared__ uint32_t s_kx;             // target | draft logit of the draft token (bf16 bits)
  __shared__ double s_xe[2];            // draft token: p(x_j); exp part of q(x_j)

  const int tid = threadIdx.x;
  const int lane = tid % WAVE, wv = tid / WAVE;
  const Unit un = unit_of(a, blockIdx.x);
  const int r = un.r;
  const bool bonus = un.bonus;
  // A pair's rows are known without any load, so its first loads go out
  // before the request checks (a unit that then turns out invalid exits
  // with them in flight; they read inside the rows either way).
  int j = un.j;
  if (bonus) j = min(max(request_k(a, r), 0), a.K_max);
  const int V = a.V, nvec = (V + VEC - 1) / VEC;
  const int Vd = a.Vd;   // the draft row's logits (ids Vd..V-1 have q = 0)
  const float rep = a.rep;
  const char* trow = target_row(a, r, j);
  const char* drow = bonus ? trow : draft_row(a, r, j);
  const __amdgpu_buffer_rsrc_t rs_t = row_rsrc(trow, nvec * 16);
  const __amdgpu_buffer_rsrc_t rs_d = row_rsrc(drow, bonus ? 0 : (Vd + VEC - 1) / VEC * 16);
  const uint32_t voff = (uint32_t)tid * 16u;
  ExactList exp_, exq;
  exp_.key = ekey[0];
  exp_.id = eid[0];
  exp_.raw = eraw[0];
  exp_.n = &s_ne[0];
  exp_.pkey = pkey_arr[0];
  exp_.pid = pid_arr[0];
  exp_.praw = praw_arr[0];
  exp_.np = &s_np[0];
  exq.key = ekey[1];
  exq.id = eid[1];
  exq.raw = eraw[1];
  exq.n = &s_ne[1];
  exq.pkey = pkey_arr[1];
  exq.pid = pid_arr[1];
  exq.praw = praw_arr[1];
  exq.np = &s_np[1];
  uint32_t* hist = hsl.slot_arr;
  uint32_t* histq = hsl.histq;
  // One load ring over the target row (rounds 0..NR-1) and the draft row
  // (rounds NR..2NR-1): NSTG loads in flight per thread throughout.  Then
  // the penalty set's first entries.
  uint4 stg[NSTG];
  static_for<NSTG>([&]<int s>() __attribute__((always_inline)) {
    stg[s] = ring_load<s>(rs_t, rs_d, voff);
  });
  __builtin_amdgcn_sched_barrier(0);   // the ring's loads go out first
  if (tid == 0) {
    s_ne[0] = 0;
    s_ne[1] = 0;
    s_np[0] = 0;
    s_np[1] = 0;
    s_npl = 0;
  }
  for (int i = tid; i < NBINW; i += NT) {   // both rows' histograms
    hist[i] = 0u;
    histq[i] = 0u;
  }
  if (tid < NBIN) {
    hneg[tid] = 0u;
    ecnt[tid] = 0u;
    emass[tid] = 0ull;
  }
  float u_j, v_j;
  uniforms(a.seed, a.offset, r, j, u_j, v_j);
  // The request's words in one round trip: the prior-id list bounds, the
  // draft token x_j, K, T, top-p and the TV budget (an absent array, and
  // the draft token of a bonus unit, read a zero word instead, which is then
  // not used).
  const bool pen_prior = a.rep != 1.0f && a.prior && a.poff;
  const ReqWords rw = request_words<PR>(pen_prior ? a.poff + r : g_zero_words,
                                    a.kpr ? a.kpr + r : g_zero_words,
                                    a.temp ? reinterpret_cast<const int32_t*>(a.temp + r) : g_zero_words,
                                    bonus ? g_zero_words : a.ids + (int64_t)r * a.K_max + j,
                                    PR && a.tpr ? reinterpret_cast<const int32_t*>(a.tpr + r) : g_zero_words,
                                    PR && a.dpr ? reinterpret_cast<const int32_t*>(a.dpr + r) : g_zero_words);
  const int K = a.kpr ? (int)rw.k : a.K_max;
  const float T = a.temp ? __uint_as_float(rw.t) : 1.0f;
  const float top_p = PR && a.tpr ? __uint_as_float(rw.tp) : a.top_p;
  const float Dr = PR && a.dpr ? __uint_as_float(rw.d) : a.D;
  if (K < 0 || K > a.K_max || (bonus ? j != K : j >= K) || !(T > 0.0f) || !(T < INFINITY) ||
      (PR && !params_ok(top_p, Dr)))
    return;
  const double tp = (double)top_p;
  const float c = 1.4426950408889634f / T;
  const int po0 = (int)(uint32_t)rw.off, po1 = (int)(uint32_t)(rw.off >> 32);
  PenSet ps;
  ps.p0 = pen_prior ? po0 : 0;
  ps.nprior = pen_prior && po1 > po0 ? po1 - po0 : 0;
  ps.npre = a.rep != 1.0f && !(a.flags & SD_PENALTY_PRIOR_ONLY) ? j : 0;
  ps.on = ps.nprior + ps.npre > 0;
  const bool pen = ps.on;
  const PenFirst pf = pen_first(a, ps, r, tid);
  // The logits of the draft token x_j, for the accept test (thread 0).
  const int xtok = bonus ? -1 : (int)rw.x;
  const uint32_t xoff = (tid == 0 && xtok >= 0 && xtok < V) ? (uint32_t)xtok * 2u : 0x7FFFFFF0u;
  // (gathers load the aligned dword that holds the logit and pick it out
  // where it is used, so that no earlier instruction waits for them)
  const uint32_t gxp = __builtin_amdgcn_raw_buffer_load_b32(rs_t, xoff & ~3u, 0, 0);
  const uint32_t gxq = __builtin_amdgcn_raw_buffer_load_b32(rs_d, xoff & ~3u, 0, 0);
  if (pen)
    for (int w = tid; w < (V + 31) / 32; w += NT) bm[w] = 0u;
  // (the anchor's block max below is the barrier that orders these clears
  // before the penalty claim in the stream's first round)
  uint32_t oflags = 0, why = 0;

  // ---- phase A: the target row ----
  // Anchor: block max of the first NSAMP rounds; the window is the 254
  // bf16 keys from UP above it downwards.
  float m0 = -INFINITY;
  static_for<NSAMP>([&]<int l>() __attribute__((always_inline)) {
    const int k = l * NT + tid;
    if (k < nvec) {
      Vec8 v;
      vec8(stg[l], l, k, V, v);
      m0 = fmaxf(m0, max8(v.z));   // logits as read: the anchor is only a reference
    }
  });
  // (block-uniform values read from LDS: moved to scalar registers)
  const float Gp = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(bar_max<NT>(m0, red_f[0]))));
  const bool anchor_ok = Gp > -1e30f && Gp < INFINITY;
  const uint32_t t1p = anchor_ok ? min(ord16f(Gp) + UP, 0xFFFEu) + 1u : 0xFFFFu;
  const float gcp = anchor_ok ? Gp * c : 0.0f;
  const Bins binp = row_bins(t1p);

  uint32_t code[NR][2];
  RowAcc ap = row_acc_init();
  if (anchor_ok) ap.mo = ord16f(Gp) * 0x00010001u;   // the max of the sampled rounds
  int x0 = -1;          // this thread's penalty-list index (set in round 1)
  uint32_t gp = 0u, gq = 0u, goff = 0u;
  auto stream_a = [&]<bool TAIL>() __attribute__((always_inline)) {
  static_for<NR>([&]<int l>() __attribute__((always_inline)) {
    const uint4 ld = stg[l % NSTG];
    if constexpr (l == 0 || l == 6 || l == 12 || l == 17)   // lagging waves first
      __builtin_amdgcn_s_setprio(l == 0 ? 3 : l == 6 ? 2 : l == 12 ? 1 : 0);
    if constexpr (l == 1) {
      // Each distinct penalized id is listed once; the thread that listed it
      // loads its target and draft logits now (stored to the list a few
      // rounds later); they are settled after each stream.
      const int id0 = pen_pick(ps, pf, tid);
      x0 = pen ? pen_claim(a, ps, r, V, id0, bm, plid, plraw, &s_npl, tid) : -1;
      goff = x0 >= 0 ? (uint32_t)id0 * 2u : 0x7FFFFFF0u;
      gp = __builtin_amdgcn_raw_buffer_load_b32(rs_t, goff & ~3u, 0, 0);
      gq = __builtin_amdgcn_raw_buffer_load_b32(rs_d, goff & ~3u, 0, 0);
    }
    if constexpr (l == NSTG - 1) {   // loaded rounds ago
      const uint32_t sh = (xoff & 2u) * 8u;
      if (tid == 0) s_kx = __builtin_amdgcn_ubfe(gxp, sh, 16u) | (__builtin_amdgcn_ubfe(gxq, sh, 16u) << 16);
    }
    if constexpr (l == 8) {
      const uint32_t sh = (goff & 2u) * 8u;
      if (x0 >= 0) plraw[x0] = __builtin_amdgcn_ubfe(gp, sh, 16u) | (__builtin_amdgcn_ubfe(gq, sh, 16u) << 16);
    }
    const int k = l * NT + tid;
    // (codes of vectors past the row end are never read: every reader
    // checks k < nvec)
    if ((!TAIL && l < NR - 1) || k < nvec) {
      Vec8 v;
      vec8<TAIL>(ld, l, k, V, v);
      const uint2 cw = row_vec<(l < NSAMP)>(v, k, t1p, binp, hist, exp_, ap);
      code[l][0] = cw.x;
      code[l][1] = cw.y;
    }
    SDV_PIN(ap.mo);
    SDV_PIN(ap.lo);
    SDV_PIN(code[l][0]);
    SDV_PIN(code[l][1]);
    // The slot's next load (next target round, or a draft round) goes out
    // once this round's words are used, into the same registers.
    __builtin_amdgcn_sched_barrier(0);
    stg[l % NSTG] = ring_load<l + NSTG>(rs_t, rs_d, voff);
    __builtin_amdgcn_sched_barrier(0);   // keep later rounds' loads in their rounds
  });
  };
  // (instances by whether a vector needs masking)
  const bool tail = (V & 7) != 0 || V <= (NR - 1) * NT_F * VEC;
  if (tail) stream_a.template operator()<true>();
  else stream_a.template operator()<false>();
  __syncthreads();   // the target stream is done: histogram, stream entries, logit list
  const int npl = s_npl;
  if (npl <= PL_CAP)
    for (int i = tid; i < npl; i += NT) {
      const int id = plid[i];
      const uint32_t g = plraw[i];
      const uint32_t raw = g == 0xFFFFFFFFu ? reinterpret_cast<const uint16_t*>(trow)[id] : g & 0xFFFFu;
      pen_fix(raw, id, t1p, rep, c, gcp, hneg, exp_, ap);
    }
  {
    const float wm = wave_max(row_max(ap));
    if (lane == 0) red_f[1][wv] = wm;
  }
  __syncthreads();   // penalized logits settled; maxima
  // Wave 0 prepares the window cut (it needs the row max, not the
  // normalizer) while waves 1.. sum the normalizer from the histogram.
  float M = 0.0f;
  bool prep_ok = false;
  const int ne0 = s_ne[0], np0 = s_np[0];
  if (wv == 0) {
    M = red_f[1][0];
#pragma unroll
    for (int i = 1; i < NT / WAVE; ++i) M = fmaxf(M, red_f[1][i]);
    prep_ok = anchor_ok && M > -INFINITY && M < INFINITY && ne0 <= E_CAP && np0 <= PE_CAP && npl <= PL_CAP;
    if (prep_ok) {
      __builtin_amdgcn_s_setprio(3);
      wave_cut_prep(hist, hneg, exp_, ne0, np0, bm, pen, t1p, M, c, ecnt, emass, cxs);
      __builtin_amdgcn_s_setprio(0);
    }
  } else {
    ap.Z += hist_z(hist, binp, t1p, c, gcp, exp_, s_ne[0], tid - WAVE, NT - WAVE);
  }
  {
    // The draft's anchor rides along: the block max of its first NSAMP
    // rounds, which the ring already holds.
    float q0 = -INFINITY;
    if (!bonus) {
      static_for<NSAMP>([&]<int l>() __attribute__((always_inline)) {
        const int k = l * NT + tid;
        if (k < nvec) {
          Vec8 v;
          vec8(stg[(NR + l) % NSTG], l, k, Vd, v);
          q0 = fmaxf(q0, max8(v.z));
        }
      });
    }
    const float wq = wave_max(q0);
    const double wz = wave_sum(ap.Z);
    if (lane == 0) {
      red_f[2][wv] = wq;
      red_d[0][wv] = wz;
    }
  }
  __syncthreads();   // partials
  if (wv == 0) {
    double Zs = 0.0;
#pragma unroll
    for (int i = 0; i < NT / WAVE; ++i) Zs += red_d[0][i];
    double zerr;
    Zs += lumped_z(hist, binp, t1p, c, gcp, &zerr);
    // (the lumped bins may move the normalizer by at most 2^-24 of itself)
    const bool good = prep_ok && Zs > 0.0 && Zs < INFINITY && zerr <= 0x1p-24 * Zs;
    Cut cc;
    cc.ok = 0;
    cc.code = 0;
    cc.key = 0.0f;
    cc.zk = 0.0;
    double TP = 0.0;
    if (good) {
      const double Zp = Zs * exp2((double)gcp - (double)M * (double)c);
      TP = tp * Zp;
      cc = wave_cut_finish(hneg, ecnt, emass, cxs, exp_, ne0, np0, bm, pen, t1p, M, c, TP, rkey, rmass, rid,
                           &s_rcnt);
    }
    if (lane == 0) {
      s_cut[0] = CutRes{good ? (cc.ok ? 1 : -1) : 0, cc.code, cc.key, M, cc.zk};
      s_tp[0] = TP;
      s_t1[0] = t1p;
    }
  }
  __syncthreads();
  const CutRes cp = s_cut[0];
  const float Mp = cp.M;
  const int nep = s_ne[0], npp = s_np[0];
  // A target crossing below the window: the row's key histogram (in the
  // slots' space) is exact for RUP keys below the window's top, which most
  // such crossings reach.  The unit streams its draft row without filing
  // slots (the window's codes do not mark that nucleus), and the exact
  // route cuts both rows from their histograms.
  const bool pmiss = cp.ok == -1;
  if (cp.ok == 0 || (pmiss && bonus)) {
    oflags = UO_FALLBACK;
    why = pmiss ? FB_P_CUT : FB_P_STATE;
    goto write_out_flags;
  }
  {
  const float kp_cut = cp.key;
  const uint32_t cut_code = (uint32_t)cp.code;
  const double Zkp = cp.zk;
  const float ip = (float)(1.0 / Zkp);
  if (tid < NBIN) {   // first touched after the draft stream's closing barrier
    hneg[tid] = 0u;
    ecnt[tid] = 0u;
    emass[tid] = 0ull;
  }

  int nslot = 0;
  const bool raise = pen && rep < 1.0f;   // penalized keys rise: all are candidates
  // Processed keys of the draft token x_j in the target and draft rows.
  auto draft_keys = [&](float& kxp, float& kxq) {
    kxp = kxq = -INFINITY;
    if (xtok >= 0 && xtok < V) {
      kxp = __uint_as_float(s_kx << 16);
      kxq = xtok < Vd ? __uint_as_float(s_kx & 0xFFFF0000u) : -INFINITY;
      if (pen && ((bm[xtok >> 5] >> (xtok & 31)) & 1u)) {
        kxp = penalize(kxp, rep);
        kxq = penalize(kxq, rep);
      }
    }
  };

  // ---- phase B: the draft row (pairs) or the nucleus from the codes (bonus) ----
  float Mq = 0.0f, kq_cut = 0.0f, iq = 0.0f;
  double Zkq = 1.0;
  if (bonus) {
    static_for<NR>([&]<int l>() __attribute__((always_inline)) {
      const int k = l * NT + tid;
      if (k < nvec && ((code[l][0] & code[l][1]) != 0xFFFFFFFFu || cut_code >= 255u)) {
        const uint32_t bits = raise ? pen_bits8(bm, k) : 0u;
        file_round(l, code[l][0], code[l][1], make_uint4(0u, 0u, 0u, 0u), false, bits, cut_code,
                   raise, slot_arr, nslot);
      }
    });
  } else {
    float Gq = red_f[2][0];
#pragma unroll
    for (int i = 1; i < NT / WAVE; ++i) Gq = fmaxf(Gq, red_f[2][i]);
    Gq = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(Gq)));
    const bool anchor_q = Gq > -1e30f && Gq < INFINITY;
    const uint32_t t1q = anchor_q ? min(ord16f(Gq) + UP, 0xFFFEu) + 1u : 0xFFFFu;
    const float gcq = anchor_q ? Gq * c : 0.0f;
    const Bins binq = row_bins(t1q);
    RowAcc aq = row_acc_init();
    if (anchor_q) aq.mo = ord16f(Gq) * 0x00010001u;
    auto stream_b = [&]<int LOW, bool RAISE, bool TAIL, bool FILE = true>() __attribute__((always_inline)) {
    static_for<NR>([&]<int l>() __attribute__((always_inline)) {
      const uint4 ld = stg[(NR + l) % NSTG];
      if constexpr (l == 0 || l == 6 || l == 12 || l == 17)
        __builtin_amdgcn_s_setprio(l == 0 ? 3 : l == 6 ? 2 : l == 12 ? 1 : 0);
      const int k = l * NT + tid;
      if ((!TAIL && l < NR - 1) || k < nvec) {
        Vec8 v;
        vec8<TAIL>(ld, l, k, Vd, v);
        const uint32_t bits = RAISE ? pen_bits8(bm, k) : 0u;
        const uint4 dv = make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]);
        (void)row_vec<(l < NSAMP)>(v, k, t1q, binq, histq, exq, aq);
        if constexpr (FILE)
          file_round<LOW>(l, code[l][0], code[l][1], dv, true, bits, cut_code, RAISE, slot_arr, nslot);
      }
      SDV_PIN(aq.mo);
      SDV_PIN(aq.lo);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (l + NSTG < NR) stg[(NR + l) % NSTG] = ring_load<NR + l + NSTG>(rs_t, rs_d, voff);
      __builtin_amdgcn_sched_barrier(0);
    });
    };
    // (instances by the target cut's half of the code range, and by whether
    // penalized keys rise or a vector needs masking)
    const bool low = cut_code < 127u;
    const bool tail_d = (Vd & 7) != 0 || Vd < V || Vd <= (NR - 1) * NT_F * VEC;
    if (pmiss) stream_b.template operator()<-1, false, true, false>();
    else if (raise || tail_d) stream_b.template operator()<-1, true, true>();
    else if (low) stream_b.template operator()<1, false, false>();
    else stream_b.template operator()<0, false, false>();
    __syncthreads();   // the draft stream is done: histogram, stream entries
    if (npl <= PL_CAP)
      for (int i = tid; i < npl; i += NT) {
        const int id = plid[i];
        const uint32_t g = plraw[i];
        const uint32_t raw = id >= Vd ? 0xFF80u   // past a shorter draft row: -inf
                             : g == 0xFFFFFFFFu ? reinterpret_cast<const uint16_t*>(drow)[id] : g >> 16;
        pen_fix(raw, id, t1q, rep, c, gcq, hneg, exq, aq);
      }
    {
      const float wm = wave_max(row_max(aq));
      const int wo = __any(nslot > CAPT) ? 1 : 0;
      if (lane == 0) {
        red_f[3][wv] = wm;
        red_i[0][wv] = wo;
      }
    }
    __syncthreads();   // penalized logits settled; maxima
    // (as for the target row: wave 0 prepares the cut meanwhile)
    float Mq0 = 0.0f;
    bool prepq = false;
    const int ne1 = s_ne[1], np1 = s_np[1];
    if (wv == 0) {
      Mq0 = red_f[3][0];
#pragma unroll
      for (int i = 1; i < NT / WAVE; ++i) Mq0 = fmaxf(Mq0, red_f[3][i]);
      prepq = anchor_q && Mq0 > -INFINITY && Mq0 < INFINITY && ne1 <= E_CAP && np1 <= PE_CAP;
      if (prepq) {
        __builtin_amdgcn_s_setprio(3);
        wave_cut_prep(histq, hneg, exq, ne1, np1, bm, pen, t1q, Mq0, c, ecnt, emass, cxs);
        __builtin_amdgcn_s_setprio(0);
      }
    } else {
      aq.Z += hist_z(histq, binq, t1q, c, gcq, exq, s_ne[1], tid - WAVE, NT - WAVE);
    }
    {
      const double wz = wave_sum(aq.Z);
      if (lane == 0) red_d[1][wv] = wz;
    }
    __syncthreads();   // partials
    if (wv == 0) {
      const float M = Mq0;
      double Zs = 0.0;
      int over = 0;
#pragma unroll
      for (int i = 0; i < NT / WAVE; ++i) {
        Zs += red_d[1][i];
        over |= red_i[0][i];
      }
      double zerr;
      Zs += lumped_z(histq, binq, t1q, c, gcq, &zerr);
      const bool good = prepq && Zs > 0.0 && Zs < INFINITY && zerr <= 0x1p-24 * Zs;
      Cut cc;
      cc.ok = 0;
      cc.code = 0;
      cc.key = 0.0f;
      cc.zk = 0.0;
      double TPq = 0.0;
      if (good) {
        const double Zqa = Zs * exp2((double)gcq - (double)M * (double)c);
        TPq = tp * Zqa;
        cc = wave_cut_finish(hneg, ecnt, emass, cxs, exq, ne1, np1, bm, pen, t1q, M, c, TPq, rkey, rmass,
                             rid, &s_rcnt);
      }
      // (a slot overflow with both cuts settled hands those cuts to the exact route)
      const int okv = !good ? 0 : !cc.ok ? -1 : over ? -2 : 1;
      if (lane == 0) {
        s_cut[1] = CutRes{okv, cc.code, cc.key, M, cc.zk};
        s_tp[1] = TPq;
        s_t1[1] = t1q;
      }
    } else if (wv == 1 && lane < 2) {
      // Meanwhile the draft token's fp64 exponentials: lane 0 p(x_j) (the
      // target cut is known), lane 1 the draft's, which its normalizer and
      // cut complete later.
      float M = Mp;
      if (lane == 1) {
        M = red_f[3][0];
#pragma unroll
        for (int i = 1; i < NT / WAVE; ++i) M = fmaxf(M, red_f[3][i]);
      }
      float kxp, kxq;
      draft_keys(kxp, kxq);
      const float kx = lane == 0 ? kxp : kxq;
      const double e = exp(((double)kx - (double)M) / (double)T);
      RowStat P;
      P.kord = ord_key(kp_cut);
      s_xe[lane] = lane == 1 ? e : kept(P, ord_key(kx)) ? e / Zkp : 0.0;
    }
    __syncthreads();
    const CutRes cq = s_cut[1];
    if (cq.ok != 1 || pmiss) {
      oflags = UO_FALLBACK;
      why = (pmiss ? FB_P_CUT : 0u) |
            (cq.ok == 1 ? 0u : cq.ok == -2 ? FB_SLOTS : cq.ok == 0 ? FB_Q_STATE : FB_Q_CUT);
      goto write_out_flags;
    }
    Mq = cq.M;
    kq_cut = cq.key;
    Zkq = cq.zk;
    iq = (float)(1.0 / Zkq);
  }
  if (bonus) {
    const int wo = __any(nslot > CAPT) ? 1 : 0;
    if (lane == 0) red_i[1][wv] = wo;
    __syncthreads();
    int over = 0;
#pragma unroll
    for (int i = 0; i < NT / WAVE; ++i) over |= red_i[1][i];
    if (over) {
      oflags = UO_FALLBACK;
      why = FB_SLOTS;
      goto write_out_flags;
    }
  }

  // Keys of slot s of this lane (penalty re-applied from the bitmap); a
  // candidate outside the target nucleus gets zp = -inf (weight 0).
  auto slot_keys = [&](int sidx, float& zp, float& zq, int& id) {
    const uint32_t w = slot_arr[sidx];
    const uint32_t ps = w >> 24;
    id = ((int)(ps >> 3) * NT + tid) * VEC + (int)(ps & 7);
    uint32_t praw = slot_praw((w >> 16) & 0xFFu, t1p);
    if (praw == SLOT_EXACT) praw = exact_raw(exp_, nep, npp, id);   // none: below the window
    zp = praw == 0xFFFFFFFFu ? -INFINITY : __uint_as_float(praw << 16);
    zq = __uint_as_float(w << 16);
    if (pen && ((bm[id >> 5] >> (id & 31)) & 1u)) {
      zp = penalize(zp, rep);
      zq = penalize(zq, rep);
    }
    if (!(zp >= kp_cut)) zp = -INFINITY;
  };

  // ---- TV, p(x), q(x), theta, pi, acceptance ----
  UnitOut out;
  out.d = out.th = out.px = out.qx = out.pix = out.S = 0.0f;
  out.u = u_j;
  out.v = v_j;
  out.accept = 1;
  out.y = -1;
  out.flags = 0;
  out.why = 0;
  if (!bonus) {
    double acc = 0.0;
    for (int sl = 0; sl < nslot; ++sl) {
      float zp, zq;
      int id;
      slot_keys(sl * NT + tid, zp, zq, id);
      acc += (double)nucleus_w(zp, zq, 0, Mp, ip, kq_cut, Mq, iq, c);
    }
    acc = wave_sum(acc);
    if (lane == 0) red_d[2][wv] = acc;
    __syncthreads();
    if (tid == 0) {
      double d = 0.0;
#pragma unroll
      for (int i = 0; i < NT / WAVE; ++i) d += red_d[2][i];
      d = fmin(d, 1.0);
      float kxp, kxq;
      draft_keys(kxp, kxq);
      RowStat Q;
      Q.kord = ord_key(kq_cut);
      const double qx = kept(Q, ord_key(kxq)) ? s_xe[1] / Zkq : 0.0;   // as prob_at
      const Decision dc = decide_from(s_xe[0], qx, (double)Dr, true, d, u_j);
      out.d = (float)d;
      out.th = (float)dc.th;
      out.px = (float)dc.px;
      out.qx = (float)dc.qx;
      out.pix = (float)dc.pix;
      out.accept = dc.accept ? 1 : 0;
      if (dc.qx == 0.0) out.flags |= UO_QZERO;
      s_acc = out.accept;
      if (dc.accept) uo[blockIdx.x] = out;
    }
    __syncthreads();
    if (s_acc) return;
  }

  // ---- correction (rejected position) or bonus draw from the nucleus ----
  // Ascending token ids run over rounds l (ids [8192 l, 8192 l + 8192)), then
  // lanes, then the 8 logits of a lane; a lane's slots are in round order.
  // Weights are summed in 64-bit fixed point (SHD fractional bits): the
  // round totals by LDS atomics in any order, the crossing round by an exact
  // scan, so every comparison with t = v S is exact and order-free.
  int mode = bonus ? 1 : 0;
  uint64_t Sf = 0, tf = 0, Rf = 0;
  int lstar = -1;
  const uint64_t vk = (uint64_t)(v_j * 0x1p24f);   // v = vk 2^-24 exactly
  for (int pass = 0; pass < 2; ++pass) {
    if (tid <= NR) rtf[tid] = 0ull;
    __syncthreads();
    for (int sl = 0; sl < nslot; ++sl) {
      float zp, zq;
      int id;
      slot_keys(sl * NT + tid, zp, zq, id);
      const float w = nucleus_w(zp, zq, mode, Mp, ip, kq_cut, Mq, iq, c);
      if (w > 0.0f)
        atomicAdd(&rtf[slot_arr[sl * NT + tid] >> 27], (unsigned long long)e_fixed(w, SHD));
    }
    __syncthreads();
    Sf = 0;
    for (int l = 0; l < NR; ++l) Sf += rtf[l];
    tf = (__umul64hi(vk, Sf) << 40) | ((vk * Sf) >> 24);   // floor(v S), exact
    uint64_t accr = 0, alast = 0;
    int last = -1;
    lstar = -1;
    for (int l = 0; l < NR; ++l) {
      const uint64_t rl = rtf[l];
      if (rl > 0) { last = l; alast = accr; }
      if (lstar < 0 && accr + rl > tf) { lstar = l; Rf = accr; }
      accr += rl;
    }
    if (lstar < 0) { lstar = last; Rf = alast; }
    __syncthreads();   // the totals are read before a second pass clears them
    if (Sf == 0 && mode == 0) {
      mode = 1;
      oflags |= UO_RESID_ZERO;
      continue;
    }
    break;
  }
  {
    // round lstar: lane totals, block scan (integers below 2^53 held exactly
    // in doubles), then the crossing lane's logits
    uint64_t sf = 0;
    int first = -1, cnt = 0;
    for (int sl = 0; sl < nslot; ++sl) {
      if ((int)(slot_arr[sl * NT + tid] >> 27) != lstar) continue;
      if (first < 0) first = sl;
      ++cnt;
      float zp, zq;
      int id;
      slot_keys(sl * NT + tid, zp, zq, id);
      sf += e_fixed(nucleus_w(zp, zq, mode, Mp, ip, kq_cut, Mq, iq, c), SHD);
    }
    // block scan with one barrier (the per-wave totals have a buffer of
    // their own); the one thread whose inclusive total first exceeds t (its
    // exclusive total, the previous thread's inclusive, does not) claims
    // the crossing with a plain store
    if (tid == 0) { si[0] = INT_MAX; si[1] = -1; }
    double xs = wave_incl_scan((double)sf);
    if (lane == WAVE - 1) scanw[wv] = xs;
    __syncthreads();
    for (int i = 0; i < wv; ++i) xs += scanw[i];
    const uint64_t incl = (uint64_t)xs;
    if (lstar >= 0 && Rf + incl > tf && Rf + incl - sf <= tf) si[0] = tid;
    __syncthreads();
    if (tid == si[0]) {
      uint64_t C = Rf + incl - sf;
      int yy = -1, lastpos = -1;
      for (int q = 0; q < cnt && yy < 0; ++q) {
        float zp, zq;
        int id;
        slot_keys((first + q) * NT + tid, zp, zq, id);
        const uint64_t wf = e_fixed(nucleus_w(zp, zq, mode, Mp, ip, kq_cut, Mq, iq, c), SHD);
        if (wf > 0) lastpos = id;
        C += wf;
        if (C > tf) yy = id;
      }
      si[1] = yy >= 0 ? yy : lastpos;
    }
    __syncthreads();
    if (tid == 0) {
      out.y = si[1];
      out.S = (float)((double)Sf * 0x1p-40);
      out.flags |= oflags;
      uo[blockIdx.x] = out;
    }
    return;
  }
  }

write_out_flags:
  // The unit leaves the single pass (oflags holds UO_FALLBACK): the exact
  // route, in the histogram and slot space.
  {
    unsigned char* const fb = reinterpret_cast<unsigned char*>(&hsl);
    ExactLds ex;
    ex.hmass = reinterpret_cast<uint64_t*>(fb);
    ex.hcnt = reinterpret_cast<uint32_t*>(fb + HBINS * 8);
    ex.su = reinterpret_cast<uint64_t*>(fb + HBINS * 12);
    ex.sd = reinterpret_cast<double*>(fb + HBINS * 12 + NT * 8);
    ex.ctot = reinterpret_cast<double*>(fb + HBINS * 12 + NT * 16);
    ex.sf = sf;
    ex.si = si;
    static_assert(HBINS * 12 + NT_F * 16 + (MAXV_FAST / VEC / WAVE + 1) * 8 <= sizeof(HistSlots),
                  "exact route LDS");
    (void)oflags;
    // (the arguments are read again from the kernel's argument segment, where
    // the first parameter starts: held in registers from the kernel's start,
    // the fields only this route uses would crowd the streams)
#if __HIP_DEVICE_COMPILE__
    auto kseg = __builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(kseg));
    typedef __attribute__((address_space(4))) const Args KArgs;
    const Args ax = *(KArgs*)kseg;
#else
    const Args ax = a;   // (the host pass only parses device code)
#endif
    // Rows whose crossing lies below the window are cut from their whole
    // key histograms: the target's (in the slots' space, no slot filed),
    // then the draft's (with the slots' space for scratch).
    auto wide_lds = [&](bool is_t) __attribute__((always_inline)) {
      WideLds w;
      w.hist = is_t ? hsl.slot_arr : hsl.histq;
      w.ecnt4 = is_t ? hsl.slot_arr + NBINW + 2 * RUP : hsl.slot_arr;
      w.emass4 = reinterpret_cast<uint64_t*>(is_t ? hsl.slot_arr + NBINW : hsl.slot_arr + RUP);
      w.ex = is_t ? exp_ : exq;
      w.ns = s_ne[is_t ? 0 : 1];
      w.plid = plid;
      w.plraw = plraw;
      w.npl = s_npl;
      w.rkey = rkey;
      w.rmass = rmass;
      w.rid = rid;
      w.scnt = &s_rcnt;
      w.wtot = sd;
      w.TP = s_tp[is_t ? 0 : 1];
      w.t1 = s_t1[is_t ? 0 : 1];
      w.cut = &s_cut[is_t ? 0 : 1];
      return w;
    };
    static_assert(NBINW + 3 * RUP <= CAPT * NT, "wide-cut scratch");
    // The cuts the single pass settled go along: the target's unless its
    // state or cut failed, the draft's with a slot overflow or after a
    // target cut below the window.
    const bool p_set = !(why & (FB_P_STATE | FB_P_CUT));
    const bool q_set = !bonus && (why == FB_SLOTS || why == FB_P_CUT);
    exact_unit<NT>(ax, uo, blockIdx.x, bm, ex, why, p_set ? &s_cut[0] : nullptr, q_set ? &s_cut[1] : nullptr,
                   wide_lds(true), wide_lds(false));
  }
}

__global__ __launch_bounds__(64) void k_fast_finalize(Args a, const UnitOut* uo, int32_t* out_acc,
                                                      int32_t* out_tok, uint32_t* out_status,
                                                      float* out_stats) {
  constexpr int NT = 64;
  static_assert(NT == WAVE && SD_MAX_K + 1 <= NT, "one wave per request, one lane per position");
  __shared__ int si[NT / WAVE + 4];
  const int r = blockIdx.x;
  const int K1 = a.K_max + 1;
  const int K = request_k(a, r);
  const float T = request_t(a, r);
  uint32_t st = request_status<NT>(a, r, K, T, true, si);
  const int64_t bonus_idx = (int64_t)a.B * a.K_max + r;
  // Lane jj < K holds pair jj's record and draft token, lane K the bonus
  // row's record, all loaded at once; the first rejection is the first bit
  // of a ballot and the drawn token comes from its lane.  (Units of a
  // request with an invalidating bit may hold no record of this call:
  // k_pair_fast skips requests with a bad K, temperature or parameter.)
  const int jj = threadIdx.x;
  UnitOut o;
  o.d = o.th = o.px = o.qx = o.pix = o.u = o.v = o.S = 0.0f;
  o.accept = 1;
  o.y = -1;
  o.flags = o.why = 0u;
  int idv = -1;
  if (!(st & SD_ST_INVALID_MASK) && jj <= K) {
    o = uo[jj < K ? (int64_t)r * a.K_max + jj : bonus_idx];
    if (jj < K) idv = a.ids[(int64_t)r * a.K_max + jj];
  }
  if (block_or<NT>((o.flags & UO_NONFINITE) ? 1 : 0, si)) st |= SD_ST_NONFINITE;
  const int64_t base = (int64_t)r * K1;
  if (st & SD_ST_INVALID_MASK) {
    if (jj < K1) {
      out_tok[base + jj] = -1;
      if (out_stats)
        for (int s = 0; s < SD_NSTAT; ++s) out_stats[(base + jj) * SD_NSTAT + s] = 0.0f;
    }
    if (jj == 0) {
      out_acc[r] = -1;
      if (out_status) out_status[r] = st;
    }
    return;
  }
  if (__any(jj < K && (o.flags & UO_QZERO))) st |= SD_ST_Q_ZERO;
  const uint64_t rej = __ballot(jj < K && !o.accept);
  const int n = rej ? __builtin_ctzll(rej) : K;
  const int y = __shfl(o.y, n);
  const float S = __shfl(o.S, n);
  if (n < K && (__shfl((int)o.flags, n) & UO_RESID_ZERO)) st |= SD_ST_RESID_ZERO;
  const bool emit = !(n == K && (a.flags & SD_NO_BONUS));
  if (jj < K1) {
    out_tok[base + jj] = jj < n ? idv : (jj == n && emit) ? y : -1;
    if (out_stats) {
      float sv[SD_NSTAT];
#pragma unroll
      for (int s = 0; s < SD_NSTAT; ++s) sv[s] = 0.0f;
      if (jj < K) {
        sv[SD_STAT_D] = o.d;
        sv[SD_STAT_THETA] = o.th;
        sv[SD_STAT_PX] = o.px;
        sv[SD_STAT_QX] = o.qx;
        sv[SD_STAT_PIX] = o.pix;
      }
      if (jj <= K) {
        sv[SD_STAT_U] = o.u;
        sv[SD_STAT_V] = o.v;
      }
      if (jj == n && emit) sv[SD_STAT_S] = S;
#pragma unroll
      for (int s = 0; s < SD_NSTAT; ++s) out_stats[(base + jj) * SD_NSTAT + s] = sv[s];
    }
  }
  if (jj == 0) {
    out_acc[r] = n;
    if (out_status) out_status[r] = st;
  }
}

// ---------------------------------------------------------------------------
// Debug export of processed rows (general-path statistics).
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(NT_ROW) void k_debug_rows(Args a, const RowStat* rs, float* out_p,
                                                      float* out_q) {
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
    load8_row<DT>(row, k, is_t ? V : a.Vd, z);
    if (pen) apply_penalty8(bm, k, 0, a.rep, z);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int id = k * VEC + e;
      if (id < V) out[id] = kept(S, ord_key(z[e])) ? e_rel(z[e], S.M, S.c) * ip : 0.0f;
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
  const int k0 = lo / VEC, k1 = (hi + VEC - 1) / VEC;
  // every vector of the thread's share is requested at once, before the
  // penalty bitmap is built (buffer loads issued whatever the range; a
  // vector past the slice reads nothing), so the slice costs one memory
  // latency instead of one per vector
  constexpr int GU = G_SLICE / VEC / NT;
  const __amdgpu_buffer_rsrc_t rs = raw_rsrc<DT>(row, V);
  RawVec<DT> rv[GU];
#pragma unroll
  for (int u = 0; u < GU; ++u) {
    const int k = k0 + (int)threadIdx.x + u * NT;
    rv[u] = load_raw<DT>(rs, k, k < k1);
  }
  const bool pen = build_penalty_bitmap<NT>(a, r, j, lo, G_SLICE, bm);
  uint32_t bo = 0;
  int bi = INT_MAX, nan = 0;
#pragma unroll
  for (int u = 0; u < GU; ++u) {
    const int k = k0 + (int)threadIdx.x + u * NT;
    if (k >= k1) break;
    float z[VEC];
    unpack<DT>(rv[u], k, V, z);
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
  constexpr int NT = 64;
  static_assert(NT == WAVE && SD_MAX_K + 1 <= NT, "one wave per request, one lane per position");
  __shared__ int g[SD_MAX_K + 1];
  __shared__ int si[NT / WAVE + 4];
  const int r = blockIdx.x;
  const int K1 = a.K_max + 1;
  const int K = request_k(a, r);
  uint32_t st = request_status<NT>(a, r, K, 1.0f, false, si);
  // Lane jj <= K reduces position jj's slice partials (the order of the
  // reduction does not matter: larger key, then lower id) and compares the
  // argmax with the draft token it loaded beforehand; the first mismatch is
  // the first set bit of a ballot, so no lane waits on a chain of loads.
  const int jj = threadIdx.x;
  int nan = 0, mism = 0, idv = -1;
  if (!(st & SD_ST_INVALID_MASK) && jj <= K) {
    if (jj < K) idv = a.ids[(int64_t)r * a.K_max + jj];
    const GPart* pj = parts + ((int64_t)r * K1 + jj) * ns;
    uint32_t bo = 0;
    int bi = INT_MAX;
    int s = 0;
    for (; s + 4 <= ns; s += 4) {
      GPart p[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) p[u] = pj[s + u];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        nan |= (int)p[u].nan;
        if (better(p[u].ord, p[u].id, bo, bi)) { bo = p[u].ord; bi = p[u].id; }
      }
    }
    for (; s < ns; ++s) {
      const GPart p = pj[s];
      nan |= (int)p.nan;
      if (better(p.ord, p.id, bo, bi)) { bo = p.ord; bi = p.id; }
    }
    g[jj] = bi;
    mism = jj < K && idv != bi;
  }
  if (block_or<NT>(nan, si)) st |= SD_ST_NONFINITE;   // (its barrier also publishes g)
  const int64_t base = (int64_t)r * K1;
  if (st & SD_ST_INVALID_MASK) {
    if (jj < K1) {
      out_tok[base + jj] = -1;
      if (out_argmax) out_argmax[base + jj] = -1;
    }
    if (jj == 0) {
      out_acc[r] = -1;
      if (out_status) out_status[r] = st;
    }
    return;
  }
  const uint64_t mm = __ballot(mism != 0);
  const int n = mm ? __builtin_ctzll(mm) : K;
  if (jj < K1) {
    int v = -1;
    if (jj < n) v = idv;
    else if (jj == n && !(n == K && (a.flags & SD_NO_BONUS))) v = g[n];
    out_tok[base + jj] = v;
    if (out_argmax) out_argmax[base + jj] = (jj <= K) ? g[jj] : -1;
  }
  if (jj == 0) {
    out_acc[r] = n;
    if (out_status) out_status[r] = st;
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
struct Layout {
  size_t rs, dtv, gp, uo, drec, ctot, rpart, total;
  int ns;
  int tvS, drS, rowS;   // slices of the general path's TV, draw and row passes
};

Layout layout(const sd_verify_args_t* a) {
  Layout L;
  const size_t B = (size_t)a->B, K = (size_t)a->K_max;
  L.ns = (a->V + G_SLICE - 1) / G_SLICE;
  size_t off = 0;
  L.tvS = tv_slices(a->B, a->K_max, a->V);
  L.drS = draw_slices(a->B, a->V);
  L.rowS = row_slices(a->B, a->K_max, a->V, a->top_p_per_row != nullptr || a->top_p < 1.0f);
  L.rs = off;  off = align_up(off + B * (2 * K + 1) * sizeof(RowStat), 256);
  L.dtv = off; off = align_up(off + B * K * (size_t)L.tvS * sizeof(double), 256);
  L.drec = off; off = align_up(off + (L.drS > 1 ? B * sizeof(int2) : 0), 256);
  L.ctot = off; off = align_up(off + (L.drS > 1 ? B * 2 * (size_t)(draw_chunks(a->V) + 1) * sizeof(double) : 0), 256);
  L.rpart = off; off = align_up(off + (L.rowS > 1 ? B * (2 * K + 1) * L.rowS * sizeof(RowPart) : 0), 256);
  L.gp = off;  off = align_up(off + B * (K + 1) * (size_t)L.ns * sizeof(GPart), 256);
  L.uo = off;  off = align_up(off + B * (K + 1) * sizeof(UnitOut), 256);
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
  if (sample && (a->V_draft < 0 || a->V_draft > a->V)) return SD_EINVAL;
  const int64_t vd = a->V_draft > 0 ? a->V_draft : a->V;
  if (sample && a->K_max > 0 &&
      (!a->draft_logits || a->ld_draft < vd || (a->ld_draft * es) % 16 != 0 ||
       (reinterpret_cast<uintptr_t>(a->draft_logits) & 15u)))
    return SD_EINVAL;
  if (!(a->rep_penalty > 0.0f) || !(a->rep_penalty < INFINITY)) return SD_EINVAL;
  if (sample) {
    if (!a->top_p_per_row && (!(a->top_p > 0.0f) || !(a->top_p <= 1.0f))) return SD_EINVAL;
    if (!a->tv_budget_per_row && !(a->tv_budget >= 0.0f)) return SD_EINVAL;
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
  a.tpr = s->top_p_per_row;
  a.dpr = s->tv_budget_per_row;
  a.prior = s->prior_ids;
  a.poff = s->prior_offsets;
  a.seed = s->seed;
  a.offset = s->offset;
  a.flags = s->flags;
  a.fp_shift = 62 - ceil_log2(s->V);
  a.Vd = s->V_draft > 0 ? s->V_draft : s->V;
  return a;
}

int bitmap_words(int V) { return (V + 31) / 32; }

size_t row_lds(int V) { return align_up((size_t)bitmap_words(V) * 4, 16) + exact_lds(V, NT_ROW); }

size_t fin_lds(int V) {
  const int nch = ((V + VEC - 1) / VEC + WAVE - 1) / WAVE;   // the draw's 64-vector chunks
  return align_up((size_t)bitmap_words(V) * 4, 16) + (size_t)(nch + 1) * 8;
}

int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SD_OK : SD_EHIP;
}

// The single-pass kernel covers bf16 rows with top-p on and V <= 155648.
bool use_fast(const Args& a) {
  return a.dtype == SD_BF16 && (a.tpr || a.top_p < 1.0f) && a.V <= MAXV_FAST;
}

// LDS of the general row pass: the penalty bitmap only with a penalty, the
// radix-select histograms only when some request truncates (top-p < 1).
size_t prepare_lds(const Args& a) {
  const bool topp = a.tpr || a.top_p < 1.0f;
  const size_t bm = align_up((size_t)bitmap_words(a.V) * 4, 16);
  if (topp) return bm + exact_lds(a.V, NT_ROW);
  return a.rep != 1.0f ? bm : 0;
}

template <int DT>
int run_prepare(const Args& a, const Layout& L, char* ws, hipStream_t st) {
  const int grid = a.B * (2 * a.K_max + 1);
  if (L.rowS > 1) {
    RowPart* parts = reinterpret_cast<RowPart*>(ws + L.rpart);
    hipLaunchKernelGGL(k_row_part<DT>, dim3(grid * L.rowS), dim3(NT_ROW),
                       a.rep != 1.0f ? align_up((size_t)bitmap_words(a.V) * 4, 16) : 0, st, a, parts, L.rowS);
    hipLaunchKernelGGL(k_row_combine<DT>, dim3(grid), dim3(WAVE), 0, st, a, parts,
                       reinterpret_cast<RowStat*>(ws + L.rs), L.rowS);
    return launch_status();
  }
  const int bmw = (a.rep != 1.0f || a.tpr || a.top_p < 1.0f) ? bitmap_words(a.V) : 0;
  hipLaunchKernelGGL(k_row_prepare<DT>, dim3(grid), dim3(NT_ROW), prepare_lds(a), st, a,
                     reinterpret_cast<RowStat*>(ws + L.rs), bmw);
  return launch_status();
}

bool needs_tv(const Args& a, const float* stats) {
  return stats != nullptr || a.dpr != nullptr || (a.D > 0.0f && a.D < 1.0f);
}

// One phase of the sampling path.  Single-pass path: 0 = k_pair_fast (with
// the exact route of the units it cannot settle), 1 = no launch,
// 2 = k_fast_finalize.  General path: 0 = k_row_prepare, 1 = k_pair_tv (when
// needed), 2 = k_finalize.
template <int DT>
int run_phase(const Args& a, const Layout& L, char* ws, int phase, int32_t* acc, int32_t* tok,
              uint32_t* status, float* stats, hipStream_t st) {
  if (DT == SD_BF16 && use_fast(a)) {
    UnitOut* uo = reinterpret_cast<UnitOut*>(ws + L.uo);
    if (phase == 0) {
      if (a.tpr || a.dpr)
        hipLaunchKernelGGL(k_pair_fast<true>, dim3(a.B * a.K_max + a.B), dim3(NT_F), 0, st, a, uo);
      else
        hipLaunchKernelGGL(k_pair_fast<false>, dim3(a.B * a.K_max + a.B), dim3(NT_F), 0, st, a, uo);
      return launch_status();
    }
    if (phase == 1) return SD_OK;   // (flagged units take the exact route inside k_pair_fast)
    hipLaunchKernelGGL(k_fast_finalize, dim3(a.B), dim3(64), 0, st, a, uo, acc, tok, status, stats);
    return launch_status();
  }
  const bool need_tv = needs_tv(a, stats);
  if (phase == 0) return run_prepare<DT>(a, L, ws, st);
  if (phase == 1) {
    if (!need_tv || a.K_max == 0) return SD_OK;
    hipLaunchKernelGGL(k_pair_tv<DT>, dim3(a.B * a.K_max * L.tvS), dim3(NT_ROW),
                       a.rep != 1.0f ? align_up((size_t)bitmap_words(a.V) * 4, 16) : 0, st, a,
                       reinterpret_cast<const RowStat*>(ws + L.rs),
                       reinterpret_cast<double*>(ws + L.dtv), L.tvS);
    return launch_status();
  }
  const RowStat* rs = reinterpret_cast<const RowStat*>(ws + L.rs);
  const double* dpart = reinterpret_cast<const double*>(ws + L.dtv);
  if (L.drS <= 1) {
    hipLaunchKernelGGL((k_finalize<DT, false>), dim3(a.B), dim3(NT_ROW), fin_lds(a.V), st, a, rs, dpart,
                       need_tv ? 1 : 0, L.tvS, bitmap_words(a.V), nullptr, acc, tok, status, stats);
    return launch_status();
  }
  // small batches: the draw split over workgroups by chunk ranges
  int2* drec = reinterpret_cast<int2*>(ws + L.drec);
  double* ctot = reinterpret_cast<double*>(ws + L.ctot);
  hipLaunchKernelGGL((k_finalize<DT, true>), dim3(a.B), dim3(NT_ROW), 0, st, a, rs, dpart, need_tv ? 1 : 0,
                     L.tvS, 0, drec, acc, tok, status, stats);
  hipLaunchKernelGGL(k_draw_tot<DT>, dim3(a.B * L.drS), dim3(NT_ROW),
                     a.rep != 1.0f ? align_up((size_t)bitmap_words(a.V) * 4, 16) : 0, st, a, rs, drec, ctot,
                     L.drS);
  hipLaunchKernelGGL(k_draw_pick<DT>, dim3(a.B), dim3(NT_ROW), 0, st, a, rs, drec, ctot, tok, status, stats);
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

// Built-in workspace of sd_verify_sample_noalloc: one array per GPU, held
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: its device address comes from hipGetSymbolAddress, once
// per device with that device current, and only that address is used.
static __device__ __align__(256) unsigned char scratch[SD_NOALLOC_MAX_WORKSPACE];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];   // device address of `scratch`, per device

// Device address of the current device's scratch array (looked up on the
// first call on that device).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return SD_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SD_EHIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SD_OK;
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

int sd_verify_sample_noalloc(const sd_verify_args_t* args, int32_t* out_accepted,
                             int32_t* out_tokens, uint32_t* out_status, float* out_stats,
                             void* stream) {
  int rc = check_common(args, true);
  if (rc) return rc;
  if (!out_accepted || !out_tokens) return SD_EINVAL;
  if (layout(args).total > SD_NOALLOC_MAX_WORKSPACE) return SD_ESCRATCH;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  // Nothing in the workspace needs to start at zero: every record a kernel
  // reads is written earlier in the same call.
  return sd_verify_sample(args, ws, SD_NOALLOC_MAX_WORKSPACE, out_accepted, out_tokens,
                          out_status, out_stats, stream);
}

const char* sd_strerror(int code) {
  switch (code) {
    case SD_OK: return "ok";
    case SD_EINVAL: return "invalid argument";
    case SD_EWORKSPACE: return "workspace missing or too small";
    case SD_EHIP: return "HIP runtime error";
    case SD_EUNSUPPORTED: return "unsupported size (K_max or V beyond this build's limits)";
    case SD_ESCRATCH: return "call needs more workspace than the built-in scratch array holds";
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
                       reinterpret_cast<const RowStat*>(ws + L.rs), out_p, out_q);
  else
    hipLaunchKernelGGL(k_debug_rows<SD_F32>, dim3(grid), dim3(NT_ROW), lds, st, a,
                       reinterpret_cast<const RowStat*>(ws + L.rs), out_p, out_q);
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

const char* sd_debug_phase_kernel(const sd_verify_args_t* args, int phase) {
  if (check_common(args, true) != SD_OK || phase < 0 || phase > 2) return nullptr;
  const Args a = make_args(args);
  if (a.dtype == SD_BF16 && use_fast(a)) {
    static const char* const fast[3] = {"k_pair_fast", nullptr, "k_fast_finalize"};
    return fast[phase];
  }
  if (phase == 0) return "k_row_prepare";
  if (phase == 1) return (needs_tv(a, nullptr) && a.K_max > 0) ? "k_pair_tv" : nullptr;
  return draw_slices(a.B, a.V) > 1 ? "k_finalize + k_draw_tot + k_draw_pick" : "k_finalize";
}

int sd_debug_fallback_units(const sd_verify_args_t* args, const void* workspace,
                            size_t workspace_bytes, int32_t* out_count, uint32_t* out_why,
                            void* stream) {
  int rc = check_common(args, true);
  if (rc) return rc;
  if (!out_count) return SD_EINVAL;
  const Args a = make_args(args);
  if (!(a.dtype == SD_BF16 && use_fast(a))) return SD_EUNSUPPORTED;
  const Layout L = layout(args);
  if (!workspace || workspace_bytes < L.total) return SD_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // The unit records' flags and the per-request K and T, copied to the host.
  const int B = a.B, nunits = B * (a.K_max + 1);
  std::vector<uint32_t> flags(2 * (size_t)nunits);   // flags, why per unit
  std::vector<int32_t> ks(B, a.K_max);
  std::vector<float> ts(B, 1.0f);
  std::vector<float> tps(B, a.top_p), ds(B, a.D);
  const char* uo = static_cast<const char*>(workspace) + L.uo;
  static_assert(offsetof(UnitOut, why) == offsetof(UnitOut, flags) + 4, "UnitOut layout");
  bool ok = hipMemcpy2DAsync(flags.data(), 2 * sizeof(uint32_t), uo + offsetof(UnitOut, flags),
                             sizeof(UnitOut), 2 * sizeof(uint32_t), nunits, hipMemcpyDeviceToHost,
                             st) == hipSuccess;
  if (ok && a.kpr)
    ok = hipMemcpyAsync(ks.data(), a.kpr, B * sizeof(int32_t), hipMemcpyDeviceToHost, st) == hipSuccess;
  if (ok && a.temp)
    ok = hipMemcpyAsync(ts.data(), a.temp, B * sizeof(float), hipMemcpyDeviceToHost, st) == hipSuccess;
  if (ok && a.tpr)
    ok = hipMemcpyAsync(tps.data(), a.tpr, B * sizeof(float), hipMemcpyDeviceToHost, st) == hipSuccess;
  if (ok && a.dpr)
    ok = hipMemcpyAsync(ds.data(), a.dpr, B * sizeof(float), hipMemcpyDeviceToHost, st) == hipSuccess;
  if (!ok || hipStreamSynchronize(st) != hipSuccess) return SD_EHIP;
  // Units the kernel skips (invalid request, position beyond K_r) hold no record.
  int n = 0;
  for (int u = 0; u < nunits; ++u) {
    if (out_why) out_why[u] = 0u;
    const bool bonus = u >= B * a.K_max;
    const int r = bonus ? u - B * a.K_max : u / a.K_max;
    const int j = bonus ? 0 : u % a.K_max;
    const int K = ks[r];
    const float T = ts[r];
    if (K < 0 || K > a.K_max || (!bonus && j >= K) || !(T > 0.0f) || !(T < INFINITY)) continue;
    if (!(tps[r] > 0.0f && tps[r] <= 1.0f) || !(ds[r] >= 0.0f)) continue;   // as params_ok
    if (flags[2 * u] & UO_FALLBACK) {
      ++n;
      if (out_why) out_why[u] = flags[2 * u + 1];
    }
  }
  *out_count = n;
  return SD_OK;
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
