// Verify step fed from hidden states through the LM heads on gfx950, with no
// V-wide logit row written to memory ("What I Gave Up to Make Speculative
// Decoding Faster", section "Finding the break-even point": the engine scores
// the verify rows with its LM head; Adaptive-SpecDecode-Lab README,
// implementation section: one target forward keeps the logits of the rows
// being verified).
//
// Logits come out of a bf16 MFMA tile engine (v_mfma_f32_32x32x16_bf16, fp32
// accumulation): a workgroup of 256 threads computes a 64-row x 128-token
// tile, hidden states (rows) times head rows (tokens), both K-contiguous,
// through LDS in K chunks of 64.  Every kernel consumes its tiles in an
// epilogue:
//   k_lm_stats      per (row, token tile): max and sum of exp2 of l = z c,
//                   and the logit of the row's draft token when the tile
//                   holds it
//   k_lm_rowstat    per row: M = max l, Z = sum 2^(l - M)
//   k_lm_tv         per (pair, tile): sum |p - q| (target and draft tiles
//                   of the same pair in one workgroup), only when a budget
//                   strictly between 0 and 1 needs d
//   k_lm_decide     per request (one lane per position): theta, pi(x),
//                   acceptance, first rejection
//   k_lm_draw_tiles per (request, tile): fixed-point totals of the draw
//                   weights (the residual max(p - q, 0) and p)
//   k_lm_draw_pick  per request: the crossing tile, recomputed, scanned
// Greedy: k_lm_greedy_part (per row and tile: max and lowest argmax) and
// k_lm_greedy_final.  A tile engine call recomputes the same logits bit for
// bit wherever it runs (same K order), so the draw's pick agrees with its
// tile totals.  Rows are taken from compacted lists of the rows each request
// uses, so a ragged K costs no work on unused rows.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <limits.h>
#include <math.h>
#include <stddef.h>

#include "sd_verify.h"
#include "sdv_device.h"

using namespace sdv;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int TM = 64;            // rows per tile
constexpr int TN = 128;           // tokens per tile
constexpr int BK = 64;            // K chunk
constexpr int LDK = BK + 8;       // LDS row stride of the A/B chunks (bf16): 144 B
constexpr int NT_L = 256;         // threads of a tile workgroup (4 waves)
constexpr int LDC = TN;           // LDS row stride of a stashed fp32 tile

// Word of element (m, n) of a stashed fp32 tile.  Within each 32-column
// group of a row the column is XORed with (m mod 8, group) so that the
// epilogues' pattern (thread 4 row + q takes columns 32 q + e of its row,
// at the same e across the wave) touches 32 different banks per half-wave,
// and the stash's (32 consecutive columns of one row per half-wave) stays
// a permutation of one group.
__device__ __forceinline__ int cidx(int m, int n) {
  return m * LDC + (n ^ (((m & 7) << 2) | ((n >> 5) & 3)));
}
// LDS words of the A/B chunks or, after the product, the stashed fp32 tile
constexpr int TILE_LDS_WORDS = (TM + TN) * LDK / 2 > TM * LDC ? (TM + TN) * LDK / 2 : TM * LDC;
// The row-statistics and greedy passes take taller tiles, MBS 64-row parts
// (each head tile is then read once per 192 rows instead of per 64), and
// stash their result one 64-row part at a time over the chunk buffers.
constexpr int MBS = 3;
constexpr int TMS = 64 * MBS;
constexpr int TALL_LDS_WORDS = (TMS + TN) * LDK / 2 > TM * LDC ? (TMS + TN) * LDK / 2 : TM * LDC;
constexpr int NXCD = 8;           // dies of the device (tile order is per die)
constexpr int SHL = 40;           // fixed-point shift of the draw weights (each <= 1)

struct LmArgs {
  const uint16_t* th;   // target hidden [B][K_max+1][Ht]
  const uint16_t* dh;   // draft hidden  [B][K_max][Hd]
  const uint16_t* wt;   // target head [V][Ht]
  const uint16_t* wd;   // draft head  [Vd][Hd]
  int Ht, Hd, B, K_max, V, Vd;
  const int32_t* ids;
  const int32_t* kpr;
  const float* temp;
  float D;
  uint64_t seed, offset;
  uint32_t flags;
};

struct RowSL {       // statistics of one listed row
  float M;           // max of l = z c (log2 units)
  float c;           // log2(e) / T
  double Z;          // sum of 2^(l - M)
  float zx;          // logit of the row's draft token (or -inf)
  uint32_t flags;    // 1: a non-finite logit
  int32_t pad0, pad1;
};
static_assert(sizeof(RowSL) == 32, "RowSL layout");

// Workspace carve-up.
struct LmLayout {
  size_t cnt, toff, doff, tlist, dlist, tcx, dcx, tpart, dpart, trs, drs, tvp, dvec, drw, wpart, gpart, total;
  int ntt, ntd;   // token tiles of the target and draft heads
};

__host__ __device__ inline size_t al256(size_t x) { return (x + 255) / 256 * 256; }

LmLayout lm_layout(int B, int K, int V, int Vd) {
  LmLayout L;
  L.ntt = (V + TN - 1) / TN;
  L.ntd = (Vd + TN - 1) / TN;
  const size_t nt = (size_t)B * (K + 1), nd = (size_t)B * K;
  size_t o = 0;
  L.cnt = o;   o = al256(o + 4 * sizeof(int));
  L.toff = o;  o = al256(o + (size_t)B * sizeof(int));
  L.doff = o;  o = al256(o + (size_t)B * sizeof(int));
  L.tlist = o; o = al256(o + nt * sizeof(int));
  L.dlist = o; o = al256(o + (nd ? nd : 1) * sizeof(int));
  L.tcx = o;   o = al256(o + nt * sizeof(int2));
  L.dcx = o;   o = al256(o + (nd ? nd : 1) * sizeof(int2));
  L.tpart = o; o = al256(o + nt * L.ntt * sizeof(float2));
  L.dpart = o; o = al256(o + (nd ? nd : 1) * L.ntd * sizeof(float2));
  L.trs = o;   o = al256(o + nt * sizeof(RowSL));
  L.drs = o;   o = al256(o + (nd ? nd : 1) * sizeof(RowSL));
  L.tvp = o;   o = al256(o + (nd ? nd : 1) * L.ntt * sizeof(float));
  L.dvec = o;  o = al256(o + (nd ? nd : 1) * sizeof(double));
  L.drw = o;   o = al256(o + (size_t)B * sizeof(int2));
  L.wpart = o; o = al256(o + (size_t)B * L.ntt * 2 * sizeof(uint64_t));
  L.gpart = o; o = al256(o + nt * L.ntt * sizeof(uint2));
  L.total = o;
  return L;
}

struct LmWs {
  int* cnt;      // [0] target rows listed, [1] draft rows listed
  int* toff;     // per request: its first target row in the list (-1: none)
  int* doff;     // per request: its first draft row in the list
  int* tlist;    // listed target rows: r (K_max + 1) + j
  int* dlist;    // listed draft rows: r K_max + j
  int2* tcx;     // per listed target row: (bits of c = log2(e) / T, draft token x_j or -1)
  int2* dcx;     // per listed draft row: the same
  float2* tpart; // [listed target row][token tile] (max l, sum 2^(l - max))
  float2* dpart;
  RowSL* trs;
  RowSL* drs;
  float* tvp;    // [pair = listed draft row][target token tile] sum |p - q|
  double* dvec;  // [pair] d
  int2* drw;     // per request: (mode, n); mode 0 residual, 1 p, -1 none
  uint64_t* wpart;   // [request][tile][2] fixed-point totals: residual, p
  uint2* gpart;  // [listed target row][tile] (orderable key, id) of the max
};

LmWs carve(char* ws, const LmLayout& L) {
  LmWs w;
  w.cnt = reinterpret_cast<int*>(ws + L.cnt);
  w.toff = reinterpret_cast<int*>(ws + L.toff);
  w.doff = reinterpret_cast<int*>(ws + L.doff);
  w.tlist = reinterpret_cast<int*>(ws + L.tlist);
  w.dlist = reinterpret_cast<int*>(ws + L.dlist);
  w.tcx = reinterpret_cast<int2*>(ws + L.tcx);
  w.dcx = reinterpret_cast<int2*>(ws + L.dcx);
  w.tpart = reinterpret_cast<float2*>(ws + L.tpart);
  w.dpart = reinterpret_cast<float2*>(ws + L.dpart);
  w.trs = reinterpret_cast<RowSL*>(ws + L.trs);
  w.drs = reinterpret_cast<RowSL*>(ws + L.drs);
  w.tvp = reinterpret_cast<float*>(ws + L.tvp);
  w.dvec = reinterpret_cast<double*>(ws + L.dvec);
  w.drw = reinterpret_cast<int2*>(ws + L.drw);
  w.wpart = reinterpret_cast<uint64_t*>(ws + L.wpart);
  w.gpart = reinterpret_cast<uint2*>(ws + L.gpart);
  return w;
}

__device__ __forceinline__ int req_k(const LmArgs& a, int r) { return a.kpr ? a.kpr[r] : a.K_max; }
__device__ __forceinline__ float req_t(const LmArgs& a, int r) { return a.temp ? a.temp[r] : 1.0f; }

// Status of request r before any logit is seen (sampling: with the
// temperature; greedy: without).  One invalidating defect, in the order K,
// draft ids, temperature.
__device__ uint32_t lm_status(const LmArgs& a, int r, bool sample) {
  const int K = req_k(a, r);
  if (K < 0 || K > a.K_max) return SD_ST_BAD_K;
  for (int j = 0; j < K; ++j) {
    const int x = a.ids[(int64_t)r * a.K_max + j];
    if (x < 0 || x >= a.V) return SD_ST_BAD_DRAFT_ID;
  }
  if (sample) {
    const float T = req_t(a, r);
    if (!(T > 0.0f) || !(T < INFINITY)) return SD_ST_BAD_TEMP;
  }
  return 0u;
}

// ---------------------------------------------------------------------------
// Row lists: one workgroup; valid requests list rows j = 0..K_r (target) and
// j = 0..K_r - 1 (draft) in request order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_lm_lists(LmArgs a, LmWs w, int sample) {
  constexpr int NT = 1024;
  __shared__ int wt_t[NT / WAVE], wt_d[NT / WAVE];
  __shared__ int base_t, base_d;
  if (threadIdx.x == 0) { base_t = 0; base_d = 0; }
  __syncthreads();
  for (int r0 = 0; r0 < a.B; r0 += NT) {
    const int r = r0 + threadIdx.x;
    int nt = 0, nd = 0;
    if (r < a.B && lm_status(a, r, sample != 0) == 0u) {
      const int K = req_k(a, r);
      nt = K + 1;
      nd = sample ? K : 0;
    }
    int tot_t, tot_d;
    const int et = block_excl_scan_int<NT>(nt, wt_t, &tot_t);
    const int ed = block_excl_scan_int<NT>(nd, wt_d, &tot_d);
    const int bt = base_t, bd = base_d;
    if (r < a.B) {
      w.toff[r] = nt ? bt + et : -1;
      w.doff[r] = nd ? bd + ed : -1;
      // (each row's c and draft token, for the statistics pass to load with
      // one access before its product)
      const int cb = __float_as_int(1.4426950408889634f / req_t(a, r));
      for (int j = 0; j < nt; ++j) {
        w.tlist[bt + et + j] = r * (a.K_max + 1) + j;
        w.tcx[bt + et + j] = make_int2(cb, j < nt - 1 ? a.ids[(int64_t)r * a.K_max + j] : -1);
      }
      for (int j = 0; j < nd; ++j) {
        w.dlist[bd + ed + j] = r * a.K_max + j;
        w.dcx[bd + ed + j] = make_int2(cb, a.ids[(int64_t)r * a.K_max + j]);
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) { base_t += tot_t; base_d += tot_d; }
    __syncthreads();
  }
  if (threadIdx.x == 0) { w.cnt[0] = base_t; w.cnt[1] = base_d; }
}

// ---------------------------------------------------------------------------
// The tile engine.
// ---------------------------------------------------------------------------
// Compile-time loop: f.template operator()<I>() for I = 0 .. N-1, so that
// register arrays indexed by I stay in registers.
template <int N, class F>
__device__ __forceinline__ void unroll_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (f.template operator()<I>(), ...);
  }(std::make_integer_sequence<int, N>{});
}

struct TileLds {
  uint16_t* a;   // [TM][LDK]
  uint16_t* b;   // [TN][LDK]
};

// Hidden-state rows of a tile engine call: A slot i of this thread holds
// tile row t / 8 + 32 i (i < 2 MB); row[i] is its row of the hidden-state
// array at base (rows of H elements, bytes in all, below 2^31), or -1 for
// a row past the list, which reads 0.
template <int MB>
struct ARows {
  const uint16_t* base;
  uint32_t bytes;
  int row[2 * MB];
};

// acc[mb][nb] = rows (64 MB) x tokens (TN) of hidden x head^T; weight rows
// n0 .. n0 + TN - 1 past nrows_w read 0.  The chunk loads are buffer loads:
// a row past the list or the head reads zeros without a memory access, and
// every load is issued unconditionally, so the wait before a chunk's LDS
// writes counts only that chunk's loads and the other sets' stay in flight.
// Wave (wr, wc) = (wave / 2, wave % 2) holds rows 32 (MB wr + mb) + m and tokens
// 64 wc + 32 b + n (b = 0, 1) in the MFMA 32x32 output layout: lane l, value
// v: n = l % 32, m = 8 (v / 4) + 4 (l / 32) + v % 4.  Every logit is the
// same K-ordered chain of MFMA steps whatever MB is, so tiles of any height
// give the same logits bit for bit.
template <int MB>
__device__ __forceinline__ void tile_gemm(const ARows<MB>& ar, const uint16_t* w, int n0, int nrows_w,
                                          int H, const TileLds& s, f32x16 (&acc)[MB][2]) {
  const int t = threadIdx.x;
  const int lane = t % WAVE, wv = t / WAVE;
  const int wr = wv >> 1, wc = wv & 1;
  const int kc = (t & 7) * 8;     // this thread's 8-element chunk of a K chunk
  const int rr = t >> 3;          // its row within a 32-row slab
  // byte offsets of the slots' rows at k = kc (a row past the end: at 2^31,
  // beyond either resource)
  const __amdgpu_buffer_rsrc_t rsa =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(ar.base), (short)0, (int)ar.bytes, 0x00020000);
  const int64_t wbytes = (int64_t)max(nrows_w - n0, 0) * H * 2;
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(w + (int64_t)n0 * H), (short)0, (int)min(wbytes, (int64_t)0x7FFFFFFF), 0x00020000);
  uint32_t aoff[2 * MB], boff[4];
#pragma unroll
  for (int i = 0; i < 2 * MB; ++i)
    aoff[i] = ar.row[i] >= 0 ? (uint32_t)ar.row[i] * (uint32_t)H * 2u + (uint32_t)kc * 2u : 0x80000000u;
#pragma unroll
  for (int i = 0; i < 4; ++i) boff[i] = (uint32_t)(rr + 32 * i) * (uint32_t)H * 2u + (uint32_t)kc * 2u;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][b][v] = 0.0f;
  // NS register sets of chunk loads: chunk k + NS is loaded while chunk k
  // is multiplied, so NS chunks' loads are in flight behind the matrix
  // cores (one chunk's latency is several times its MFMA work).  Three for
  // the 64-row tiles, whose passes stream each head tile once (their
  // registers allow it); two for the taller tiles.
  constexpr int NS = MB == 1 ? 3 : 2;
  uint4 ra[NS][2 * MB], rb[NS][4];
  auto load = [&](int k0, uint4 (&ra)[2 * MB], uint4 (&rb)[4]) __attribute__((always_inline)) {
    const uint32_t kb = (uint32_t)k0 * 2u;
#pragma unroll
    for (int i = 0; i < 2 * MB; ++i) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsa, aoff[i] + kb, 0, 0);
      ra[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsb, boff[i] + kb, 0, 0);
      rb[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };
  const int ko = 8 * (lane >> 5);
  // one K chunk: its loads to LDS, the load of the chunk NS ahead into the
  // same registers, then the products
  auto chunk = [&](int k0, uint4 (&ra)[2 * MB], uint4 (&rb)[4]) __attribute__((always_inline)) {
    __syncthreads();   // the previous chunk's fragments are read
#pragma unroll
    for (int i = 0; i < 2 * MB; ++i)
      *reinterpret_cast<uint4*>(s.a + (rr + 32 * i) * LDK + kc) = ra[i];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(s.b + (rr + 32 * i) * LDK + kc) = rb[i];
    __syncthreads();
    // (issued every time, the last chunk again past the end, so that every
    // wait counts the same loads)
    load(min(k0 + NS * BK, H - BK), ra, rb);
#pragma unroll
    for (int st = 0; st < BK / 16; ++st) {
      bf16x8 af[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        af[mb] = *reinterpret_cast<const bf16x8*>(s.a + (32 * (MB * wr + mb) + (lane & 31)) * LDK + 16 * st + ko);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int bn = 64 * wc + 32 * b + (lane & 31);
        const bf16x8 bfr = *reinterpret_cast<const bf16x8*>(s.b + bn * LDK + 16 * st + ko);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr, acc[mb][b], 0, 0, 0);
      }
    }
  };
  unroll_for<NS>([&]<int I>() __attribute__((always_inline)) { load(min(I * BK, H - BK), ra[I], rb[I]); });
  int k0 = 0;
  for (; k0 + (NS - 1) * BK < H; k0 += NS * BK)
    unroll_for<NS>([&]<int I>() __attribute__((always_inline)) { chunk(k0 + I * BK, ra[I], rb[I]); });
  // (fewer than NS chunks left, in the sets that hold them)
  unroll_for<NS - 1>([&]<int I>() __attribute__((always_inline)) {
    if (k0 + I * BK < H) chunk(k0 + I * BK, ra[I], rb[I]);
  });
}

// Rows 64 p .. 64 p + 63 of a tile of 64 MB rows into an fp32 LDS tile
// C[64][LDC] (the waves holding other rows write nothing).
template <int MB>
__device__ __forceinline__ void stash_part(const f32x16 (&acc)[MB][2], float* C, int p) {
  const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
  const int wr = wv >> 1, wc = wv & 1;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int row0 = 32 * (MB * wr + mb) - 64 * p;
    if (row0 < 0 || row0 >= 64) continue;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = row0 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int n = 64 * wc + 32 * b + (lane & 31);
        C[cidx(m, n)] = acc[mb][b][v];
      }
  }
}

// The accumulators into an fp32 LDS tile C[TM][LDC].
__device__ __forceinline__ void stash(const f32x16 (&acc)[2], float* C) {
  const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
  const int wr = wv >> 1, wc = wv & 1;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = 32 * wr + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      const int n = 64 * wc + 32 * b + (lane & 31);
      C[cidx(m, n)] = acc[b][v];
    }
}

// Tile order: the blocks of one die take consecutive tiles, row blocks
// fastest, so a head tile is fetched into that die's L2 once for all its row
// blocks.  Returns false for padding blocks.
__device__ __forceinline__ bool tile_of(int nm, int nn, int& m, int& n) {
  const int per = (int)gridDim.x / NXCD;
  const int g = ((int)blockIdx.x % NXCD) * per + (int)blockIdx.x / NXCD;
  if (g >= nm * nn) return false;
  m = g % nm;
  n = g / nm;
  return true;
}

// The tile engine's view of the target or draft hidden states, no row yet.
template <int MB>
__device__ __forceinline__ ARows<MB> hidden_rows(const LmArgs& a, bool target) {
  ARows<MB> r;
  r.base = target ? a.th : a.dh;
  r.bytes = (uint32_t)((int64_t)a.B * (target ? a.K_max + 1 : a.K_max) * (target ? a.Ht : a.Hd) * 2);
#pragma unroll
  for (int i = 0; i < 2 * MB; ++i) r.row[i] = -1;
  return r;
}

// ---------------------------------------------------------------------------
// Pass 1: per (listed row, token tile) max and exp2 sum; the draft token's logit.
// ---------------------------------------------------------------------------
template <bool TGT>
__global__ __launch_bounds__(NT_L, 2) void k_lm_stats(LmArgs a, LmWs w, int nm, int nn) {
  // (each fp32 part is stashed over the A/B chunks once the product is done)
  __shared__ __align__(16) float lds_ab_c[TALL_LDS_WORDS];
  uint16_t* const sa = reinterpret_cast<uint16_t*>(lds_ab_c);
  uint16_t* const sb = sa + TMS * LDK;
  float* const C = lds_ab_c;
  int mb, nb;
  if (!tile_of(nm, nn, mb, nb)) return;
  const int nrows = w.cnt[TGT ? 0 : 1];
  const int m0 = mb * TMS, n0 = nb * TN;
  if (m0 >= nrows) return;
  const int* list = TGT ? w.tlist : w.dlist;
  const int rr = threadIdx.x >> 3;
  ARows<MBS> ar = hidden_rows<MBS>(a, TGT);
#pragma unroll
  for (int i = 0; i < 2 * MBS; ++i) {
    const int li = m0 + rr + 32 * i;
    ar.row[i] = li < nrows ? list[li] : -1;
  }
  const int Vs = TGT ? a.V : a.Vd;
  // the epilogue's (c, draft token) of this thread's row in each part,
  // loaded now so that their latency hides behind the product
  int2 cx[MBS];
#pragma unroll
  for (int p = 0; p < MBS; ++p) {
    const int li = m0 + 64 * p + (int)(threadIdx.x >> 2);
    cx[p] = li < nrows ? (TGT ? w.tcx : w.dcx)[li] : make_int2(__float_as_int(1.0f), -1);
  }
  f32x16 acc[MBS][2];
  tile_gemm<MBS>(ar, TGT ? a.wt : a.wd, n0, Vs, TGT ? a.Ht : a.Hd, TileLds{sa, sb}, acc);
  const int nv = min(TN, Vs - n0);
  // (unrolled: each part reads its own accumulators where it stashes them)
#pragma unroll
  for (int part = 0; part < MBS; ++part) {
    if (m0 + 64 * part >= nrows) continue;
    __syncthreads();   // the chunk buffers, or the previous part, are read
    stash_part<MBS>(acc, C, part);
    __syncthreads();
    // four threads per row, 32 tokens each
    const int row = threadIdx.x >> 2, q4 = threadIdx.x & 3;
    const int li = m0 + 64 * part + row;
    const bool live = li < nrows;
    const float c = __int_as_float(cx[part].x);
    const int x = live ? cx[part].y : -1;
    float m = -INFINITY;
    int bad = 0;
    for (int e = 0; e < 32; ++e) {
      const int n = q4 * 32 + e;
      if (n < nv) {
        const float z = C[cidx(row, n)];
        bad |= nonfinite(z);
        m = fmaxf(m, z * c);
      }
      if (live && n0 + n == x && n < nv) {
        RowSL* rs = (TGT ? w.trs : w.drs) + li;
        rs->zx = C[cidx(row, n)];
      }
    }
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    float s = 0.0f;
    if (m > -INFINITY)
      for (int e = 0; e < 32; ++e) {
        const int n = q4 * 32 + e;
        if (n < nv) s += fast_exp2(C[cidx(row, n)] * c - m);
      }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    bad |= __shfl_xor(bad, 1);
    bad |= __shfl_xor(bad, 2);
    if (live && q4 == 0) {
      float2* part_out = (TGT ? w.tpart : w.dpart) + (int64_t)li * nn + nb;
      *part_out = make_float2(bad ? NAN : m, s);
    }
  }
}

// Per listed row: M, Z from the tile partials (fp64 combine in tile order).
template <bool TGT>
__global__ __launch_bounds__(256) void k_lm_rowstat(LmArgs a, LmWs w, int nn) {
  __shared__ float sf[256 / WAVE];
  __shared__ double sd[256 / WAVE];
  __shared__ int si[256 / WAVE + 4];
  const int li = blockIdx.x;
  if (li >= w.cnt[TGT ? 0 : 1]) return;
  const float2* part = (TGT ? w.tpart : w.dpart) + (int64_t)li * nn;
  float m = -INFINITY;
  int bad = 0;
  for (int t = threadIdx.x; t < nn; t += 256) {
    const float2 p = part[t];
    bad |= (p.x != p.x);
    m = fmaxf(m, p.x);
  }
  const float M = block_max<256>(m, sf);
  bad = block_or<256>(bad, si);
  double z = 0.0;
  for (int t = threadIdx.x; t < nn; t += 256) {
    const float2 p = part[t];
    if (p.x > -INFINITY) z += (double)p.y * exp2((double)p.x - (double)M);
  }
  const double Z = block_sum<256>(z, sd);
  if (threadIdx.x == 0) {
    RowSL* rs = (TGT ? w.trs : w.drs) + li;
    const int enc = (TGT ? w.tlist : w.dlist)[li];
    const int r = TGT ? enc / (a.K_max + 1) : enc / a.K_max;
    rs->M = M;
    rs->c = 1.4426950408889634f / req_t(a, r);
    rs->Z = Z;
    rs->flags = (bad || !(M > -INFINITY) || !(M < INFINITY)) ? 1u : 0u;
  }
}

// Clears the draft-token logits before pass 1 writes the ones it finds (a
// token past a short draft head is never found: -inf).
__global__ void k_lm_clear_zx(LmWs w, int nt_max, int nd_max) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nt_max) w.trs[i].zx = -INFINITY;
  if (i < nd_max) w.drs[i].zx = -INFINITY;
}

// ---------------------------------------------------------------------------
// The pair kernels: a tile of 64 pairs (or requests) x 128 tokens, the
// target tile stashed in LDS, the draft tile in registers.
// ---------------------------------------------------------------------------
struct PairRows {
  int tli, dli;   // listed target / draft row (-1: none)
};

// TV partials: pair p = listed draft row (r, j); its target row is listed at
// toff[r] + j.
__global__ __launch_bounds__(NT_L) void k_lm_tv(LmArgs a, LmWs w, int nm, int nn) {
  __shared__ __align__(16) float Ct[TM * LDC];
  __shared__ __align__(16) float U[TM * LDC];   // A/B chunks, then the draft tile
  __shared__ int s_tli[TM];
  int mb, nb;
  if (!tile_of(nm, nn, mb, nb)) return;
  const int npairs = w.cnt[1];
  const int m0 = mb * TM, n0 = nb * TN;
  if (m0 >= npairs) return;
  if (threadIdx.x < TM) {
    const int p = m0 + threadIdx.x;
    int tli = -1;
    if (p < npairs) {
      const int enc = w.dlist[p];
      const int r = enc / a.K_max, j = enc % a.K_max;
      tli = w.toff[r] + j;
    }
    s_tli[threadIdx.x] = tli;
  }
  __syncthreads();
  const int rr = threadIdx.x >> 3;
  TileLds s{reinterpret_cast<uint16_t*>(U), reinterpret_cast<uint16_t*>(U) + TM * LDK};
  f32x16 acc[1][2];
  {
    ARows<1> ar = hidden_rows<1>(a, true);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int tli = s_tli[rr + 32 * i];
      ar.row[i] = tli >= 0 ? w.tlist[tli] : -1;
    }
    tile_gemm<1>(ar, a.wt, n0, a.V, a.Ht, s, acc);
    stash(acc[0], Ct);
  }
  {
    ARows<1> ar = hidden_rows<1>(a, false);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = m0 + rr + 32 * i;
      ar.row[i] = p < npairs ? w.dlist[p] : -1;
    }
    tile_gemm<1>(ar, a.wd, n0, a.Vd, a.Hd, s, acc);
  }
  __syncthreads();
  stash(acc[0], U);
  __syncthreads();
  const int row = threadIdx.x >> 2, q4 = threadIdx.x & 3;
  const int p = m0 + row;
  float sum = 0.0f;
  if (p < npairs) {
    const RowSL P = w.trs[s_tli[row]], Q = w.drs[p];
    const float ip = (float)(1.0 / P.Z), iq = (float)(1.0 / Q.Z);
    const int nv = min(TN, a.V - n0);
    for (int e = 0; e < 32; ++e) {
      const int n = q4 * 32 + e;
      if (n >= nv) continue;
      const float pp = fast_exp2(Ct[cidx(row, n)] * P.c - P.M) * ip;
      const float qq = (n0 + n < a.Vd) ? fast_exp2(U[cidx(row, n)] * Q.c - Q.M) * iq : 0.0f;
      sum += fabsf(pp - qq);
    }
  }
  sum += __shfl_xor(sum, 1);
  sum += __shfl_xor(sum, 2);
  if (p < npairs && q4 == 0) w.tvp[(int64_t)p * nn + nb] = sum;
}

__global__ __launch_bounds__(256) void k_lm_tv_reduce(LmWs w, int nn) {
  __shared__ double sd[256 / WAVE];
  const int p = blockIdx.x;
  if (p >= w.cnt[1]) return;
  double s = 0.0;
  for (int t = threadIdx.x; t < nn; t += 256) s += (double)w.tvp[(int64_t)p * nn + t];
  s = block_sum<256>(s, sd);
  if (threadIdx.x == 0) w.dvec[p] = fmin(0.5 * s, 1.0);
}

// p(x) or q(x) of a listed row in fp64.
__device__ __forceinline__ double prob_x(const RowSL& s) {
  if (!(s.zx > -INFINITY)) return 0.0;
  return exp2((double)s.zx * (double)s.c - (double)s.M) / s.Z;
}

// Decisions of one request: one wave per request, lane jj for position jj
// (its uniforms, p(x), q(x), d and acceptance); the first rejection is the
// first bit of a ballot.
__global__ __launch_bounds__(64) void k_lm_decide(LmArgs a, LmWs w, int tv_valid, int32_t* out_acc,
                                                  int32_t* out_tok, uint32_t* out_status,
                                                  float* out_stats) {
  static_assert(WAVE == 64 && SD_MAX_K + 1 <= WAVE, "one lane per position");
  const int r = blockIdx.x;
  const int jj = threadIdx.x;
  const int K1 = a.K_max + 1;
  const int64_t base = (int64_t)r * K1;
  uint32_t st = lm_status(a, r, true);
  const int K = st ? 0 : req_k(a, r);
  int nonf = 0;
  if (!st) {
    const int t0 = w.toff[r], d0 = w.doff[r];
    if (jj <= K && w.trs[t0 + jj].flags) nonf = 1;
    if (jj < K && w.drs[d0 + jj].flags) nonf = 1;
  }
  if (__any(nonf)) st |= SD_ST_NONFINITE;
  if (st & SD_ST_INVALID_MASK) {
    if (jj < K1) {
      out_tok[base + jj] = -1;
      if (out_stats)
        for (int s2 = 0; s2 < SD_NSTAT; ++s2) out_stats[(base + jj) * SD_NSTAT + s2] = 0.0f;
    }
    if (jj == 0) {
      out_acc[r] = -1;
      if (out_status) out_status[r] = st;
      w.drw[r] = make_int2(-1, 0);
    }
    return;
  }
  float sv[SD_NSTAT] = {0, 0, 0, 0, 0, 0, 0, 0};
  bool acc = true, qzero = false;
  if (jj <= K) {
    float u, v;
    uniforms(a.seed, a.offset, r, jj, u, v);
    sv[SD_STAT_U] = u;
    sv[SD_STAT_V] = v;
    if (jj < K) {
      const int t0 = w.toff[r], d0 = w.doff[r];
      const double px = prob_x(w.trs[t0 + jj]);
      const double qx = prob_x(w.drs[d0 + jj]);
      const double d = tv_valid ? w.dvec[d0 + jj] : 0.0;
      double th;
      if (tv_valid) th = (d <= (double)a.D) ? 1.0 : (double)a.D / d;
      else th = (a.D >= 1.0f) ? 1.0 : 0.0;   // D = 0: theta matters only where p = q
      const double pix = (1.0 - th) * px + th * qx;
      acc = (double)u * qx < pix;
      qzero = qx == 0.0;
      sv[SD_STAT_D] = (float)d;
      sv[SD_STAT_THETA] = (float)th;
      sv[SD_STAT_PX] = (float)px;
      sv[SD_STAT_QX] = (float)qx;
      sv[SD_STAT_PIX] = (float)pix;
    }
  }
  if (__any(qzero)) st |= SD_ST_Q_ZERO;
  const uint64_t rej = __ballot(jj < K && !acc);
  const int n = rej ? __builtin_ctzll(rej) : K;
  if (jj < K1) {
    if (out_stats)
      for (int s2 = 0; s2 < SD_NSTAT; ++s2) out_stats[(base + jj) * SD_NSTAT + s2] = sv[s2];
    out_tok[base + jj] = jj < n ? a.ids[(int64_t)r * a.K_max + jj] : -1;
  }
  if (jj == 0) {
    const bool emit = !(n == K && (a.flags & SD_NO_BONUS));
    out_acc[r] = n;
    if (out_status) out_status[r] = st;
    w.drw[r] = make_int2(emit ? (n < K ? 0 : 1) : -1, n);
  }
}

// Draw weights of one token: residual max(p - q, 0) (mode 0) and p.
__device__ __forceinline__ void draw_w(float zt, float zd, bool has_q, const RowSL& P,
                                       const RowSL& Q, float ip, float iq, float& wres,
                                       float& wp) {
  const float pp = fast_exp2(zt * P.c - P.M) * ip;
  const float qq = has_q ? fast_exp2(zd * Q.c - Q.M) * iq : 0.0f;
  wp = pp;
  wres = fmaxf(pp - qq, 0.0f);
}

// The tiles of a draw: requests r with a draw, 64 per block, the target row
// (r, n) and (mode 0) the draft row (r, n).
__device__ __forceinline__ void draw_tiles_gemm(const LmArgs& a, const LmWs& w, const int* reqs,
                                                int n0, float* Ct, float* U, f32x16 (&acc)[1][2]) {
  const int rr = threadIdx.x >> 3;
  TileLds s{reinterpret_cast<uint16_t*>(U), reinterpret_cast<uint16_t*>(U) + TM * LDK};
  {
    ARows<1> ar = hidden_rows<1>(a, true);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = reqs[rr + 32 * i];
      if (r >= 0) {
        const int2 dr = w.drw[r];
        ar.row[i] = w.tlist[w.toff[r] + dr.y];
      }
    }
    tile_gemm<1>(ar, a.wt, n0, a.V, a.Ht, s, acc);
    stash(acc[0], Ct);
  }
  {
    ARows<1> ar = hidden_rows<1>(a, false);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = reqs[rr + 32 * i];
      if (r >= 0) {
        const int2 dr = w.drw[r];
        if (dr.x == 0) ar.row[i] = w.dlist[w.doff[r] + dr.y];
      }
    }
    tile_gemm<1>(ar, a.wd, n0, a.Vd, a.Hd, s, acc);
  }
  __syncthreads();
  stash(acc[0], U);
  __syncthreads();
}

__global__ __launch_bounds__(NT_L) void k_lm_draw_tiles(LmArgs a, LmWs w, int nm, int nn) {
  __shared__ __align__(16) float Ct[TM * LDC];
  __shared__ __align__(16) float U[TM * LDC];
  __shared__ int reqs[TM];
  int mb, nb;
  if (!tile_of(nm, nn, mb, nb)) return;
  const int m0 = mb * TM, n0 = nb * TN;
  if (threadIdx.x < TM) {
    const int r = m0 + threadIdx.x;
    reqs[threadIdx.x] = (r < a.B && w.drw[r].x >= 0) ? r : -1;
  }
  __syncthreads();
  int any = 0;
  for (int i = 0; i < TM; ++i) any |= reqs[i] >= 0;
  if (!any) return;
  f32x16 acc[1][2];
  draw_tiles_gemm(a, w, reqs, n0, Ct, U, acc);
  const int row = threadIdx.x >> 2, q4 = threadIdx.x & 3;
  const int r = reqs[row];
  uint64_t sres = 0, sp = 0;
  if (r >= 0) {
    const int2 dr = w.drw[r];
    const RowSL P = w.trs[w.toff[r] + dr.y];
    RowSL Q = P;
    if (dr.x == 0) Q = w.drs[w.doff[r] + dr.y];
    const float ip = (float)(1.0 / P.Z), iq = (float)(1.0 / Q.Z);
    const int nv = min(TN, a.V - n0);
    for (int e = 0; e < 32; ++e) {
      const int n = q4 * 32 + e;
      if (n >= nv) continue;
      float wres, wp;
      draw_w(Ct[cidx(row, n)], U[cidx(row, n)], dr.x == 0 && n0 + n < a.Vd, P, Q, ip, iq, wres, wp);
      sres += e_fixed(wres, SHL);
      sp += e_fixed(wp, SHL);
    }
  }
  sres += __shfl_xor(sres, 1);
  sres += __shfl_xor(sres, 2);
  sp += __shfl_xor(sp, 1);
  sp += __shfl_xor(sp, 2);
  if (r >= 0 && q4 == 0) {
    w.wpart[((int64_t)r * nn + nb) * 2 + 0] = sres;
    w.wpart[((int64_t)r * nn + nb) * 2 + 1] = sp;
  }
}

// One request per block: the crossing tile from the tile totals (ascending
// token id), that tile recomputed, the crossing token.  A residual of zero
// mass falls back to p (status bit).
__global__ __launch_bounds__(NT_L) void k_lm_draw_pick(LmArgs a, LmWs w, int nn, int32_t* out_tok,
                                                       uint32_t* out_status, float* out_stats) {
  __shared__ __align__(16) float Ct[TM * LDC];
  __shared__ __align__(16) float U[TM * LDC];
  __shared__ int reqs[TM];
  __shared__ uint64_t su[NT_L];
  __shared__ int s_tile, s_y;
  __shared__ uint64_t s_R, s_tf, s_S;
  __shared__ int s_mode;
  const int r = blockIdx.x;
  const int2 dr = w.drw[r];
  if (dr.x < 0) return;
  const int K1 = a.K_max + 1;
  float u, v;
  uniforms(a.seed, a.offset, r, dr.y, u, v);
  // Totals in tile order, spread over the block: thread t sums tiles
  // [t CH, t CH + CH); a block scan of those sums finds the thread whose
  // range holds the crossing, and that thread walks its tiles.  (All sums
  // are exact integers, so the order of the additions does not matter.)
  {
    const int t = threadIdx.x;
    const int CH = (nn + NT_L - 1) / NT_L;
    const int t0 = min(t * CH, nn), t1 = min(t0 + CH, nn);
    uint64_t own0 = 0, own1 = 0;
    for (int q = t0; q < t1; ++q) {
      own0 += w.wpart[((int64_t)r * nn + q) * 2 + 0];
      own1 += w.wpart[((int64_t)r * nn + q) * 2 + 1];
    }
    const uint64_t S0 = block_sum_u64<NT_L>(own0, su);
    const uint64_t S1 = block_sum_u64<NT_L>(own1, su);
    int mode = dr.x;
    if (mode == 0 && S0 == 0) mode = 1;
    const uint64_t S = mode == 0 ? S0 : S1;
    const uint64_t own = mode == 0 ? own0 : own1;
    const uint64_t vk = (uint64_t)(v * 0x1p24f);
    const uint64_t tf = (__umul64hi(vk, S) << 40) | ((vk * S) >> 24);   // floor(v S)
    // inclusive scan of the per-thread sums (Hillis-Steele in LDS)
    __syncthreads();
    su[t] = own;
    __syncthreads();
    for (int o = 1; o < NT_L; o <<= 1) {
      const uint64_t y = t >= o ? su[t - o] : 0ull;
      __syncthreads();
      su[t] += y;
      __syncthreads();
    }
    const uint64_t incl = su[t], excl = incl - own;
    if (t == 0) {
      s_tile = -1;
      s_tf = tf;
      s_S = S;
      s_mode = mode;
      s_y = -1;
      if (mode != dr.x && out_status) out_status[r] |= SD_ST_RESID_ZERO;
    }
    __syncthreads();
    if (excl <= tf && incl > tf) {   // the one thread whose range crosses t
      uint64_t acc = excl;
      for (int q = t0; q < t1; ++q) {
        const uint64_t x = w.wpart[((int64_t)r * nn + q) * 2 + mode];
        if (acc + x > tf) {
          s_tile = q;
          s_R = acc;
          break;
        }
        acc += x;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x < TM) reqs[threadIdx.x] = threadIdx.x == 0 ? r : -1;
  __syncthreads();
  const int tile = s_tile;
  if (tile < 0) {
    if (threadIdx.x == 0) {
      out_tok[(int64_t)r * K1 + dr.y] = -1;
      if (out_stats) out_stats[((int64_t)r * K1 + dr.y) * SD_NSTAT + SD_STAT_S] = 0.0f;
    }
    return;
  }
  const int n0 = tile * TN;
  f32x16 acc[1][2];
  draw_tiles_gemm(a, w, reqs, n0, Ct, U, acc);
  // row 0 of the tile: per-token fixed weights, two per thread in id order
  const RowSL P = w.trs[w.toff[r] + dr.y];
  RowSL Q = P;
  if (dr.x == 0) Q = w.drs[w.doff[r] + dr.y];
  const float ip = (float)(1.0 / P.Z), iq = (float)(1.0 / Q.Z);
  const int mode = s_mode;
  const int nv = min(TN, a.V - n0);
  uint64_t wf = 0;
  const int n = threadIdx.x;   // token n0 + n (threads >= TN hold nothing)
  if (n < nv) {
    float wres, wp;
    draw_w(Ct[cidx(0, n)], U[cidx(0, n)], dr.x == 0 && n0 + n < a.Vd, P, Q, ip, iq, wres, wp);
    wf = e_fixed(mode == 0 ? wres : wp, SHL);
  }
  su[threadIdx.x] = wf;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t C = s_R;
    int y = -1, lastpos = -1;
    for (int i = 0; i < nv; ++i) {
      if (su[i] > 0) lastpos = n0 + i;
      C += su[i];
      if (C > s_tf) { y = n0 + i; break; }
    }
    if (y < 0) y = lastpos;
    out_tok[(int64_t)r * K1 + dr.y] = y;
    if (out_stats) out_stats[((int64_t)r * K1 + dr.y) * SD_NSTAT + SD_STAT_S] = (float)((double)s_S * 0x1p-40);
  }
}

// ---------------------------------------------------------------------------
// Greedy: per (listed target row, tile) the largest logit and its lowest id.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NT_L, 2) void k_lm_greedy_part(LmArgs a, LmWs w, int nm, int nn) {
  // (each fp32 part is stashed over the A/B chunks once the product is done)
  __shared__ __align__(16) float lds_ab_c[TALL_LDS_WORDS];
  uint16_t* const sa = reinterpret_cast<uint16_t*>(lds_ab_c);
  uint16_t* const sb = sa + TMS * LDK;
  float* const C = lds_ab_c;
  int mb, nb;
  if (!tile_of(nm, nn, mb, nb)) return;
  const int nrows = w.cnt[0];
  const int m0 = mb * TMS, n0 = nb * TN;
  if (m0 >= nrows) return;
  const int rr = threadIdx.x >> 3;
  ARows<MBS> ar = hidden_rows<MBS>(a, true);
#pragma unroll
  for (int i = 0; i < 2 * MBS; ++i) {
    const int li = m0 + rr + 32 * i;
    ar.row[i] = li < nrows ? w.tlist[li] : -1;
  }
  f32x16 acc[MBS][2];
  tile_gemm<MBS>(ar, a.wt, n0, a.V, a.Ht, TileLds{sa, sb}, acc);
  const int nv = min(TN, a.V - n0);
  // (unrolled: each part reads its own accumulators where it stashes them)
#pragma unroll
  for (int part = 0; part < MBS; ++part) {
    if (m0 + 64 * part >= nrows) continue;
    __syncthreads();   // the chunk buffers, or the previous part, are read
    stash_part<MBS>(acc, C, part);
    __syncthreads();
    const int row = threadIdx.x >> 2, q4 = threadIdx.x & 3;
    const int li = m0 + 64 * part + row;
    uint32_t bo = 0u;
    int bi = INT_MAX;
    int nan = 0;
    for (int e = 0; e < 32; ++e) {
      const int n = q4 * 32 + e;
      if (n >= nv) continue;
      const float z = C[cidx(row, n)];
      if (z != z) { nan = 1; continue; }
      const uint32_t o = ord_key(z);
      if (o > bo || (o == bo && n0 + n < bi)) { bo = o; bi = n0 + n; }
    }
#pragma unroll
    for (int off = 1; off < 4; off <<= 1) {
      const uint32_t o2 = __shfl_xor(bo, off);
      const int i2 = __shfl_xor(bi, off);
      if (o2 > bo || (o2 == bo && i2 < bi)) { bo = o2; bi = i2; }
      nan |= __shfl_xor(nan, off);
    }
    if (li < nrows && q4 == 0) w.gpart[(int64_t)li * nn + nb] = make_uint2(nan ? 0xFFFFFFFFu : bo, (uint32_t)bi);
  }
}

// One wave per request: for each position, the lanes reduce the tile
// partials (larger key, then lower id: any order gives the same result),
// lane jj keeps position jj's argmax, and the first mismatch with the draft
// tokens is the first bit of a ballot.
__global__ __launch_bounds__(64) void k_lm_greedy_final(LmArgs a, LmWs w, int nn, int32_t* out_acc,
                                                        int32_t* out_tok, uint32_t* out_status,
                                                        int32_t* out_argmax) {
  static_assert(WAVE == 64 && SD_MAX_K + 1 <= WAVE, "one lane per position");
  const int r = blockIdx.x;
  const int lane = threadIdx.x;
  const int K1 = a.K_max + 1;
  const int64_t base = (int64_t)r * K1;
  uint32_t st = lm_status(a, r, false);
  const int K = st ? 0 : req_k(a, r);
  int myg = INT_MAX;
  if (!st) {
    const int t0 = w.toff[r];
    for (int jj = 0; jj <= K; ++jj) {
      const uint2* pj = w.gpart + (int64_t)(t0 + jj) * nn;
      uint32_t bo = 0u;
      int bi = INT_MAX, nan = 0;
      for (int t = lane; t < nn; t += WAVE) {
        const uint2 p = pj[t];
        if (p.x == 0xFFFFFFFFu) { nan = 1; continue; }
        if (p.x > bo || (p.x == bo && (int)p.y < bi)) { bo = p.x; bi = (int)p.y; }
      }
#pragma unroll
      for (int off = WAVE / 2; off > 0; off >>= 1) {
        const uint32_t o2 = __shfl_xor(bo, off);
        const int i2 = __shfl_xor(bi, off);
        if (o2 > bo || (o2 == bo && i2 < bi)) { bo = o2; bi = i2; }
      }
      if (__any(nan)) st |= SD_ST_NONFINITE;
      if (lane == jj) myg = bi;
    }
  }
  if (st & SD_ST_INVALID_MASK) {
    if (lane < K1) {
      out_tok[base + lane] = -1;
      if (out_argmax) out_argmax[base + lane] = -1;
    }
    if (lane == 0) {
      out_acc[r] = -1;
      if (out_status) out_status[r] = st;
    }
    return;
  }
  const int idv = lane < K ? a.ids[(int64_t)r * a.K_max + lane] : -1;
  const uint64_t mis = __ballot(lane < K && idv != myg);
  const int n = mis ? __builtin_ctzll(mis) : K;
  const int gn = __shfl(myg, n);
  if (lane < K1) {
    int v = -1;
    if (lane < n) v = idv;
    else if (lane == n && !(n == K && (a.flags & SD_NO_BONUS))) v = gn;
    out_tok[base + lane] = v;
    if (out_argmax) out_argmax[base + lane] = lane <= K ? myg : -1;
  }
  if (lane == 0) {
    out_acc[r] = n;
    if (out_status) out_status[r] = st;
  }
}

// Test export: the logits of every listed row, written densely.
template <bool TGT>
__global__ __launch_bounds__(NT_L) void k_lm_dump(LmArgs a, LmWs w, int nm, int nn, float* out) {
  // (the fp32 tile is stashed over the A/B chunks once the product is done:
  // 32 KB of LDS instead of 60, so more workgroups share a CU)
  __shared__ __align__(16) float lds_ab_c[TILE_LDS_WORDS];
  uint16_t* const sa = reinterpret_cast<uint16_t*>(lds_ab_c);
  uint16_t* const sb = sa + TM * LDK;
  float* const C = lds_ab_c;
  int mb, nb;
  if (!tile_of(nm, nn, mb, nb)) return;
  const int nrows = w.cnt[TGT ? 0 : 1];
  const int m0 = mb * TM, n0 = nb * TN;
  if (m0 >= nrows) return;
  const int* list = TGT ? w.tlist : w.dlist;
  const int rr = threadIdx.x >> 3;
  ARows<1> ar = hidden_rows<1>(a, TGT);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int li = m0 + rr + 32 * i;
    ar.row[i] = li < nrows ? list[li] : -1;
  }
  const int Vs = TGT ? a.V : a.Vd;
  f32x16 acc[1][2];
  tile_gemm<1>(ar, TGT ? a.wt : a.wd, n0, Vs, TGT ? a.Ht : a.Hd, TileLds{sa, sb}, acc);
  __syncthreads();
  stash(acc[0], C);
  __syncthreads();
  for (int i = threadIdx.x; i < TM * TN; i += NT_L) {
    const int row = i / TN, n = i % TN;
    if (m0 + row < nrows && n0 + n < Vs) out[(int64_t)list[m0 + row] * Vs + n0 + n] = C[cidx(row, n)];
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
int lm_check(const sd_lmhead_args_t* s, bool sample) {
  if (!s) return SD_EINVAL;
  if (s->B < 1 || s->K_max < 0 || s->V < 1) return SD_EINVAL;
  if (s->K_max > SD_MAX_K) return SD_EUNSUPPORTED;
  if (!s->target_hidden || !s->target_weight) return SD_EINVAL;
  if (s->H_target < BK || s->H_target % BK) return SD_EINVAL;
  if ((reinterpret_cast<uintptr_t>(s->target_hidden) | reinterpret_cast<uintptr_t>(s->target_weight)) & 15u)
    return SD_EINVAL;
  if (s->K_max > 0 && !s->draft_ids) return SD_EINVAL;
  if ((int64_t)s->B * (s->K_max + 1) > INT_MAX / 4) return SD_EUNSUPPORTED;
  // (the tile engine addresses a hidden-state array by 32-bit byte offsets)
  if ((int64_t)s->B * (s->K_max + 1) * s->H_target * 2 > INT_MAX) return SD_EUNSUPPORTED;
  if ((s->flags & ~(uint32_t)SD_NO_BONUS)) return SD_EINVAL;
  if (sample) {
    if (s->V_draft < 0 || s->V_draft > s->V) return SD_EINVAL;
    if (!(s->tv_budget >= 0.0f)) return SD_EINVAL;
    if (s->K_max > 0) {
      if (!s->draft_hidden || !s->draft_weight) return SD_EINVAL;
      if (s->H_draft < BK || s->H_draft % BK) return SD_EINVAL;
      if ((int64_t)s->B * s->K_max * s->H_draft * 2 > INT_MAX) return SD_EUNSUPPORTED;
      if ((reinterpret_cast<uintptr_t>(s->draft_hidden) | reinterpret_cast<uintptr_t>(s->draft_weight)) & 15u)
        return SD_EINVAL;
    }
  }
  return SD_OK;
}

LmArgs lm_args(const sd_lmhead_args_t* s) {
  LmArgs a;
  a.th = static_cast<const uint16_t*>(s->target_hidden);
  a.dh = static_cast<const uint16_t*>(s->draft_hidden);
  a.wt = static_cast<const uint16_t*>(s->target_weight);
  a.wd = static_cast<const uint16_t*>(s->draft_weight);
  a.Ht = s->H_target;
  a.Hd = s->H_draft > 0 ? s->H_draft : BK;
  a.B = s->B;
  a.K_max = s->K_max;
  a.V = s->V;
  a.Vd = s->V_draft > 0 ? s->V_draft : s->V;
  a.ids = s->draft_ids;
  a.kpr = s->k_per_row;
  a.temp = s->temperature;
  a.D = s->tv_budget;
  a.seed = s->seed;
  a.offset = s->offset;
  a.flags = s->flags;
  return a;
}

int lm_launch_status() { return hipGetLastError() == hipSuccess ? SD_OK : SD_EHIP; }

// A 1-D grid of tile blocks, a multiple of the die count.
unsigned tile_grid(int nm, int nn) {
  const long long n = (long long)nm * nn;
  return (unsigned)((n + NXCD - 1) / NXCD * NXCD);
}

int lm_prepare(const LmArgs& a, const LmLayout& L, const LmWs& w, bool sample, hipStream_t st) {
  const int nt_max = a.B * (a.K_max + 1), nd_max = sample ? a.B * a.K_max : 0;
  hipLaunchKernelGGL(k_lm_lists, dim3(1), dim3(1024), 0, st, a, w, sample ? 1 : 0);
  if (sample) {
    const int nmx = nt_max > nd_max ? nt_max : nd_max;
    hipLaunchKernelGGL(k_lm_clear_zx, dim3((nmx + 255) / 256), dim3(256), 0, st, w, nt_max, nd_max);
  }
  (void)L;
  return lm_launch_status();
}

}  // namespace

extern "C" {

int sd_lmhead_workspace_bytes(const sd_lmhead_args_t* args, size_t* bytes) {
  if (!args || !bytes) return SD_EINVAL;
  if (args->B < 1 || args->K_max < 0 || args->V < 1 || args->V_draft < 0 || args->V_draft > args->V)
    return SD_EINVAL;
  if (args->K_max > SD_MAX_K) return SD_EUNSUPPORTED;
  *bytes = lm_layout(args->B, args->K_max, args->V, args->V_draft > 0 ? args->V_draft : args->V).total;
  return SD_OK;
}

int sd_lmhead_verify_sample(const sd_lmhead_args_t* args, void* workspace, size_t workspace_bytes,
                            int32_t* out_accepted, int32_t* out_tokens, uint32_t* out_status,
                            float* out_stats, void* stream) {
  int rc = lm_check(args, true);
  if (rc) return rc;
  if (!out_accepted || !out_tokens) return SD_EINVAL;
  const LmArgs a = lm_args(args);
  const LmLayout L = lm_layout(a.B, a.K_max, a.V, a.Vd);
  if (!workspace || workspace_bytes < L.total) return SD_EWORKSPACE;
  const LmWs w = carve(static_cast<char*>(workspace), L);
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = lm_prepare(a, L, w, true, st);
  if (rc) return rc;
  const int nt_max = a.B * (a.K_max + 1), nd_max = a.B * a.K_max;
  const int nmd = (nd_max + TM - 1) / TM;   // 64-row tiles of the pair kernels
  const int nst = (nt_max + TMS - 1) / TMS, nsd = (nd_max + TMS - 1) / TMS;   // tall tiles
  hipLaunchKernelGGL(k_lm_stats<true>, dim3(tile_grid(nst, L.ntt)), dim3(NT_L), 0, st, a, w, nst, L.ntt);
  if (nd_max > 0)
    hipLaunchKernelGGL(k_lm_stats<false>, dim3(tile_grid(nsd, L.ntd)), dim3(NT_L), 0, st, a, w, nsd, L.ntd);
  hipLaunchKernelGGL(k_lm_rowstat<true>, dim3(nt_max), dim3(256), 0, st, a, w, L.ntt);
  if (nd_max > 0)
    hipLaunchKernelGGL(k_lm_rowstat<false>, dim3(nd_max), dim3(256), 0, st, a, w, L.ntd);
  // d is needed where theta depends on it (0 < D < 1) or when statistics are asked for
  const bool tv = nd_max > 0 && ((a.D > 0.0f && a.D < 1.0f) || out_stats);
  if (tv) {
    hipLaunchKernelGGL(k_lm_tv, dim3(tile_grid(nmd, L.ntt)), dim3(NT_L), 0, st, a, w, nmd, L.ntt);
    hipLaunchKernelGGL(k_lm_tv_reduce, dim3(nd_max), dim3(256), 0, st, w, L.ntt);
  }
  hipLaunchKernelGGL(k_lm_decide, dim3(a.B), dim3(64), 0, st, a, w, tv ? 1 : 0,
                     out_accepted, out_tokens, out_status, out_stats);
  const int nmr = (a.B + TM - 1) / TM;
  hipLaunchKernelGGL(k_lm_draw_tiles, dim3(tile_grid(nmr, L.ntt)), dim3(NT_L), 0, st, a, w, nmr, L.ntt);
  hipLaunchKernelGGL(k_lm_draw_pick, dim3(a.B), dim3(NT_L), 0, st, a, w, L.ntt, out_tokens,
                     out_status, out_stats);
  return lm_launch_status();
}

int sd_lmhead_verify_greedy(const sd_lmhead_args_t* args, void* workspace, size_t workspace_bytes,
                            int32_t* out_accepted, int32_t* out_tokens, uint32_t* out_status,
                            int32_t* out_argmax, void* stream) {
  int rc = lm_check(args, false);
  if (rc) return rc;
  if (!out_accepted || !out_tokens) return SD_EINVAL;
  const LmArgs a = lm_args(args);
  const LmLayout L = lm_layout(a.B, a.K_max, a.V, a.Vd);
  if (!workspace || workspace_bytes < L.total) return SD_EWORKSPACE;
  const LmWs w = carve(static_cast<char*>(workspace), L);
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = lm_prepare(a, L, w, false, st);
  if (rc) return rc;
  const int nmt = (a.B * (a.K_max + 1) + TMS - 1) / TMS;
  hipLaunchKernelGGL(k_lm_greedy_part, dim3(tile_grid(nmt, L.ntt)), dim3(NT_L), 0, st, a, w, nmt, L.ntt);
  hipLaunchKernelGGL(k_lm_greedy_final, dim3(a.B), dim3(64), 0, st, a, w, L.ntt,
                     out_accepted, out_tokens, out_status, out_argmax);
  return lm_launch_status();
}

int sd_debug_lmhead_logits(const sd_lmhead_args_t* args, void* workspace, size_t workspace_bytes,
                           float* out_target, float* out_draft, void* stream) {
  const bool sample = out_draft != nullptr;
  int rc = lm_check(args, sample);
  if (rc) return rc;
  if (!out_target) return SD_EINVAL;
  const LmArgs a = lm_args(args);
  const LmLayout L = lm_layout(a.B, a.K_max, a.V, a.Vd);
  if (!workspace || workspace_bytes < L.total) return SD_EWORKSPACE;
  const LmWs w = carve(static_cast<char*>(workspace), L);
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = lm_prepare(a, L, w, sample, st);
  if (rc) return rc;
  const int nmt = (a.B * (a.K_max + 1) + TM - 1) / TM;
  hipLaunchKernelGGL(k_lm_dump<true>, dim3(tile_grid(nmt, L.ntt)), dim3(NT_L), 0, st, a, w, nmt, L.ntt,
                     out_target);
  if (sample && a.K_max > 0) {
    const int nmd = (a.B * a.K_max + TM - 1) / TM;
    hipLaunchKernelGGL(k_lm_dump<false>, dim3(tile_grid(nmd, L.ntd)), dim3(NT_L), 0, st, a, w, nmd,
                       L.ntd, out_draft);
  }
  return lm_launch_status();
}

}  // extern "C"
