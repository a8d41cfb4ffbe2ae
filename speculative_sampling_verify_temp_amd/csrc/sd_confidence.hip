// Draft-side confidence on gfx950: the top-1 probability of each draft row
// and the draft length an early-stop threshold implies ("What I Gave Up to
// Make Speculative Decoding Faster", section "Confidence-guided early stop":
// after each draft token, the probability of the most likely token is taken
// from the logits already produced; below a threshold the draft stops, and
// that last token is still verified).
//
// Two launches on the caller's stream:
//   k_draft_confidence  one 256-thread workgroup per draft row: one pass over
//                       the row from HBM, a running max and a running sum of
//                       exp2((z - max) c) per thread (rescaled when the max
//                       moves, once per 4 vectors), then a block max and an
//                       fp64 block sum: top1 = 1 / sum.
//   k_confidence_k      one thread per request: the first row below the
//                       threshold ends the proposal.
// HBM-bound: every logit is read once, 16 bytes per load, 4 loads in flight
// per thread, several workgroups per CU.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "sd_verify.h"
#include "sdv_device.h"

using namespace sdv;

namespace {

constexpr int NT_C = 256;   // threads per row
constexpr int UC = 4;       // 16-byte loads in flight per thread

// Elements of logit e of a 16-byte word group as fp32 (bf16: 8 per word
// group, fp32: 4).
template <int DT>
struct Lane16 {
  static constexpr int N = DT == SD_BF16 ? 8 : 4;
  __device__ static void unpack(const uint4& w, float (&z)[8]) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
    if constexpr (DT == SD_BF16) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        z[2 * e] = __uint_as_float(u[e] << 16);
        z[2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) z[e] = __uint_as_float(u[e]);
    }
  }
};

template <int DT>
__global__ __launch_bounds__(NT_C) void k_draft_confidence(const char* __restrict__ base,
                                                           int64_t row_bytes, int K, int V,
                                                           const float* __restrict__ temp,
                                                           float* __restrict__ top1) {
  constexpr int N = Lane16<DT>::N;
  __shared__ float sf[NT_C / WAVE];
  __shared__ double sd[NT_C / WAVE];
  __shared__ int si[NT_C / WAVE];
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int r = row / K;
  const char* p = base + (int64_t)row * row_bytes;
  const float T = temp ? temp[r] : 1.0f;
  const bool t_ok = T > 0.0f && T < INFINITY;
  const float c = t_ok ? 1.4426950408889634f / T : 1.0f;
  const int nvec = (V + N - 1) / N;
  // The row as a buffer resource over its 16-byte extent: loads past it
  // read zeros and touch no memory.
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0, nvec * 16, 0x00020000);
  float m = -INFINITY, s = 0.0f;
  int nan_seen = 0;   // NaNs in groups with no other value above -inf
  for (int k0 = 0; k0 < nvec; k0 += NT_C * UC) {
    uint4 w[UC];
#pragma unroll
    for (int u = 0; u < UC; ++u) {
      const uint32_t off = (uint32_t)(k0 + u * NT_C + tid) * 16u;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2);   // read once
      w[u] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    float z[UC][8];
    float gm = -INFINITY;
#pragma unroll
    for (int u = 0; u < UC; ++u) {
      Lane16<DT>::unpack(w[u], z[u]);
      const int i0 = (k0 + u * NT_C + tid) * N;
      if (i0 + N > V) {   // the vector that holds the row end, or one past it
#pragma unroll
        for (int e = 0; e < N; ++e)
          if (i0 + e >= V) z[u][e] = -INFINITY;
      }
#pragma unroll
      for (int e = 0; e < N; ++e) gm = fmaxf(gm, z[u][e]);
    }
    if (gm > -INFINITY) {
      const float mn = fmaxf(m, gm);
      const float g = mn * c;
      s *= fast_exp2(fmaf(m, c, -g));   // 0 while m = -inf
      float t = 0.0f;
#pragma unroll
      for (int u = 0; u < UC; ++u)
#pragma unroll
        for (int e = 0; e < N; ++e) t += fast_exp2(fmaf(z[u][e], c, -g));
      s += t;
      m = mn;
    } else {
      // (fmaxf passes over NaN, so a group of -inf and NaN lands here)
#pragma unroll
      for (int u = 0; u < UC; ++u)
#pragma unroll
        for (int e = 0; e < N; ++e) nan_seen |= z[u][e] != z[u][e];
    }
  }
  // A NaN logit makes the running sum NaN, a +inf one the max +inf (and its
  // own term NaN): no per-logit test is needed.
  const int bad = (m == INFINITY) || (s != s) || nan_seen;
  const float M = block_max<NT_C>(m, sf);
  const double part = (m > -INFINITY && !bad) ? (double)s * (double)fast_exp2((m - M) * c) : 0.0;
  const double Z = block_sum<NT_C>(part, sd);
  const int any_bad = block_or<NT_C>(bad, si);
  if (tid == 0) top1[row] = (any_bad || !t_ok || !(Z > 0.0)) ? __builtin_nanf("") : (float)(1.0 / Z);
}

__global__ void k_confidence_k(const float* __restrict__ top1, int B, int K, float threshold,
                               int32_t* __restrict__ out_k) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= B) return;
  int k = K;
  for (int j = 0; j < K; ++j)
    if (top1[(int64_t)r * K + j] < threshold) {   // NaN compares false
      k = j + 1;
      break;
    }
  out_k[r] = k;
}

}  // namespace

extern "C" int sd_draft_confidence(const void* draft_logits, int32_t dtype, int32_t B, int32_t K_max,
                                   int32_t V, int64_t ld_draft, const float* temperature,
                                   float threshold, float* out_top1, int32_t* out_k, void* stream) {
  if (dtype != SD_F32 && dtype != SD_BF16) return SD_EINVAL;
  const int es = dtype == SD_BF16 ? 2 : 4;
  if (!draft_logits || !out_top1 || B < 1 || K_max < 1 || V < 1 || ld_draft < V ||
      (ld_draft * es) % 16 != 0 || ((uintptr_t)draft_logits % 16) != 0 || threshold != threshold)
    return SD_EINVAL;
  if ((int64_t)B * K_max > 0x7FFFFFFF) return SD_EUNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int rows = B * K_max;
  if (dtype == SD_BF16)
    hipLaunchKernelGGL(k_draft_confidence<SD_BF16>, dim3(rows), dim3(NT_C), 0, st,
                       static_cast<const char*>(draft_logits), ld_draft * es, (int)K_max, (int)V,
                       temperature, out_top1);
  else
    hipLaunchKernelGGL(k_draft_confidence<SD_F32>, dim3(rows), dim3(NT_C), 0, st,
                       static_cast<const char*>(draft_logits), ld_draft * es, (int)K_max, (int)V,
                       temperature, out_top1);
  if (hipGetLastError() != hipSuccess) return SD_EHIP;
  if (out_k) {
    hipLaunchKernelGGL(k_confidence_k, dim3((B + 255) / 256), dim3(256), 0, st, out_top1, (int)B,
                       (int)K_max, threshold, out_k);
    if (hipGetLastError() != hipSuccess) return SD_EHIP;
  }
  return SD_OK;
}
