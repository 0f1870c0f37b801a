// Activation / weight quantizers and global-scale calibration.
//
// fp8r ("BFL (fp8r / nvfp4)", fp8r bullet): one E4M3 scale per row,
//   d = fp32(amax / 448), r = fp32(1 / d), q = E4M3(fp32(x * r)).
// nvfp4 (same page, nvfp4 bullet): E4M3 scale per 16 elements times an fp32
//   global g, G = fp32(1 / g), sf = E4M3(fp32(fp32(a_b / 6) * G)),
//   r_b = fp32(G / sf), q = E2M1(fp32(x * r_b)).
// Every fp32 step is a single IEEE-rounded operation: this file is built
// with -ffp-contract=off and correctly rounded division.
#include "bsq_device.hpp"
#include "bsq_launch.hpp"

namespace bsq {

// ---- fp8r: one wave per row ---------------------------------------------------
// Each lane owns the 16-byte chunks (8 bf16) c = lane + 64 i of the row. The
// first NCH of them stay in registers between the amax pass and the encode
// pass; chunks beyond 64 * NCH (rows longer than 512 * NCH) are read twice.
// (absmax8 and encode8_fp8, the per-chunk steps, are shared with the fused
// adapter kernel.)
template <int NCH>
__global__ __launch_bounds__(256) void quant_fp8r_rows(const uint16_t* __restrict__ x, int64_t M, int K,
                                                        int64_t ldx, uint8_t* __restrict__ xq,
                                                        float* __restrict__ sx) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const uint16_t* xr = x + row * ldx;
  uint8_t* qr = xq + row * (int64_t)K;
  const int nch = K >> 3;
  uint4 buf[NCH];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      buf[i] = *reinterpret_cast<const uint4*>(xr + (int64_t)c * 8);
      amax = fmaxf(amax, absmax8(buf[i]));
    }
  }
  for (int c = lane + 64 * NCH; c < nch; c += 64)
    amax = fmaxf(amax, absmax8(*reinterpret_cast<const uint4*>(xr + (int64_t)c * 8)));
  amax = wave_max(amax);
  const float d = amax / kE4M3Max;
  const float r = d > 0.0f ? 1.0f / d : 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) *reinterpret_cast<uint2*>(qr + (int64_t)c * 8) = encode8_fp8(buf[i], r);
  }
  for (int c = lane + 64 * NCH; c < nch; c += 64)
    *reinterpret_cast<uint2*>(qr + (int64_t)c * 8) =
        encode8_fp8(*reinterpret_cast<const uint4*>(xr + (int64_t)c * 8), r);
  if (lane == 0) sx[row] = d;
}

// The same quantizer with wider per-lane pieces: each of TPR threads of a row (one wave, or a
// whole workgroup for long rows) takes pairs of adjacent 8-value chunks -- 32 bytes in, one
// 16-byte store out -- and the row maximum is combined across the row's waves through LDS.
// Measured against quant_fp8r_rows: 4096 x 3072 7.2 -> 6.5 us, 512 x 3072 3.7 -> 3.1 us, with
// identical bits.
//
// With PM, the row's maximum is not taken over the row but over pmax[row][s], s < nseg: the
// maxima of the row's 64-value segments that a GEMM epilogue already wrote (the same value,
// since the maximum is exact); everything else is unchanged.
template <int NP, int TPR, bool PM = false>
__global__ __launch_bounds__(256) void quant_fp8r_pairs(const uint16_t* __restrict__ x, int64_t M, int K,
                                                         int64_t ldx, uint8_t* __restrict__ xq,
                                                         float* __restrict__ sx, const float* __restrict__ pmax,
                                                         int nseg) {
  constexpr int WPR = TPR / 64;  // waves per row
  __shared__ float red[4];
  const int t = threadIdx.x % TPR, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const bool live = row < M;  // uniform per row, so per wave
  const uint16_t* xr = x + (live ? row : 0) * ldx;
  uint8_t* qr = xq + row * (int64_t)K;
  const int np = K >> 4;
  uint4 buf[NP][2];
  float amax = 0.0f;
  if constexpr (PM) {
    for (int sg = t; live && sg < nseg; sg += TPR) amax = fmaxf(amax, pmax[row * nseg + sg]);
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int c = t + TPR * i;
    if (live && c < np) {
      buf[i][0] = *reinterpret_cast<const uint4*>(xr + (int64_t)c * 16);
      buf[i][1] = *reinterpret_cast<const uint4*>(xr + (int64_t)c * 16 + 8);
      if constexpr (!PM) amax = fmaxf(amax, fmaxf(absmax8(buf[i][0]), absmax8(buf[i][1])));
    }
  }
  amax = wave_max(amax);
  if constexpr (WPR > 1) {
    if (lane == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < WPR; ++w) amax = fmaxf(amax, red[w]);
  }
  if (!live) return;
  const float d = amax / kE4M3Max;
  const float r = d > 0.0f ? 1.0f / d : 0.0f;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int c = t + TPR * i;
    if (c < np) {
      const uint2 lo = encode8_fp8(buf[i][0], r), hi = encode8_fp8(buf[i][1], r);
      *reinterpret_cast<uint4*>(qr + (int64_t)c * 16) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  }
  if (t == 0) sx[row] = d;
}

hipError_t launch_quant_fp8r(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* xq,
                             float* sx, hipStream_t s) {
  if (K <= 64 * 16 * 4) {  // a wave per row, four rows per workgroup
    hipLaunchKernelGGL((quant_fp8r_pairs<4, 64>), dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, x, M, (int)K,
                       ldx, xq, sx, nullptr, 0);
    return hipGetLastError();
  }
  if (K <= 256 * 16 * 4) {  // a workgroup per row
    hipLaunchKernelGGL((quant_fp8r_pairs<4, 256>), dim3((unsigned)M), dim3(256), 0, s, x, M, (int)K, ldx, xq, sx,
                       nullptr, 0);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((M + 3) / 4)), block(256);
  if (K <= 512 * 8)
    hipLaunchKernelGGL(quant_fp8r_rows<8>, grid, block, 0, s, x, M, (int)K, ldx, xq, sx);
  else
    hipLaunchKernelGGL(quant_fp8r_rows<24>, grid, block, 0, s, x, M, (int)K, ldx, xq, sx);
  return hipGetLastError();
}

hipError_t launch_encode_fp8r_rows(const uint16_t* y, int64_t M, int64_t N, int64_t ldy, const float* pmax,
                                   uint8_t* yq, float* yd, hipStream_t s) {
  const int nseg = (int)ypmax_segments(N);
  if (N <= 64 * 16 * 4) {
    hipLaunchKernelGGL((quant_fp8r_pairs<4, 64, true>), dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, y, M,
                       (int)N, ldy, yq, yd, pmax, nseg);
    return hipGetLastError();
  }
  if (N <= 256 * 16 * 4) {
    hipLaunchKernelGGL((quant_fp8r_pairs<4, 256, true>), dim3((unsigned)M), dim3(256), 0, s, y, M, (int)N, ldy, yq,
                       yd, pmax, nseg);
    return hipGetLastError();
  }
  // longer rows: the quantizer's own maximum (one more read of each row; same bits)
  return launch_quant_fp8r(y, M, N, ldy, yq, yd, s);
}

// ---- nvfp4: one thread per 16-element block ---------------------------------
__global__ __launch_bounds__(256) void quant_nvfp4_blocks(const uint16_t* __restrict__ x, int64_t M, int K,
                                                           int64_t ldx, const float* __restrict__ gptr,
                                                           uint8_t* __restrict__ xq, uint8_t* __restrict__ xs) {
  const int nb = K >> 4;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= M * nb) return;
  const int64_t row = t / nb;
  const int b = (int)(t - row * nb);
  const uint16_t* p = x + row * ldx + (int64_t)b * 16;
  const uint4 v0 = *reinterpret_cast<const uint4*>(p);
  const uint4 v1 = *reinterpret_cast<const uint4*>(p + 8);
  float f[16];
  bf16x16_to_f32(v0, v1, f);
  const float G = 1.0f / gptr[0];
  uint2 o;
  const uint32_t sf = quant_block16_nvfp4(f, G, o);
  *reinterpret_cast<uint2*>(xq + row * (int64_t)(K >> 1) + (int64_t)b * 8) = o;
  xs[row * (int64_t)nb + b] = (uint8_t)sf;
}

hipError_t launch_quant_nvfp4(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const float* g,
                              uint8_t* xq, uint8_t* xs, hipStream_t s) {
  const int64_t total = M * (K >> 4);
  hipLaunchKernelGGL(quant_nvfp4_blocks, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, x, M,
                     (int)K, ldx, g, xq, xs);
  return hipGetLastError();
}

// ---- calibration: amax over the tensor, two deterministic passes -------------
constexpr int kCalibMaxBlocks = 1024;
int calibrate_partials(int64_t M) {
  const int64_t b = (M + 3) / 4;
  return (int)(b < kCalibMaxBlocks ? b : kCalibMaxBlocks);
}

__global__ __launch_bounds__(256) void amax_partial(const uint16_t* __restrict__ x, int64_t M, int K,
                                                     int64_t ldx, float* __restrict__ partials) {
  __shared__ float red[4];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int k8 = K >> 3;  // 8-value chunks per row
  float a = 0.0f, b = 0.0f, c2 = 0.0f, d = 0.0f;
  for (int64_t row = (int64_t)blockIdx.x * 4 + wv; row < M; row += (int64_t)gridDim.x * 4) {
    const uint4* xr = reinterpret_cast<const uint4*>(x + row * ldx);
    int c = lane;
    // four loads in flight per lane (independent maxima), then the row's remainder
    for (; c + 192 < k8; c += 256) {
      const uint4 v0 = xr[c], v1 = xr[c + 64], v2 = xr[c + 128], v3 = xr[c + 192];
      a = fmaxf(a, absmax8(v0));
      b = fmaxf(b, absmax8(v1));
      c2 = fmaxf(c2, absmax8(v2));
      d = fmaxf(d, absmax8(v3));
    }
    for (; c < k8; c += 64) a = fmaxf(a, absmax8(xr[c]));
  }
  a = wave_max(fmaxf(fmaxf(a, b), fmaxf(c2, d)));
  if (lane == 0) red[wv] = a;
  __syncthreads();
  if (threadIdx.x == 0) partials[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__global__ __launch_bounds__(256) void amax_final(const float* __restrict__ partials, int n, float* out) {
  __shared__ float red[4];
  float a = 0.0f;
  for (int i = threadIdx.x; i < n; i += 256) a = fmaxf(a, partials[i]);
  a = wave_max(a);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    out[0] = m > 0.0f ? m / (kE2M1Max * kE4M3Max) : 1.0f;
  }
}

hipError_t launch_calibrate(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, float* out,
                            float* partials, hipStream_t s) {
  const int nb = calibrate_partials(M);
  hipLaunchKernelGGL(amax_partial, dim3(nb), dim3(256), 0, s, x, M, (int)K, ldx, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(amax_final, dim3(1), dim3(256), 0, s, partials, nb, out);
  return hipGetLastError();
}

}  // namespace bsq
