// Fallback dequantization to bf16 ("BFL (fp8r / nvfp4)", last paragraph of
// "Kernels": weights are dequantized to the compute dtype and the layer runs
// as a regular linear). Streaming kernels, bound by HBM bandwidth.
//   nvfp4: bf16( fp32( (e2m1 * e4m3(sf)) * g ) )   the inner product is exact
//   fp8r : bf16( fp32( e4m3(q) * d_row ) )
#include "bsq_device.hpp"
#include "bsq_launch.hpp"

namespace bsq {

// one thread per 16 packed bytes = 32 values = two 16-element blocks
template <int sel>
__device__ __forceinline__ uint32_t nvfp4_pair_bf16(uint32_t w, float sf, float g) {
  const v2f e = dec_e2m1x2_f32<sel>(w);
  return pack_bf16x2((e.x * sf) * g, (e.y * sf) * g);
}

__global__ __launch_bounds__(256) void dequant_nvfp4_kernel(const uint8_t* __restrict__ w,
                                                             const uint8_t* __restrict__ sf,
                                                             const float* __restrict__ gptr, int64_t N,
                                                             int K, uint16_t* __restrict__ out) {
  const int per_row = K >> 5;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= N * per_row) return;
  const int64_t row = t / per_row;
  const int c = (int)(t - row * per_row);
  const uint4 q = *reinterpret_cast<const uint4*>(w + row * (int64_t)(K >> 1) + (int64_t)c * 16);
  const uint32_t s2 = *reinterpret_cast<const uint16_t*>(sf + row * (int64_t)(K >> 4) + (int64_t)c * 2);
  const float s0 = dec_e4m3<0>(s2), s1 = dec_e4m3<1>(s2);
  const float g = gptr[0];
  uint4 o0, o1, o2, o3;
  o0.x = nvfp4_pair_bf16<0>(q.x, s0, g); o0.y = nvfp4_pair_bf16<1>(q.x, s0, g);
  o0.z = nvfp4_pair_bf16<2>(q.x, s0, g); o0.w = nvfp4_pair_bf16<3>(q.x, s0, g);
  o1.x = nvfp4_pair_bf16<0>(q.y, s0, g); o1.y = nvfp4_pair_bf16<1>(q.y, s0, g);
  o1.z = nvfp4_pair_bf16<2>(q.y, s0, g); o1.w = nvfp4_pair_bf16<3>(q.y, s0, g);
  o2.x = nvfp4_pair_bf16<0>(q.z, s1, g); o2.y = nvfp4_pair_bf16<1>(q.z, s1, g);
  o2.z = nvfp4_pair_bf16<2>(q.z, s1, g); o2.w = nvfp4_pair_bf16<3>(q.z, s1, g);
  o3.x = nvfp4_pair_bf16<0>(q.w, s1, g); o3.y = nvfp4_pair_bf16<1>(q.w, s1, g);
  o3.z = nvfp4_pair_bf16<2>(q.w, s1, g); o3.w = nvfp4_pair_bf16<3>(q.w, s1, g);
  uint4* dst = reinterpret_cast<uint4*>(out + row * (int64_t)K + (int64_t)c * 32);
  dst[0] = o0; dst[1] = o1; dst[2] = o2; dst[3] = o3;
}

hipError_t launch_dequant_nvfp4(const uint8_t* w, const uint8_t* sf, const float* g, int64_t N,
                                int64_t K, uint16_t* out, hipStream_t s) {
  const int64_t total = N * (K >> 5);
  hipLaunchKernelGGL(dequant_nvfp4_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, w, sf,
                     g, N, (int)K, out);
  return hipGetLastError();
}

// one thread per 16 E4M3 codes
__device__ __forceinline__ uint2 fp8_quad_bf16(uint32_t w, float d) {
  const v2f a = dec_e4m3x2<false>(w), b = dec_e4m3x2<true>(w);
  return make_uint2(pack_bf16x2(a.x * d, a.y * d), pack_bf16x2(b.x * d, b.y * d));
}

__global__ __launch_bounds__(256) void dequant_fp8r_kernel(const uint8_t* __restrict__ w,
                                                            const float* __restrict__ sw, int64_t N, int K,
                                                            uint16_t* __restrict__ out) {
  const int per_row = K >> 4;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= N * per_row) return;
  const int64_t row = t / per_row;
  const int c = (int)(t - row * per_row);
  const uint4 q = *reinterpret_cast<const uint4*>(w + row * (int64_t)K + (int64_t)c * 16);
  const float d = sw[row];
  const uint2 a = fp8_quad_bf16(q.x, d), b = fp8_quad_bf16(q.y, d);
  const uint2 e = fp8_quad_bf16(q.z, d), f = fp8_quad_bf16(q.w, d);
  uint4* dst = reinterpret_cast<uint4*>(out + row * (int64_t)K + (int64_t)c * 16);
  dst[0] = make_uint4(a.x, a.y, b.x, b.y);
  dst[1] = make_uint4(e.x, e.y, f.x, f.y);
}

hipError_t launch_dequant_fp8r(const uint8_t* w, const float* sw, int64_t N, int64_t K, uint16_t* out,
                               hipStream_t s) {
  const int64_t total = N * (K >> 4);
  hipLaunchKernelGGL(dequant_fp8r_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, w, sw,
                     N, (int)K, out);
  return hipGetLastError();
}

}  // namespace bsq
