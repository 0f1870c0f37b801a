// fp8r W8A8 GEMM on the gfx950 FP8 matrix cores.
//
// "BFL (fp8r / nvfp4)", "Kernels" table: the fp8r scheme multiplies E4M3
// activations (quantized per row at run time) by E4M3 weights and applies the
// two row-wise scale vectors to the fp32 result:
//   y[m][n] = bf16( (sum_k e4m3(xq[m][k]) * e4m3(w[n][k])) * sx[m] * sw[n] ).
// Both scale vectors are rank-1 over (m, n), so they are applied once in the
// epilogue; the K loop is a plain E4M3 x E4M3 -> fp32 contraction on
// v_mfma_f32_32x32x64_f8f6f4 (no per-block scaling inside the loop).
//
// Tiling: a workgroup of 4 waves computes a BM x BN tile of Y (m x n); each
// wave owns a (BM/2) x (BN/2) quadrant as 32x32 MFMA tiles. The MFMA "A"
// operand is a 32-row slice of W and "B" a 32-row slice of Xq, so each lane's
// accumulator holds one token m and four consecutive output channels n per
// 4-register group, which makes the bf16 stores 8-byte vectors along n.
// K advances 128 bytes per iteration through a double-buffered LDS stage
// holding Xq rows then W rows, 128 bytes per row, 16-byte chunks XOR-swizzled
// by (row & 7) so that MFMA operand reads (8 rows per 128-byte phase) and
// the staging writes are bank-conflict free.
#include "bsq_device.hpp"
#include "bsq_launch.hpp"

namespace bsq {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 128;  // bytes (= E4M3 elements) of K per iteration

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

template <int BM, int BN>
struct Cfg {
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int ROWS = BM + BN;
  static constexpr int CPT = ROWS * 8 / kThreads;  // 16-byte chunks each thread stages
  static constexpr int STAGE = ROWS * 128;
  static_assert(ROWS * 8 % kThreads == 0, "tile rows must be a multiple of 32");
};

template <int BM, int BN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_fp8_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ sx,
                     const uint8_t* __restrict__ w, const float* __restrict__ sw,
                     uint16_t* __restrict__ y, int64_t ldy, int M, int N, int K) {
  using C = Cfg<BM, BN>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  grouped_tile(xcd_contiguous_id(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, 8, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // ---- staging map: chunk q = tid + 256 j -> (row, chunk) of the stage
  const uint8_t* gsrc[C::CPT];
  bool gok[C::CPT];
  int soff[C::CPT];
#pragma unroll
  for (int j = 0; j < C::CPT; ++j) {
    const int q = tid + kThreads * j, row = q >> 3, c = q & 7;
    if (row < BM) {
      const int gm = m0 + row;
      gok[j] = gm < M;
      gsrc[j] = xq + (int64_t)(gok[j] ? gm : 0) * K + c * 16;
    } else {
      const int gn = n0 + row - BM;
      gok[j] = gn < N;
      gsrc[j] = w + (int64_t)(gok[j] ? gn : 0) * K + c * 16;
    }
    soff[j] = swz(row, c);
  }
  const int nk = (K + kBK - 1) / kBK;
  uint4 stage[C::CPT];
  auto gload = [&](int kt) {
    const int kb = kt * kBK;
#pragma unroll
    for (int j = 0; j < C::CPT; ++j) {
      const int c = (tid + kThreads * j) & 7;
      stage[j] = make_uint4(0, 0, 0, 0);
      if (gok[j] && kb + c * 16 < K) stage[j] = *reinterpret_cast<const uint4*>(gsrc[j] + kb);
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* base = smem + buf * C::STAGE;
#pragma unroll
    for (int j = 0; j < C::CPT; ++j) *reinterpret_cast<uint4*>(base + soff[j]) = stage[j];
  };

  v16f acc[C::TN][C::TM];
#pragma unroll
  for (int i = 0; i < C::TN; ++i)
#pragma unroll
    for (int j = 0; j < C::TM; ++j) acc[i][j] = v16f{};

  const int lr = lane & 31, lh = lane >> 5;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* base = smem + cur * C::STAGE;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int c0 = 4 * t + 2 * lh;
      v8i a[C::TN], b[C::TM];
#pragma unroll
      for (int i = 0; i < C::TN; ++i) {
        const int row = BM + wn * C::WN + i * 32 + lr;
        const uint4 lo = *reinterpret_cast<const uint4*>(base + swz(row, c0));
        const uint4 hi = *reinterpret_cast<const uint4*>(base + swz(row, c0 + 1));
        a[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int j = 0; j < C::TM; ++j) {
        const int row = wm * C::WM + j * 32 + lr;
        const uint4 lo = *reinterpret_cast<const uint4*>(base + swz(row, c0));
        const uint4 hi = *reinterpret_cast<const uint4*>(base + swz(row, c0 + 1));
        b[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int i = 0; i < C::TN; ++i)
#pragma unroll
        for (int j = 0; j < C::TM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 0, 0, 0, 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  const bool vec_ok = (ldy & 3) == 0;  // 8-byte stores need 4-element aligned rows
  // ---- epilogue: y = bf16(acc * sx[m] * sw[n]); lane holds m = .. + lr, n = .. + 8g + 4 lh + (0..3)
#pragma unroll
  for (int j = 0; j < C::TM; ++j) {
    const int m = m0 + wm * C::WM + j * 32 + lr;
    if (m >= M) continue;
    const float xs = sx[m];
    uint16_t* yr = y + (int64_t)m * ldy;
#pragma unroll
    for (int i = 0; i < C::TN; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * C::WN + i * 32 + 8 * g + 4 * lh;
        const v16f& A = acc[i][j];
        if (n + 3 < N && vec_ok) {
          const float v0 = A[4 * g + 0] * xs * sw[n + 0], v1 = A[4 * g + 1] * xs * sw[n + 1];
          const float v2 = A[4 * g + 2] * xs * sw[n + 2], v3 = A[4 * g + 3] * xs * sw[n + 3];
          *reinterpret_cast<uint2*>(yr + n) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) yr[n + e] = (uint16_t)(pack_bf16x2(A[4 * g + e] * xs * sw[n + e], 0.0f) & 0xFFFFu);
        }
      }
    }
  }
}

template <int BM, int BN>
hipError_t run(const uint8_t* xq, const float* sx, const uint8_t* w, const float* sw, uint16_t* y,
               int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  using C = Cfg<BM, BN>;
  const size_t lds = 2 * C::STAGE;
  static std::atomic<unsigned long long> lds_set{0};
  hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(&gemm_fp8_kernel<BM, BN>), (int)lds, lds_set);
  if (e != hipSuccess) return e;
  const int tiles = (int)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
  hipLaunchKernelGGL((gemm_fp8_kernel<BM, BN>), dim3(tiles), dim3(kThreads), lds, s, xq, sx, w, sw, y, ldy,
                     (int)M, (int)N, (int)K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp8(const uint8_t* xq, const float* sx, const uint8_t* w, const float* sw,
                           uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  // pick the tile whose grid best fills the 256 compute units
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t t192 = ((M + 255) / 256) * ((N + 191) / 192);
  if (t256 >= 256 && t256 % 256 == 0) return run<256, 256>(xq, sx, w, sw, y, ldy, M, N, K, s);
  if (t192 >= 192) return run<256, 192>(xq, sx, w, sw, y, ldy, M, N, K, s);
  return run<128, 128>(xq, sx, w, sw, y, ldy, M, N, K, s);
}

}  // namespace bsq
