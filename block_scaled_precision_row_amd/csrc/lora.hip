// Low-rank adapter (LoRA) down projection on the matrix cores: T = bf16(s * X A^T).
//
// "FLUX 3 Image Klein vs Qwen-Image-2.1" (model overview) and the FLUX 3 Image
// Klein open-source release page (section three, speed figures): the quantized
// model can run with a LoRA attached. The adapter adds s * B (A x) to the
// linear's output; its rank-r intermediate T = s * X A^T [M][r] is computed
// here from the unquantized bf16 activations and held in bf16 (the adapter
// scale applied before that rounding), and the GEMM epilogues add T B^T.
//
// A workgroup owns 32 rows of X; its 8 waves split K in 64-deep chunks (wave
// w takes chunks w, w + 8, ...). v_mfma_f32_32x32x16_bf16 takes 32 adapter
// rows as the A operand (RT tiles of 32 cover the rank) and the 32 X rows as
// the B operand, so a lane accumulates token m = lane % 32 and adapter rows
// j = 32 r + 8 g + 4 (lane / 32) + e in register 4 g + e of tile r. In a chunk
// starting at kc, lane half h holds K values [kc + 32 h, kc + 32 h + 32) of
// both operands in 4 MFMA steps of 8, so each lane reads 64 contiguous bytes
// of each of its rows. The adapter matrix (r x K bf16) is read by every
// workgroup and stays in L2; X streams from HBM once. The 8 partial tiles
// are summed through LDS in wave order, so the result does not depend on
// timing.
#include "bsq_device.hpp"
#include "bsq_launch.hpp"

namespace bsq {

namespace {

constexpr int kDownWaves = 8;
constexpr int kDownRows = 32;

template <int RT>
struct DownOps {
  uint4 x[4];      // this lane's 32 values of its X row
  uint4 a[RT][4];  // and of adapter rows 32 r + lane % 32
};

__device__ __forceinline__ v8bf as_v8bf(uint4 u) {
  union {
    uint4 u;
    v8bf h;
  } c;
  c.u = u;
  return c.h;
}

template <int RT>
__global__ __launch_bounds__(64 * kDownWaves) void lora_down_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                                     const uint16_t* __restrict__ a, int M, int K,
                                                                     int rank, float scale,
                                                                     uint16_t* __restrict__ t) {
  __shared__ float red[kDownWaves * RT * 16 * 64];
  const int m0 = blockIdx.x * kDownRows;
  const int rows = M - m0 < kDownRows ? M - m0 : kDownRows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lh = lane >> 5;

  // rows past M and adapter rows past the rank read as zeros (offsets past the records)
  const rsrc_t rx = make_rsrc(x + (int64_t)m0 * ldx, (uint32_t)rows * (uint32_t)ldx * 2u);
  const rsrc_t ra = make_rsrc(a, (uint32_t)rank * (uint32_t)K * 2u);
  const uint32_t xrow = (uint32_t)lr * (uint32_t)ldx * 2u;
  uint32_t arow[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) arow[r] = (uint32_t)(32 * r + lr) * (uint32_t)K * 2u;

  const int nch = (K + 63) / 64;
  auto load = [&](DownOps<RT>& o, int c) __attribute__((always_inline)) {
    const int kc = c * 64 + 32 * lh;  // K % 32 == 0: a lane's 32 values are all inside K or all past it
    const bool ok = c < nch && kc < K;
#pragma unroll
    for (int q = 0; q < 4; ++q) o.x[q] = bload16(rx, ok ? xrow + (uint32_t)kc * 2u + 16u * q : kBufOut);
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) o.a[r][q] = bload16(ra, ok ? arow[r] + (uint32_t)kc * 2u + 16u * q : kBufOut);
  };

  v16f acc[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) acc[r] = v16f{};
  DownOps<RT> cur, nxt;
  load(cur, wave);
  for (int c = wave; c < nch; c += kDownWaves) {
    load(nxt, c + kDownWaves);  // past the wave's last chunk: reads zeros, unused
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < RT; ++r)
        acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_v8bf(cur.a[r][q]), as_v8bf(cur.x[q]), acc[r], 0, 0, 0);
    cur = nxt;
  }

#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int e = 0; e < 16; ++e) red[((wave * RT + r) * 16 + e) * 64 + lane] = acc[r][e];
  __syncthreads();

  // output (ml, j): adapter row j = 32 r + jj sits in register 4 (jj / 8) + jj % 4 of lane
  // ml + 32 ((jj / 4) % 2); consecutive threads write consecutive j of a row
  for (int idx = tid; idx < kDownRows * rank; idx += 64 * kDownWaves) {
    const int ml = idx / rank, j = idx - ml * rank;
    if (ml >= rows) break;  // rows only grow with idx
    const int r = j >> 5, jj = j & 31;
    const int reg = 4 * (jj >> 3) + (jj & 3), ln = ml + 32 * ((jj >> 2) & 1);
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kDownWaves; ++w) sum += red[((w * RT + r) * 16 + reg) * 64 + ln];
    t[(int64_t)(m0 + ml) * rank + j] = (uint16_t)(pack_bf16x2(scale * sum, 0.0f) & 0xFFFFu);
  }
}

template <int RT>
hipError_t run_down(const uint16_t* x, int64_t ldx, const uint16_t* a, int64_t M, int64_t K, int rank, float scale,
                    uint16_t* t, hipStream_t s) {
  const unsigned blocks = (unsigned)((M + kDownRows - 1) / kDownRows);
  hipLaunchKernelGGL((lora_down_kernel<RT>), dim3(blocks), dim3(64 * kDownWaves), 0, s, x, ldx, a, (int)M, (int)K,
                     rank, scale, t);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lora_down(const uint16_t* x, int64_t ldx, const uint16_t* a, int64_t M, int64_t K, int rank,
                            float scale, uint16_t* t, hipStream_t s) {
  if (rank <= 32) return run_down<1>(x, ldx, a, M, K, rank, scale, t, s);
  if (rank <= 64) return run_down<2>(x, ldx, a, M, K, rank, scale, t, s);
  return run_down<4>(x, ldx, a, M, K, rank, scale, t, s);
}

}  // namespace bsq
