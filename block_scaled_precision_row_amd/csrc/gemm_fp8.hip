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
// Pipeline (layout conventions in gemm_common.hpp): each stage is 128 K
// values = 128 bytes (one full cache line) of every W row and every Xq row,
// fetched by LDS DMA into a ring of NS stage buffers; full-line rows halve
// the number of memory requests against 64-byte stages. A stage is two
// 64-deep MFMA K steps. Iteration s reads step 1 of stage s into registers
// while the MFMAs of step 0 run, waits until stage s + 1 has landed, and at
// the barrier that follows no wave reads stage s any more, so its buffer is
// refilled with stage s + NS at once; step 0 of stage s + 1 is then read
// while the MFMAs of step 1 run. NS - 1 stages are in flight behind the one
// being multiplied.
// K permutation: in step t of a stage, lane half h of an MFMA operand holds
// the 32 bytes [64 h + 32 t, 64 h + 32 t + 32) of its row -- the same for W
// and Xq, so every product pairs equal K indices.
// The epilogue scales the accumulators, converts them to bf16 into an LDS
// copy of the output tile, and writes the tile back in 16-byte row chunks.
#include "gemm_common.hpp"
#include "bsq_launch.hpp"

namespace bsq {

namespace {

using namespace gemm;

constexpr int kStageK = 128;  // K values (bytes) per row per stage

template <int BM, int BN, int NS>
struct Cfg {
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int TM = WM / 32, TN = WN / 32;
  using RA = Region<128, BN, kStageK>;  // W rows
  using RB = Region<128, BM, kStageK>;  // Xq rows
  static constexpr int A_BYTES = BN * 128, STAGE = (BN + BM) * 128;
  static constexpr int LOADS_MIN = RA::MIN_PER_WAVE + RB::MIN_PER_WAVE;  // per wave per stage
  static constexpr int TROW = BN * 2 + 16;  // bytes per row of the bf16 output tile in LDS (padded)
  static constexpr int LDS = NS * STAGE > BM * TROW ? NS * STAGE : BM * TROW;
  static_assert(NS >= 2, "one stage in flight behind the one being multiplied");
  static_assert(RA::MIN_PER_WAVE == RA::MAX_PER_WAVE && RB::MIN_PER_WAVE == RB::MAX_PER_WAVE,
                "every wave issues the same number of loads (exact vmcnt accounting)");
  static_assert((NS - 1) * LOADS_MIN < 64, "vmcnt range");
  static_assert(LDS + 4 * (BM + BN) <= 160 * 1024, "LDS budget");
};

// operands of K step t (0 or 1) of a stage: W rows from region A at `base`, Xq rows from region B at `bbase`
template <int TN, int TM>
__device__ __forceinline__ void read_ops(const uint8_t* base, const uint8_t* bbase, int rowa, int rowb, int lh, int t,
                                         v8i (&a)[TN], v8i (&b)[TM]) {
  const int c = 4 * lh + 2 * t;
#pragma unroll
  for (int i = 0; i < TN; ++i) {
    const int row = rowa + i * 32;
    const uint4 lo = *reinterpret_cast<const uint4*>(base + swz_off<128>(row, c));
    const uint4 hi = *reinterpret_cast<const uint4*>(base + swz_off<128>(row, c + 1));
    a[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int row = rowb + j * 32;
    const uint4 lo = *reinterpret_cast<const uint4*>(bbase + swz_off<128>(row, c));
    const uint4 hi = *reinterpret_cast<const uint4*>(bbase + swz_off<128>(row, c + 1));
    b[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
}

template <int TN, int TM>
__device__ __forceinline__ void mfma_all(v16f (&acc)[TN][TM], const v8i (&a)[TN], const v8i (&b)[TM]) {
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 0, 0, 0, 0, 0, 0);
}

template <int BM, int BN, int NS, bool LORA>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_fp8_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ sx,
                     const uint8_t* __restrict__ w, const float* __restrict__ sw,
                     uint16_t* __restrict__ y, int64_t ldy, int M, int N, int K, const uint16_t* lt,
                     const uint16_t* lb, int rank, int stream_y) {
  using C = Cfg<BM, BN, NS>;
  constexpr int TN = C::TN, TM = C::TM;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];
  __shared__ __attribute__((aligned(16))) float s_sx[BM];
  __shared__ __attribute__((aligned(16))) float s_sw[BN];

  int m0, n0;
  tile_of_block(M, N, BM, BN, m0, n0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  const int rows_x = M - m0 < BM ? M - m0 : BM, rows_w = N - n0 < BN ? N - n0 : BN;
  const v4i rx = buffer_rsrc(xq + (int64_t)m0 * K, (uint32_t)(rows_x * K));
  const v4i rw = buffer_rsrc(w + (int64_t)n0 * K, (uint32_t)(rows_w * K));
  const uint32_t lds0 = lds_offset(smem);

  auto issue_stage = [&](int kt) {
    const int kb = kt * kStageK;
    const uint32_t base = lds0 + (uint32_t)((kt % NS) * C::STAGE);
    dma_region<typename C::RA>(rw, base, wave, lane, K, kb, kb, K);
    dma_region<typename C::RB>(rx, base + C::A_BYTES, wave, lane, K, kb, kb, K);
  };

  // row / column scales of the tile, for the epilogue
  for (int i = tid; i < BM; i += kThreads) s_sx[i] = m0 + i < M ? sx[m0 + i] : 0.0f;
  for (int i = tid; i < BN; i += kThreads) s_sw[i] = n0 + i < N ? sw[n0 + i] : 0.0f;

  v16f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v16f{};

  const int lr = lane & 31, lh = lane >> 5;
  const int rowa = wn * C::WN + lr, rowb = wm * C::WM + lr;  // region-local rows
  const int nk = (K + kStageK - 1) / kStageK;

  // prologue: NS stages in flight, wait for the first
#pragma unroll
  for (int p = 0; p < NS; ++p) issue_stage(p);
  wait_vmcnt<(NS - 1) * C::LOADS_MIN>();
  __syncthreads();
  v8i a0[TN], b0[TM], a1[TN], b1[TM];
  read_ops<TN, TM>(smem, smem + C::A_BYTES, rowa, rowb, lh, 0, a0, b0);

  // MFMAs of one K step with the LDS reads of the next one interleaved
  auto sched = [&]() {
#pragma unroll
    for (int i = 0; i < TN * TM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                       // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, (2 * (TN + TM) + TN * TM - 1) / (TN * TM), 0);  // LDS read
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // stage s, its step 0 already in a0/b0. Stages past K read as zeros and go unused.
  for (int s = 0; s < nk; ++s) {
    const uint8_t* cur = smem + (s % NS) * C::STAGE;
    const uint8_t* nxt = smem + ((s + 1) % NS) * C::STAGE;
    read_ops<TN, TM>(cur, cur + C::A_BYTES, rowa, rowb, lh, 1, a1, b1);
    mfma_all<TN, TM>(acc, a0, b0);
    sched();
    wait_vmcnt<(NS - 2) * C::LOADS_MIN>();  // this wave's share of stage s + 1 has landed
    __syncthreads();                         // everybody's has; nobody reads stage s any more
    issue_stage(s + NS);                     // refill the buffer of stage s
    read_ops<TN, TM>(nxt, nxt + C::A_BYTES, rowa, rowb, lh, 0, a0, b0);
    mfma_all<TN, TM>(acc, a1, b1);
    sched();
  }

  // ---- epilogue: y = bf16(acc * sx[m] * sw[n]) via an LDS copy of the tile [BM][BN]
  if constexpr (LORA) {
    // with an adapter: y = bf16(acc * sx[m] * sw[n] + T B^T), the adapter's MFMAs accumulating
    // onto the scaled accumulators
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const float xs = s_sx[wm * C::WM + j * 32 + lr];
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 s4 = *reinterpret_cast<const float4*>(&s_sw[wn * C::WN + i * 32 + 8 * g + 4 * lh]);
          acc[i][j][4 * g + 0] = acc[i][j][4 * g + 0] * xs * s4.x;
          acc[i][j][4 * g + 1] = acc[i][j][4 * g + 1] * xs * s4.y;
          acc[i][j][4 * g + 2] = acc[i][j][4 * g + 2] * xs * s4.z;
          acc[i][j][4 * g + 3] = acc[i][j][4 * g + 3] * xs * s4.w;
        }
    }
    lora_update<TN, TM>(acc, lt, lb, rank, M, N, n0 + wn * C::WN, m0 + wm * C::WM, lane);
  }
  wait_vmcnt<0>();
  __syncthreads();  // all stage buffers are free now
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int ml = wm * C::WM + j * 32 + lr;
    const float xs = LORA ? 1.0f : s_sx[ml];
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nl = wn * C::WN + i * 32 + 8 * g + 4 * lh;
        const v16f& A = acc[i][j];
        const float4 s4 = LORA ? make_float4(1.0f, 1.0f, 1.0f, 1.0f) : *reinterpret_cast<const float4*>(&s_sw[nl]);
        *reinterpret_cast<uint2*>(smem + ml * C::TROW + nl * 2) =
            make_uint2(pack_bf16x2(A[4 * g + 0] * xs * s4.x, A[4 * g + 1] * xs * s4.y),
                       pack_bf16x2(A[4 * g + 2] * xs * s4.z, A[4 * g + 3] * xs * s4.w));
      }
    }
  }
  __syncthreads();
  store_tile_rows<BM, BN, C::TROW>(smem, y, ldy, M, N, m0, n0, tid, stream_y != 0);
}

template <int BM, int BN, int NS>
hipError_t run(const uint8_t* xq, const float* sx, const uint8_t* w, const float* sw, uint16_t* y,
               int64_t ldy, int64_t M, int64_t N, int64_t K, const uint16_t* lt, const uint16_t* lb, int rank,
               hipStream_t s) {
  const int tiles = (int)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
  constexpr bool kAdapter = !(BM == 256 && BN == 256);  // the 256 x 256 tile never carries one (launch_gemm_fp8)
  if (kAdapter && lt)
    hipLaunchKernelGGL((gemm_fp8_kernel<BM, BN, NS, kAdapter>), dim3(tiles), dim3(kThreads), 0, s, xq, sx, w, sw, y,
                       ldy, (int)M, (int)N, (int)K, lt, lb, rank, (int)stream_output((M + N) * K, M, N));
  else
    hipLaunchKernelGGL((gemm_fp8_kernel<BM, BN, NS, false>), dim3(tiles), dim3(kThreads), 0, s, xq, sx, w, sw, y,
                       ldy, (int)M, (int)N, (int)K, lt, lb, rank, (int)stream_output((M + N) * K, M, N));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp8(const uint8_t* xq, const float* sx, const uint8_t* w, const float* sw,
                           uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, const uint16_t* lt,
                           const uint16_t* lb, int rank, hipStream_t s) {
  // A grid of few tiles leaves compute units idle, and each busy unit is bound by the latency
  // of its own loads (three stages in flight); more, smaller tiles keep more loads in flight
  // across the chip. So while its grid fits one round on the 256 units, the smallest tile is
  // taken: 64 x 64 (its 64 KB of LDS lets two workgroups share a unit), then 64 tokens x 128
  // weight rows. Measured at K = 3072: 512 x 3072 14.8 -> 10.0 us, 320 x 3072 14.2 -> 8.4 us,
  // 512 x 3072 x 12288 46.4 -> 33.8 us.
  //
  // Larger grids take the tile of least expected time over whole rounds, with per-tile times
  // measured at K = 3072 with every unit busy: 256 x 256 46 us, 256 x 192 36 us, 128 x 128
  // 15.5 us. The square tile moves 12 % fewer operand bytes per flop through the L2 -> LDS
  // path that bounds this kernel, so it wins when the rounds come out even (16384 x 3072:
  // 7-11 % faster); the rounds decide elsewhere -- 3072 x 4096 78 -> 45.5 us on 256 x 256,
  // 3072 x 12288 131 -> 107 us on 256 x 192, 1024 x 3072 22 -> 14.7 us on 128 x 128. With an
  // adapter the square tile is left out (its epilogue does not fit the square tile's
  // registers). Every tile shape gives the same bits (the same MFMA sequence per output).
  const int64_t t64 = ((M + 63) / 64) * ((N + 63) / 64), t64x128 = ((M + 63) / 64) * ((N + 127) / 128);
  if (t64 <= 256) return run<64, 64, 4>(xq, sx, w, sw, y, ldy, M, N, K, lt, lb, rank, s);
  if (t64x128 <= 256) return run<64, 128, 4>(xq, sx, w, sw, y, ldy, M, N, K, lt, lb, rank, s);
  const int64_t c256 = lt ? INT64_MAX : rounds_cost(M, N, 256, 256, 92);
  const int64_t c192 = rounds_cost(M, N, 256, 192, 72), c128 = rounds_cost(M, N, 128, 128, 31);
  if (c256 <= c192 && c256 <= c128) return run<256, 256, 2>(xq, sx, w, sw, y, ldy, M, N, K, lt, lb, rank, s);
  if (c192 <= c128) return run<256, 192, 2>(xq, sx, w, sw, y, ldy, M, N, K, lt, lb, rank, s);
  return run<128, 128, 4>(xq, sx, w, sw, y, ldy, M, N, K, lt, lb, rank, s);
}

}  // namespace bsq
