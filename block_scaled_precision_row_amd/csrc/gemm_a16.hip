// Weight-only GEMMs (W4A16, W8A16): bf16 activations as stored, weights decoded
// to exact bf16 in registers, bf16 matrix cores.
//
// "BFL (fp8r / nvfp4)", "Kernels" table and its last paragraph: the weight-only
// fallback keeps the activations in bf16 and dequantizes the weights,
//   W4A16: y[m][n] = bf16( (sum_k x[m][k] * wh[n][k]) * gw ),
//          wh = e2m1(wq) * e4m3(block scale of its 16 K values)
//   W8A16: y[m][n] = bf16( (sum_k x[m][k] * e4m3(w[n][k])) * sw[n] ).
// Both decoded weight values are exact in bf16 (e2m1 x e4m3 has at most six
// significant bits; an E4M3 value has four), so the contraction runs on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation, the same products as the
// dequantize-then-multiply fallback without rounding W to bf16 first.
//
// Data movement (conventions in gemm_common.hpp): a stage is 128 K values --
// 256 bytes of every bf16 X row, 64 bytes of packed E2M1 (plus 8 block-scale
// bytes) or 128 bytes of E4M3 of every W row -- copied to LDS by LDS DMA into
// one of two stage buffers while the other is multiplied. X fragments go from
// LDS to the MFMA as they are; W fragments are read once per 64-deep group and
// decoded right before each 16-deep K step: nvfp4 pairs through fp32 (one
// v_cvt_scalef32_pk_f32_fp4, two multiplies by the block scale, one packing
// conversion: every step exact), E4M3 pairs with one v_cvt_scalef32_pk_bf16_fp8.
//
// K permutation: lane half h of both MFMA operands covers K values
// [64 h, 64 h + 64) of a stage, eight per K step t at [64 h + 8 t, + 8): one
// 16-byte X chunk, four bytes of packed W (or eight of E4M3), inside one block
// of 16 for the scale. Every product pairs equal K indices.
#include "gemm_common.hpp"
#include "bsq_launch.hpp"

namespace bsq {

namespace {

using namespace gemm;

constexpr int kAK = 128;  // K values per stage

// nvfp4 block scales of a stage: 8 bytes (the stage's 8 blocks of 16) per W row, copied by
// dword LDS DMA, two lanes per row and 32 rows per load, spread over the waves. Loads of K
// past the end read zeros (their offset is out of range).
template <int ROWS>
__device__ __forceinline__ void dma_scales8(const v4i& rsrc, uint32_t lds_base, int wave, int lane, int ks, int kb,
                                            int K) {
  constexpr int LOADS = Scales8<ROWS>::LOADS;
#pragma unroll
  for (int i = 0; i < (LOADS + 3) / 4; ++i) {
    const int ld = wave + 4 * i;
    if (ld >= LOADS) break;  // wave-uniform
    const DmaAddr d = scales8_load(ld, lane, ks, kb, K);
    dma4(rsrc, lds_base + ld * 256, d.voff, d.soff);
  }
}

__device__ __forceinline__ uint32_t bf2u(v2bf v) {
  union { v2bf h; uint32_t u; } c;
  c.h = v;
  return c.u;
}

// eight E2M1 values (one dword, low nibble first) times the block scale s -> bf16
template <int P>
__device__ __forceinline__ uint32_t dec_fp4x2(uint32_t w, float s) {
  const v2f f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, P);
  return bf2u(v2bf{(__bf16)(f.x * s), (__bf16)(f.y * s)});
}
__device__ __forceinline__ uint4 dec_fp4x8(uint32_t w, float s) {
  return make_uint4(dec_fp4x2<0>(w, s), dec_fp4x2<1>(w, s), dec_fp4x2<2>(w, s), dec_fp4x2<3>(w, s));
}
// eight E4M3 values (two dwords) -> bf16
__device__ __forceinline__ uint4 dec_e4m3x8(uint32_t lo, uint32_t hi) {
  return make_uint4(bf2u(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
                    bf2u(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
                    bf2u(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
                    bf2u(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true)));
}

template <int BM, int BN, int MODE, bool LORA>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_a16_kernel(DecArgs a) {
  constexpr bool FP4 = MODE == kW4A16;
  using C = ACfg<BM, BN, FP4>;
  constexpr int TN = C::TN, TM = C::TM;
  constexpr int RQ = FP4 ? 1 : 2;  // 16-byte weight chunks per lane and 64-deep group
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];
  __shared__ __attribute__((aligned(16))) float s_sw[BN];

  const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
  int m0, n0;
  tile_of_block(M, N, BM, BN, m0, n0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  const int rows_x = M - m0 < BM ? M - m0 : BM, rows_w = N - n0 < BN ? N - n0 : BN;
  const int xpitch = (int)a.ldx * 2, wpitch = FP4 ? K / 2 : K, ks = K / 16;
  const v4i rx = buffer_rsrc(a.x + (int64_t)m0 * a.ldx, (uint32_t)(rows_x * xpitch));
  const v4i rw = buffer_rsrc(a.w + (int64_t)n0 * wpitch, (uint32_t)(rows_w * wpitch));
  const v4i rs = FP4 ? buffer_rsrc(a.ws + (int64_t)n0 * ks, (uint32_t)(rows_w * ks)) : v4i{};
  const uint32_t lds0 = lds_offset(smem);

  // fetch stage kt into buffer kt % 2 (stages past K read as zeros)
  auto issue_stage = [&](int kt) {
    const int kb = kt * kAK;
    const uint32_t base = lds0 + (uint32_t)((kt & 1) * C::STAGE);
    dma_region<typename C::RX>(rx, base + C::X_OFF, wave, lane, xpitch, 2 * kb, kb, K);
    dma_region<typename C::RW>(rw, base + C::W_OFF, wave, lane, wpitch, FP4 ? kb / 2 : kb, kb, K);
    if constexpr (FP4) dma_scales8<BN>(rs, base + C::S_OFF, wave, lane, ks, kb, K);
  };

  if (MODE == kW8A16)
    for (int i = tid; i < BN; i += kThreads) s_sw[i] = n0 + i < N ? a.sw[n0 + i] : 0.0f;

  v16f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v16f{};

  const int lr = lane & 31, lh = lane >> 5;
  const int rowa = wn * C::WN + lr, rowb = wm * C::WM + lr;  // region-local rows (W, X)
  const int nk = (K + kAK - 1) / kAK;

  uint4 r0[TN][RQ], r1[TN][RQ];  // raw weight bytes of the current / next 64-deep group
  uint32_t sc[TN];               // nvfp4: the lane's 4 block scales of the stage, as E4M3 bytes
  uint4 x0[TM], x1[TM];          // X fragments of two consecutive K steps
  uint4 d0[TN], d1[TN];          // decoded W fragments of two consecutive K steps

  // group g (0, 1) of the stage at `st`: this lane's K values [64 h + 32 g, + 32) of each W row
  auto read_w = [&](const uint8_t* st, int g, uint4 (&r)[TN][RQ]) {
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const int row = rowa + i * 32;
      if constexpr (FP4) {
        r[i][0] = *reinterpret_cast<const uint4*>(st + C::W_OFF + swz_off<64>(row, 2 * lh + g));
      } else {
        r[i][0] = *reinterpret_cast<const uint4*>(st + C::W_OFF + swz_off<128>(row, 4 * lh + 2 * g));
        r[i][1] = *reinterpret_cast<const uint4*>(st + C::W_OFF + swz_off<128>(row, 4 * lh + 2 * g + 1));
      }
    }
  };
  auto read_sc = [&](const uint8_t* st) {
    if constexpr (FP4) {
#pragma unroll
      for (int i = 0; i < TN; ++i)
        sc[i] = *reinterpret_cast<const uint32_t*>(st + C::S_OFF + (rowa + i * 32) * 8 + 4 * lh);
    }
  };
  // K step t (0..7) of the stage at `st`: X chunk 8 h + t of each row
  auto read_x = [&](const uint8_t* st, int t, uint4 (&x)[TM]) {
#pragma unroll
    for (int j = 0; j < TM; ++j)
      x[j] = *reinterpret_cast<const uint4*>(st + C::X_OFF + swz_off<256>(rowb + j * 32, 8 * lh + t));
  };
  // W fragments of step u (0..3) of group g from the group's raw bytes
  auto decode = [&](const uint4 (&r)[TN][RQ], int g, int u, uint4 (&d)[TN]) {
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      if constexpr (FP4) {
        const uint32_t w = u == 0 ? r[i][0].x : u == 1 ? r[i][0].y : u == 2 ? r[i][0].z : r[i][0].w;
        const int b = 2 * g + (u >> 1);  // block 4 h + b of the stage
        const float s = __builtin_amdgcn_cvt_f32_fp8((int)(sc[i] >> (8 * b)), 0);
        d[i] = dec_fp4x8(w, s);
      } else {
        const uint4& q = r[i][u >> 1];
        d[i] = (u & 1) ? dec_e4m3x8(q.z, q.w) : dec_e4m3x8(q.x, q.y);
      }
    }
  };
  auto mfmas = [&](const uint4 (&d)[TN], const uint4 (&x)[TM]) {
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        union { uint4 u; v8bf h; } p, q;
        p.u = d[i];
        q.u = x[j];
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p.h, q.h, acc[i][j], 0, 0, 0);
      }
  };

  issue_stage(0);
  issue_stage(1);
  wait_vmcnt<0>();
  __syncthreads();
  read_sc(smem);
  read_w(smem, 0, r0);
  read_x(smem, 0, x0);
  decode(r0, 0, 0, d0);

  // the epilogue's scaling and bf16 conversion of accumulator tile t into the LDS copy of the
  // output tile (see the epilogue below); without an adapter the last K stage does it
  const float gw = FP4 ? a.gw[0] : 1.0f;
  constexpr bool kLoopOut = !LORA;
  auto tile_out = [&](int t) {
    const int i = t / TM, j = t % TM;
    const int ml = wm * C::WM + j * 32 + lr;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int nl = wn * C::WN + i * 32 + 8 * g + 4 * lh;
      const v16f& A = acc[i][j];
      float sv[4] = {gw, gw, gw, gw};
      if (LORA) {
        sv[0] = sv[1] = sv[2] = sv[3] = 1.0f;
      } else if (!FP4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[e] = s_sw[nl + e];
      }
      *reinterpret_cast<uint2*>(smem + ml * C::TROW + nl * 2) =
          make_uint2(pack_bf16x2(A[4 * g + 0] * sv[0], A[4 * g + 1] * sv[1]),
                     pack_bf16x2(A[4 * g + 2] * sv[2], A[4 * g + 3] * sv[3]));
    }
  };

  // Stage s sits in buffer s % 2 and stage s + 1 in the other. Each K step's MFMAs run while
  // the next step's X chunks are read and its W fragments decoded. Once the last step's chunks
  // are read, every wave waits for stage s + 1, the barrier publishes it (and ends all reads
  // of stage s), and stage s + 2 is fetched into buffer s % 2. Without an adapter the last
  // stage is peeled: after its barrier no stage buffer is read any more (and no load is in
  // flight), so each tile is written to the output copy under the next tile's last MFMA.
  auto stage = [&](int s, auto last) __attribute__((always_inline)) {
    constexpr bool LAST = decltype(last)::value;
    const uint8_t* cur = smem + (s & 1) * C::STAGE;
    const uint8_t* nxt = smem + ((s + 1) & 1) * C::STAGE;
    read_x(cur, 1, x1);
    decode(r0, 0, 1, d1);
    mfmas(d0, x0);
    read_x(cur, 2, x0);
    decode(r0, 0, 2, d0);
    mfmas(d1, x1);
    read_x(cur, 3, x1);
    read_w(cur, 1, r1);
    decode(r0, 0, 3, d1);
    mfmas(d0, x0);
    read_x(cur, 4, x0);
    decode(r1, 1, 0, d0);
    mfmas(d1, x1);
    read_x(cur, 5, x1);
    decode(r1, 1, 1, d1);
    mfmas(d0, x0);
    read_x(cur, 6, x0);
    decode(r1, 1, 2, d0);
    mfmas(d1, x1);
    read_x(cur, 7, x1);
    decode(r1, 1, 3, d1);
    mfmas(d0, x0);
    // every read of stage s is issued: the barrier (and the refill of its buffer) go between
    // the last two steps' MFMAs, which run on while the wave waits and the next stage's first
    // operands are read
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();
    __syncthreads();
    if constexpr (LAST) {
#pragma unroll
      for (int k = 0; k < TN * TM; ++k) {
        const int i = k / TM, j = k % TM;
        union { uint4 u; v8bf h; } p, q;
        p.u = d1[i];
        q.u = x1[j];
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p.h, q.h, acc[i][j], 0, 0, 0);
        if (k > 0) tile_out(k - 1);
      }
      tile_out(TN * TM - 1);
    } else {
      issue_stage(s + 2);
      read_sc(nxt);
      read_w(nxt, 0, r0);
      read_x(nxt, 0, x0);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(d1, x1);
      decode(r0, 0, 0, d0);
    }
  };
  int s = 0;
  for (; s + 1 < nk; ++s) stage(s, std::false_type{});
  stage(s, std::integral_constant<bool, kLoopOut>{});

  // ---- epilogue: y = bf16(acc * gw) (W4A16) or bf16(acc * sw[n]) (W8A16), via an LDS copy of
  // the tile [BM][BN]
  if constexpr (LORA) {
    // with an adapter: y = bf16(acc * scale + T B^T), the adapter's MFMAs accumulating onto the
    // scaled accumulators
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nl = wn * C::WN + i * 32 + 8 * g + 4 * lh;
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][4 * g + e] *= FP4 ? gw : s_sw[nl + e];
      }
    lora_update<TN, TM>(acc, a.lt, a.lb, a.rank, M, N, n0 + wn * C::WN, m0 + wm * C::WM, lane);
  }
  wait_vmcnt<0>();
  __syncthreads();  // all stage buffers are free now
#pragma unroll
  for (int j = 0; j < (kLoopOut ? 0 : TM); ++j) {
    const int ml = wm * C::WM + j * 32 + lr;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nl = wn * C::WN + i * 32 + 8 * g + 4 * lh;
        const v16f& A = acc[i][j];
        float s[4] = {gw, gw, gw, gw};
        if (LORA) {
          s[0] = s[1] = s[2] = s[3] = 1.0f;
        } else if (!FP4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) s[e] = s_sw[nl + e];
        }
        *reinterpret_cast<uint2*>(smem + ml * C::TROW + nl * 2) =
            make_uint2(pack_bf16x2(A[4 * g + 0] * s[0], A[4 * g + 1] * s[1]),
                       pack_bf16x2(A[4 * g + 2] * s[2], A[4 * g + 3] * s[3]));
      }
    }
  }
  __syncthreads();
  if (a.y) store_tile_rows<BM, BN, C::TROW>(smem, a.y, a.ldy, M, N, m0, n0, tid, a.stream_y != 0);
  // optionally Y encoded for the next quantized linear ("BFL (fp8r / nvfp4)": every quantized
  // linear quantizes its input at run time), from the same bf16 values: nvfp4 16-blocks along
  // this N (inside the tile), or the row maxima of an fp8r encoding (its row scale spans every
  // tile of the row; one pass after the GEMM encodes)
  if (a.yq) quant_tile_rows<BM, BN, C::TROW>(smem, a.yq, a.ys, 1.0f / a.gy[0], M, N, m0, n0, tid);
  if (a.ypmax) rowmax_tile<BM, BN, C::TROW>(smem, a.ypmax, M, N, m0, n0, tid);
}

template <int BM, int BN, int MODE>
hipError_t run(const DecArgs& a, hipStream_t s) {
  const int tiles = (int)(((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN));
  if (a.lt)
    hipLaunchKernelGGL((gemm_a16_kernel<BM, BN, MODE, true>), dim3(tiles), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_a16_kernel<BM, BN, MODE, false>), dim3(tiles), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int MODE>
hipError_t pick(const DecArgs& args, hipStream_t s) {
  constexpr bool FP4 = MODE == kW4A16;
  DecArgs a = args;
  a.stream_y = stream_output(a.M * 2 * a.K + a.N * (FP4 ? a.K / 2 + a.K / 16 : a.K), a.M, a.N);  // bf16 X + W
  // While its grid fits one round on the 256 compute units, the smallest tile, as in the other
  // tiled GEMMs. Larger grids take the tile of least expected time over whole rounds (a partial
  // last round costs a full one), with per-tile times measured at K = 3072 with every unit busy:
  //   nvfp4 256 x 192 75 us, 256 x 128 55 us, 128 x 128 34 us (the widest tile re-reads X for
  //     the fewest weight rows: 4096 x 12288 333 -> 299 us, 3072 x 3072 105 -> 73 us);
  //   E4M3 (cheap to decode) 128 x 256 48 us, 128 x 192 39.5 us, 128 x 128 29 us (3072 x 3072
  //     90 -> 73 us, 4096 x 3072 92 -> 81 us on 128 x 192).
  // Costs below are those times in half-microseconds for E4M3, microseconds for nvfp4.
  const int64_t t64 = ((a.M + 63) / 64) * ((a.N + 63) / 64), t64x128 = ((a.M + 63) / 64) * ((a.N + 127) / 128);
  if (t64 <= 256) return run<64, 64, MODE>(a, s);
  if (t64x128 <= 256) return run<64, 128, MODE>(a, s);
  constexpr int LBM = FP4 ? 256 : 128, LBN = FP4 ? 192 : 256, MBM = FP4 ? 256 : 128, MBN = FP4 ? 128 : 192;
  const int64_t cl = rounds_cost(a.M, a.N, LBM, LBN, FP4 ? 75 : 96);
  const int64_t cm = rounds_cost(a.M, a.N, MBM, MBN, FP4 ? 55 : 79);
  const int64_t cs = rounds_cost(a.M, a.N, 128, 128, FP4 ? 34 : 58);
  if (cl <= cm && cl <= cs) return run<LBM, LBN, MODE>(a, s);
  if (cm <= cs) return run<MBM, MBN, MODE>(a, s);
  return run<128, 128, MODE>(a, s);
}

}  // namespace

bool gemm_a16_supported(DecMode mode, const DecArgs& a) {
  if (mode != kW4A16 && mode != kW8A16) return false;
  // dword block-scale copies need K % 64 == 0; buffer offsets of 256 X rows stay below 2^30
  if (mode == kW4A16 && a.K % 64 != 0) return false;
  return a.ldx < ((int64_t)1 << 21) && a.K < ((int64_t)1 << 22);
}

hipError_t launch_gemm_a16(DecMode mode, const DecArgs& a, hipStream_t s) {
  return mode == kW4A16 ? pick<kW4A16>(a, s) : pick<kW8A16>(a, s);
}

}  // namespace bsq
