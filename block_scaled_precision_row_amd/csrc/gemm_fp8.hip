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
#include <cmath>

#include "gemm_common.hpp"
#include "bsq_launch.hpp"

namespace bsq {

namespace {

using namespace gemm;

constexpr int kStageK = 128;  // K values (bytes) per row per stage

template <int BM, int BN, int NS>
using Cfg = Fp8Cfg<BM, BN, NS>;

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

// one operand fragment (32 bytes of K step t) of MFMA operand row `row` of a stage buffer
__device__ __forceinline__ v8i frag(const uint8_t* base, int row, int lh, int t) {
  const int c = 4 * lh + 2 * t;
  const uint4 lo = *reinterpret_cast<const uint4*>(base + swz_off<128>(row, c));
  const uint4 hi = *reinterpret_cast<const uint4*>(base + swz_off<128>(row, c + 1));
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int TN, int TM>
__device__ __forceinline__ void mfma_all(v16f (&acc)[TN][TM], const v8i (&a)[TN], const v8i (&b)[TM]) {
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 0, 0, 0, 0, 0, 0);
}

// Where the epilogue's adapter MFMAs find the tile's T rows and B rows (rank % 8 == 0; other
// ranks read them from global memory in the epilogue, where their load latency is exposed after
// the K loop -- about 2 us at 4096 x 3072 x 3072, rank 32):
//  * kLoraAhead (ranks 8..32): copied by LDS DMA ahead of the first stage into an LDS array of
//    their own, 64-byte rows ((BM + BN) * 64 bytes; the prologue's wait covers them);
//  * kLoraLate (ranks 40..64, hand-ordered loop): copied by LDS DMA into the stage buffer that
//    the last two stages leave free, 128-byte rows ((BM + BN) * 128 bytes: one stage buffer),
//    issued after the barrier of the second-to-last stage, so the last stage's MFMAs cover it;
//  * kLoraLate2 (ranks 72..128, hand-ordered loop): rank values 0..63 as kLoraLate, values
//    64..127 into the other stage buffer after the last stage's barrier (its K step 1 and the
//    first half's adapter MFMAs cover that copy).
// Rows are swizzled as in the stage regions; values past the rank and rows past M or N read as
// zeros.
enum LoraLds { kLoraGlobal = 0, kLoraAhead = 1, kLoraLate = 2, kLoraLate2 = 3 };
constexpr int kLoraLdsRow = 64;  // bytes a row of the kLoraAhead copy (rank 32)
constexpr int lora_lds_host(int rank, bool hand) {
  return (rank & 7) || rank > 128 ? kLoraGlobal
         : rank <= 32             ? kLoraAhead
         : !hand                  ? kLoraGlobal
         : rank <= 64             ? kLoraLate
                                  : kLoraLate2;
}
// rank values k_lo .. k_lo + R / 2 - 1 of the tile's T rows and B rows into R-byte LDS rows
template <int BM, int BN, int R>
__device__ __forceinline__ void lora_stage(const uint16_t* lt, const uint16_t* lb, int M, int N, int m0, int n0,
                                           int rank, int k_lo, uint32_t lds, int wave, int lane) {
  const int rows_t = M - m0 < BM ? M - m0 : BM, rows_b = N - n0 < BN ? N - n0 : BN;
  const v4i rt = buffer_rsrc(lt + (int64_t)m0 * rank, (uint32_t)(rows_t * rank * 2));
  const v4i rb = buffer_rsrc(lb + (int64_t)n0 * rank, (uint32_t)(rows_b * rank * 2));
  dma_region<Region<R, BM, R / 2>>(rt, lds, wave, lane, 2 * rank, 2 * k_lo, k_lo, rank);
  dma_region<Region<R, BN, R / 2>>(rb, lds + BM * R, wave, lane, 2 * rank, 2 * k_lo, k_lo, rank);
}
// this wave's LDS DMAs of one lora_stage call
template <int BM, int BN, int R>
constexpr int lora_stage_loads() {
  return Region<R, BM, R / 2>::MIN_PER_WAVE + Region<R, BN, R / 2>::MIN_PER_WAVE;
}
// acc += T B^T over rank values k_lo .. k_lo + R / 2 - 1 from an LDS copy of them with R-byte rows
// (tile-local rows: n at nl0 + 32 i, m at ml0 + 32 j), 32 rank values per batch
template <int BM, int R, int TN, int TM>
__device__ __forceinline__ void lora_update_lds(v16f (&acc)[TN][TM], const uint8_t* lds, int rank, int k_lo, int nl0,
                                                int ml0, int lane) {
  const int lr = lane & 31, lh = lane >> 5;
  auto chunk = [&](const uint8_t* base, int row, int c) {
    union {
      uint4 u;
      v8bf h;
    } v;
    v.u = *reinterpret_cast<const uint4*>(base + row * R + (swz_chunk<R>(row, c) << 4));
    return v.h;
  };
  for (int k0 = k_lo; k0 < k_lo + R / 2 && k0 < rank; k0 += 32) {
    LoraRegs<TN, TM, 2> r;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = (k0 - k_lo) / 8 + 2 * s + lh;
#pragma unroll
      for (int i = 0; i < TN; ++i) r.b[s][i] = chunk(lds + BM * R, nl0 + 32 * i + lr, c);
#pragma unroll
      for (int j = 0; j < TM; ++j) r.t[s][j] = chunk(lds, ml0 + 32 * j + lr, c);
    }
    lora_mfma(acc, r, k0, rank);
  }
}

// The K loop, two ways. The general loop (any K, any ring depth) leaves the order of its
// LDS reads, DMAs and MFMAs to the compiler, within scheduling groups. The hand-ordered loop
// (two stage buffers, K % 128 == 0, with or without an adapter) fixes the order per MFMA, which took the large tiles 8-13 %
// faster (4096 x 3072 x 3072 on 256 x 192: 38 -> 34 us; 16384 x 3072 x 3072 and
// 4096 x 12288 x 3072 on 256 x 256: 147 -> 128 us, same bits):
//  * K step 0 of stage s: one MFMA, then the LDS reads of RPM fragments of K step 1 (B
//    fragments first, the order step 1's MFMAs consume them), so every read has landed long
//    before step 1 needs it;
//  * the barrier (stage s read by every wave, stage s + 1 landed);
//  * K step 1: one MFMA, then one DMA of stage s + 2 into stage s's buffers (lane offsets
//    hoisted: with K % 128 == 0 every chunk of a real stage lies inside K), and from MFMA KD on
//    the reads of K step 0 of stage s + 1. The last two stages fetch nothing (no stage past K
//    is ever loaded).
// Without the fixed order the compiler bunched the DMAs' address arithmetic between the two
// K steps (the matrix pipe drained there) and waited for every read at the loop head.
template <int NS>
constexpr bool hand_ordered() { return NS == 2; }

// OQ: quantized output for the next linear -- 0 none, 1 nvfp4 blocks in the epilogue, 2 the
// row maxima of the fp8r encoding (YQuant). HS: the hand-ordered K loop (K % 128 == 0). LL:
// where the adapter's T and B rows are read (LoraLds). WPE: waves per SIMD the registers are
// budgeted for (2: two workgroups share a compute unit).
// One output tile: workgroup `bid` of the grid of BM x BN tiles over M x N.
template <int BM, int BN, int NS, bool LORA, int OQ, bool HS, int LL>
__device__ __forceinline__ void fp8_tile(const uint8_t* __restrict__ xq, const float* __restrict__ sx,
                                         const uint8_t* __restrict__ w, const float* __restrict__ sw,
                                         uint16_t* __restrict__ y, int64_t ldy, int M, int N, int K,
                                         const uint16_t* lt, const uint16_t* lb, int rank, int stream_y,
                                         const YQuant& q, int bid) {
  using C = Cfg<BM, BN, NS>;
  constexpr int TN = C::TN, TM = C::TM;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];
  __shared__ __attribute__((aligned(16))) float s_sx[BM];
  __shared__ __attribute__((aligned(16))) float s_sw[BN];
  __shared__ __attribute__((aligned(16))) uint8_t s_lora[LL == kLoraAhead ? (BM + BN) * kLoraLdsRow : 16];

  int m0, n0;
  tile_of_id(bid, M, N, BM, BN, m0, n0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  const int rows_x = M - m0 < BM ? M - m0 : BM, rows_w = N - n0 < BN ? N - n0 : BN;
  const v4i rx = buffer_rsrc(xq + (int64_t)m0 * K, (uint32_t)(rows_x * K));
  const v4i rw = buffer_rsrc(w + (int64_t)n0 * K, (uint32_t)(rows_w * K));
  const uint32_t lds0 = lds_offset(smem);
  // the adapter's T and B rows of this tile, ahead of the first stage (older than every stage
  // load, so the prologue's wait covers them)
  if constexpr (LL == kLoraAhead)
    lora_stage<BM, BN, kLoraLdsRow>(lt, lb, M, N, m0, n0, rank, 0, lds_offset(s_lora), wave, lane);

  auto issue_stage = [&](int kt) {
    const int kb = kt * kStageK;
    const uint32_t base = lds0 + (uint32_t)((kt % NS) * C::STAGE);
    dma_region<typename C::RA>(rw, base, wave, lane, K, kb, kb, K);
    dma_region<typename C::RB>(rx, base + C::A_BYTES, wave, lane, K, kb, kb, K);
  };

  // row / column scales of the tile, for the epilogue: dword LDS DMA of 64 rows a load (rows past
  // M or N read as zeros), issued ahead of the first stage -- older than every stage load, so the
  // prologue's wait covers them, and no wave waits for them before its first stage is in flight
  {
    const v4i rsx = buffer_rsrc(sx + m0, (uint32_t)(rows_x * 4));
    const v4i rsw = buffer_rsrc(sw + n0, (uint32_t)(rows_w * 4));
    for (int i = wave; i < BM / 64; i += 4) dma4(rsx, lds_offset(s_sx) + 256 * i, (64 * i + lane) * 4, 0);
    for (int i = wave; i < BN / 64; i += 4) dma4(rsw, lds_offset(s_sw) + 256 * i, (64 * i + lane) * 4, 0);
  }

  v16f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v16f{};

  const int lr = lane & 31, lh = lane >> 5;
  const int rowa = wn * C::WN + lr, rowb = wm * C::WM + lr;  // region-local rows
  const int nk = (K + kStageK - 1) / kStageK;

  // the epilogue's scaling and bf16 conversion of accumulator tile t into the LDS copy of the
  // output tile (see the epilogue below). The last K stage does it without an adapter; in the
  // general loop only for the tiles whose registers hold it (the 256-row ones would spill).
  constexpr bool kLoopOut = !LORA && (HS || BM * BN <= 128 * 128);
  auto tile_out = [&](int t) {
    const int i = t / TM, j = t % TM;
    const int ml = wm * C::WM + j * 32 + lr;
    const float xs = s_sx[ml];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int nl = wn * C::WN + i * 32 + 8 * g + 4 * lh;
      const v16f& A = acc[i][j];
      const float4 s4 = *reinterpret_cast<const float4*>(&s_sw[nl]);
      *reinterpret_cast<uint2*>(smem + ml * C::TROW + nl * 2) =
          make_uint2(pack_bf16x2(A[4 * g + 0] * xs * s4.x, A[4 * g + 1] * xs * s4.y),
                     pack_bf16x2(A[4 * g + 2] * xs * s4.z, A[4 * g + 3] * xs * s4.w));
    }
  };
  v8i a0[TN], b0[TM], a1[TN], b1[TM];
  if constexpr (HS) {
    static_assert(NS == 2, "two stage buffers");
    constexpr int NM = TN * TM, NF = TN + TM;
    constexpr int LA = C::RA::MIN_PER_WAVE, LD = C::LOADS_MIN;  // this wave's DMAs per stage (W first)
    constexpr int RPM = NM >= 16 ? 1 : 2;  // fragment reads per MFMA
    constexpr int KD = 8;                  // K-step-1 MFMAs before the next stage's reads start
    static_assert(C::RA::C == 8 && C::RB::C == 8, "128-byte rows");
    // load i of a stage: this wave's loads of region A (W) then of region B (Xq)
    auto load_addr = [&](int i, int kb) {
      const int ld = wave + 4 * (i < LA ? i : i - LA);
      return i < LA ? region_load<typename C::RA>(ld, lane, K, kb, kb, K)
                    : region_load<typename C::RB>(ld, lane, K, kb, kb, K);
    };
    int voff[LD];  // every chunk of a real stage lies inside K: the lane offsets of stage 0 hold
#pragma unroll
    for (int i = 0; i < LD; ++i) voff[i] = load_addr(i, 0).voff;
    auto dma = [&](int i, int kt) {
      const bool isA = i < LA;
      const int ld = wave + 4 * (isA ? i : i - LA);
      const uint32_t lb = lds0 + (uint32_t)((kt % NS) * C::STAGE) + (isA ? 0u : (uint32_t)C::A_BYTES) + ld * 1024;
      dma16(isA ? rw : rx, lb, voff[i], load_addr(i, kt * kStageK).soff);
    };
    auto abuf = [&](int kt) { return smem + (kt % NS) * C::STAGE; };
    const int nk = K / kStageK;
#pragma unroll
    for (int i = 0; i < LD; ++i) dma(i, 0);
    // kLoraLate(2): rank values 0..63 go to the stage buffer of stage nk - 2 once it is read
    // (stage buffer 1 for a single stage), values 64..127 to that of stage nk - 1
    static_assert(LL < kLoraLate || C::STAGE == (BM + BN) * 128, "64 rank values of the rows fill one stage buffer");
    auto lora_late = [&](int buf, int k_lo) {
      if constexpr (LL >= kLoraLate)
        lora_stage<BM, BN, 128>(lt, lb, M, N, m0, n0, rank, k_lo, lds0 + (uint32_t)(buf * C::STAGE), wave, lane);
    };
    if (nk > 1) {
#pragma unroll
      for (int i = 0; i < LD; ++i) dma(i, 1);
      wait_vmcnt<LD>();
    } else {
      lora_late(1, 0);
      wait_vmcnt<0>();
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TN; ++i) a0[i] = frag(abuf(0), rowa + 32 * i, lh, 0);
#pragma unroll
    for (int j = 0; j < TM; ++j) b0[j] = frag(abuf(0) + C::A_BYTES, rowb + 32 * j, lh, 0);

    auto iter = [&](int s, auto fetch, auto last) {
      constexpr bool F = decltype(fetch)::value, LAST = decltype(last)::value;
      const uint8_t* ca = abuf(s);
      const uint8_t* cb = ca + C::A_BYTES;
#pragma unroll
      for (int k = 0; k < NM; ++k) {
        const int i = k / TM, j = k % TM;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0[i], b0[j], acc[i][j], 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < RPM; ++r) {
          const int f = k * RPM + r;
          if (f < TM) b1[f] = frag(cb, rowb + 32 * f, lh, 1);
          else if (f < NF) a1[f - TM] = frag(ca, rowa + 32 * (f - TM), lh, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (LL < kLoraLate || s + 1 < nk) wait_vmcnt<0>();  // (the last stage leaves the adapter copy in flight)
      __syncthreads();  // stage s read by every wave; stage s + 1 landed
      if constexpr (!F) {
        if (s == nk - 2) lora_late(s % NS, 0);
        if (LL == kLoraLate2 && s == nk - 1) lora_late(s % NS, 64);
      }
      if constexpr (LAST) {
        // the last stage without an adapter: once every wave has passed the barrier above no
        // stage buffer is read any more, so each tile is scaled and written to the output copy
        // while the next tile's last MFMA runs
#pragma unroll
        for (int k = 0; k < NM; ++k) {
          const int i = k / TM, j = k % TM;
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1[i], b1[j], acc[i][j], 0, 0, 0, 0, 0, 0);
          if (k > 0) tile_out(k - 1);
        }
        tile_out(NM - 1);
        return;
      }
      const uint8_t* na = abuf(s + 1);
      const uint8_t* nb = na + C::A_BYTES;
#pragma unroll
      for (int k = 0; k < NM; ++k) {
        const int i = k / TM, j = k % TM;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1[i], b1[j], acc[i][j], 0, 0, 0, 0, 0, 0);
        if constexpr (F) {
          if (k < LD) dma(k, s + 2);
        }
        if (k >= KD) {
#pragma unroll
          for (int r = 0; r < RPM; ++r) {
            const int f = (k - KD) * RPM + r;
            if (f < TM) b0[f] = frag(nb, rowb + 32 * f, lh, 0);
            else if (f < NF) a0[f - TM] = frag(na, rowa + 32 * (f - TM), lh, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (F) {
#pragma unroll
        for (int di = NM; di < LD; ++di) dma(di, s + 2);
      }
      constexpr int done = (NM - KD) * RPM;
#pragma unroll
      for (int f = done; f < NF; ++f) {  // past the last stage these read unused bytes
        if (f < TM) b0[f] = frag(nb, rowb + 32 * f, lh, 0);
        else a0[f - TM] = frag(na, rowa + 32 * (f - TM), lh, 0);
      }
    };
    int s = 0;
    for (; s + 2 < nk; ++s) iter(s, std::true_type{}, std::false_type{});
    for (; s + 1 < nk; ++s) iter(s, std::false_type{}, std::false_type{});
    iter(s, std::false_type{}, std::integral_constant<bool, !LORA>{});
  } else {
  // prologue: NS stages in flight, wait for the first
#pragma unroll
  for (int p = 0; p < NS; ++p) issue_stage(p);
  wait_vmcnt<(NS - 1) * C::LOADS_MIN>();
  __syncthreads();
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
  for (int s = 0; s < nk - (kLoopOut ? 1 : 0); ++s) {
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
  if constexpr (kLoopOut) {
    // the last stage without an adapter: once the loads of the stages past K (zeros, into the
    // stage buffers) have landed and every wave has passed the barrier, no stage buffer is used
    // any more, and each tile is written to the output copy under the next one's MFMA
    const uint8_t* cur = smem + ((nk - 1) % NS) * C::STAGE;
    read_ops<TN, TM>(cur, cur + C::A_BYTES, rowa, rowb, lh, 1, a1, b1);
    mfma_all<TN, TM>(acc, a0, b0);
    sched();
    wait_vmcnt<0>();
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TN * TM; ++k) {
      const int i = k / TM, j = k % TM;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1[i], b1[j], acc[i][j], 0, 0, 0, 0, 0, 0);
      if (k > 0) tile_out(k - 1);
    }
    tile_out(TN * TM - 1);
  }
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
    if constexpr (LL == kLoraAhead) {
      lora_update_lds<BM, kLoraLdsRow>(acc, s_lora, rank, 0, wn * C::WN, wm * C::WM, lane);
    } else if constexpr (LL >= kLoraLate) {
      // rank values 0..63 (with kLoraLate2 the copy of 64..127, issued later, may still be in flight)
      wait_vmcnt<LL == kLoraLate2 ? lora_stage_loads<BM, BN, 128>() : 0>();
      __syncthreads();  // every wave's part of the copy has landed
      lora_update_lds<BM, 128>(acc, smem + (nk >= 2 ? (nk - 2) % NS : 1) * C::STAGE, rank, 0, wn * C::WN, wm * C::WM,
                               lane);
      if constexpr (LL == kLoraLate2) {
        wait_vmcnt<0>();
        __syncthreads();
        lora_update_lds<BM, 128>(acc, smem + ((nk - 1) % NS) * C::STAGE, rank, 64, wn * C::WN, wm * C::WM, lane);
      }
    } else
      lora_update<TN, TM>(acc, lt, lb, rank, M, N, n0 + wn * C::WN, m0 + wm * C::WM, lane);
  }
  wait_vmcnt<0>();
  __syncthreads();  // all stage buffers are free now
  // (the K loop has written the output copy in its last stage)
  constexpr bool kWritten = kLoopOut;
#pragma unroll
  for (int j = 0; j < (kWritten ? 0 : TM); ++j) {
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
  if (y) store_tile_rows<BM, BN, C::TROW>(smem, y, ldy, M, N, m0, n0, tid, stream_y != 0);
  // the next linear's input, quantized from the same bf16 tile ("BFL (fp8r / nvfp4)": every
  // quantized linear quantizes its input at run time)
  if constexpr (OQ == 1) quant_tile_rows<BM, BN, C::TROW>(smem, q.yq, q.ys, 1.0f / q.gy[0], M, N, m0, n0, tid);
  if constexpr (OQ == 2) rowmax_tile<BM, BN, C::TROW>(smem, q.pmax, M, N, m0, n0, tid);
}

template <int BM, int BN, int NS, bool LORA, int OQ = 0, bool HS = false, int LL = kLoraGlobal, int WPE = 1>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void gemm_fp8_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ sx,
                     const uint8_t* __restrict__ w, const float* __restrict__ sw,
                     uint16_t* __restrict__ y, int64_t ldy, int M, int N, int K, const uint16_t* lt,
                     const uint16_t* lb, int rank, int stream_y, YQuant q) {
  fp8_tile<BM, BN, NS, LORA, OQ, HS, LL>(xq, sx, w, sw, y, ldy, M, N, K, lt, lb, rank, stream_y, q, blockIdx.x);
}

// The tiles of several W8A8 GEMMs in one grid (hand-ordered loop, two stage buffers): the
// problem of each workgroup, then that problem's tile, exactly as its own launch would compute
// it (same tile shape, same bits).
struct Fp8Group {
  Fp8Problem p[kMaxGroup];
  int start[kMaxGroup + 1];
  int count;
};
template <int BM, int BN, int WPE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void gemm_fp8_grouped_kernel(Fp8Group g) {
  const int bid = blockIdx.x;
  const int p = group_problem(g.start, g.count, bid);
  const Fp8Problem& q = g.p[p];
  fp8_tile<BM, BN, 2, false, 0, true, kLoraGlobal>(q.xq, q.sx, q.w, q.sw, q.y, q.ldy, q.M, q.N, q.K, nullptr,
                                                   nullptr, 0, q.stream_y, YQuant{}, bid - g.start[p]);
}

template <int BM, int BN, int NS, bool HS, int WPE = 1>
hipError_t launch_oq(int oq, int tiles, const uint8_t* xq, const float* sx, const uint8_t* w, const float* sw,
                     uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, int st, const YQuant& qv,
                     hipStream_t s) {
  if (oq == 1)
    hipLaunchKernelGGL((gemm_fp8_kernel<BM, BN, NS, false, 1, HS, kLoraGlobal, WPE>), dim3(tiles), dim3(kThreads), 0,
                       s, xq, sx, w, sw, y, ldy, (int)M, (int)N, (int)K, nullptr, nullptr, 0, st, qv);
  else if (oq == 2)
    hipLaunchKernelGGL((gemm_fp8_kernel<BM, BN, NS, false, 2, HS, kLoraGlobal, WPE>), dim3(tiles), dim3(kThreads), 0,
                       s, xq, sx, w, sw, y, ldy, (int)M, (int)N, (int)K, nullptr, nullptr, 0, st, qv);
  else
    hipLaunchKernelGGL((gemm_fp8_kernel<BM, BN, NS, false, 0, HS, kLoraGlobal, WPE>), dim3(tiles), dim3(kThreads), 0,
                       s, xq, sx, w, sw, y, ldy, (int)M, (int)N, (int)K, nullptr, nullptr, 0, st, qv);
  return hipGetLastError();
}

// 128 x 128 tiles with two stage buffers and the hand-ordered loop, two workgroups per compute
// unit (65 KB of LDS and at most 256 registers a lane each), so one workgroup's barrier waits,
// prologue and output write overlap the other's K loop: 512 tiles a round
hipError_t run_pair(const uint8_t* xq, const float* sx, const uint8_t* w, const float* sw, uint16_t* y, int64_t ldy,
                    int64_t M, int64_t N, int64_t K, hipStream_t s, const YQuant* q) {
  const int tiles = (int)(((M + 127) / 128) * ((N + 127) / 128));
  const int st = (int)stream_output((M + N) * K, M, N);
  const YQuant qv = q ? *q : YQuant{};
  const int oq = qv.yq ? 1 : qv.pmax ? 2 : 0;
  return launch_oq<128, 128, 2, true, 2>(oq, tiles, xq, sx, w, sw, y, ldy, M, N, K, st, qv, s);
}

template <int BM, int BN, int NS>
hipError_t run(const uint8_t* xq, const float* sx, const uint8_t* w, const float* sw, uint16_t* y,
               int64_t ldy, int64_t M, int64_t N, int64_t K, const uint16_t* lt, const uint16_t* lb, int rank,
               hipStream_t s, const YQuant* q) {
  const int tiles = (int)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
  constexpr bool kAdapter = !(BM == 256 && BN == 256);  // the 256 x 256 tile never carries one (launch_gemm_fp8)
  const int st = (int)stream_output((M + N) * K, M, N);
  const YQuant qv = q ? *q : YQuant{};
  if (kAdapter && lt) {
    constexpr bool kHand = hand_ordered<NS>();
    constexpr int kAhead = kAdapter ? kLoraAhead : kLoraGlobal, kLate = kAdapter && kHand ? kLoraLate : kLoraGlobal,
                  kLate2 = kAdapter && kHand ? kLoraLate2 : kLoraGlobal;
    const bool hs = kHand && K % kStageK == 0;
    const int ll = lora_lds_host(rank, hs);
    if (hs && ll == kLoraAhead)
      hipLaunchKernelGGL((gemm_fp8_kernel<BM, BN, NS, kAdapter, 0, kHand, kAhead>), dim3(tiles), dim3(kThreads), 0, s,
                         xq, sx, w, sw, y, ldy, (int)M, (int)N, (int)K, lt, lb, rank, st, qv);
    else if (hs && ll == kLoraLate)
      hipLaunchKernelGGL((gemm_fp8_kernel<BM, BN, NS, kAdapter, 0, kHand, kLate>), dim3(tiles), dim3(kThreads), 0, s,
                         xq, sx, w, sw, y, ldy, (int)M, (int)N, (int)K, lt, lb, rank, st, qv);
    else if (hs && ll == kLoraLate2)
      hipLaunchKernelGGL((gemm_fp8_kernel<BM, BN, NS, kAdapter, 0, kHand, kLate2>), dim3(tiles), dim3(kThreads), 0, s,
                         xq, sx, w, sw, y, ldy, (int)M, (int)N, (int)K, lt, lb, rank, st, qv);
    else if (hs)
      hipLaunchKernelGGL((gemm_fp8_kernel<BM, BN, NS, kAdapter, 0, kHand>), dim3(tiles), dim3(kThreads), 0, s, xq, sx,
                         w, sw, y, ldy, (int)M, (int)N, (int)K, lt, lb, rank, st, qv);
    else if (ll == kLoraAhead)
      hipLaunchKernelGGL((gemm_fp8_kernel<BM, BN, NS, kAdapter, 0, false, kAhead>), dim3(tiles), dim3(kThreads), 0, s,
                         xq, sx, w, sw, y, ldy, (int)M, (int)N, (int)K, lt, lb, rank, st, qv);
    else
      hipLaunchKernelGGL((gemm_fp8_kernel<BM, BN, NS, kAdapter>), dim3(tiles), dim3(kThreads), 0, s, xq, sx, w, sw,
                         y, ldy, (int)M, (int)N, (int)K, lt, lb, rank, st, qv);
    return hipGetLastError();
  }
  const int oq = qv.yq ? 1 : qv.pmax ? 2 : 0;
  if (hand_ordered<NS>() && K % kStageK == 0)
    return launch_oq<BM, BN, NS, hand_ordered<NS>()>(oq, tiles, xq, sx, w, sw, y, ldy, M, N, K, st, qv, s);
  return launch_oq<BM, BN, NS, false>(oq, tiles, xq, sx, w, sw, y, ldy, M, N, K, st, qv, s);
}

}  // namespace

// Grouped W8A8: every problem on the hand-ordered loop (K % 128 == 0). Below three rounds of
// 256 x 192 tiles the group runs on 128 x 128 tiles two to a compute unit, once those fill one
// round of pairs (512 tiles); beyond, on the 256 x 256 or 256 x 192 tile of least expected time
// over whole rounds (each tile's time in proportion to its K; round times as for one GEMM, at
// K = 3072) when it fills two rounds. Smaller groups run one launch per problem, whose own tile
// choice fills the compute units. A joint block's four linears (qkv, proj, up, down; cold
// weights) as one grid against four launches, fp8r / nvfp4 (us): 384 tokens 96 / 102 vs 114 /
// 150, 512 tokens 104 / 111 vs 129 / 171, 768 tokens 104 / 158 vs 145 / 218, 1024 tokens 144 /
// 200 vs 156 / 242 (all on 128 x 128 pairs), 2048 tokens 221 / 356 vs 290 / 443 (256 x 192),
// 4096 tokens 410 / 672 vs 440 / 716 (256 x 256). On 128 x 128 pairs 2048 and 4096 tokens took
// 262 / 406 and 505 / 803 us; on 256-row tiles 512 tokens (288 tiles) took 145 / 196 us.
namespace {
struct GroupTile {
  int bm, bn, per_round, round_us;
};
constexpr GroupTile kFp8GroupTiles[3] = {{256, 256, 256, 92}, {256, 192, 256, 72}, {128, 128, 512, 52}};
// the group's tile (index into kFp8GroupTiles), or -1 when no tile fills two rounds
int fp8_group_tile(const Fp8Problem* p, int count) {
  auto tiles_of = [&](const GroupTile& c, double* work) {
    int64_t tiles = 0;
    double w = 0;  // tiles times K / 3072
    for (int i = 0; i < count; ++i) {
      const int64_t n = ((int64_t)(p[i].M + c.bm - 1) / c.bm) * ((p[i].N + c.bn - 1) / c.bn);
      tiles += n;
      w += (double)n * (double)p[i].K / 3072.0;
    }
    if (work) *work = w;
    return tiles;
  };
  // under three rounds of 256 x 192 tiles, 128 x 128 tiles two to a compute unit once they fill a
  // round of pairs (measured below); otherwise the 256-row tile of fewer whole rounds
  if (tiles_of(kFp8GroupTiles[1], nullptr) < 3 * 256) {
    const int64_t t = tiles_of(kFp8GroupTiles[2], nullptr);
    return t >= 512 && t < ((int64_t)1 << 31) ? 2 : -1;
  }
  int best = -1;
  double best_cost = 0;
  for (int t = 0; t < 2; ++t) {
    const GroupTile& c = kFp8GroupTiles[t];
    double work = 0;
    const int64_t tiles = tiles_of(c, &work);
    if (tiles < 2 * (int64_t)c.per_round || tiles >= ((int64_t)1 << 31)) continue;  // 32-bit workgroup ids
    const double cost = std::ceil(work / c.per_round - 1e-9) * c.round_us;
    if (best < 0 || cost < best_cost) best = t, best_cost = cost;
  }
  return best;
}
template <int BM, int BN, int WPE>
hipError_t run_fp8_group(const Fp8Problem* p, int count, hipStream_t s) {
  Fp8Group g{};
  g.count = count;
  int64_t total = 0;
  for (int i = 0; i < count; ++i) {
    g.p[i] = p[i];
    g.p[i].stream_y = (int)stream_output((int64_t)(p[i].M + p[i].N) * p[i].K, p[i].M, p[i].N);
    g.start[i] = (int)total;
    total += ((int64_t)(p[i].M + BM - 1) / BM) * ((p[i].N + BN - 1) / BN);
  }
  for (int i = count; i <= kMaxGroup; ++i) g.start[i] = (int)total;
  hipLaunchKernelGGL((gemm_fp8_grouped_kernel<BM, BN, WPE>), dim3((unsigned)total), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}
}  // namespace

bool gemm_fp8_grouped_supported(const Fp8Problem* p, int count) {
  if (count < 2 || count > kMaxGroup) return false;
  for (int i = 0; i < count; ++i)
    if (p[i].K % kStageK != 0) return false;
  return fp8_group_tile(p, count) >= 0;
}

hipError_t launch_gemm_fp8_grouped(const Fp8Problem* p, int count, hipStream_t s) {
  switch (fp8_group_tile(p, count)) {
    case 0: return run_fp8_group<256, 256, 1>(p, count, s);
    case 1: return run_fp8_group<256, 192, 1>(p, count, s);
    default: return run_fp8_group<128, 128, 2>(p, count, s);
  }
}

hipError_t launch_gemm_fp8(const uint8_t* xq, const float* sx, const uint8_t* w, const float* sw,
                           uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, const uint16_t* lt,
                           const uint16_t* lb, int rank, hipStream_t s, const YQuant* q) {
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
  if (t64 <= 256) return run<64, 64, 4>(xq, sx, w, sw, y, ldy, M, N, K, lt, lb, rank, s, q);
  if (t64x128 <= 256) return run<64, 128, 4>(xq, sx, w, sw, y, ldy, M, N, K, lt, lb, rank, s, q);
  const int64_t c256 = lt ? INT64_MAX : rounds_cost(M, N, 256, 256, 92);
  const int64_t c192 = rounds_cost(M, N, 256, 192, 72), c128 = rounds_cost(M, N, 128, 128, 31);
  // 128 x 128 tiles two to a compute unit (no adapter, K % 128 == 0): 512 tiles a round at
  // about 26 us (K = 3072), which wins between 256 and 512 of them -- 2048 x 3072 28.3 -> 22.7 us,
  // 1536 x 3072 28.0 -> 21.7 us, 2048 x 4096 31.3 -> 26.6 us, 2500 x 3072 30.5 -> 25.7 us
  const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
  const int64_t c2 = lt || K % kStageK != 0 || t128 <= 256 ? INT64_MAX : (t128 + 511) / 512 * 52;
  if (c2 < c256 && c2 < c192 && c2 < c128) return run_pair(xq, sx, w, sw, y, ldy, M, N, K, s, q);
  if (c256 <= c192 && c256 <= c128) return run<256, 256, 2>(xq, sx, w, sw, y, ldy, M, N, K, lt, lb, rank, s, q);
  if (c192 <= c128) return run<256, 192, 2>(xq, sx, w, sw, y, ldy, M, N, K, lt, lb, rank, s, q);
  return run<128, 128, 4>(xq, sx, w, sw, y, ldy, M, N, K, lt, lb, rank, s, q);
}

}  // namespace bsq
