// nvfp4 W4A4 GEMM: packed E2M1 operands decoded in registers, f16 matrix cores.
//
// "BFL (fp8r / nvfp4)", nvfp4 bullet: a value is e2m1 * e4m3(scale of its
// 16-element block) * global scale, and activations are quantized the same
// way with the calibrated input_scale before an fp4 GEMM ("Kernels" table):
//   y[m][n] = bf16( (sum_k xh[m][k] * wh[n][k]) * gx * gw ),
//   xh = e2m1(xq) * e4m3(sfx),  wh = e2m1(wq) * e4m3(sfw).
// An E2M1 value (2 significant bits) times an E4M3 scale (4 significant bits)
// has at most 6 significant bits and lies in [2^-10, 2688], so xh and wh are
// exact in f16; the contraction runs on v_mfma_f32_32x32x16_f16 with fp32
// accumulation and the two fp32 global scales go to the epilogue. (gfx950's
// block-scaled FP4 MFMA applies power-of-two scales per 32 elements, which
// cannot carry an E4M3 scale per 16.)
//
// Data movement (conventions in gemm_common.hpp): a stage is 256 K values
// of every W and Xq row -- 128 bytes of packed codes (one full cache line)
// plus 16 block-scale bytes -- copied to LDS as stored by LDS DMA into one of
// two stage buffers while the other is multiplied. Long stages keep the
// number of memory requests low (small per-row segments would cost one
// request each). Every wave reads its operands' packed bytes from LDS one
// 64-deep K group ahead and decodes them in registers right before the MFMAs
// of each 16-deep K step: per byte one v_cvt_scalef32_pk_f16_fp4 (exact
// E2M1 -> f16 pair) and one v_pk_mul_f16 by the block scale. LDS traffic
// stays at the packed size; the decode work (about 4 VALU per MFMA) issues
// under the MFMAs.
//
// K permutation: lane half h of an MFMA operand covers K values
// [128 h, 128 h + 128) of a stage -- 32 of them per 64-deep K group q, at
// [128 h + 32 q, 128 h + 32 q + 32), one 8-value group per K step -- for both
// operands alike, so every product pairs equal K indices. A lane's 8 block
// scales of a stage are then 8 consecutive bytes, read once per stage.
#include <cmath>

#include "gemm_common.hpp"
#include "bsq_launch.hpp"

namespace bsq {

namespace {

using namespace gemm;

constexpr int kStageK = 256;  // K values per stage

// packed operand bytes of one K group for one lane: 32 E2M1 values (4 dwords)
struct Raw {
  uint4 q;
};

// packed bytes of K group q (0..3) of a stage for this lane: chunk 4h + q of the row
template <int TN, int TM>
__device__ __forceinline__ void read_raw(const uint8_t* st, int a_off, int b_off, int rowa, int rowb, int lh, int q,
                                         Raw (&ra)[TN], Raw (&rb)[TM]) {
#pragma unroll
  for (int i = 0; i < TN; ++i)
    ra[i].q = *reinterpret_cast<const uint4*>(st + a_off + swz_off<128>(rowa + i * 32, 4 * lh + q));
#pragma unroll
  for (int j = 0; j < TM; ++j)
    rb[j].q = *reinterpret_cast<const uint4*>(st + b_off + swz_off<128>(rowb + j * 32, 4 * lh + q));
}

// this lane's 8 block scales of a stage (blocks 8h .. 8h + 7 of the row)
template <int TN, int TM>
__device__ __forceinline__ void read_scales(const uint8_t* st, int sa_off, int sb_off, int rowa, int rowb, int lh,
                                            uint2 (&sa)[TN], uint2 (&sb)[TM]) {
#pragma unroll
  for (int i = 0; i < TN; ++i) sa[i] = *reinterpret_cast<const uint2*>(st + sa_off + (rowa + i * 32) * 16 + 8 * lh);
#pragma unroll
  for (int j = 0; j < TM; ++j) sb[j] = *reinterpret_cast<const uint2*>(st + sb_off + (rowb + j * 32) * 16 + 8 * lh);
}

// block scale bytes 2 hi and 2 hi + 1 of `s` as f16 (E4M3 -> f16 is exact)
__device__ __forceinline__ v2h scale_pairs(uint32_t s, int hi) {
  return hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, true)
            : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, false);
}

__device__ __forceinline__ uint32_t h2u(v2h v) {
  union { v2h h; uint32_t u; } c;
  c.h = v;
  return c.u;
}

// decode the 8 values of K step t (dword t of the packed chunk) times its block scale
__device__ __forceinline__ v8h decode8(uint32_t w, v2h s) {
  union { uint4 u; v8h h; } r;
  r.u = make_uint4(h2u(dec_e2m1x2_f16<0>(w) * s), h2u(dec_e2m1x2_f16<1>(w) * s),
                   h2u(dec_e2m1x2_f16<2>(w) * s), h2u(dec_e2m1x2_f16<3>(w) * s));
  return r.h;
}

template <int T>
__device__ __forceinline__ uint32_t dword_of(const uint4& q) {
  return T == 0 ? q.x : T == 1 ? q.y : T == 2 ? q.z : q.w;
}

// One output tile: workgroup `bid` of the grid of BM x BN tiles over M x N.
template <int BM, int BN, bool LORA>
__device__ __forceinline__ void w4a4_tile(const DecArgs& a, int bid) {
  using C = W4Cfg<BM, BN>;
  constexpr int TN = C::TN, TM = C::TM;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];
  __shared__ __attribute__((aligned(16))) float s_g[2][64];  // gx, gw (lane 0 of two dword DMAs)

  const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
  int m0, n0;
  tile_of_id(bid, M, N, BM, BN, m0, n0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  const int rows_x = M - m0 < BM ? M - m0 : BM, rows_w = N - n0 < BN ? N - n0 : BN;
  const int kp = K >> 1, ks = K >> 4;  // packed bytes and scale bytes per row
  const v4i rxq = buffer_rsrc(a.xq + (int64_t)m0 * kp, (uint32_t)(rows_x * kp));
  const v4i rwq = buffer_rsrc(a.w + (int64_t)n0 * kp, (uint32_t)(rows_w * kp));
  const v4i rxs = buffer_rsrc(a.xs + (int64_t)m0 * ks, (uint32_t)(rows_x * ks));
  const v4i rws = buffer_rsrc(a.ws + (int64_t)n0 * ks, (uint32_t)(rows_w * ks));
  const uint32_t lds0 = lds_offset(smem);
  // the two global scales, by dword LDS DMA ahead of the first stage (older than every stage
  // load, so the prologue's wait covers them): the last stage scales the accumulators in the loop
  if (wave == 0) {
    dma4(buffer_rsrc(a.gx, 4u), lds_offset(s_g[0]), lane == 0 ? 0 : kOutOfRange, 0);
    dma4(buffer_rsrc(a.gw, 4u), lds_offset(s_g[1]), lane == 0 ? 0 : kOutOfRange, 0);
  }

  // fetch stage kt into buffer kt % 2 (stages past K read as zeros)
  auto issue_stage = [&](int kt) {
    const int kb = kt * kStageK;
    const uint32_t base = lds0 + (uint32_t)((kt & 1) * C::STAGE);
    dma_region<typename C::RA>(rwq, base + C::A_OFF, wave, lane, kp, kb >> 1, kb, K);
    dma_region<typename C::RB>(rxq, base + C::B_OFF, wave, lane, kp, kb >> 1, kb, K);
    dma_region<typename C::SA>(rws, base + C::SA_OFF, wave, lane, ks, kb >> 4, kb, K);
    dma_region<typename C::SB>(rxs, base + C::SB_OFF, wave, lane, ks, kb >> 4, kb, K);
  };

  v16f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v16f{};

  const int lr = lane & 31, lh = lane >> 5;
  const int rowa = wn * C::WN + lr, rowb = wm * C::WM + lr;  // region-local rows
  const int nk = K / kStageK;

  Raw r0a[TN], r0b[TM], r1a[TN], r1b[TM];  // packed operands of the current / next K group
  uint2 s0a[TN], s0b[TM], s1a[TN], s1b[TM];  // block scales of the current / next stage
  v8h d0a[TN], d0b[TM], d1a[TN], d1b[TM];  // decoded operands of two consecutive K steps
  v2h spa[TN][2], spb[TM][2];              // block-scale pairs of the K group being decoded

  // scale pairs of K group q from the stage's scale bytes (bytes 2q, 2q + 1 of the lane's 8)
  // (one conversion gives both scales of the group; the multiplies broadcast one half of it)
  auto scales_of = [&](const uint2 (&sa)[TN], const uint2 (&sb)[TM], int q) {
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const v2h p = scale_pairs(q < 2 ? sa[i].x : sa[i].y, q & 1);
      spa[i][0] = v2h{p.x, p.x};
      spa[i][1] = v2h{p.y, p.y};
    }
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const v2h p = scale_pairs(q < 2 ? sb[j].x : sb[j].y, q & 1);
      spb[j][0] = v2h{p.x, p.x};
      spb[j][1] = v2h{p.y, p.y};
    }
  };
  auto decode_step = [&](auto tc, const Raw (&ra)[TN], const Raw (&rb)[TM], v8h (&da)[TN], v8h (&db)[TM]) {
    constexpr int T = decltype(tc)::value;
#pragma unroll
    for (int i = 0; i < TN; ++i) da[i] = decode8(dword_of<T>(ra[i].q), spa[i][T >> 1]);
#pragma unroll
    for (int j = 0; j < TM; ++j) db[j] = decode8(dword_of<T>(rb[j].q), spb[j][T >> 1]);
  };
  auto mfmas = [&](const v8h (&da)[TN], const v8h (&db)[TM]) {
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(da[i], db[j], acc[i][j], 0, 0, 0);
  };
  // one K step's MFMAs with the next step's decode (VALU) and LDS reads issued between them
  auto pipeline = [&](auto vc, auto dc) {
    constexpr int NV = decltype(vc)::value, ND = decltype(dc)::value;
#pragma unroll
    for (int i = 0; i < TN * TM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
      if (ND) __builtin_amdgcn_sched_group_barrier(0x100, ND, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using NV = std::integral_constant<int, 8 * (TN + TM) / (TN * TM) + 1>;  // decode VALU per MFMA
  using NV2 = std::integral_constant<int, 8 * (TN + TM) / (TN * TM) + 3>;

  // the epilogue's scaling by gx gw and bf16 conversion of accumulator tile t into the LDS copy
  // of the output tile [BM][BN]
  auto tile_out = [&](int t, float alpha) {
    const int i = t / TM, j = t % TM;
    const int ml = wm * C::WM + j * 32 + lr;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int nl = wn * C::WN + i * 32 + 8 * g + 4 * lh;
      const v16f& A = acc[i][j];
      *reinterpret_cast<uint2*>(smem + ml * C::TROW + nl * 2) =
          make_uint2(pack_bf16x2(A[4 * g + 0] * alpha, A[4 * g + 1] * alpha),
                     pack_bf16x2(A[4 * g + 2] * alpha, A[4 * g + 3] * alpha));
    }
  };

  // K group q of a stage: operands in ca/cb (K step 0 decoded in d0, scale pairs of the group
  // in spa/spb); the next group's packed bytes are read into na/nb from `nst` (group nq, whose
  // scales are in nsa/nsb) and its K step 0 decoded into d0. The last group of the last stage
  // (LG) reads nothing ahead; once every wave has passed the last stage's barrier no stage
  // buffer is read any more, so each accumulator tile is scaled and written to the output copy
  // while the next tile's last MFMA runs.
  auto group = [&](const Raw (&ca)[TN], const Raw (&cb)[TM], Raw (&na)[TN], Raw (&nb)[TM], const uint8_t* nst,
                   int nq, const uint2 (&nsa)[TN], const uint2 (&nsb)[TM], auto lg) {
    constexpr bool LG = decltype(lg)::value;
    if constexpr (!LG) read_raw<TN, TM>(nst, C::A_OFF, C::B_OFF, rowa, rowb, lh, nq, na, nb);
    decode_step(I1{}, ca, cb, d1a, d1b);
    mfmas(d0a, d0b);
    pipeline(NV{}, std::integral_constant<int, LG ? 0 : 1>{});
    decode_step(I2{}, ca, cb, d0a, d0b);
    mfmas(d1a, d1b);
    pipeline(NV{}, I0{});
    decode_step(I3{}, ca, cb, d1a, d1b);
    if constexpr (!LG) scales_of(nsa, nsb, nq);
    mfmas(d0a, d0b);
    pipeline(NV2{}, I0{});
    if constexpr (LG) {
      const float alpha = s_g[0][0] * s_g[1][0];
#pragma unroll
      for (int k = 0; k < TN * TM; ++k) {
        const int i = k / TM, j = k % TM;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(d1a[i], d1b[j], acc[i][j], 0, 0, 0);
        if (k > 0) tile_out(k - 1, alpha);
      }
      tile_out(TN * TM - 1, alpha);
    } else {
      decode_step(I0{}, na, nb, d0a, d0b);
      mfmas(d1a, d1b);
      pipeline(NV{}, I0{});
    }
  };

  if constexpr (LORA) {
    // low-rank adapter: the accumulators start at T' B^T with T' = T / (gx gw) (the down
    // projection divides), so the epilogue's scaling by gx gw leaves y = bf16(base + T B^T).
    // Its first 64 rank values are loaded alongside the first stage; larger ranks follow.
    const rsrc_t rt = make_rsrc(a.lt, (uint32_t)M * (uint32_t)a.rank * 2u);
    const rsrc_t rb = make_rsrc(a.lb, (uint32_t)N * (uint32_t)a.rank * 2u);
    const int nw0 = n0 + wn * C::WN, mw0 = m0 + wm * C::WM;
    LoraRegs<TN, TM, 4> lo;
    lora_load(lo, rt, rb, 0, a.rank, nw0, mw0, lane);
    issue_stage(0);
    // both sets of loads are in flight before anything waits (the scheduler would otherwise
    // hoist the adapter MFMAs, and their wait, above the stage's DMA)
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();
    lora_mfma(acc, lo, 0, a.rank);
    for (int k0 = 64; k0 < a.rank; k0 += 64) {
      lora_load(lo, rt, rb, k0, a.rank, nw0, mw0, lane);
      lora_mfma(acc, lo, k0, a.rank);
    }
  } else {
    issue_stage(0);
    wait_vmcnt<0>();
  }
  __syncthreads();
  issue_stage(1);
  read_raw<TN, TM>(smem, C::A_OFF, C::B_OFF, rowa, rowb, lh, 0, r0a, r0b);
  read_scales<TN, TM>(smem, C::SA_OFF, C::SB_OFF, rowa, rowb, lh, s0a, s0b);
  scales_of(s0a, s0b, 0);
  decode_step(I0{}, r0a, r0b, d0a, d0b);

  // Stage s sits in buffer s % 2 and stage s + 1 is in flight into the other one. Before the
  // last K group reads ahead into stage s + 1, every wave waits for its share of stage s + 1,
  // the barrier publishes it (and ends all reads of stage s), and stage s + 2 (if there is one)
  // is fetched into buffer s % 2. Past the second-to-last stage the read-ahead sees a stale
  // buffer and goes unused; the last stage reads nothing ahead.
  using F = std::false_type;
  auto stage = [&](int s, const uint2 (&csa)[TN], const uint2 (&csb)[TM], uint2 (&nsa)[TN], uint2 (&nsb)[TM],
                   auto last) {
    constexpr bool LAST = decltype(last)::value;
    const uint8_t* cur = smem + (s & 1) * C::STAGE;
    const uint8_t* nxt = smem + ((s + 1) & 1) * C::STAGE;
    group(r0a, r0b, r1a, r1b, cur, 1, csa, csb, F{});
    group(r1a, r1b, r0a, r0b, cur, 2, csa, csb, F{});
    group(r0a, r0b, r1a, r1b, cur, 3, csa, csb, F{});
    wait_vmcnt<0>();
    __syncthreads();
    if (s + 2 < nk) issue_stage(s + 2);
    if constexpr (!LAST) read_scales<TN, TM>(nxt, C::SA_OFF, C::SB_OFF, rowa, rowb, lh, nsa, nsb);
    group(r1a, r1b, r0a, r0b, nxt, 0, nsa, nsb, last);
  };
  using T = std::true_type;
  int s = 0;
  for (; s + 2 < nk; s += 2) {
    stage(s, s0a, s0b, s1a, s1b, F{});
    stage(s + 1, s1a, s1b, s0a, s0b, F{});
  }
  if (s + 2 == nk) {
    stage(s, s0a, s0b, s1a, s1b, F{});
#pragma unroll
    for (int i = 0; i < TN; ++i) s0a[i] = s1a[i];
#pragma unroll
    for (int j = 0; j < TM; ++j) s0b[j] = s1b[j];
    ++s;
  }
  stage(s, s0a, s0b, s1a, s1b, T{});

  // ---- epilogue: y = bf16(acc * gx * gw), written to the LDS copy of the tile [BM][BN] by the
  // last stage above, then stored
  __syncthreads();
  if (a.y) store_tile_rows<BM, BN, C::TROW>(smem, a.y, a.ldy, M, N, m0, n0, tid, a.stream_y != 0);
  // optionally the nvfp4 encoding of Y for the next linear ("BFL (fp8r / nvfp4)": every
  // quantized linear quantizes its input at run time); its 16-blocks run along this N, inside
  // the tile
  if (a.yq) quant_tile_rows<BM, BN, C::TROW>(smem, a.yq, a.ys, 1.0f / a.gy[0], M, N, m0, n0, tid);
  // or the row maxima of an fp8r encoding, whose per-row scale spans every tile of the row
  if (a.ypmax) rowmax_tile<BM, BN, C::TROW>(smem, a.ypmax, M, N, m0, n0, tid);
}

template <int BM, int BN, bool LORA, int WPE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void gemm_w4a4_kernel(DecArgs a) {
  w4a4_tile<BM, BN, LORA>(a, blockIdx.x);
}

// The tiles of several W4A4 GEMMs in one grid: the problem of each workgroup, then that
// problem's tile, exactly as its own launch would compute it (same tile shape, same bits).
struct W4Group {
  DecArgs p[kMaxGroup];
  int start[kMaxGroup + 1];
  int count;
};
template <int BM, int BN, int WPE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void gemm_w4a4_grouped_kernel(W4Group g) {
  const int bid = blockIdx.x;
  const int p = group_problem(g.start, g.count, bid);
  w4a4_tile<BM, BN, false>(g.p[p], bid - g.start[p]);
}

// WPE: waves per SIMD the registers are budgeted for. The 128 x 128 tile takes 72 KB of LDS, so
// two of its workgroups share a compute unit when each wave keeps to 256 registers; the decode
// VALU of one then overlaps the other's MFMAs.
template <int BM, int BN>
hipError_t run(const DecArgs& a, hipStream_t s) {
  constexpr int WPE = BM == 128 && BN == 128 ? 2 : 1;
  const int tiles = (int)(((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN));
  if (a.lt)
    hipLaunchKernelGGL((gemm_w4a4_kernel<BM, BN, true, WPE>), dim3(tiles), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_w4a4_kernel<BM, BN, false, WPE>), dim3(tiles), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool gemm_w4a4_supported(const DecArgs& a) { return a.K % kStageK == 0; }

// Grouped W4A4: every problem with K % 256 == 0 and plain bf16 output (no adapter, no quantized
// output). The tile rule and its measurements are those of the grouped fp8r launch (128 x 128
// tiles two to a compute unit below three rounds of 256 x 192 tiles, else the 256 x 256 or
// 256 x 192 tile of least expected time over whole rounds), except that the decode-heavier W4A4
// tile already pays from 256 pair tiles (half a round): a joint block at 192 / 256 / 320 tokens
// as one grid 91.3 / 91.1 / 94.2 us against four launches 99.2 / 106.0 / 121.3 us, where the fp8r
// block lost (93.3 / 100.9 / 91.8 vs 76.6 / 83.3 / 86.7 us) and keeps the full round.
namespace {
struct GroupTile {
  int bm, bn, per_round, round_us;
};
constexpr GroupTile kW4GroupTiles[3] = {{256, 256, 256, 76}, {256, 192, 256, 60}, {128, 128, 512, 49}};
// the group's tile (index into kW4GroupTiles), or -1 when no tile fills two rounds
int w4a4_group_tile(const DecArgs* p, int count) {
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
  if (tiles_of(kW4GroupTiles[1], nullptr) < 3 * 256) {
    const int64_t t = tiles_of(kW4GroupTiles[2], nullptr);
    return t >= 256 && t < ((int64_t)1 << 31) ? 2 : -1;  // half a round of pairs already pays
  }
  int best = -1;
  double best_cost = 0;
  for (int t = 0; t < 2; ++t) {
    const GroupTile& c = kW4GroupTiles[t];
    double work = 0;
    const int64_t tiles = tiles_of(c, &work);
    if (tiles < 2 * (int64_t)c.per_round || tiles >= ((int64_t)1 << 31)) continue;  // 32-bit workgroup ids
    const double cost = std::ceil(work / c.per_round - 1e-9) * c.round_us;
    if (best < 0 || cost < best_cost) best = t, best_cost = cost;
  }
  return best;
}
template <int BM, int BN, int WPE>
hipError_t run_w4a4_group(const DecArgs* p, int count, hipStream_t s) {
  W4Group g{};
  g.count = count;
  int64_t total = 0;
  for (int i = 0; i < count; ++i) {
    g.p[i] = p[i];
    g.p[i].stream_y = stream_output((p[i].M + p[i].N) * (p[i].K / 2 + p[i].K / 16), p[i].M, p[i].N);
    g.start[i] = (int)total;
    total += ((p[i].M + BM - 1) / BM) * ((p[i].N + BN - 1) / BN);
  }
  for (int i = count; i <= kMaxGroup; ++i) g.start[i] = (int)total;
  hipLaunchKernelGGL((gemm_w4a4_grouped_kernel<BM, BN, WPE>), dim3((unsigned)total), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}
}  // namespace

bool gemm_w4a4_grouped_supported(const DecArgs* p, int count) {
  if (count < 2 || count > kMaxGroup) return false;
  for (int i = 0; i < count; ++i)
    if (p[i].K % kStageK != 0 || p[i].lt || p[i].yq || p[i].ypmax || !p[i].y) return false;
  return w4a4_group_tile(p, count) >= 0;
}

hipError_t launch_gemm_w4a4_grouped(const DecArgs* p, int count, hipStream_t s) {
  switch (w4a4_group_tile(p, count)) {
    case 0: return run_w4a4_group<256, 256, 1>(p, count, s);
    case 1: return run_w4a4_group<256, 192, 1>(p, count, s);
    default: return run_w4a4_group<128, 128, 2>(p, count, s);
  }
}

bool lora_pre_scaled_w4a4(const DecArgs& a) { return gemm_w4a4_supported(a); }

hipError_t launch_gemm_w4a4(const DecArgs& args, hipStream_t s) {
  DecArgs a = args;
  a.stream_y = stream_output((a.M + a.N) * (a.K / 2 + a.K / 16), a.M, a.N);
  // While its grid fits one round on the 256 compute units, the smallest tile (64 x 64, then
  // 64 tokens x 128 weight rows): a grid of few large tiles leaves units idle while each busy
  // one waits on its own loads. Measured at K = 3072: 512 x 3072 26.6 -> 19.2 us, 256 x 3072
  // 27 -> 13.3 us, 64 x 12288 29 -> 14 us, 512 x 3072 x 12288 88 -> 64 us.
  //
  // Larger grids take the tile of least expected time over whole rounds, with round times
  // measured at K = 3072 with every unit busy: 256 x 256 76 us and 256 x 192 60 us for 256
  // tiles, 128 x 128 49 us for 512 (two workgroups a compute unit). The square tile does the
  // most work per operand byte and per decode, so it wins when the rounds come out even, as at
  // 4096 x 12288: 230 vs 240 us. Where they do not: 3072 x 3072 75 -> 53 us and 4096 x 6144
  // 136 -> 122 us on 256 x 192; 2048 x 3072 54 -> 43 us and 1536 x 3072 48 -> 41 us on
  // 128 x 128. Every tile shape gives the same bits.
  const int64_t t64 = ((a.M + 63) / 64) * ((a.N + 63) / 64), t64x128 = ((a.M + 63) / 64) * ((a.N + 127) / 128);
  if (t64 <= 256) return run<64, 64>(a, s);
  if (t64x128 <= 256) return run<64, 128>(a, s);
  const int64_t c256 = rounds_cost(a.M, a.N, 256, 256, 76), c192 = rounds_cost(a.M, a.N, 256, 192, 60);
  const int64_t c128 = ((a.M + 127) / 128 * ((a.N + 127) / 128) + 511) / 512 * 49;
  if (c256 <= c192 && c256 <= c128) return run<256, 256>(a, s);
  if (c192 <= c128) return run<256, 192>(a, s);
  return run<128, 128>(a, s);
}

}  // namespace bsq
