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
// Data movement (conventions in gemm_common.hpp): each 64-deep K stage of
// every W and Xq row -- 32 bytes of packed codes plus 4 block-scale bytes --
// is copied to LDS as stored, by LDS DMA, into a ring of NS stage buffers.
// Every wave reads its operands' packed bytes from LDS one stage ahead and
// decodes them in registers right before the MFMAs of each 16-deep K step:
// per byte one v_cvt_scalef32_pk_f16_fp4 (exact E2M1 -> f16 pair) and one
// v_pk_mul_f16 by the block scale. LDS traffic stays at the packed size; the
// decode work (about 4 VALU per MFMA) issues under the MFMAs.
//
// K permutation: within a stage, lane half h of an MFMA operand covers K
// values [32 h, 32 h + 32) of the stage, one 8-value group per K step, for
// both operands alike, so every product pairs equal K indices.
#include "gemm_common.hpp"
#include "bsq_launch.hpp"

namespace bsq {

namespace {

using namespace gemm;

template <int BM, int BN, int NS>
struct W4Cfg {
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int TM = WM / 32, TN = WN / 32;
  using RA = Region<32, BN>;  // packed W rows, 32 bytes per stage
  using RB = Region<32, BM>;  // packed Xq rows
  using SA = ScaleRegion<BN>;
  using SB = ScaleRegion<BM>;
  static constexpr int A_OFF = 0, B_OFF = BN * 32, SA_OFF = (BN + BM) * 32, SB_OFF = SA_OFF + BN * 4;
  static constexpr int STAGE = (BN + BM) * 36;
  static constexpr int LOADS_MIN = RA::MIN_PER_WAVE + RB::MIN_PER_WAVE + SA::MIN_PER_WAVE + SB::MIN_PER_WAVE;
  static constexpr int TROW = BN * 2 + 16;  // bytes per row of the bf16 output tile in LDS
  static constexpr int LDS = NS * STAGE > BM * TROW ? NS * STAGE : BM * TROW;
  static_assert(NS >= 3, "at least one stage in flight behind the next");
  static_assert((NS - 3) * LOADS_MIN < 64, "vmcnt range");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// packed operand bytes of one stage for one lane: 32 E2M1 values (4 dwords)
// and the two E4M3 scales of its two 16-value blocks as f16 pairs
struct Raw {
  uint4 q;
  uint32_t s;  // two scale bytes in bits 15:0
};

template <int TN, int TM>
__device__ __forceinline__ void read_raw(const uint8_t* st, int a_off, int b_off, int sa_off, int sb_off, int rowa,
                                         int rowb, int lh, Raw (&ra)[TN], Raw (&rb)[TM]) {
#pragma unroll
  for (int i = 0; i < TN; ++i) {
    const int row = rowa + i * 32;
    ra[i].q = *reinterpret_cast<const uint4*>(st + a_off + swz_off<32>(row, lh));
    ra[i].s = *reinterpret_cast<const uint16_t*>(st + sa_off + row * 4 + 2 * lh);
  }
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int row = rowb + j * 32;
    rb[j].q = *reinterpret_cast<const uint4*>(st + b_off + swz_off<32>(row, lh));
    rb[j].s = *reinterpret_cast<const uint16_t*>(st + sb_off + row * 4 + 2 * lh);
  }
}

// block scale byte b (0 or 1) of `s` as an f16 pair (E4M3 -> f16 is exact)
__device__ __forceinline__ v2h scale_pair(uint32_t s, int b) {
  const uint32_t dup = __builtin_amdgcn_perm(s, s, b ? 0x01010101u : 0x00000000u);
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(dup, 1.0f, false);
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

template <int BM, int BN, int NS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_w4a4_kernel(DecArgs a) {
  using C = W4Cfg<BM, BN, NS>;
  constexpr int TN = C::TN, TM = C::TM;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];

  const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
  int m0, n0;
  tile_of_block(M, N, BM, BN, m0, n0);
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

  auto issue_stage = [&](int kt) {
    const int kb = kt * kKS;
    const uint32_t base = lds0 + (uint32_t)((kt % NS) * C::STAGE);
    dma_region<typename C::RA>(rwq, base + C::A_OFF, wave, lane, kp, kb >> 1, kb, K);
    dma_region<typename C::RB>(rxq, base + C::B_OFF, wave, lane, kp, kb >> 1, kb, K);
    dma_scales<typename C::SA>(rws, base + C::SA_OFF, wave, lane, ks, kb < K ? kb : kOutOfRange);
    dma_scales<typename C::SB>(rxs, base + C::SB_OFF, wave, lane, ks, kb < K ? kb : kOutOfRange);
  };

  v16f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v16f{};

  const int lr = lane & 31, lh = lane >> 5;
  const int rowa = wn * C::WN + lr, rowb = wm * C::WM + lr;  // region-local rows
  const int nk = K / kKS;

#pragma unroll
  for (int p = 0; p < NS - 1; ++p) issue_stage(p);
  wait_vmcnt<(NS - 2) * C::LOADS_MIN>();
  __syncthreads();

  Raw r0a[TN], r0b[TM], r1a[TN], r1b[TM];  // packed operands of the current / next stage
  v8h d0a[TN], d0b[TM], d1a[TN], d1b[TM];  // decoded operands of two consecutive K steps
  v2h spa[TN][2], spb[TM][2];              // block-scale pairs of the stage being decoded

  auto scales_of = [&](const Raw (&ra)[TN], const Raw (&rb)[TM]) {
#pragma unroll
    for (int i = 0; i < TN; ++i) { spa[i][0] = scale_pair(ra[i].s, 0); spa[i][1] = scale_pair(ra[i].s, 1); }
#pragma unroll
    for (int j = 0; j < TM; ++j) { spb[j][0] = scale_pair(rb[j].s, 0); spb[j][1] = scale_pair(rb[j].s, 1); }
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
  // one K step's MFMAs with the next step's decode (VALU) and reads (LDS) issued between them
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
  constexpr int DEC_VALU = 8 * (TN + TM) / (TN * TM) + 1;  // decode VALU per MFMA (rounded up)

  read_raw<TN, TM>(smem, C::A_OFF, C::B_OFF, C::SA_OFF, C::SB_OFF, rowa, rowb, lh, r0a, r0b);
  scales_of(r0a, r0b);
  decode_step(I0{}, r0a, r0b, d0a, d0b);

  // stage s: its packed operands in ca/cb, K step 0 already decoded in d0; stage s + 1 is read
  // into na/nb and its K step 0 decoded into d0 at the end. Past the last stage this reads a
  // buffer of zeros (stages beyond K are fetched as zeros) and the result goes unused.
  auto iteration = [&](int s, const Raw (&ca)[TN], const Raw (&cb)[TM], Raw (&na)[TN], Raw (&nb)[TM]) {
    {
      wait_vmcnt<(NS - 3) * C::LOADS_MIN>();  // this wave's share of stage s + 1 has landed
      __syncthreads();                         // everybody's has; nobody reads stage s - 1 any more
      issue_stage(s + NS - 1);
      const uint8_t* st = smem + ((s + 1) % NS) * C::STAGE;
      read_raw<TN, TM>(st, C::A_OFF, C::B_OFF, C::SA_OFF, C::SB_OFF, rowa, rowb, lh, na, nb);
    }
    decode_step(I1{}, ca, cb, d1a, d1b);
    mfmas(d0a, d0b);
    pipeline(std::integral_constant<int, DEC_VALU>{}, std::integral_constant<int, 2>{});
    decode_step(I2{}, ca, cb, d0a, d0b);
    mfmas(d1a, d1b);
    pipeline(std::integral_constant<int, DEC_VALU>{}, I0{});
    decode_step(I3{}, ca, cb, d1a, d1b);
    mfmas(d0a, d0b);
    pipeline(std::integral_constant<int, DEC_VALU>{}, I0{});
    scales_of(na, nb);
    decode_step(I0{}, na, nb, d0a, d0b);
    mfmas(d1a, d1b);
    pipeline(std::integral_constant<int, DEC_VALU + 2>{}, I0{});
  };
  int s = 0;
  for (; s + 1 < nk; s += 2) {
    iteration(s, r0a, r0b, r1a, r1b);
    iteration(s + 1, r1a, r1b, r0a, r0b);
  }
  if (s < nk) iteration(s, r0a, r0b, r1a, r1b);

  // ---- epilogue: y = bf16(acc * gx * gw) via an LDS copy of the tile [BM][BN]
  const float alpha = a.gx[0] * a.gw[0];
  wait_vmcnt<0>();
  __syncthreads();  // all stage buffers are free now
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int ml = wm * C::WM + j * 32 + lr;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nl = wn * C::WN + i * 32 + 8 * g + 4 * lh;
        const v16f& A = acc[i][j];
        *reinterpret_cast<uint2*>(smem + ml * C::TROW + nl * 2) =
            make_uint2(pack_bf16x2(A[4 * g + 0] * alpha, A[4 * g + 1] * alpha),
                       pack_bf16x2(A[4 * g + 2] * alpha, A[4 * g + 3] * alpha));
      }
    }
  }
  __syncthreads();
  store_tile_rows<BM, BN, C::TROW>(smem, a.y, a.ldy, M, N, m0, n0, tid);
}

template <int BM, int BN, int NS>
hipError_t run(const DecArgs& a, hipStream_t s) {
  const int tiles = (int)(((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN));
  hipLaunchKernelGGL((gemm_w4a4_kernel<BM, BN, NS>), dim3(tiles), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool gemm_w4a4_supported(const DecArgs& a) { return a.K % kKS == 0; }

hipError_t launch_gemm_w4a4(const DecArgs& a, hipStream_t s) {
  const int64_t t256 = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  if (t256 >= 192) return run<256, 256, 4>(a, s);
  return run<128, 128, 6>(a, s);
}

}  // namespace bsq
