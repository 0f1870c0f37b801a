// Decode-to-16-bit GEMMs for nvfp4 (W4A4, W4A16) and fp8r weight-only (W8A16)
// on the gfx950 bf16 / f16 matrix cores.
//
// "BFL (fp8r / nvfp4)", nvfp4 bullet: a weight value is e2m1 * e4m3(block
// scale over 16) * weight_scale_2, and activations are quantized the same way
// with input_scale ("Kernels" table). The product of an E2M1 value (2
// significant bits) and an E4M3 scale (4 significant bits) has at most 6
// significant bits and lies in [2^-10, 2688], so it is exact in both f16 and
// bf16. The decoder therefore turns each 16-element block into exact 16-bit
// values and the contraction runs on the 16-bit matrix cores with fp32
// accumulation; the two fp32 global scales are rank-0 and go to the
// epilogue. (gfx950's block-scaled FP4 MFMA takes power-of-two scales per 32
// elements, which cannot represent an E4M3 scale per 16 exactly.)
//
//   W4A4 : X and W both nvfp4, decoded to f16, v_mfma_f32_32x32x16_f16,
//          y = bf16(acc * (gx * gw)).
//   W4A16: X bf16 as stored, W nvfp4 decoded to bf16, v_mfma_f32_32x32x16_bf16,
//          y = bf16(acc * gw)         (the fallback's arithmetic, "Kernels"
//                                       last paragraph, without rounding W).
//   W8A16: X bf16, W E4M3 decoded to bf16, y = bf16(acc * sw[n]).
//
// Tiling as in the FP8 kernel: 4 waves, each a (BM/2) x (BN/2) quadrant of
// 32x32 MFMA tiles; W rows feed the MFMA A operand so each lane stores four
// consecutive n. One LDS stage holds 64 K-values (128 bytes) of every X row
// then every W row, decoded, with 16-byte chunks XOR-swizzled by (row & 7).
// Each thread stages whole rows: it loads the packed row segment (32 bytes
// of E2M1 plus 4 block scales, 64 bytes of E4M3 or 128 bytes of bf16),
// decodes it in registers and writes 8 swizzled 16-byte chunks.
#include "bsq_launch.hpp"
#include "gemm_common.hpp"

namespace bsq {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;  // K values per iteration

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

enum RowKind : int { kNvfp4F16 = 0, kNvfp4Bf16 = 1, kE4m3Bf16 = 2, kBf16 = 3 };

// Registers holding one row's segment of one stage, before decoding.
struct RowRaw {
  uint4 d[8];   // packed data (how many are used depends on the kind)
  uint32_t s;   // 4 block scales (nvfp4 kinds)
};

template <int KIND>
__device__ __forceinline__ void load_row(RowRaw& r, const uint8_t* src, const uint8_t* ssrc, bool ok, int kb,
                                         int K) {
  if (KIND == kNvfp4F16 || KIND == kNvfp4Bf16) {
    // src: row start of packed bytes, ssrc: row start of block scales
    r.d[0] = make_uint4(0, 0, 0, 0);
    r.d[1] = make_uint4(0, 0, 0, 0);
    uint32_t s0 = 0, s1 = 0;
    if (ok) {
      r.d[0] = *reinterpret_cast<const uint4*>(src + (kb >> 1));
      s0 = *reinterpret_cast<const uint16_t*>(ssrc + (kb >> 4));
      if (kb + 32 < K) {
        r.d[1] = *reinterpret_cast<const uint4*>(src + (kb >> 1) + 16);
        s1 = *reinterpret_cast<const uint16_t*>(ssrc + (kb >> 4) + 2);
      }
    }
    r.s = s0 | (s1 << 16);
  } else if (KIND == kE4m3Bf16) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      r.d[c] = make_uint4(0, 0, 0, 0);
      if (ok && kb + 16 * c < K) r.d[c] = *reinterpret_cast<const uint4*>(src + kb + 16 * c);
    }
  } else {  // bf16, src is a uint16 row viewed as bytes
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      r.d[c] = make_uint4(0, 0, 0, 0);
      if (ok && kb + 8 * c < K) r.d[c] = *reinterpret_cast<const uint4*>(src + 2 * (kb + 8 * c));
    }
  }
}

__device__ __forceinline__ uint32_t h2bits(v2h v) {
  union { v2h h; uint32_t u; } x;
  x.h = v;
  return x.u;
}

// 8 packed E2M1 values (one dword) times block scale -> 8 f16 (one 16-byte chunk)
__device__ __forceinline__ uint4 dec8_f16(uint32_t q, v2h s) {
  return make_uint4(h2bits(dec_e2m1x2_f16<0>(q) * s), h2bits(dec_e2m1x2_f16<1>(q) * s),
                    h2bits(dec_e2m1x2_f16<2>(q) * s), h2bits(dec_e2m1x2_f16<3>(q) * s));
}
template <int sel>
__device__ __forceinline__ uint32_t dec2_bf16(uint32_t q, float s) {
  const v2f e = dec_e2m1x2_f32<sel>(q);
  return pack_bf16x2(e.x * s, e.y * s);
}
__device__ __forceinline__ uint4 dec8_bf16(uint32_t q, float s) {
  return make_uint4(dec2_bf16<0>(q, s), dec2_bf16<1>(q, s), dec2_bf16<2>(q, s), dec2_bf16<3>(q, s));
}
__device__ __forceinline__ uint2 e4m3x4_bf16(uint32_t q) {
  const v2f a = dec_e4m3x2<false>(q), b = dec_e4m3x2<true>(q);
  return make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(b.x, b.y));
}

// E4M3 block scale b (0..3) of a scale word; b is a constant after unrolling
__device__ __forceinline__ float scale_of(uint32_t s, int b) {
  switch (b) {
    case 0: return dec_e4m3<0>(s);
    case 1: return dec_e4m3<1>(s);
    case 2: return dec_e4m3<2>(s);
    default: return dec_e4m3<3>(s);
  }
}

template <int KIND>
__device__ __forceinline__ void store_row(const RowRaw& r, uint8_t* base, int row) {
  if (KIND == kNvfp4F16) {
    const uint32_t q[8] = {r.d[0].x, r.d[0].y, r.d[0].z, r.d[0].w, r.d[1].x, r.d[1].y, r.d[1].z, r.d[1].w};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const _Float16 sh = (_Float16)scale_of(r.s, b);
      const v2h s = v2h{sh, sh};
      *reinterpret_cast<uint4*>(base + swz(row, 2 * b)) = dec8_f16(q[2 * b], s);
      *reinterpret_cast<uint4*>(base + swz(row, 2 * b + 1)) = dec8_f16(q[2 * b + 1], s);
    }
  } else if (KIND == kNvfp4Bf16) {
    const uint32_t q[8] = {r.d[0].x, r.d[0].y, r.d[0].z, r.d[0].w, r.d[1].x, r.d[1].y, r.d[1].z, r.d[1].w};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float s = scale_of(r.s, b);
      *reinterpret_cast<uint4*>(base + swz(row, 2 * b)) = dec8_bf16(q[2 * b], s);
      *reinterpret_cast<uint4*>(base + swz(row, 2 * b + 1)) = dec8_bf16(q[2 * b + 1], s);
    }
  } else if (KIND == kE4m3Bf16) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint2 a = e4m3x4_bf16(r.d[c].x), b = e4m3x4_bf16(r.d[c].y);
      const uint2 e = e4m3x4_bf16(r.d[c].z), f = e4m3x4_bf16(r.d[c].w);
      *reinterpret_cast<uint4*>(base + swz(row, 2 * c)) = make_uint4(a.x, a.y, b.x, b.y);
      *reinterpret_cast<uint4*>(base + swz(row, 2 * c + 1)) = make_uint4(e.x, e.y, f.x, f.y);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) *reinterpret_cast<uint4*>(base + swz(row, c)) = r.d[c];
  }
}

template <int MODE>
struct ModeTraits;
template <>
struct ModeTraits<kW4A4> {
  static constexpr int XK = kNvfp4F16, WK = kNvfp4F16;
  static constexpr bool F16 = true;
};
template <>
struct ModeTraits<kW4A16> {
  static constexpr int XK = kBf16, WK = kNvfp4Bf16;
  static constexpr bool F16 = false;
};
template <>
struct ModeTraits<kW8A16> {
  static constexpr int XK = kBf16, WK = kE4m3Bf16;
  static constexpr bool F16 = false;
};

template <int MODE, int BM, int BN, bool LORA>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_dec_kernel(DecArgs a) {
  using T = ModeTraits<MODE>;
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
  constexpr int ROWS = BM + BN, STAGE = ROWS * 128;
  constexpr int RPT = (ROWS + kThreads - 1) / kThreads;  // rows staged per thread
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  grouped_tile(xcd_contiguous_id(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, 8, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // staging map: row r = tid + 256 j of the stage (X rows first, then W rows)
  const uint8_t* src[RPT];
  const uint8_t* ssrc[RPT];
  bool ok[RPT], isx[RPT], act[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int r = tid + kThreads * j;
    act[j] = r < ROWS;
    isx[j] = r < BM;
    src[j] = nullptr;
    ssrc[j] = nullptr;
    if (isx[j]) {
      const int gm = m0 + r;
      ok[j] = gm < M;
      const int64_t gr = ok[j] ? gm : 0;
      if (T::XK == kNvfp4F16) {
        src[j] = a.xq + gr * (K >> 1);
        ssrc[j] = a.xs + gr * (K >> 4);
      } else {
        src[j] = reinterpret_cast<const uint8_t*>(a.x + gr * a.ldx);
      }
    } else {
      const int gn = n0 + r - BM;
      ok[j] = act[j] && gn < N;
      const int64_t gr = ok[j] ? gn : 0;
      if (T::WK == kE4m3Bf16) {
        src[j] = a.w + gr * K;
      } else {
        src[j] = a.w + gr * (K >> 1);
        ssrc[j] = a.ws + gr * (K >> 4);
      }
    }
  }
  RowRaw raw[RPT];
  auto gload = [&](int kt) {
    const int kb = kt * kBK;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      if (!act[j]) continue;
      if (isx[j]) load_row<T::XK>(raw[j], src[j], ssrc[j], ok[j], kb, K);
      else load_row<T::WK>(raw[j], src[j], ssrc[j], ok[j], kb, K);
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* base = smem + buf * STAGE;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      if (!act[j]) continue;
      const int r = tid + kThreads * j;
      if (isx[j]) store_row<T::XK>(raw[j], base, r);
      else store_row<T::WK>(raw[j], base, r);
    }
  };

  v16f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v16f{};

  const int lr = lane & 31, lh = lane >> 5;
  const int nk = (K + kBK - 1) / kBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* base = smem + cur * STAGE;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c = 4 * lh + t;
      uint4 av[TN], bv[TM];
#pragma unroll
      for (int i = 0; i < TN; ++i) av[i] = *reinterpret_cast<const uint4*>(base + swz(BM + wn * WN + i * 32 + lr, c));
#pragma unroll
      for (int j = 0; j < TM; ++j) bv[j] = *reinterpret_cast<const uint4*>(base + swz(wm * WM + j * 32 + lr, c));
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) {
          if (T::F16) {
            union { uint4 u; v8h h; } x, z;
            x.u = av[i];
            z.u = bv[j];
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(x.h, z.h, acc[i][j], 0, 0, 0);
          } else {
            union { uint4 u; v8bf h; } x, z;
            x.u = av[i];
            z.u = bv[j];
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x.h, z.h, acc[i][j], 0, 0, 0);
          }
        }
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue
  const bool vec_ok = (a.ldy & 3) == 0;  // 8-byte stores need 4-element aligned rows
  float alpha = 1.0f;
  if (MODE == kW4A4) alpha = a.gx[0] * a.gw[0];
  if (MODE == kW4A16) alpha = a.gw[0];
  if constexpr (LORA) {
    // with an adapter: y = bf16(acc * scale + T B^T), the adapter's MFMAs accumulating onto the
    // scaled accumulators
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * WN + i * 32 + 8 * g + 4 * lh;
        float s[4] = {alpha, alpha, alpha, alpha};
        if (MODE == kW8A16) {
#pragma unroll
          for (int e = 0; e < 4; ++e) s[e] = (n + e < N) ? a.sw[n + e] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][4 * g + e] *= s[e];
      }
    gemm::lora_update<TN, TM>(acc, a.lt, a.lb, a.rank, M, N, n0 + wn * WN, m0 + wm * WM, lane);
    alpha = 1.0f;
  }
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int m = m0 + wm * WM + j * 32 + lr;
    if (m >= M) continue;
    uint16_t* yr = a.y + (int64_t)m * a.ldy;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * WN + i * 32 + 8 * g + 4 * lh;
        const v16f& A = acc[i][j];
        float s[4] = {alpha, alpha, alpha, alpha};
        if (MODE == kW8A16 && !LORA) {
#pragma unroll
          for (int e = 0; e < 4; ++e) s[e] = (n + e < N) ? a.sw[n + e] : 0.0f;
        }
        if (n + 3 < N && vec_ok) {
          *reinterpret_cast<uint2*>(yr + n) = make_uint2(pack_bf16x2(A[4 * g] * s[0], A[4 * g + 1] * s[1]),
                                                         pack_bf16x2(A[4 * g + 2] * s[2], A[4 * g + 3] * s[3]));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) yr[n + e] = (uint16_t)(pack_bf16x2(A[4 * g + e] * s[e], 0.0f) & 0xFFFFu);
        }
      }
    }
  }
}

template <int MODE, int BM, int BN, bool LORA>
hipError_t run_kernel(const DecArgs& a, hipStream_t s) {
  const size_t lds = 2 * (size_t)(BM + BN) * 128;
  static std::atomic<unsigned long long> lds_set{0};
  hipError_t e =
      ensure_lds_limit(reinterpret_cast<const void*>(&gemm_dec_kernel<MODE, BM, BN, LORA>), (int)lds, lds_set);
  if (e != hipSuccess) return e;
  const int tiles = (int)(((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN));
  hipLaunchKernelGGL((gemm_dec_kernel<MODE, BM, BN, LORA>), dim3(tiles), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}
template <int MODE, int BM, int BN>
hipError_t run(const DecArgs& a, hipStream_t s) {
  return a.lt ? run_kernel<MODE, BM, BN, true>(a, s) : run_kernel<MODE, BM, BN, false>(a, s);
}

template <int MODE>
hipError_t pick(const DecArgs& a, hipStream_t s) {
  const int64_t t256 = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  const int64_t t192 = ((a.M + 255) / 256) * ((a.N + 191) / 192);
  if (t256 >= 256) return run<MODE, 256, 256>(a, s);
  if (t192 >= 192) return run<MODE, 256, 192>(a, s);
  return run<MODE, 128, 128>(a, s);
}

}  // namespace

hipError_t launch_gemm_dec(DecMode mode, const DecArgs& a, hipStream_t s) {
  switch (mode) {
    case kW4A4: return gemm_w4a4_supported(a) ? launch_gemm_w4a4(a, s) : pick<kW4A4>(a, s);
    case kW4A16: return gemm_a16_supported(mode, a) ? launch_gemm_a16(mode, a, s) : pick<kW4A16>(a, s);
    default: return gemm_a16_supported(mode, a) ? launch_gemm_a16(mode, a, s) : pick<kW8A16>(a, s);
  }
}

}  // namespace bsq
