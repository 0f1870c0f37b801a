// Skinny GEMMs for few tokens (small M), all four schemes of the linear layer.
//
// With few activation rows the layer is a stream over the weights ("BFL
// (fp8r / nvfp4)", "Kernels" table: the weight is read once per call), and a
// tiled GEMM with one workgroup per output tile leaves most compute units
// idle and walks K serially. Here every workgroup owns one MFMA block of 32
// weight rows (N) and MB blocks of 32 activation rows (M), and its waves
// split K: wave w of NW takes the 128-deep K stages w, w + NW, w + 2 NW, ...
// The NW partial tiles are summed through LDS in wave order, so the result
// does not depend on timing, and the epilogue applies the scheme's scales:
//   W4A4 : y = bf16(acc * gx * gw)          f16 MFMA on exact decoded nvfp4
//   W4A16: y = bf16(acc * gw)               bf16 MFMA, X as given
//   W8A8 : y = bf16(acc * sx[m] * sw[n])    fp8 MFMA on the E4M3 codes
//   W8A16: y = bf16(acc * sw[n])            bf16 MFMA, W decoded exactly
//
// Operand fetch, two variants:
//  - E4M3 weights (W8A8, W8A16): each wave streams its stages through a
//    private ring of two LDS stage buffers with LDS DMA -- whole 128- or
//    256-byte row segments per request, so a 1 KB request touches 4 to 8
//    cache lines, where loading the MFMA operand layout directly (each lane
//    its own row) touches 32 -- and reads its operands from there. A wave
//    only reads what it fetched itself, so the K loop has no workgroup
//    barrier.
//  - nvfp4 weights (W4A4, W4A16): operands go from global memory straight
//    into the MFMA operand registers with buffer loads, two stages in flight
//    per wave (8 waves per workgroup).
//
// K layout of a stage (kb = first K value): lane half h of an MFMA operand
// holds the 64 values [kb + 64 h, kb + 64 h + 64), in MFMA K steps of 8
// (16-bit MFMAs) or 32 (fp8 MFMA) consecutive values -- the same for both
// operands, so every product pairs equal K indices. Workgroups start their walk over K at
// different stages (see stage_k).
#include "gemm_common.hpp"
#include "bsq_launch.hpp"

namespace bsq {

namespace {

using namespace gemm;


// ---- operands of one stage for one lane -------------------------------------------
// nvfp4: 64 values = 32 packed bytes (q[g] holds values 32 g .. 32 g + 31 of the lane's
// window) and their 4 E4M3 block scales (byte b scales values 16 b .. 16 b + 15)
struct OpNv {
  uint4 q[2];
  uint32_t s;
};
// fp8: 64 E4M3 codes
struct OpF8 {
  uint4 d[4];
};
// bf16: 64 values
struct OpBf {
  uint4 d[8];
};

// ---- decoders ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t h2u(v2h v) {
  union { v2h h; uint32_t u; } c;
  c.h = v;
  return c.u;
}
// block scale byte b of s as an f16 pair / as fp32 (E4M3 is exact in both)
__device__ __forceinline__ v2h scale_h2(uint32_t s, int b) {
  const uint32_t dup = __builtin_amdgcn_perm(s, s, 0x01010101u * (uint32_t)b);
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(dup, 1.0f, false);
}
__device__ __forceinline__ float scale_f(uint32_t s, int b) {
  switch (b) {
    case 0: return dec_e4m3<0>(s);
    case 1: return dec_e4m3<1>(s);
    case 2: return dec_e4m3<2>(s);
    default: return dec_e4m3<3>(s);
  }
}
// 8 E2M1 values (one packed dword) times their block scale, as 8 f16 / 8 bf16; both exact
__device__ __forceinline__ v8h nv8_f16(uint32_t w, v2h s) {
  union { uint4 u; v8h h; } r;
  r.u = make_uint4(h2u(dec_e2m1x2_f16<0>(w) * s), h2u(dec_e2m1x2_f16<1>(w) * s), h2u(dec_e2m1x2_f16<2>(w) * s),
                   h2u(dec_e2m1x2_f16<3>(w) * s));
  return r.h;
}
template <int sel>
__device__ __forceinline__ uint32_t nv2_bf16(uint32_t w, float s) {
  const v2f e = dec_e2m1x2_f32<sel>(w);
  return pack_bf16x2(e.x * s, e.y * s);
}
__device__ __forceinline__ v8bf nv8_bf16(uint32_t w, float s) {
  union { uint4 u; v8bf b; } r;
  r.u = make_uint4(nv2_bf16<0>(w, s), nv2_bf16<1>(w, s), nv2_bf16<2>(w, s), nv2_bf16<3>(w, s));
  return r.b;
}
// 8 E4M3 codes (two dwords) as 8 bf16 (exact)
__device__ __forceinline__ v8bf f8x8_bf16(uint32_t lo, uint32_t hi) {
  const v2f a = dec_e4m3x2<false>(lo), b = dec_e4m3x2<true>(lo), c = dec_e4m3x2<false>(hi), d = dec_e4m3x2<true>(hi);
  union { uint4 u; v8bf b; } r;
  r.u = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(b.x, b.y), pack_bf16x2(c.x, c.y), pack_bf16x2(d.x, d.y));
  return r.b;
}
__device__ __forceinline__ v8bf as_bf(uint4 u) {
  union { uint4 u; v8bf b; } r;
  r.u = u;
  return r.b;
}
__device__ __forceinline__ uint32_t dw(const uint4& q, int t) { return t == 0 ? q.x : t == 1 ? q.y : t == 2 ? q.z : q.w; }

// ---- per-scheme stage: operand types, loads and MFMAs ---------------------------------
template <int MODE>
struct Scheme;

template <>
struct Scheme<kW4A4> {
  using WOp = OpNv;
  using XOp = OpNv;
  template <int MB>
  __device__ static void mma(v16f (&acc)[MB], const WOp& w, const XOp (&x)[MB]) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int b = 2 * g + (t >> 1);
        const v8h a = nv8_f16(dw(w.q[g], t), scale_h2(w.s, b));
#pragma unroll
        for (int j = 0; j < MB; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, nv8_f16(dw(x[j].q[g], t), scale_h2(x[j].s, b)), acc[j],
                                                          0, 0, 0);
      }
  }
};
template <>
struct Scheme<kW4A16> {
  using WOp = OpNv;
  using XOp = OpBf;
  template <int MB>
  __device__ static void mma(v16f (&acc)[MB], const WOp& w, const XOp (&x)[MB]) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const v8bf a = nv8_bf16(dw(w.q[g], t), scale_f(w.s, 2 * g + (t >> 1)));
#pragma unroll
        for (int j = 0; j < MB; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf(x[j].d[4 * g + t]), acc[j], 0, 0, 0);
      }
  }
};
template <>
struct Scheme<kW8A8> {
  using WOp = OpF8;
  using XOp = OpF8;
  template <int MB>
  __device__ static void mma(v16f (&acc)[MB], const WOp& w, const XOp (&x)[MB]) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint4 l = w.d[2 * s], h = w.d[2 * s + 1];
      const v8i a = v8i{(int)l.x, (int)l.y, (int)l.z, (int)l.w, (int)h.x, (int)h.y, (int)h.z, (int)h.w};
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const uint4 xl = x[j].d[2 * s], xh = x[j].d[2 * s + 1];
        const v8i b = v8i{(int)xl.x, (int)xl.y, (int)xl.z, (int)xl.w, (int)xh.x, (int)xh.y, (int)xh.z, (int)xh.w};
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, 0, 0, 0, 0, 0);
      }
    }
  }
};
template <>
struct Scheme<kW8A16> {
  using WOp = OpF8;
  using XOp = OpBf;
  template <int MB>
  __device__ static void mma(v16f (&acc)[MB], const WOp& w, const XOp (&x)[MB]) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint4& q = w.d[c >> 1];
      const v8bf a = (c & 1) ? f8x8_bf16(q.z, q.w) : f8x8_bf16(q.x, q.y);
#pragma unroll
      for (int j = 0; j < MB; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf(x[j].d[c]), acc[j], 0, 0, 0);
    }
  }
};

// sum the NW partial tiles (red = [NW][MB][16 registers][64 lanes]) in wave order, scale,
// convert and store the tile
// Low-rank adapter tile of the workgroup: T B^T for its 32 weight rows and activation block j
// = wave (waves 0 .. MB - 1), on the bf16 matrix cores, 64 rank values per batch of loads, into
// lred [MB][16][64] in the accumulator layout (lane: token, register: weight row).
template <int MB>
__device__ __forceinline__ void skinny_lora_tile(const DecArgs& a, float* lred, int m0, int n0, int wave, int lane) {
  if (wave >= MB) return;
  const rsrc_t rt = make_rsrc(a.lt, (uint32_t)a.M * (uint32_t)a.rank * 2u);
  const rsrc_t rb = make_rsrc(a.lb, (uint32_t)a.N * (uint32_t)a.rank * 2u);
  v16f l[1][1] = {{v16f{}}};
  for (int k0 = 0; k0 < a.rank; k0 += 64) {
    LoraRegs<1, 1, 4> r;
    lora_load(r, rt, rb, k0, a.rank, n0, m0 + 32 * wave, lane);
    lora_mfma(l, r, k0, a.rank);
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) lred[(wave * 16 + e) * 64 + lane] = l[0][0][e];
}

// lred: the adapter tiles (LORA), added to the scaled sums: y = bf16(acc * scale + T B^T)
template <int MODE, int MB, int NW, bool LORA>
__device__ __forceinline__ void skinny_epilogue(const DecArgs& a, const float* red, const float* lred, int m0, int n0,
                                                int tid) {
  const int M = (int)a.M, N = (int)a.N;
  float alpha = 1.0f;
  if constexpr (MODE == kW4A4) alpha = a.gx[0] * a.gw[0];
  if constexpr (MODE == kW4A16) alpha = a.gw[0];
  // thread -> (row ml of the tile, output pair p): consecutive threads write consecutive pairs
  for (int idx = tid; a.y && idx < 32 * MB * 16; idx += 64 * NW) {
    const int ml = idx >> 4, p = idx & 15;
    const int m = m0 + ml;
    if (m >= M) break;
    const int j = ml >> 5, lm = ml & 31;
    float v[2], lv[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int nl = 2 * p + e;  // n = 8 G + 4 H + q is held by lane lm + 32 H in register 4 G + q
      const int r = 4 * (nl >> 3) + (nl & 3), ln = lm + 32 * ((nl >> 2) & 1);
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += red[((w * MB + j) * 16 + r) * 64 + ln];
      v[e] = s;
      lv[e] = LORA ? lred[(j * 16 + r) * 64 + ln] : 0.0f;
    }
    const int n = n0 + 2 * p;
    float s0 = alpha, s1 = alpha;
    if constexpr (MODE == kW8A8 || MODE == kW8A16) {
      s0 = n < N ? a.sw[n] : 0.0f;
      s1 = n + 1 < N ? a.sw[n + 1] : 0.0f;
    }
    if constexpr (MODE == kW8A8) {
      const float xs = a.sx[m];
      v[0] = v[0] * xs;
      v[1] = v[1] * xs;
    }
    float y0 = v[0] * s0, y1 = v[1] * s1;
    if constexpr (LORA) {  // y = bf16(acc * scale + T B^T)
      y0 += lv[0];
      y1 += lv[1];
    }
    const uint32_t pk = pack_bf16x2(y0, y1);
    uint16_t* yr = a.y + (int64_t)m * a.ldy;
    if (n + 1 < N) {
      *reinterpret_cast<uint32_t*>(yr + n) = pk;
    } else if (n < N) {
      yr[n] = (uint16_t)(pk & 0xFFFFu);
    }
  }
  // W4A4 only: the nvfp4 encoding of Y for the next linear, from the same bf16 values
  if constexpr (MODE == kW4A4) {
    if (a.yq) {
      const float G = 1.0f / a.gy[0];
      for (int idx = tid; idx < 32 * MB * 2; idx += 64 * NW) {  // (row, 16-block) of the tile
        const int ml = idx >> 1, blk = idx & 1;
        const int m = m0 + ml, n = n0 + 16 * blk;
        if (m >= M) break;
        if (n >= N) continue;
        const int j = ml >> 5, lm = ml & 31;
        float f[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int nl = 16 * blk + e;
          const int r = 4 * (nl >> 3) + (nl & 3), ln = lm + 32 * ((nl >> 2) & 1);
          float sum = 0.0f;
#pragma unroll
          for (int w = 0; w < NW; ++w) sum += red[((w * MB + j) * 16 + r) * 64 + ln];
          float yv = sum * alpha;
          if constexpr (LORA) yv += lred[(j * 16 + r) * 64 + ln];
          f[e] = bf16_lo(pack_bf16x2(yv, 0.0f));  // the value the bf16 output holds
        }
        uint2 codes;
        const uint32_t sf = quant_block16_nvfp4(f, G, codes);
        *reinterpret_cast<uint2*>(a.yq + (int64_t)m * (N >> 1) + (n >> 1)) = codes;
        a.ys[(int64_t)m * (N >> 4) + (n >> 4)] = (uint8_t)sf;
      }
    }
  }
}

// ---- direct operand loads (nvfp4 schemes) --------------------------------------------
constexpr uint32_t kSkOut = kBufOut;  // buffer offset past every tile's records
// K offset of a wave's i-th stage. Every workgroup reads the same activation rows; starting
// the walk over K at a different stage per workgroup spreads those reads over the cache
// channels instead of having all workgroups hit the same lines at once. Stages past the
// wave's share return K (their loads read zeros).
__device__ __forceinline__ int stage_k(int wave, int nw, int i, int nk, int rot, int K) {
  const int v = wave + nw * i;
  if (v >= nk) return K;
  const int s = v + rot < nk ? v + rot : v + rot - nk;
  return s * kSkK;
}

// ---- register-staged variant (nvfp4 weights) -------------------------------------------
// A wave's share of one 128-deep stage is fetched with row-contiguous buffer loads (4 or 16
// lanes per row segment), so one 1 KB load touches 8 cache lines; it lands in registers, is
// written to the wave's LDS stage buffer in the MFMA operand layout, and read back as in the
// DMA variant. Three stages of loads are in flight per wave.
constexpr int kSkStagedWaves = 8;

// nvfp4 operand of a stage: 32 rows x 64 packed bytes (2 loads of 16 rows) + 32 rows x 8 scale
// bytes (lane l: dword l % 2 of row l / 2)
struct RawNv {
  uint4 c[2];
  uint32_t s;
};
// `rows` = rows of the tile inside the matrix: a load that would only cover rows past it is
// skipped (those rows only feed outputs that are never stored)
__device__ __forceinline__ void fetch_nv(RawNv& r, rsrc_t rq, rsrc_t rs, int lane, int kp, int ks, int kv, int K,
                                         bool dword_scales, int rows) {
#pragma unroll
  for (int ld = 0; ld < 2; ++ld) {
    const int row = 16 * ld + (lane >> 2), c = lane & 3;
    r.c[ld] = 16 * ld < rows ? bload16(rq, kv + 32 * c < K ? (uint32_t)(row * kp + (kv >> 1) + 16 * c) : kSkOut)
                             : make_uint4(0, 0, 0, 0);
  }
  const int row = lane >> 1, d = lane & 1;
  const bool ok = kv + 64 * d < K;
  const uint32_t off = (uint32_t)(row * ks + (kv >> 4) + 4 * d);
  if (dword_scales) {  // K % 64 == 0: the dword is 4-byte aligned
    r.s = __builtin_amdgcn_raw_buffer_load_b32(rs, ok ? (int)off : (int)kSkOut, 0, 0);
  } else {
    const uint32_t lo = bload2(rs, ok ? off : kSkOut), hi = bload2(rs, ok ? off + 2 : kSkOut);
    r.s = (lo & 0xFFFFu) | (hi << 16);
  }
}
__device__ __forceinline__ void stash_nv(const RawNv& r, uint8_t* codes, uint8_t* scales, int lane) {
#pragma unroll
  for (int ld = 0; ld < 2; ++ld) {
    const int row = 16 * ld + (lane >> 2), c = lane & 3;
    *reinterpret_cast<uint4*>(codes + swz_off<64>(row, c)) = r.c[ld];
  }
  *reinterpret_cast<uint32_t*>(scales + 4 * lane) = r.s;  // row lane / 2, dword lane % 2
}
// bf16 operand of a stage: 32 rows x 256 bytes (8 loads of 4 rows)
struct RawBf {
  uint4 c[8];
};
__device__ __forceinline__ void fetch_bf(RawBf& r, rsrc_t rx, int lane, int pitch, int kv, int K, int rows) {
#pragma unroll
  for (int ld = 0; ld < 8; ++ld) {
    const int row = 4 * ld + (lane >> 4), c = lane & 15;
    r.c[ld] = 4 * ld < rows ? bload16(rx, kv + 8 * c < K ? (uint32_t)(row * pitch + 2 * kv + 16 * c) : kSkOut)
                            : make_uint4(0, 0, 0, 0);
  }
}
__device__ __forceinline__ void stash_bf(const RawBf& r, uint8_t* codes, int lane) {
#pragma unroll
  for (int ld = 0; ld < 8; ++ld) {
    const int row = 4 * ld + (lane >> 4), c = lane & 15;
    *reinterpret_cast<uint4*>(codes + swz_off<256>(row, c)) = r.c[ld];
  }
}
// operand reads in the MFMA layout
__device__ __forceinline__ void read_nv(OpNv& o, const uint8_t* codes, const uint8_t* scales, int lr, int lh,
                                        int kv, int K) {
  o.q[0] = *reinterpret_cast<const uint4*>(codes + swz_off<64>(lr, 2 * lh));
  o.q[1] = *reinterpret_cast<const uint4*>(codes + swz_off<64>(lr, 2 * lh + 1));
  const uint32_t s = *reinterpret_cast<const uint32_t*>(scales + lr * 8 + 4 * lh);
  const int nvalid = (K - (kv + 64 * lh)) >> 4;  // blocks of this lane's window inside K
  o.s = nvalid >= 4 ? s : nvalid <= 0 ? 0u : s & ((1u << (8 * nvalid)) - 1u);
}
__device__ __forceinline__ void read_bf16(OpBf& o, const uint8_t* codes, int lr, int lh) {
#pragma unroll
  for (int c = 0; c < 8; ++c) o.d[c] = *reinterpret_cast<const uint4*>(codes + swz_off<256>(lr, 8 * lh + c));
}

// One workgroup's 32 weight rows and MB activation blocks: workgroup `bid` of the grid.
template <int MODE, int MB, bool LORA, int NWV>
__device__ __forceinline__ void skinny_staged_tile(const DecArgs& a, int bid) {
  static_assert(MODE == kW4A4 || MODE == kW4A16, "nvfp4 weights only");
  using S = Scheme<MODE>;
  constexpr int NW = NWV;
  constexpr bool XBF = MODE == kW4A16;
  using RawX = typename std::conditional<XBF, RawBf, RawNv>::type;
  constexpr int NV_BYTES = 32 * 64 + 256;                   // codes + scales of one nvfp4 operand
  constexpr int X_BYTES = XBF ? 32 * 256 : NV_BYTES;        // per activation block
  constexpr int STAGE = NV_BYTES + MB * X_BYTES;            // one buffer per wave
  constexpr int RED = NW * MB * 16 * 64 * 4 + (LORA ? MB * 16 * 64 * 4 : 0);  // partial tiles, adapter tiles
  constexpr int LDS = NW * STAGE > RED ? NW * STAGE : RED;
  static_assert(LDS <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS];

  const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
  const int nblk = (N + 31) / 32;
  const int n0 = (bid % nblk) * 32, m0 = (bid / nblk) * (32 * MB);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lh = lane >> 5;
  const int rows_w = N - n0 < 32 ? N - n0 : 32;
  const int kp = K >> 1, ks = K >> 4;
  const bool dword_scales = (K & 63) == 0;

  const rsrc_t wq = make_rsrc(a.w + (int64_t)n0 * kp, (uint32_t)(rows_w * kp));
  const rsrc_t ws = make_rsrc(a.ws + (int64_t)n0 * ks, (uint32_t)(rows_w * ks));
  const int xpitch = XBF ? (int)(a.ldx * 2) : kp;
  rsrc_t xq[MB], xs[MB];
  int xrows[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int mj = m0 + 32 * j;
    const int rows = M - mj <= 0 ? 0 : M - mj < 32 ? M - mj : 32;
    xrows[j] = rows;
    if constexpr (XBF) {
      xq[j] = make_rsrc(a.x + (int64_t)mj * a.ldx, rows ? (uint32_t)((rows - 1) * xpitch + 2 * K) : 0u);
      xs[j] = xq[j];
    } else {
      xq[j] = make_rsrc(a.xq + (int64_t)mj * kp, (uint32_t)(rows * kp));
      xs[j] = make_rsrc(a.xs + (int64_t)mj * ks, (uint32_t)(rows * ks));
    }
  }

  uint8_t* buf = smem + wave * STAGE;
  v16f acc[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) acc[j] = v16f{};

  const int nk = (K + kSkK - 1) / kSkK;
  const int mine = nk > wave ? (nk - wave + NW - 1) / NW : 0;  // uniform per wave
  const int rot = (int)((unsigned)bid % (unsigned)nk);
  RawNv w0, w1, w2;
  RawX x0[MB], x1[MB], x2[MB];
  auto fetch = [&](RawNv& w, RawX (&x)[MB], int i) {
    const int kv = stage_k(wave, NW, i, nk, rot, K);
    fetch_nv(w, wq, ws, lane, kp, ks, kv, K, dword_scales, rows_w);
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      if constexpr (XBF) fetch_bf(x[j], xq[j], lane, xpitch, kv, K, xrows[j]);
      else fetch_nv(x[j], xq[j], xs[j], lane, kp, ks, kv, K, dword_scales, xrows[j]);
    }
  };
  // stage i: registers -> LDS (after this wave's reads of stage i - 1, which precede in the
  // LDS queue), operands back in the MFMA layout, MFMAs
  auto consume = [&](const RawNv& w, const RawX (&x)[MB], int i) {
    const int kv = stage_k(wave, NW, i, nk, rot, K);
    stash_nv(w, buf, buf + 32 * 64, lane);
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      uint8_t* xb = buf + NV_BYTES + j * X_BYTES;
      if constexpr (XBF) stash_bf(x[j], xb, lane);
      else stash_nv(x[j], xb, xb + 32 * 64, lane);
    }
    typename S::WOp wo;
    typename S::XOp xo[MB];
    read_nv(wo, buf, buf + 32 * 64, lr, lh, kv, K);
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const uint8_t* xb = buf + NV_BYTES + j * X_BYTES;
      if constexpr (XBF) read_bf16(xo[j], xb, lr, lh);
      else read_nv(xo[j], xb, xb + 32 * 64, lr, lh, kv, K);
    }
    S::template mma<MB>(acc, wo, xo);
  };
  // Three stages in flight (a wave's whole share at K = 3072); nothing is fetched past the
  // wave's share (the address unit is the scarce resource here)
  if (mine > 0) fetch(w0, x0, 0);
  if (mine > 1) fetch(w1, x1, 1);
  if (mine > 2) fetch(w2, x2, 2);
  for (int i = 0; i < mine; i += 3) {
    consume(w0, x0, i);
    if (i + 3 < mine) fetch(w0, x0, i + 3);
    if (i + 1 < mine) {
      consume(w1, x1, i + 1);
      if (i + 4 < mine) fetch(w1, x1, i + 4);
    }
    if (i + 2 < mine) {
      consume(w2, x2, i + 2);
      if (i + 5 < mine) fetch(w2, x2, i + 5);
    }
  }
  __syncthreads();  // LDS is reused for the reduction

  float* red = reinterpret_cast<float*>(smem);  // [NW][MB][16][64], then the adapter tiles [MB][16][64]
  float* lred = red + NW * MB * 16 * 64;
#pragma unroll
  for (int j = 0; j < MB; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[((wave * MB + j) * 16 + r) * 64 + lane] = acc[j][r];
  if constexpr (LORA) skinny_lora_tile<MB>(a, lred, m0, n0, wave, lane);
  __syncthreads();
  skinny_epilogue<MODE, MB, NW, LORA>(a, red, lred, m0, n0, tid);
}

template <int MODE, int MB, bool LORA, int NWV = kSkStagedWaves>
__global__ __launch_bounds__(64 * NWV) void gemm_skinny_staged_kernel(DecArgs a) {
  skinny_staged_tile<MODE, MB, LORA, NWV>(a, blockIdx.x);
}

// ---- LDS-DMA variant (E4M3 weights): stage layout of one wave -----------------------
// A code region holds 32 rows of R bytes (R = 128 for E4M3, 256 for bf16 at a 128-deep
// stage), 16-byte chunks XOR-swizzled as in gemm_common.hpp.
template <int MODE>
using Layout = SkLayout<MODE>;

// a buffer resource as the scalar operand the DMA instruction takes (the values are
// wave-uniform; this keeps them in scalar registers when they come from an array)
__device__ __forceinline__ v4i sgpr(const v4i& r) {
  return v4i{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
             __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3])};
}

// DMA of one code region: load ld covers rows RPL * ld .. RPL * ld + RPL - 1; lane l writes
// physical chunk l % C of its row, so it fetches the logical chunk the swizzle puts there.
// `kv` is the first K value of the stage, `vpc` the K values per 16-byte chunk.
// Loads that would only cover rows past `rows` (the tile's rows inside the matrix) are
// skipped: those rows only feed outputs that are never stored.
template <int R>
__device__ __forceinline__ void dma_codes(const v4i& r, uint32_t lds, int lane, int pitch, int kbyte, int kv, int vpc,
                                          int K, int rows) {
  using G = CodeRegion<R>;
  const v4i rs = sgpr(r);
#pragma unroll
  for (int ld = 0; ld < G::LOADS; ++ld) {
    if (ld * G::RPL >= rows) break;  // uniform
    const DmaAddr d = code_load<R>(ld, lane, pitch, kbyte, kv, vpc, K);
    dma16(rs, lds + ld * 1024, d.voff, d.soff);
  }
}

// s_waitcnt that the compiler may not move memory accesses across
template <int n>
__device__ __forceinline__ void wait_vm_fence() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
  __asm__ volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_lds_fence() { __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// operand reads from a wave's stage buffer
__device__ __forceinline__ void read_f8(OpF8& o, const uint8_t* codes, int lr, int lh) {
#pragma unroll
  for (int c = 0; c < 4; ++c) o.d[c] = *reinterpret_cast<const uint4*>(codes + swz_off<128>(lr, 4 * lh + c));
}
__device__ __forceinline__ void read_bf(OpBf& o, const uint8_t* codes, int lr, int lh) {
#pragma unroll
  for (int c = 0; c < 8; ++c) o.d[c] = *reinterpret_cast<const uint4*>(codes + swz_off<256>(lr, 8 * lh + c));
}

// One workgroup's 32 weight rows and MB activation blocks: workgroup `bid` of the grid.
template <int MODE, int MB, int NW, bool LORA>
__device__ __forceinline__ void skinny_tile(const DecArgs& a, int bid) {
  using S = Scheme<MODE>;
  using L = Layout<MODE>;
  using SC = SkCfg<MODE, MB, NW, LORA>;
  constexpr int STAGE = SC::STAGE, WAVE = SC::WAVE;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SC::LDS];

  const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
  const int nblk = (N + 31) / 32;
  const int n0 = (bid % nblk) * 32, m0 = (bid / nblk) * (32 * MB);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lh = lane >> 5;
  const int rows_w = N - n0 < 32 ? N - n0 : 32;

  // buffer resources over this tile's rows: rows past the matrix read as zeros
  const v4i rwq = buffer_rsrc(a.w + (int64_t)n0 * K, (uint32_t)(rows_w * K));
  const int xpitch = L::XBF ? (int)(a.ldx * 2) : K;
  v4i rxq[MB];
  int xrows[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int mj = m0 + 32 * j;
    const int rows = M - mj <= 0 ? 0 : M - mj < 32 ? M - mj : 32;
    xrows[j] = rows;
    if constexpr (L::XBF)
      rxq[j] = buffer_rsrc(a.x + (int64_t)mj * a.ldx, rows ? (uint32_t)((rows - 1) * xpitch + 2 * K) : 0u);
    else
      rxq[j] = buffer_rsrc(a.xq + (int64_t)mj * K, (uint32_t)(rows * K));
  }

  const uint32_t wave_lds = lds_offset(smem) + (uint32_t)(wave * WAVE);
  const uint8_t* wave_mem = smem + wave * WAVE;
  const int nk = (K + kSkK - 1) / kSkK;
  const int rot = (int)((unsigned)bid % (unsigned)nk);
  // fetch this wave's i-th stage into ring buffer i % 2 (stages past K read as zeros)
  auto issue = [&](int i) {
    const int kv = stage_k(wave, NW, i, nk, rot, K);
    const uint32_t base = wave_lds + (uint32_t)((i & 1) * STAGE);
    // activation rows first, weight rows last: the weight loads of a stage are its last
    // L::W_LOADS memory operations (the wait below relies on it)
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const uint32_t xb = base + L::W_BYTES + j * L::X_BYTES;
      if constexpr (L::XBF) dma_codes<256>(rxq[j], xb, lane, xpitch, 2 * kv, kv, 8, K, xrows[j]);
      else dma_codes<128>(rxq[j], xb, lane, xpitch, kv, kv, 16, K, xrows[j]);
    }
    dma_codes<128>(rwq, base, lane, K, kv, kv, 16, K, 32);
  };

  v16f acc[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) acc[j] = v16f{};

  const int mine = nk > wave ? (nk - wave + NW - 1) / NW : 0;  // uniform per wave
  // Nothing is fetched past the wave's share. A stage issues a variable number of activation
  // loads (rows past M are skipped) followed by exactly L::W_LOADS weight loads, and loads
  // complete in order: once at most L::W_LOADS are outstanding, stage i has landed.
  if (mine > 0) issue(0);
  if (mine > 1) issue(1);
  for (int i = 0; i < mine; ++i) {
    if (i + 1 < mine) wait_vm_fence<L::W_LOADS>();  // stage i has landed
    else wait_vm_fence<0>();
    const uint8_t* st = wave_mem + (i & 1) * STAGE;
    typename S::WOp w;
    typename S::XOp x[MB];
    read_f8(w, st, lr, lh);
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const uint8_t* xb = st + L::W_BYTES + j * L::X_BYTES;
      if constexpr (L::XBF) read_bf(x[j], xb, lr, lh);
      else read_f8(x[j], xb, lr, lh);
    }
    wait_lds_fence();  // the buffer is free again
    if (i + 2 < mine) issue(i + 2);
    S::template mma<MB>(acc, w, x);
  }
  wait_vm_fence<0>();
  __syncthreads();  // every ring is idle: the LDS is reused for the reduction

  // sum the NW partial tiles in wave order
  float* red = reinterpret_cast<float*>(smem);  // [NW][MB][16][64], then the adapter tiles [MB][16][64]
  float* lred = red + NW * MB * 16 * 64;
#pragma unroll
  for (int j = 0; j < MB; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[((wave * MB + j) * 16 + r) * 64 + lane] = acc[j][r];
  if constexpr (LORA) skinny_lora_tile<MB>(a, lred, m0, n0, wave, lane);
  __syncthreads();

  skinny_epilogue<MODE, MB, NW, LORA>(a, red, lred, m0, n0, tid);
}

template <int MODE, int MB, int NW, bool LORA>
__global__ __launch_bounds__(64 * NW) void gemm_skinny_kernel(DecArgs a) {
  skinny_tile<MODE, MB, NW, LORA>(a, blockIdx.x);
}

// The workgroups of several few-token GEMMs of one scheme in one grid: each workgroup finds its
// problem and computes what that problem's own launch computes in its workgroup (same bits).
struct SkGroup {
  DecArgs p[kMaxGroup];
  int start[kMaxGroup + 1];
  int count;
};
template <int MODE, int MB, int NW>
__global__ __launch_bounds__(64 * NW) void gemm_skinny_staged_grouped_kernel(SkGroup g) {
  const int bid = blockIdx.x;
  const int p = group_problem(g.start, g.count, bid);
  skinny_staged_tile<MODE, MB, false, NW>(g.p[p], bid - g.start[p]);
}
template <int MODE, int MB, int NW>
__global__ __launch_bounds__(64 * NW) void gemm_skinny_grouped_kernel(SkGroup g) {
  const int bid = blockIdx.x;
  const int p = group_problem(g.start, g.count, bid);
  skinny_tile<MODE, MB, NW, false>(g.p[p], bid - g.start[p]);
}

template <int MODE, int MB, int NW>
hipError_t run(const DecArgs& a, hipStream_t s) {
  const int64_t blocks = ((a.N + 31) / 32) * ((a.M + 32 * MB - 1) / (32 * MB));
  if (a.lt)
    hipLaunchKernelGGL((gemm_skinny_kernel<MODE, MB, NW, true>), dim3((unsigned)blocks), dim3(64 * NW), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<MODE, MB, NW, false>), dim3((unsigned)blocks), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}
template <int MODE, int MB, int NW = kSkStagedWaves>
hipError_t run_staged(const DecArgs& a, hipStream_t s) {
  const int64_t blocks = ((a.N + 31) / 32) * ((a.M + 32 * MB - 1) / (32 * MB));
  if (a.lt)
    hipLaunchKernelGGL((gemm_skinny_staged_kernel<MODE, MB, true, NW>), dim3((unsigned)blocks), dim3(64 * NW), 0, s,
                       a);
  else
    hipLaunchKernelGGL((gemm_skinny_staged_kernel<MODE, MB, false, NW>), dim3((unsigned)blocks), dim3(64 * NW), 0, s,
                       a);
  return hipGetLastError();
}

template <int MODE>
hipError_t pick(const DecArgs& a, hipStream_t s) {
  // One 32-token activation block per workgroup while two per workgroup would leave the grid
  // short of the 256 compute units (measured with cold weights, K = 3072, N = 3072: W4A4 48 and
  // 64 tokens 15.9 / 16.7 -> 9.4 / 11.1 us, W8A8 48 / 64 / 96 / 128 tokens 9.1 / 9.8 / 9.2 / 9.9
  // -> 7.1 / 7.6 / 8.8 / 9.3 us); past 64 tokens W4A4 does better with two blocks (96 tokens
  // 13.1 vs 14.2 us), which halve its weight decodes per output.
  const bool short_grid = ((a.N + 31) / 32) * ((a.M + 63) / 64) < 256;
  if constexpr (MODE == kW4A4) {
    // With a full grid (>= 256 workgroups) and 16 or more tokens, four waves per workgroup
    // (twice the stages each, more workgroups per compute unit) beat eight: cold weights,
    // K = 3072, N = 12288: 16 / 32 / 64 tokens 12.7 / 15.8 / 20.5 -> 12.3 / 14.5 / 19.3 us; at
    // N = 3072 (96 workgroups) and for a single token eight stay ahead (8.0 vs 8.5, 10.7 vs 11.3).
    if (a.M <= 64) {
      if (a.M >= 16 && (a.N + 31) / 32 >= 256) return run_staged<MODE, 1, 4>(a, s);
      return run_staged<MODE, 1>(a, s);
    }
    return run_staged<MODE, 2>(a, s);
  } else if constexpr (MODE == kW4A16) {
    // bf16 activations fill registers and LDS fastest: one activation block per workgroup; on a
    // full grid four waves (N = 12288: 1 / 16 / 32 tokens 14.4 / 17.4 / 21.1 -> 13.0 / 14.8 /
    // 17.4 us; at N = 3072 eight stay ahead, 9.2 vs 10.4 at 16 tokens)
    if ((a.N + 31) / 32 >= 256) return run_staged<MODE, 1, 4>(a, s);
    return run_staged<MODE, 1>(a, s);
  } else if constexpr (MODE == kW8A16) {
    // two waves per workgroup once the grid fills the compute units (cold weights, K = 3072,
    // N = 12288, 1 / 16 tokens: 12.7 / 14.2 -> 11.8 / 13.4 us; at N = 3072 four stay ahead)
    if (a.M <= 16 && (a.N + 31) / 32 >= 256) return run<MODE, 1, 2>(a, s);
    return run<MODE, 1, 4>(a, s);
  } else {
    // eight waves for a handful of tokens on a small grid (1 x 3072 x 3072: 6.1 -> 5.5 us)
    if (a.M <= 8 && short_grid) return run<MODE, 1, 8>(a, s);
    if (a.M <= 32 || short_grid) return run<MODE, 1, 4>(a, s);
    return run<MODE, 2, 4>(a, s);
  }
}

}  // namespace

bool gemm_skinny_supported(DecMode mode, const DecArgs& a) {
  // 32-bit buffer offsets: every operand tile (up to 64 rows) stays below the out-of-range offset
  const int64_t xpitch = (mode == kW4A16 || mode == kW8A16) ? 2 * a.ldx : a.K;
  return 64 * a.K < kOutOfRange && 64 * xpitch < (int64_t)kOutOfRange;
}

hipError_t launch_gemm_skinny(DecMode mode, const DecArgs& a, hipStream_t s) {
  switch (mode) {
    case kW4A4: return pick<kW4A4>(a, s);
    case kW4A16: return pick<kW4A16>(a, s);
    case kW8A8: return pick<kW8A8>(a, s);
    default: return pick<kW8A16>(a, s);
  }
}

// Grouped few-token launch (any scheme; no adapter): one grid over every problem's workgroups,
// the variant (activation blocks and waves per workgroup) picked for the whole group from the
// largest token count and the group's total grid. A group's grid holds several problems' worth
// of workgroups, which favours more waves per workgroup than one launch of the same token count
// would take: a joint block's four linears (qkv, proj, up, down; cold weights) at 16 tokens
// took 34.5 us as one grid of four-wave W4A4 workgroups and 27.0 us with eight waves; W8A8 took
// 27.9 us with four waves and 30.0 us with eight, but 25.8 -> 24.8 us with eight at one token.
bool gemm_skinny_grouped_supported(DecMode mode, const DecArgs* p, int count) {
  if (count < 2 || count > kMaxGroup) return false;
  int64_t blocks = 0;  // at one activation block a workgroup, the most the grid can hold
  for (int i = 0; i < count; ++i) {
    if (p[i].lt || p[i].yq || p[i].ypmax || !p[i].y || !gemm_skinny_supported(mode, p[i])) return false;
    blocks += ((p[i].N + 31) / 32) * ((p[i].M + 31) / 32);
  }
  return blocks < ((int64_t)1 << 31);  // the grid's workgroup ids are 32-bit
}

namespace {
template <int MODE, int MB, int NW, bool STAGED>
hipError_t run_grouped(const DecArgs* p, int count, hipStream_t s) {
  SkGroup g{};
  g.count = count;
  int64_t total = 0;
  for (int i = 0; i < count; ++i) {
    g.p[i] = p[i];
    g.start[i] = (int)total;
    total += ((p[i].N + 31) / 32) * ((p[i].M + 32 * MB - 1) / (32 * MB));
  }
  for (int i = count; i <= kMaxGroup; ++i) g.start[i] = (int)total;
  if constexpr (STAGED)
    hipLaunchKernelGGL((gemm_skinny_staged_grouped_kernel<MODE, MB, NW>), dim3((unsigned)total), dim3(64 * NW), 0, s,
                       g);
  else
    hipLaunchKernelGGL((gemm_skinny_grouped_kernel<MODE, MB, NW>), dim3((unsigned)total), dim3(64 * NW), 0, s, g);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_skinny_grouped(DecMode mode, const DecArgs* p, int count, hipStream_t s) {
  int64_t mmax = 0, grid64 = 0;
  for (int i = 0; i < count; ++i) {
    mmax = p[i].M > mmax ? p[i].M : mmax;
    grid64 += ((p[i].N + 31) / 32) * ((p[i].M + 63) / 64);
  }
  // weight-only linears: one activation block a workgroup, eight waves (W4A16) or four (W8A16),
  // the shapes one launch of a short grid takes
  if (mode == kW4A16) return run_grouped<kW4A16, 1, kSkStagedWaves, true>(p, count, s);
  if (mode == kW8A16) return run_grouped<kW8A16, 1, 4, false>(p, count, s);
  if (mode == kW4A4) {
    if (mmax > 64) return run_grouped<kW4A4, 2, kSkStagedWaves, true>(p, count, s);
    return run_grouped<kW4A4, 1, kSkStagedWaves, true>(p, count, s);
  }
  const bool short_grid = grid64 < 256;
  if (mmax <= 8) return run_grouped<kW8A8, 1, 8, false>(p, count, s);
  if (mmax <= 32 || short_grid) return run_grouped<kW8A8, 1, 4, false>(p, count, s);
  return run_grouped<kW8A8, 2, 4, false>(p, count, s);
}

}  // namespace bsq
