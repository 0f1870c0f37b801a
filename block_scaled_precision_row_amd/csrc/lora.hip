// Low-rank adapter (LoRA) down projection on the matrix cores: T = bf16(s * X A^T).
//
// "FLUX 3 Image Klein vs Qwen-Image-2.1" (model overview) and the FLUX 3 Image
// Klein open-source release page (section three, speed figures): the quantized
// model can run with a LoRA attached. The adapter adds s * B (A x) to the
// linear's output; its rank-r intermediate T = s * X A^T [M][r] is computed
// here from the unquantized bf16 activations and held in bf16 (the adapter
// scale applied before that rounding), and the GEMMs add T B^T. For a GEMM
// whose output scale is one number alpha (the nvfp4 W4A4 kernel: gx * gw),
// T may be produced as T / alpha, so that the GEMM can accumulate T B^T into
// its accumulators before the main loop and let its own epilogue scale it.
//
// This is a tall, thin GEMM (r <= 128 columns): X streams from HBM once and
// the adapter matrix A (r x K) must reach every compute unit that works on
// some rows. A workgroup takes 128 rows of X and one slice of K; its 8 waves
// own 16 rows each and share the adapter slice, which the workgroup stages in
// LDS 256 K values at a time, so A is read once per 128 rows instead of once
// per wave. Every load of a 256-deep step (the adapter chunks and the wave's
// 16 rows x 256 values of X, 128 bytes per lane) is issued at once, so a step
// costs one memory latency. Slicing K gives enough workgroups to fill the chip
// at a few thousand tokens with one or a few steps each; the slices' fp32
// partial tiles go to a workspace and a second kernel adds them in slice order
// (deterministic), scales and rounds. With one slice the first kernel writes
// T itself.
//
// MFMA v_mfma_f32_16x16x32_bf16: the A operand is 16 adapter rows (RT tiles of
// 16 cover the rank), the B operand the wave's 16 X rows, so a lane accumulates
// token m = lane % 16 and adapter rows j = 16 r + 4 (lane / 16) + e in register
// e of tile r. Within a 64-deep chunk at kc, lane group g = lane / 16 holds K
// values [kc + 16 g, kc + 16 g + 16) of both operands (two MFMA steps of 8):
// four lanes read one full 128-byte line of each X row.
#include "bsq_device.hpp"
#include "bsq_launch.hpp"

namespace bsq {

namespace {

constexpr int kDownWaves = 8;
constexpr int kDownRows = 16 * kDownWaves;  // rows of X per workgroup
constexpr int kStep = 256;                  // K values per step (adapter stage in LDS, X in registers)
constexpr int kAPitch = kStep * 2 + 16;     // bytes per adapter row in LDS (padded against bank conflicts)
constexpr int kMaxSlices = 16;

__device__ __forceinline__ v8bf as_v8bf(uint4 u) {
  union {
    uint4 u;
    v8bf h;
  } c;
  c.u = u;
  return c.h;
}

__device__ __forceinline__ float out_factor(float scale, const float* ga, const float* gb) {
  return ga ? scale / (ga[0] * gb[0]) : scale;
}

// adapter step at kb: chunk c (thread tid + 512 i) is adapter row c / 32, values kb + 8 (c % 32) .. + 7
template <int APT, int ACH>
__device__ __forceinline__ void load_adapter(uint4 (&areg)[APT], rsrc_t ra, int tid, int kb, int k1, int K) {
#pragma unroll
  for (int i = 0; i < APT; ++i) {
    const int c = tid + 64 * kDownWaves * i;
    const int row = c >> 5, k = kb + 8 * (c & 31);
    const bool ok = c < ACH && k < k1;
    areg[i] = bload16(ra, ok ? (uint32_t)(row * K + k) * 2u : kBufOut);
  }
}
// this lane's X values of the step at kb: 16 values at kb + 64 c + 16 g for c = 0 .. 3
__device__ __forceinline__ void load_rows(uint4 (&r)[8], rsrc_t rx, uint32_t xrow, int lg, int kb, int k1) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int k = kb + 64 * c + 16 * lg;  // K % 32 == 0: all 16 values inside the slice or none
    const bool ok = k < k1;
#pragma unroll
    for (int q = 0; q < 2; ++q) r[2 * c + q] = bload16(rx, ok ? xrow + (uint32_t)k * 2u + 16u * q : kBufOut);
  }
}

// Grid (K slices, row blocks): the slices of a row block are neighbours in launch order, so
// the workgroups running together read whole rows of X rather than one segment of every row.
// Slice z covers K values [z * kr, min(K, (z + 1) * kr)), kr a multiple of kStep. With one slice: t = bf16(f * acc); otherwise the fp32 partial tile goes to
// part [slices][M][rank].
// With QUANT the kernel also writes X's nvfp4 encoding with global scale *gq (what the
// activation quantizer writes): a lane's 16 values of a 64-deep chunk are one 16-element block,
// so every block is encoded once, from the registers the projection uses.
template <int RT, bool QUANT>
__global__ __launch_bounds__(64 * kDownWaves) void lora_down_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                                     const uint16_t* __restrict__ a, int M, int K,
                                                                     int rank, int kr, float scale, const float* ga,
                                                                     const float* gb, float* __restrict__ part,
                                                                     uint16_t* __restrict__ t, const float* gq,
                                                                     uint8_t* __restrict__ xq,
                                                                     uint8_t* __restrict__ xs) {
  constexpr int AROWS = 16 * RT;
  constexpr int ACH = AROWS * (kStep / 8);                              // 16-byte chunks per adapter step
  constexpr int APT = (ACH + 64 * kDownWaves - 1) / (64 * kDownWaves);  // chunks per thread
  constexpr int TP = 16 * RT + 4;  // floats per row of the output tile in LDS (padded)
  constexpr int SA = AROWS * kAPitch > kDownRows * TP * 4 ? AROWS * kAPitch : kDownRows * TP * 4;
  __shared__ __attribute__((aligned(16))) uint8_t sa[SA];

  const int m0 = blockIdx.y * kDownRows;
  const int k0 = blockIdx.x * kr;
  const int k1 = K - k0 < kr ? K : k0 + kr;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int rows = M - m0 < kDownRows ? M - m0 : kDownRows;

  // this wave's rows of X (rows past M read as zeros) and the adapter (rows past the rank too)
  // (readfirstlane: the compiler computes the clamp on the vector unit, and a buffer resource
  // it cannot prove uniform turns every load into a loop over lanes)
  const int wrow0 = 16 * wave;
  const int wrows = __builtin_amdgcn_readfirstlane(rows - wrow0 < 0 ? 0 : (rows - wrow0 < 16 ? rows - wrow0 : 16));
  const rsrc_t rx = make_rsrc(x + (int64_t)(m0 + (wrows ? wrow0 : 0)) * ldx, (uint32_t)wrows * (uint32_t)ldx * 2u);
  const rsrc_t ra = make_rsrc(a, (uint32_t)rank * (uint32_t)K * 2u);
  const uint32_t xrow = (uint32_t)lr * (uint32_t)ldx * 2u;

  v4f acc[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) acc[r] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  for (int kb = k0; kb < k1; kb += kStep) {
    uint4 areg[APT], xr[8];
    load_adapter<APT, ACH>(areg, ra, tid, kb, k1, K);  // adapter first: its wait leaves X in flight
    load_rows(xr, rx, xrow, lg, kb, k1);
    __builtin_amdgcn_sched_barrier(0);  // keep every load of the step ahead of its first use
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const int c = tid + 64 * kDownWaves * i;
      if (c < ACH) *reinterpret_cast<uint4*>(&sa[(c >> 5) * kAPitch + 16 * (c & 31)]) = areg[i];
    }
    __syncthreads();
    if constexpr (QUANT) {
      const float G = 1.0f / gq[0];
      const int64_t row = m0 + wrow0 + lr;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int k = kb + 64 * c + 16 * lg;
        if (lr < wrows && k < k1) {
          float fv[16];
          bf16x16_to_f32(xr[2 * c], xr[2 * c + 1], fv);
          uint2 codes;
          const uint32_t sf = quant_block16_nvfp4(fv, G, codes);
          *reinterpret_cast<uint2*>(xq + row * (K >> 1) + (k >> 1)) = codes;
          xs[row * (K >> 4) + (k >> 4)] = (uint8_t)sf;
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const uint4 av =
              *reinterpret_cast<const uint4*>(sa + (16 * r + lr) * kAPitch + 2 * (64 * c + 16 * lg) + 16 * q);
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(av), as_v8bf(xr[2 * c + q]), acc[r], 0, 0, 0);
        }
    __syncthreads();  // the adapter stage is rewritten by the next step
  }

  // The block's result is one contiguous run of rows * rank values (T or this slice's partials):
  // stage the tile [128][16 RT] fp32 in LDS (lane: row 16 wave + m, adapter rows 16 r + 4 g + e)
  // and write the run with consecutive threads on consecutive values.
  float* tile = reinterpret_cast<float*>(sa);
#pragma unroll
  for (int r = 0; r < RT; ++r)
    *reinterpret_cast<float4*>(&tile[(wrow0 + lr) * TP + 16 * r + 4 * lg]) =
        make_float4(acc[r][0], acc[r][1], acc[r][2], acc[r][3]);
  __syncthreads();
  const int n = rows * rank;
  if (gridDim.x == 1) {
    const float f = out_factor(scale, ga, gb);
    uint16_t* dst = t + (int64_t)m0 * rank;  // 16-byte aligned: m0 * rank * 2 is a multiple of 256
    for (int i = 8 * tid; i < n; i += 8 * 64 * kDownWaves) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i0 = i + 2 * e, i1 = i0 + 1;
        const float v0 = i0 < n ? tile[(i0 / rank) * TP + i0 % rank] : 0.0f;
        const float v1 = i1 < n ? tile[(i1 / rank) * TP + i1 % rank] : 0.0f;
        w[e] = pack_bf16x2(f * v0, f * v1);
      }
      if (i + 8 <= n) {
        *reinterpret_cast<uint4*>(dst + i) = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (i + e < n) dst[i + e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
      }
    }
  } else {
    float* dst = part + ((int64_t)blockIdx.x * M + m0) * rank;
    const bool vec = ((reinterpret_cast<uintptr_t>(dst) & 15) == 0);
    for (int i = 4 * tid; i < n; i += 4 * 64 * kDownWaves) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = i + e < n ? tile[((i + e) / rank) * TP + (i + e) % rank] : 0.0f;
      if (vec && i + 4 <= n) {
        *reinterpret_cast<float4*>(dst + i) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (i + e < n) dst[i + e] = v[e];
      }
    }
  }
}

// t[i] = bf16(f * sum over slices z in order of part[z][i]), i over M * rank; four consecutive
// values per thread, all slices' loads issued before the sums
template <int Z>
__global__ __launch_bounds__(256) void lora_down_finish_kernel(const float* __restrict__ part, int64_t n, int slices,
                                                               float scale, const float* ga, const float* gb,
                                                               uint16_t* __restrict__ t) {
  const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i0 >= n) return;
  const float f = out_factor(scale, ga, gb);
  if (i0 + 4 <= n && (n & 3) == 0) {
    float4 v[Z];
#pragma unroll
    for (int z = 0; z < Z; ++z)
      v[z] = z < slices ? *reinterpret_cast<const float4*>(part + z * n + i0) : make_float4(0.f, 0.f, 0.f, 0.f);
    float4 s = v[0];
#pragma unroll
    for (int z = 1; z < Z; ++z)
      if (z < slices) {
        s.x += v[z].x;
        s.y += v[z].y;
        s.z += v[z].z;
        s.w += v[z].w;
      }
    *reinterpret_cast<uint2*>(t + i0) = make_uint2(pack_bf16x2(f * s.x, f * s.y), pack_bf16x2(f * s.z, f * s.w));
  } else {
    for (int64_t i = i0; i < n && i < i0 + 4; ++i) {
      float s = 0.0f;
      for (int z = 0; z < slices; ++z) s += part[z * n + i];
      t[i] = (uint16_t)(pack_bf16x2(f * s, 0.0f) & 0xFFFFu);
    }
  }
}

// ---- whole rows: the down projection, optionally fused with X's encoding -----------------
// The fp8r encoding of a row needs the row's maximum before any value is encoded, so it
// cannot ride on the K-sliced kernel above. Here a workgroup owns 16 whole rows: each of its
// (at most 8) waves holds 64 NC consecutive K values of all 16 rows in registers (NC = 6
// 64-deep chunks for K <= 3072, 12 for K <= 6144; lane (lr, lg) holds the 16 values
// kc + 16 lg .. + 15 of row lr of chunk kc, the layout of the kernel above), so X is read from
// HBM once (with twelve chunks fewer adapter pieces are requested ahead, which keeps the
// kernel within 256 registers a lane). With ENC the row maxima combine across the four
// lanes of a row and then across the waves through LDS, and each wave encodes its values
// with the quantizer's own steps (d = fp32(amax / 448), r = fp32(1 / d), E4M3(fp32(x r))).
// The nvfp4 encoding needs no row maximum: a lane's 16 values of a chunk are one block,
// encoded by the quantizer's block function (without the K slices' finishing pass this kernel
// beats the sliced one at most shapes). Every wave multiplies the same registers into T on
// the matrix cores, with the adapter read from L2 (A is the MFMA A operand, X the B operand).
// The waves' fp32 tiles (all rank tiles, behind one barrier) are added in wave order through
// LDS, scaled and rounded to bf16. For an fp8r linear one launch replaces the quantizer, the
// sliced down projection and its finishing pass.
// Measured at 4096 x 3072 (us, no profiler): the quantizer alone 6.5; this kernel 9.1 / 10.6 /
// 13.1 / 18.5 at rank 16 / 32 / 64 / 128 (with one reduction barrier per rank tile and the
// adapter after the encoding it was 9.1 / 11.5 / 14.7 / 21.2); at 4096 x 6144 13.5 for the
// quantizer, 17.1 / 19.6 / 24.0 / 33.3 here. The phases mostly add up because each compute
// unit holds one workgroup (256 of them at 4096 rows): X's loads, the encoded stores and the
// adapter's loads and MFMAs.
constexpr int kFusedWaves = 8;      // at most; 256 registers a lane
constexpr int kFusedMaxChunks = 12;  // 64-deep chunks a wave (6 up to K = 3072)
constexpr int kRingSlots = 4;    // adapter pieces (16 rows x 64 values) staged at a time per wave

template <int RT, DownEnc ENC, int NC>
__global__ __launch_bounds__(64 * kFusedWaves) void lora_down_rows_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                                   const uint16_t* __restrict__ a, int M, int K,
                                                                   int rank, float scale, const float* ga,
                                                                   const float* gb, uint16_t* __restrict__ t,
                                                                   uint8_t* __restrict__ xq, float* __restrict__ sx,
                                                                   uint8_t* __restrict__ xs, const float* gq) {
  constexpr int WMAX = kFusedWaves, KW = 64 * NC;
  __shared__ float red[WMAX][16];
  __shared__ __attribute__((aligned(16))) float part[WMAX][RT][16 * 16];
  __shared__ __attribute__((aligned(16))) uint8_t aring[WMAX][kRingSlots][2048];
  const int waves = __builtin_amdgcn_readfirstlane(blockDim.x >> 6);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int m0 = blockIdx.x * 16;
  const int rows = __builtin_amdgcn_readfirstlane(M - m0 < 16 ? M - m0 : 16);
  const int kw0 = wave * KW;
  // rows past M and values past K read as zeros: they raise no maximum and add nothing to T
  const rsrc_t rx = make_rsrc(x + (int64_t)m0 * ldx, (uint32_t)rows * (uint32_t)ldx * 2u);
  const rsrc_t ra = make_rsrc(a, (uint32_t)rank * (uint32_t)K * 2u);
  const uint32_t xrow = (uint32_t)lr * (uint32_t)ldx * 2u;

  // The adapter: piece i = RT c + r is rank tile r's 16 rows x 64 values of chunk c. Read with
  // eight lanes per 128-byte row segment (whole lines per load; in the MFMA layout the lanes
  // of a quarter wave would each address a different row) and staged through a ring of
  // kRingSlots pieces in this wave's LDS, XOR-swizzled by row, from which each lane reads its
  // MFMA operands. The first PRE pieces are requested with X, so that they arrive while X does
  // (and, after the encoding, while the row maxima are combined and X is encoded).
  constexpr int NP = NC * RT, PRE = NC == 6 ? (NP <= 12 ? NP : 8) : (ENC == kDownFp8r ? 2 : 4);
  const int gr = lane >> 3, gp = lane & 7;  // this lane's row (and row + 8) and piece of a load
  uint4 xr[NC][2], aw[NP][2];
  auto load_a = [&](int i) {
    const int c = i / RT, r = i % RT;
    const int k = kw0 + 64 * c + 8 * gp;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      aw[i][h] = bload16(ra, k < K ? (uint32_t)((16 * r + 8 * h + gr) * K + k) * 2u : kBufOut);
  };
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int k = kw0 + 64 * c + 16 * lg;  // K % 32 == 0: all 16 values inside K or none
#pragma unroll
    for (int q = 0; q < 2; ++q) xr[c][q] = bload16(rx, k < K ? xrow + (uint32_t)k * 2u + 16u * q : kBufOut);
  }
#pragma unroll
  for (int i = 0; i < PRE; ++i) load_a(i);
  // The adapter's MFMAs need X but not the row maxima. In the six-chunk fp8r kernel they run
  // before the maxima are combined (what a wave computes while others' X is still arriving
  // shortens the wait at the barrier; 4096 x 3072, rank 32: 11.5 -> 10.6 us, same bits); with
  // twelve chunks (register-bound) and in the other modes they run after the encoding.
  constexpr bool kAdapterFirst = ENC == kDownFp8r && NC == 6;
  v4f acc[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) acc[r] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  auto adapter = [&]() {
    uint8_t* ring = aring[wave][0];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int c = i / RT, r = i % RT;
      if (i + PRE < NP) load_a(i + PRE);  // PRE pieces in flight
      uint8_t* slot = ring + (i % kRingSlots) * 2048;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 8 * h + gr;
        *reinterpret_cast<uint4*>(slot + row * 128 + ((gp ^ (row & 7)) << 4)) = aw[i][h];
      }
      // lane (lr, lg): row lr, values 16 lg + 8 q of the chunk, as in xr[c][q]
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4 av = *reinterpret_cast<const uint4*>(slot + lr * 128 + (((2 * lg + q) ^ (lr & 7)) << 4));
        acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(av), as_v8bf(xr[c][q]), acc[r], 0, 0, 0);
      }
      if constexpr (NP > PRE) __builtin_amdgcn_sched_barrier(0);  // no loads hoisted past the window
    }
  };
  if constexpr (kAdapterFirst) adapter();

  if constexpr (ENC == kDownFp8r) {
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) amax = fmaxf(amax, fmaxf(absmax8(xr[c][0]), absmax8(xr[c][1])));
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    if (lg == 0) red[wave][lr] = amax;
    __syncthreads();  // every wave's row maxima are in red

    for (int w = 0; w < waves; ++w) amax = fmaxf(amax, red[w][lr]);
    if (lr < rows) {
      const float d = amax / kE4M3Max;
      const float rc = d > 0.0f ? 1.0f / d : 0.0f;
      uint8_t* qrow = xq + (int64_t)(m0 + lr) * K;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int k = kw0 + 64 * c + 16 * lg;
        if (k < K) {
          const uint2 lo = encode8_fp8(xr[c][0], rc), hi = encode8_fp8(xr[c][1], rc);
          *reinterpret_cast<uint4*>(qrow + k) = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
      }
      if (wave == 0 && lg == 0) sx[m0 + lr] = d;
    }
  }
  if constexpr (ENC == kDownNvfp4) {
    // a lane's 16 values of a chunk are one 16-element block: encoded as the quantizer does
    if (lr < rows) {
      const float G = 1.0f / gq[0];
      const int64_t row = m0 + lr;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int k = kw0 + 64 * c + 16 * lg;
        if (k < K) {
          float fv[16];
          bf16x16_to_f32(xr[c][0], xr[c][1], fv);
          uint2 codes;
          const uint32_t sf = quant_block16_nvfp4(fv, G, codes);
          *reinterpret_cast<uint2*>(xq + row * (K >> 1) + (k >> 1)) = codes;
          xs[row * (K >> 4) + (k >> 4)] = (uint8_t)sf;
        }
      }
    }
  }

  if constexpr (!kAdapterFirst) adapter();

  // T: lane (lr, lg) holds token lr, adapter rows 16 r + 4 lg + e; every wave stages its tiles
  // in part[wave][r][token][16] and one barrier later the waves are added in wave order
  const float f = out_factor(scale, ga, gb);
#pragma unroll
  for (int r = 0; r < RT; ++r)
    *reinterpret_cast<float4*>(&part[wave][r][lr * 16 + 4 * lg]) = make_float4(acc[r][0], acc[r][1], acc[r][2], acc[r][3]);
  __syncthreads();
  for (int i = tid; i < 256 * RT; i += 64 * waves) {  // i = 256 r + 16 token + adapter row within tile r
    const int r = i >> 8, n = (i >> 4) & 15, j = i & 15;
    float s = part[0][r][i & 255];
    for (int w = 1; w < waves; ++w) s += part[w][r][i & 255];
    if (n < rows && 16 * r + j < rank)
      t[(int64_t)(m0 + n) * rank + 16 * r + j] = (uint16_t)(pack_bf16x2(f * s, 0.0f) & 0xFFFFu);
  }
}

template <int RT, int NC>
hipError_t run_down_rows_nc(const uint16_t* x, int64_t ldx, const uint16_t* a, int64_t M, int64_t K, int rank,
                            float scale, const float* ga, const float* gb, uint16_t* t, const RowsEncode& en,
                            hipStream_t s) {
  const int waves = (int)((K + 64 * NC - 1) / (64 * NC));
  const dim3 grid((unsigned)((M + 15) / 16)), block((unsigned)(64 * waves));
  if (en.enc == kDownFp8r)
    hipLaunchKernelGGL((lora_down_rows_kernel<RT, kDownFp8r, NC>), grid, block, 0, s, x, ldx, a, (int)M, (int)K, rank,
                       scale, ga, gb, t, en.xq, en.sx, en.xs, en.gq);
  else if (en.enc == kDownNvfp4)
    hipLaunchKernelGGL((lora_down_rows_kernel<RT, kDownNvfp4, NC>), grid, block, 0, s, x, ldx, a, (int)M, (int)K, rank,
                       scale, ga, gb, t, en.xq, en.sx, en.xs, en.gq);
  else
    hipLaunchKernelGGL((lora_down_rows_kernel<RT, kDownPlain, NC>), grid, block, 0, s, x, ldx, a, (int)M, (int)K, rank,
                       scale, ga, gb, t, en.xq, en.sx, en.xs, en.gq);
  return hipGetLastError();
}
template <int RT>
hipError_t run_down_rows(const uint16_t* x, int64_t ldx, const uint16_t* a, int64_t M, int64_t K, int rank,
                         float scale, const float* ga, const float* gb, uint16_t* t, const RowsEncode& en,
                         hipStream_t s) {
  if (K <= 64 * 6 * kFusedWaves) return run_down_rows_nc<RT, 6>(x, ldx, a, M, K, rank, scale, ga, gb, t, en, s);
  return run_down_rows_nc<RT, 12>(x, ldx, a, M, K, rank, scale, ga, gb, t, en, s);
}

template <int RT>
hipError_t run_down(const uint16_t* x, int64_t ldx, const uint16_t* a, int64_t M, int64_t K, int rank, float scale,
                    const float* ga, const float* gb, float* part, uint16_t* t, const float* gq, uint8_t* xq,
                    uint8_t* xs, hipStream_t s) {
  const int slices = lora_down_slices(M, K, rank);
  const int64_t kr = lora_down_slice_k(K, slices);
  const dim3 grid((unsigned)slices, (unsigned)((M + kDownRows - 1) / kDownRows));
  if (xq)
    hipLaunchKernelGGL((lora_down_kernel<RT, true>), grid, dim3(64 * kDownWaves), 0, s, x, ldx, a, (int)M, (int)K,
                       rank, (int)kr, scale, ga, gb, part, t, gq, xq, xs);
  else
    hipLaunchKernelGGL((lora_down_kernel<RT, false>), grid, dim3(64 * kDownWaves), 0, s, x, ldx, a, (int)M, (int)K,
                       rank, (int)kr, scale, ga, gb, part, t, gq, xq, xs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || slices == 1) return e;
  const int64_t n = M * rank;
  const dim3 fgrid((unsigned)((n + 1023) / 1024));
  hipLaunchKernelGGL(lora_down_finish_kernel<kMaxSlices>, fgrid, dim3(256), 0, s, part, n, slices, scale, ga, gb, t);
  return hipGetLastError();
}

}  // namespace

// K slices: enough workgroups (row blocks x slices) to cover the 256 compute units twice, at
// most kMaxSlices, and few enough that the partial products (slices x M x rank fp32, written
// and read once) stay within a quarter of X's bytes; slices are whole steps, all but the last
// of equal length.
int64_t lora_down_slice_k(int64_t K, int slices) {
  const int64_t steps = (K + kStep - 1) / kStep;
  return ((steps + slices - 1) / slices) * kStep;
}
int lora_down_slices(int64_t M, int64_t K, int rank) {
  const int64_t blocks = (M + kDownRows - 1) / kDownRows;
  int64_t z = (512 + blocks - 1) / blocks;
  const int64_t steps = (K + kStep - 1) / kStep;
  if (z > steps) z = steps;
  if (z > kMaxSlices) z = kMaxSlices;
  if (z > K / (8 * (int64_t)rank)) z = K / (8 * (int64_t)rank);
  if (z < 1) z = 1;
  const int64_t kr = lora_down_slice_k(K, (int)z);
  return (int)((K + kr - 1) / kr);  // no empty slice
}

// Whole-row kernel or K-sliced kernel. Each whole-row workgroup reads all of A (r x K) from L2,
// so its cost grows with rank x rounds of 256 workgroups (4096 rows), while the sliced kernel
// shares each adapter stage among 128 rows but needs a finishing pass (and, on the fp8r path,
// the separate quantizer). Measured at K = 3072 (us, sliced vs whole-row without encoding):
// 4096 rows 10.2 / 12.1 / 15.1 / 27.3 vs 6.5 / 8.8 / 11.6 / 17.7 at rank 16 / 32 / 64 / 128;
// 16384 rows 20.8 / 23.0 / 28.6 / 36.8 vs 19.9 / 33.7 / 44.9 / 67.8; 256-1024 rows about 7 / 8 /
// 12 / 25 vs 6.4 / 8.4 / 11.2 / 17.0; 16 rows 5.6 / 6.0 / 8.3 / 17.0 vs 6.2 / 8.1 / 10.8 / 16.4.
bool lora_down_rows_fits(int64_t K) { return K <= 64 * kFusedMaxChunks * kFusedWaves; }
bool lora_down_rows_pick(int64_t M, int64_t K, int rank, DownEnc enc) {
  if (!lora_down_rows_fits(K)) return false;
  if (M > 4096) return rank <= 16;  // one rank tile keeps the adapter reads short
  // rows over 3072 values (twelve chunks a wave): from 2048 rows at any rank and encoding --
  // K = 4096 / 6144 at 4096 rows, rank 32, fp8r linear: quantizer + sliced 21.4 / 31.1 us
  // against 17.1 / 21.2; below 2048 rows the sliced kernel wins from rank 32 on
  if (K > 64 * 6 * kFusedWaves) return M >= 2048;
  // fp8r: the fused kernel also replaces the quantizer's launch
  if (enc == kDownFp8r) return true;
  // nvfp4 (the sliced kernel encodes too, with a finishing pass) and no encoding: below 256
  // rows the sliced kernel's spread over K wins up to rank 64 (16 x 12288 x 3072 nvfp4 linear,
  // rank 16: 23.0 us against 25.2), and without an encoding at ranks 17-32 below 2048 rows
  if (M < 256) return rank > 64;
  return enc == kDownNvfp4 || rank <= 16 || rank > 32 || M >= 2048;
}

hipError_t launch_lora_down_rows(const uint16_t* x, int64_t ldx, const uint16_t* a, int64_t M, int64_t K, int rank,
                                 float scale, const float* ga, const float* gb, uint16_t* t, const RowsEncode& en,
                                 hipStream_t s) {
  if (!lora_down_rows_fits(K)) return hipErrorInvalidValue;
  if (rank <= 16) return run_down_rows<1>(x, ldx, a, M, K, rank, scale, ga, gb, t, en, s);
  if (rank <= 32) return run_down_rows<2>(x, ldx, a, M, K, rank, scale, ga, gb, t, en, s);
  if (rank <= 64) return run_down_rows<4>(x, ldx, a, M, K, rank, scale, ga, gb, t, en, s);
  return run_down_rows<8>(x, ldx, a, M, K, rank, scale, ga, gb, t, en, s);
}

hipError_t launch_lora_down(const uint16_t* x, int64_t ldx, const uint16_t* a, int64_t M, int64_t K, int rank,
                            float scale, const float* ga, const float* gb, float* part, uint16_t* t, hipStream_t s,
                            const float* gq, uint8_t* xq, uint8_t* xs) {
  if (rank <= 16) return run_down<1>(x, ldx, a, M, K, rank, scale, ga, gb, part, t, gq, xq, xs, s);
  if (rank <= 32) return run_down<2>(x, ldx, a, M, K, rank, scale, ga, gb, part, t, gq, xq, xs, s);
  if (rank <= 64) return run_down<4>(x, ldx, a, M, K, rank, scale, ga, gb, part, t, gq, xq, xs, s);
  return run_down<8>(x, ldx, a, M, K, rank, scale, ga, gb, part, t, gq, xq, xs, s);
}

}  // namespace bsq
