// Building blocks shared by the GEMM kernels: tile mapping, LDS swizzles,
// the LDS-DMA stage loader and the bf16 epilogue.
//
// All GEMMs compute Y[m][n] = sum_k X[m][k] W[n][k] for row-major X [M][K]
// and W [N][K] (both K-contiguous). A workgroup of 4 waves owns a BM x BN
// tile of Y; each wave a (BM/2) x (BN/2) quadrant of 32x32 MFMA tiles. The
// MFMA "A" operand is a 32-row slice of W and "B" a 32-row slice of X, so the
// accumulator of a lane holds one token m (lane % 32) and, per 4-register
// group g, the four consecutive outputs n = 8 g + 4 (lane / 32) + (0..3).
//
// K is walked in stages (64 to 256 values deep, per kernel). Every stage of
// every operand lands in LDS untouched (packed codes stay packed) through
// buffer_load ... lds, in a ring of stage buffers so that the next stages are
// in flight while the MFMAs work on an older one. Operands are read from LDS
// into registers ahead of their K step and, where needed, decoded there right
// before the MFMA. Tile sizes (BM tokens x BN weight rows) are chosen per
// launch from the grid they give on the 256 compute units.
#pragma once

#include "bsq_device.hpp"
#include "gemm_tiles.hpp"

namespace bsq {
namespace gemm {

constexpr int kThreads = 256;
constexpr int kKS = 64;                  // default K values per stage of a Region
// s_waitcnt with vmcnt <= n (n in 0..63), lgkmcnt and expcnt unconstrained (gfx9 encoding)
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Issue this wave's loads of region `Rg` for the stage starting at K value kb.
// rsrc covers the tile's rows (rows past the matrix read as zeros), `stride`
// is the row pitch in bytes, `kbyte` the byte offset of the stage in a row.
template <class Rg>
__device__ __forceinline__ void dma_region(const v4i& rsrc, uint32_t lds_base, int wave, int lane, int stride,
                                           int kbyte, int kb, int K) {
#pragma unroll
  for (int i = 0; i < Rg::MAX_PER_WAVE; ++i) {
    const int ld = wave + 4 * i;
    if (i >= Rg::MIN_PER_WAVE && ld >= Rg::LOADS) break;  // wave-uniform
    const DmaAddr d = region_load<Rg>(ld, lane, stride, kbyte, kb, K);
    dma16(rsrc, lds_base + ld * 1024, d.voff, d.soff);
  }
}

// dword LDS DMA: lane l's 4 bytes land at M0 + 4 l (inline asm like dma16, with the same
// caveat on VALU-written SGPR operands)
__device__ __forceinline__ void dma4(v4i rsrc, uint32_t lds, int voff, int soff) {
  asm volatile("buffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds));
}

// ---- bf16 epilogue --------------------------------------------------------------
// acc[i][j] is the 32x32 tile (n-tile i, m-tile j) of this wave; `scale(n)`
// gives the per-output factor (row scales and global scales folded in by the
// caller: y = bf16(acc * rowscale(m) * scale(n))).
template <int TN, int TM, class RowScale, class ColScale>
__device__ __forceinline__ void store_tile(const v16f (&acc)[TN][TM], uint16_t* __restrict__ y, int64_t ldy, int M,
                                           int N, int mw0, int nw0, int lane, RowScale rs, ColScale cs) {
  const int lr = lane & 31, lh = lane >> 5;
  const bool vec_ok = (ldy & 3) == 0;  // 8-byte stores need 4-element aligned rows
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int m = mw0 + j * 32 + lr;
    if (m >= M) continue;
    const float xs = rs(m);
    uint16_t* yr = y + (int64_t)m * ldy;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = nw0 + i * 32 + 8 * g + 4 * lh;
        const v16f& A = acc[i][j];
        if (n + 3 < N && vec_ok) {
          const float v0 = A[4 * g + 0] * xs * cs(n + 0), v1 = A[4 * g + 1] * xs * cs(n + 1);
          const float v2 = A[4 * g + 2] * xs * cs(n + 2), v3 = A[4 * g + 3] * xs * cs(n + 3);
          *reinterpret_cast<uint2*>(yr + n) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) yr[n + e] = (uint16_t)(pack_bf16x2(A[4 * g + e] * xs * cs(n + e), 0.0f) & 0xFFFFu);
        }
      }
    }
  }
}

// Copy a bf16 output tile [BM][BN] (rows TROW bytes apart in LDS) to Y in
// 16-byte row chunks: consecutive threads write consecutive chunks of a row.
// Whole tiles use non-temporal stores when `stream` is set (stream_output():
// outputs that would push the operands out of the last-level cache), plain
// cached stores otherwise.
template <int BM, int BN, int TROW>
__device__ __forceinline__ void store_tile_rows(const uint8_t* tile, uint16_t* __restrict__ y, int64_t ldy, int M,
                                                int N, int m0, int n0, int tid, bool stream) {
  constexpr int CPR = BN / 8;  // 16-byte chunks per row
  const bool vec_ok = (ldy & 7) == 0;
  constexpr int IT = BM * CPR / kThreads;
  if (BM * CPR % kThreads == 0 && IT % 8 == 0 && vec_ok && m0 + BM <= M && n0 + BN <= N) {
    // Whole tile inside the matrix: read eight chunks from LDS before storing them, so the
    // LDS latency is paid once per eight stores instead of once per store.
#pragma unroll
    for (int i0 = 0; i0 < IT; i0 += 8) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = tid + (i0 + u) * kThreads, ml = idx / CPR, c = idx - ml * CPR;
        v[u] = *reinterpret_cast<const uint4*>(tile + ml * TROW + c * 16);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = tid + (i0 + u) * kThreads, ml = idx / CPR, c = idx - ml * CPR;
        uint4* dst = reinterpret_cast<uint4*>(y + (int64_t)(m0 + ml) * ldy + n0 + 8 * c);
        if (stream)
          store_stream(dst, v[u]);
        else
          *dst = v[u];
      }
    }
    return;
  }
  for (int idx = tid; idx < BM * CPR; idx += kThreads) {
    const int ml = idx / CPR, c = idx - ml * CPR;
    const int m = m0 + ml, n = n0 + 8 * c;
    if (m >= M) break;  // rows only grow with idx
    const uint4 v = *reinterpret_cast<const uint4*>(tile + ml * TROW + c * 16);
    uint16_t* dst = y + (int64_t)m * ldy + n;
    if (n + 8 <= N && vec_ok) {
      *reinterpret_cast<uint4*>(dst) = v;
    } else {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n + e < N) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
  }
}

// Quantize a bf16 output tile [BM][BN] (rows TROW bytes apart in LDS) to nvfp4 for the next
// linear: each 16-value block along n becomes 8 bytes of E2M1 codes in yq [M][N/2] and one
// E4M3 scale in ys [M][N/16], with the activation quantizer's arithmetic (N % 32 == 0, so
// blocks never straddle the matrix edge). Consecutive threads take consecutive blocks of a row.
template <int BM, int BN, int TROW>
__device__ __forceinline__ void quant_tile_rows(const uint8_t* tile, uint8_t* __restrict__ yq, uint8_t* __restrict__ ys,
                                                float G, int M, int N, int m0, int n0, int tid) {
  constexpr int BPR = BN / 16;  // blocks per tile row
  for (int idx = tid; idx < BM * BPR; idx += kThreads) {
    const int ml = idx / BPR, b = idx - ml * BPR;
    const int m = m0 + ml, n = n0 + 16 * b;
    if (m >= M) break;  // rows only grow with idx
    if (n >= N) continue;
    const uint4 v0 = *reinterpret_cast<const uint4*>(tile + ml * TROW + 32 * b);
    const uint4 v1 = *reinterpret_cast<const uint4*>(tile + ml * TROW + 32 * b + 16);
    float f[16];
    bf16x16_to_f32(v0, v1, f);
    uint2 codes;
    const uint32_t sf = quant_block16_nvfp4(f, G, codes);
    *reinterpret_cast<uint2*>(yq + (int64_t)m * (N >> 1) + (n >> 1)) = codes;
    ys[(int64_t)m * (N >> 4) + (n >> 4)] = (uint8_t)sf;
  }
}

// Row maxima of |y| over 64-column segments of a bf16 output tile [BM][BN] (rows TROW bytes
// apart in LDS), for an fp8r encoding of Y whose per-row scale needs the whole row: segment s
// of row m goes to pmax[m][s] (s counted over the whole row, ceil(N/64) per row, N % 32 == 0),
// and a later pass takes each row's maximum over its segments, reading them contiguously.
// Consecutive threads take consecutive segments of a row. The bf16 bit pattern with the sign
// cleared orders magnitudes as unsigned integers, so the maximum is exact and order-free.
template <int BM, int BN, int TROW>
__device__ __forceinline__ void rowmax_tile(const uint8_t* tile, float* __restrict__ pmax, int M, int N, int m0,
                                            int n0, int tid) {
  constexpr int SEG = BN / 64;
  static_assert(BN % 64 == 0, "tiles cover whole 64-column segments");
  const int nseg = (N + 63) >> 6;
  for (int idx = tid; idx < BM * SEG; idx += kThreads) {
    const int ml = idx / SEG, sg = idx % SEG;
    const int m = m0 + ml, n = n0 + 64 * sg;
    if (m >= M || n >= N) continue;
    const int nc = (N - n < 64 ? N - n : 64) >> 3;  // whole 8-value chunks (N % 32 == 0)
    uint32_t mx = 0;
    for (int c = 0; c < nc; ++c) {
      const uint4 v = *reinterpret_cast<const uint4*>(tile + ml * TROW + (64 * sg + 8 * c) * 2);
      const uint32_t w[4] = {v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu, v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu};
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = max(mx, max(w[e] & 0xFFFFu, w[e] >> 16));
    }
    pmax[(int64_t)m * nseg + (n0 >> 6) + sg] = __uint_as_float(mx << 16);
  }
}

// ---- low-rank adapter (LoRA) up-projection on the accumulators ---------------------------
// An adapter adds T B^T to the layer's output, with T = s X A^T [M][rank] (bf16, the adapter's
// scale already applied by the down-projection kernel) and B [N][rank] (bf16). The tiled GEMMs
// run it after their K loop on their own accumulators, once those hold output units:
// acc[i][j] += (B rows as the MFMA A operand, n) x (T rows as the B operand, m) over the rank,
// 16 values per step on the bf16 matrix cores, in the accumulator layout of the main loop.
// Rows past M or N and values past the rank read as zero.

// values k8 .. k8 + 7 (k8 a multiple of 8) of row `row` of the bf16 [rows][rank] matrix behind r
__device__ __forceinline__ v8bf lora_chunk(rsrc_t r, int row, int k8, int rank) {
  union {
    uint4 u;
    v8bf h;
  } c;
  if ((rank & 7) == 0) {
    c.u = bload16(r, k8 < rank ? (uint32_t)(row * rank + k8) * 2u : kBufOut);
  } else {  // rows are not 16-byte aligned: two-byte loads
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = k8 + 2 * e;
      const uint32_t off = (uint32_t)(row * rank + k) * 2u;
      const uint32_t lo = bload2(r, k < rank ? off : kBufOut), hi = bload2(r, k + 1 < rank ? off + 2u : kBufOut);
      w[e] = (lo & 0xFFFFu) | (hi << 16);
    }
    c.u = make_uint4(w[0], w[1], w[2], w[3]);
  }
  return c.h;
}

// S rank steps of 16 of this lane's adapter operands (B rows for the MFMA A operand, T rows for B)
template <int TN, int TM, int S>
struct LoraRegs {
  v8bf b[S][TN];
  v8bf t[S][TM];
};
template <int TN, int TM, int S>
__device__ __forceinline__ void lora_load(LoraRegs<TN, TM, S>& r, rsrc_t rt, rsrc_t rb, int k0, int rank, int nw0,
                                          int mw0, int lane) {
  const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int s = 0; s < S; ++s) {
#pragma unroll
    for (int i = 0; i < TN; ++i) r.b[s][i] = lora_chunk(rb, nw0 + 32 * i + lr, k0 + 16 * s + 8 * lh, rank);
#pragma unroll
    for (int j = 0; j < TM; ++j) r.t[s][j] = lora_chunk(rt, mw0 + 32 * j + lr, k0 + 16 * s + 8 * lh, rank);
  }
}
// the adapter MFMAs of rank steps k0 / 16 .. k0 / 16 + S - 1 (steps past the rank are skipped)
template <int TN, int TM, int S>
__device__ __forceinline__ void lora_mfma(v16f (&acc)[TN][TM], const LoraRegs<TN, TM, S>& r, int k0, int rank) {
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if (k0 + 16 * s >= rank) break;  // uniform
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.b[s][i], r.t[s][j], acc[i][j], 0, 0, 0);
  }
}

// acc[i][j] (n-tile i at n = nw0 + 32 i, m-tile j at m = mw0 + 32 j) += T[m][:] . B[n][:],
// 64 rank values per batch of loads (32 for the larger wave tiles, whose accumulators leave
// fewer registers)
template <int TN, int TM>
__device__ __forceinline__ void lora_update(v16f (&acc)[TN][TM], const uint16_t* lt, const uint16_t* lb, int rank,
                                            int M, int N, int nw0, int mw0, int lane) {
  constexpr int S = TN + TM >= 7 ? 2 : 4;
  const rsrc_t rt = make_rsrc(lt, (uint32_t)M * (uint32_t)rank * 2u);
  const rsrc_t rb = make_rsrc(lb, (uint32_t)N * (uint32_t)rank * 2u);
  for (int k0 = 0; k0 < rank; k0 += 16 * S) {
    LoraRegs<TN, TM, S> r;
    lora_load(r, rt, rb, k0, rank, nw0, mw0, lane);
    lora_mfma(acc, r, k0, rank);
  }
}

// tile index of this workgroup (XCD-contiguous, grouped along M)
// tile of workgroup `bid` of a grid of BM x BN tiles over M x N (bid < the tile count)
__device__ __forceinline__ void tile_of_id(int bid, int M, int N, int BM, int BN, int& m0, int& n0) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  grouped_tile(xcd_contiguous_id(bid, tiles_m * tiles_n), tiles_m, tiles_n, 8, tm, tn);
  m0 = tm * BM;
  n0 = tn * BN;
}
__device__ __forceinline__ void tile_of_block(int M, int N, int BM, int BN, int& m0, int& n0) {
  tile_of_id(blockIdx.x, M, N, BM, BN, m0, n0);
}

// A grouped launch runs the tiles of several independent GEMMs in one grid: problem p owns
// workgroups [start[p], start[p + 1]). Returns the problem of workgroup `bid` (uniform).
template <int S>
__device__ __forceinline__ int group_problem(const int (&start)[S], int count, int bid) {
  int p = 0;
#pragma unroll
  for (int i = 1; i < S - 1; ++i) p += (i < count && bid >= start[i]) ? 1 : 0;
  return p;
}

}  // namespace gemm
}  // namespace bsq
