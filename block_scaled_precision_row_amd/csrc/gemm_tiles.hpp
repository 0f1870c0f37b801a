// Tile configurations of the LDS-DMA GEMMs and the address arithmetic of every LDS-DMA load,
// as host- and device-callable integer functions. The kernels issue their loads through
// these functions, and a host program (tests/dma_audit.hip) enumerates every load of every
// launched configuration through the same functions and checks its LDS destination and its
// buffer offsets.
//
// An LDS-DMA load (buffer_load_dword[x4] ... lds) makes lane l fetch 4 or 16 bytes at
// rsrc.base + voffset(l) + soffset (the buffer's range check covers both offsets: reads at or
// past num_records return zeros) and write them to LDS at M0 + 4 l or M0 + 16 l. A DmaAddr
// describes one lane of one load: `lds` is that lane's destination relative to the region's
// base (M0 - region base + 4 or 16 lane), voff and soff the two buffer offsets.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsq_launch.hpp"

namespace bsq {
namespace gemm {

constexpr int kOutOfRange = 0x40000000;  // buffer offset beyond any tile's records

struct DmaAddr {
  int lds;
  int voff;
  int soff;
};

// LDS rows of R bytes hold R/16 chunks of 16 bytes. A ds_read_b128 serves 16 lanes per
// 256-byte LDS window; 16 consecutive rows reading the same logical chunk must land on 16
// distinct 16-byte slots of the window, so the physical chunk is the logical one XOR-ed with
// (row / rows-per-window) mod chunks. The swizzle is an involution.
template <int R>
__host__ __device__ constexpr int swz_chunk(int row, int c) {
  constexpr int C = R / 16, RPW = 16 / C;
  return c ^ ((row / RPW) % C);
}
template <int R>
__host__ __device__ constexpr int swz_off(int row, int c) {
  return row * R + (swz_chunk<R>(row, c) << 4);
}

// One operand region of a stage: ROWS rows of R bytes each, holding KSTAGE K values per row
// (for a 64-deep stage: 128 bytes of bf16, 64 of E4M3, 32 of packed E2M1, 4 of E4M3 block
// scales). A 1 KB DMA load covers 1024 / R rows; lane l writes physical chunk l % C of row
// l / C, so it fetches the logical chunk that the swizzle places there. Loads are spread
// round-robin over the 4 waves of a workgroup.
template <int R, int ROWS, int KSTAGE>
struct Region {
  static constexpr int C = R / 16;
  static constexpr int RPL = 1024 / R;            // rows per load
  static constexpr int LOADS = ROWS / RPL;        // loads per stage
  static constexpr int MIN_PER_WAVE = LOADS / 4;  // loads issued by every wave
  static constexpr int MAX_PER_WAVE = (LOADS + 3) / 4;
  static_assert(ROWS % RPL == 0, "region rows must fill whole loads");
  static constexpr int VPC = 16 * KSTAGE / R;     // K values per 16-byte chunk
};

// Load `ld` of region Rg for the stage starting at K value kb, `kbyte` bytes into each row of
// pitch `stride`; chunks at or past K get the out-of-range offset (they read zeros).
template <class Rg>
__host__ __device__ constexpr DmaAddr region_load(int ld, int lane, int stride, int kbyte, int kb, int K) {
  const int lrow = lane / Rg::C, phys = lane % Rg::C;
  const int row = ld * Rg::RPL + lrow;
  const int c = swz_chunk<Rg::C * 16>(row, phys);
  const int voff = (kb + c * Rg::VPC < K) ? lrow * stride + (c << 4) : kOutOfRange;
  return DmaAddr{ld * 1024 + 16 * lane, voff, ld * Rg::RPL * stride + kbyte};
}

// nvfp4 block scales of a 128-deep weight-only stage: 8 bytes per weight row, dword loads of
// 32 rows (two lanes per row), K past the end out of range.
template <int ROWS>
struct Scales8 {
  static constexpr int LOADS = ROWS / 32;
  static_assert(ROWS % 32 == 0, "whole scale loads");
};
__host__ __device__ constexpr DmaAddr scales8_load(int ld, int lane, int ks, int kb, int K) {
  const int half = lane & 1, lrow = lane >> 1;
  const int voff = (kb + 64 * half < K) ? lrow * ks + 4 * half : kOutOfRange;
  return DmaAddr{ld * 256 + 4 * lane, voff, ld * 32 * ks + (kb >> 4)};
}

// A few-token code region: 32 rows of R bytes; load ld covers rows RPL ld .. RPL ld + RPL - 1,
// the row offset in voffset (soffset 0). `kv` is the stage's first K value, `vpc` the K values
// per 16-byte chunk, `kbyte` the stage's byte offset in a row.
template <int R>
struct CodeRegion {
  static constexpr int C = R / 16, RPL = 1024 / R, LOADS = 32 / RPL, BYTES = 32 * R;
};
template <int R>
__host__ __device__ constexpr DmaAddr code_load(int ld, int lane, int pitch, int kbyte, int kv, int vpc, int K) {
  using G = CodeRegion<R>;
  const int lrow = lane / G::C, phys = lane % G::C;
  const int row = ld * G::RPL + lrow;
  const int c = swz_chunk<R>(row, phys);
  const int voff = kv + c * vpc < K ? row * pitch + kbyte + 16 * c : kOutOfRange;
  return DmaAddr{ld * 1024 + 16 * lane, voff, 0};
}

// ---- tile configurations ----------------------------------------------------------------
// fp8r W8A8 (gemm_fp8.hip): 128-deep stages of W rows (region A) then Xq rows (region B), a
// ring of NS stages; the bf16 output tile reuses the LDS.
template <int BM, int BN, int NS>
struct Fp8Cfg {
  static constexpr int KSTAGE = 128;
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int TM = WM / 32, TN = WN / 32;
  using RA = Region<128, BN, KSTAGE>;  // W rows
  using RB = Region<128, BM, KSTAGE>;  // Xq rows
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

// nvfp4 W4A4 (gemm_w4a4.hip): 256-deep stages of packed W and Xq rows (128 bytes each) and
// their block scales (16 bytes each), two stage buffers.
template <int BM, int BN>
struct W4Cfg {
  static constexpr int KSTAGE = 256;
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int TM = WM / 32, TN = WN / 32;
  using RA = Region<128, BN, KSTAGE>;  // packed W rows, 128 bytes per stage
  using RB = Region<128, BM, KSTAGE>;  // packed Xq rows
  using SA = Region<16, BN, KSTAGE>;   // W block scales, 16 bytes per stage
  using SB = Region<16, BM, KSTAGE>;   // Xq block scales
  static constexpr int A_OFF = 0, B_OFF = BN * 128, SA_OFF = (BN + BM) * 128, SB_OFF = SA_OFF + BN * 16;
  static constexpr int STAGE = (BN + BM) * 144;
  static constexpr int LOADS = RA::MAX_PER_WAVE + RB::MAX_PER_WAVE + SA::MAX_PER_WAVE + SB::MAX_PER_WAVE;
  static constexpr int TROW = BN * 2 + 16;  // bytes per row of the bf16 output tile in LDS
  static constexpr int LDS = 2 * STAGE > BM * TROW ? 2 * STAGE : BM * TROW;
  static_assert(LOADS < 64, "vmcnt range");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// weight-only W4A16 / W8A16 (gemm_a16.hip): 128-deep stages of bf16 X rows (256 bytes), packed
// E2M1 (64 bytes) or E4M3 (128 bytes) W rows, and for nvfp4 8 block-scale bytes per W row.
template <int BM, int BN, bool FP4>
struct ACfg {
  static constexpr int KSTAGE = 128;
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int WR = FP4 ? 64 : 128;  // weight bytes per row and stage
  using RX = Region<256, BM, KSTAGE>;        // X rows: 128 bf16 values
  using RW = Region<WR, BN, KSTAGE>;         // W rows: packed E2M1 or E4M3
  static constexpr int X_OFF = 0, W_OFF = BM * 256, S_OFF = W_OFF + BN * WR;
  static constexpr int STAGE = S_OFF + (FP4 ? BN * 8 : 0);  // nvfp4: 8 block scales per row
  static constexpr int TROW = BN * 2 + 16;  // bytes per row of the bf16 output tile in LDS
  static constexpr int LDS = 2 * STAGE > BM * TROW ? 2 * STAGE : BM * TROW;
  static_assert(LDS + 4 * BN <= 160 * 1024, "LDS budget");
};

// few-token LDS-DMA kernel (gemm_skinny.hip, E4M3 weights): per wave a ring of two stages, each
// 32 weight rows then MB activation blocks of 32 rows, 128 K values deep.
constexpr int kSkRing = 2;  // stage buffers per wave
constexpr int kSkK = 128;   // K values per stage
template <int MODE>
struct SkLayout {
  static_assert(MODE == kW8A8 || MODE == kW8A16, "E4M3 weights only");
  static constexpr bool XBF = MODE == kW8A16;
  using WC = CodeRegion<128>;
  using XC = CodeRegion<XBF ? 256 : 128>;
  static constexpr int W_BYTES = WC::BYTES, X_BYTES = XC::BYTES;  // X per M block
  static constexpr int W_LOADS = WC::LOADS, X_LOADS = XC::LOADS;
};
template <int MODE, int MB, int NW, bool LORA>
struct SkCfg {
  using L = SkLayout<MODE>;
  static constexpr int STAGE = L::W_BYTES + MB * L::X_BYTES;
  static constexpr int WAVE = kSkRing * STAGE;
  static constexpr int LOADS = L::W_LOADS + MB * L::X_LOADS;  // DMA instructions per stage
  static constexpr int RED = NW * MB * 16 * 64 * 4 + (LORA ? MB * 16 * 64 * 4 : 0);  // partial tiles, adapter tiles
  static constexpr int LDS = NW * WAVE > RED ? NW * WAVE : RED;
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert((kSkRing - 1) * LOADS < 64, "vmcnt range");
};

}  // namespace gemm
}  // namespace bsq
