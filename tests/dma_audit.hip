// Host-side audit of every LDS-DMA load of the GEMM kernels (built and run by
// tests/test_dma_audit.py; no GPU involved).
//
// The kernels compute each load's addresses with the functions of gemm_tiles.hpp; this program
// calls the same functions for every launched tile configuration, over ragged shapes, the
// tiles at the matrix edges, every wave, load, lane and stage (stages past K included where
// the kernel issues them), and checks for each lane:
//  * LDS: the destination lies inside the kernel's LDS array and inside its stage slot;
//  * buffer offsets: voffset + soffset does not wrap 32 bits; an offset marked out of range
//    really is at or past num_records (it reads zeros); any other offset reads bytes that lie
//    wholly inside num_records, inside one row, inside that row's data (never the padding past
//    its last element), and in range exactly when the chunk's K values are below K.
// It prints one line per configuration and exits with status 1 on the first violation.
#include <cstdio>
#include <cstdlib>
#include <cstdint>
#include <algorithm>
#include <vector>
#include <utility>

#include "gemm_tiles.hpp"

using namespace bsq;
using namespace bsq::gemm;

namespace {

long g_lanes = 0;

[[noreturn]] void fail(const char* cfg, const char* what, long a, long b, long c, long d) {
  std::printf("VIOLATION %s: %s (%ld %ld %ld %ld)\n", cfg, what, a, b, c, d);
  std::exit(1);
}

// one lane of one load: `bytes` per lane, region destination `dst` in an LDS array of
// `lds_size` bytes whose stage slot is [slot0, slot1); a buffer of `records` bytes holding
// `rows` rows of `pitch` bytes with `row_data` bytes of data each; `want_in` says whether the
// chunk's K values are inside K
void check_lane(const char* cfg, const DmaAddr& d, int region_base, int bytes, int lds_size, int slot0, int slot1,
                uint32_t records, int rows, long pitch, long row_data, bool want_in) {
  ++g_lanes;
  const long dst = (long)region_base + d.lds;
  if (dst < 0 || dst + bytes > lds_size) fail(cfg, "LDS destination outside the LDS array", dst, bytes, lds_size, 0);
  if (dst < slot0 || dst + bytes > slot1) fail(cfg, "LDS destination outside its stage slot", dst, slot0, slot1, 0);
  const uint64_t off = (uint64_t)(uint32_t)d.voff + (uint64_t)(uint32_t)d.soff;
  if (off >= (1ull << 32)) fail(cfg, "voffset + soffset wraps 32 bits", d.voff, d.soff, 0, 0);
  if (d.voff == kOutOfRange) {
    if (off < records) fail(cfg, "out-of-range mark lands inside the records", d.voff, d.soff, records, 0);
    if (want_in) fail(cfg, "chunk inside K marked out of range", d.voff, d.soff, 0, 0);
    return;
  }
  if (off >= records) {
    // rows past the tile's rows inside the matrix read zeros; they only feed outputs that are
    // never stored, and their K chunk must still be a real one
    if (off / pitch < rows) fail(cfg, "in-range row read as out of range", (long)off, records, rows, pitch);
    return;
  }
  if (!want_in) fail(cfg, "chunk past K not marked out of range", (long)off, records, 0, 0);
  if (off + bytes > records) fail(cfg, "read straddles the end of the records", (long)off, bytes, records, 0);
  const long r = (long)(off / pitch), in_row = (long)(off % pitch);
  if (r >= rows) fail(cfg, "read past the tile's rows", (long)off, r, rows, pitch);
  if (in_row + bytes > row_data) fail(cfg, "read past a row's data", (long)off, in_row, row_data, pitch);
}

std::vector<int> edge_tiles(int extent, int tile) {
  const int n = (extent + tile - 1) / tile;
  std::vector<int> t{0};
  if (n > 1) t.push_back(n - 1);
  if (n > 2) t.push_back(n - 2);
  return t;
}

// a region of a tiled GEMM stage, all waves and loads
template <class Rg>
void audit_region(const char* cfg, int region_base, int lds_size, int slot0, int slot1, uint32_t records, int rows,
                  long pitch, long row_data, int stride, int kbyte, int kb, int K, int vpc, bool all_waves_equal) {
  (void)all_waves_equal;
  for (int wave = 0; wave < 4; ++wave)
    for (int i = 0; i < Rg::MAX_PER_WAVE; ++i) {
      const int ld = wave + 4 * i;
      if (i >= Rg::MIN_PER_WAVE && ld >= Rg::LOADS) break;
      for (int lane = 0; lane < 64; ++lane) {
        const DmaAddr d = region_load<Rg>(ld, lane, stride, kbyte, kb, K);
        const int c = swz_chunk<Rg::C * 16>(ld * Rg::RPL + lane / Rg::C, lane % Rg::C);
        check_lane(cfg, d, region_base, 16, lds_size, slot0, slot1, records, rows, pitch, row_data,
                   kb + c * vpc < K);
      }
    }
}

// ---- fp8r W8A8 adapter rows (gemm_fp8.hip, ranks 8 / 16 / 24 / 32): the tile's T rows and B
// rows copied once into a separate LDS array of (BM + BN) rows of 64 bytes
template <int BM, int BN>
void audit_lora_rows(int M, int N, int rank) {
  constexpr int R = 64;
  using RT = Region<R, BM, R / 2>;
  using RBr = Region<R, BN, R / 2>;
  char cfg[96];
  std::snprintf(cfg, sizeof cfg, "fp8 adapter rows %dx%d, %dx%d rank %d", BM, BN, M, N, rank);
  const int lds = (BM + BN) * R;
  for (int tm : edge_tiles(M, BM))
    for (int tn : edge_tiles(N, BN)) {
      const int rows_t = std::min(BM, M - tm * BM), rows_b = std::min(BN, N - tn * BN);
      audit_region<RT>(cfg, 0, lds, 0, BM * R, (uint32_t)(rows_t * rank * 2), rows_t, 2 * rank, 2 * rank, 2 * rank,
                       0, 0, rank, 8, false);
      audit_region<RBr>(cfg, BM * R, lds, BM * R, lds, (uint32_t)(rows_b * rank * 2), rows_b, 2 * rank, 2 * rank,
                        2 * rank, 0, 0, rank, 8, false);
    }
  std::printf("ok %s\n", cfg);
}

// ---- fp8r W8A8 row / column scales (gemm_fp8.hip): dword LDS DMA of 64 rows a load into the
// tile's scale arrays (BM and BN floats), rows past M or N past the records
void audit_fp8_scales(int BM, int BN, int M, int N) {
  char cfg[96];
  std::snprintf(cfg, sizeof cfg, "fp8 scales %dx%d, %dx%d", BM, BN, M, N);
  for (int tm : edge_tiles(M, BM))
    for (int tn : edge_tiles(N, BN)) {
      const int rows[2] = {std::min(BM, M - tm * BM), std::min(BN, N - tn * BN)}, len[2] = {BM, BN};
      for (int v = 0; v < 2; ++v)
        for (int wave = 0; wave < 4; ++wave)
          for (int i = wave; i < len[v] / 64; i += 4)
            for (int lane = 0; lane < 64; ++lane) {
              const DmaAddr d{256 * i + 4 * lane, (64 * i + lane) * 4, 0};
              // one float per row: pitch 4, row data 4; the scale array is its own LDS array
              check_lane(cfg, d, 0, 4, 4 * len[v], 0, 4 * len[v], (uint32_t)(rows[v] * 4), rows[v], 4, 4, true);
            }
    }
  std::printf("ok %s\n", cfg);
}

// ---- fp8r W8A8 adapter rows late (gemm_fp8.hip, hand-ordered 256 x 192 loop, ranks 40..64): the
// tile's T rows and B rows copied into one stage buffer (128-byte rows) of the two
template <int BM, int BN>
void audit_lora_late(int M, int N, int rank, int buf, int k_lo = 0) {
  using C = Fp8Cfg<BM, BN, 2>;
  constexpr int R = 128;
  using RT = Region<R, BM, R / 2>;
  using RBr = Region<R, BN, R / 2>;
  static_assert(C::STAGE == (BM + BN) * R, "one stage buffer");
  char cfg[112];
  std::snprintf(cfg, sizeof cfg, "fp8 adapter rows late %dx%d, %dx%d rank %d from %d buffer %d", BM, BN, M, N, rank,
                k_lo, buf);
  const int s0 = buf * C::STAGE, s1 = s0 + C::STAGE;
  for (int tm : edge_tiles(M, BM))
    for (int tn : edge_tiles(N, BN)) {
      const int rows_t = std::min(BM, M - tm * BM), rows_b = std::min(BN, N - tn * BN);
      audit_region<RT>(cfg, s0, C::LDS, s0, s1, (uint32_t)(rows_t * rank * 2), rows_t, 2 * rank, 2 * rank, 2 * rank,
                       2 * k_lo, k_lo, rank, 8, false);
      audit_region<RBr>(cfg, s0 + BM * R, C::LDS, s0, s1, (uint32_t)(rows_b * rank * 2), rows_b, 2 * rank, 2 * rank,
                        2 * rank, 2 * k_lo, k_lo, rank, 8, false);
    }
  std::printf("ok %s\n", cfg);
}

// ---- fp8r W8A8 (gemm_fp8.hip): general loop (stages 0 .. nk + NS - 1) and, for two stage
// buffers with K % 128 == 0, the hand-ordered loop (stages 0 .. nk - 1, lane offsets of stage 0)
template <int BM, int BN, int NS>
void audit_fp8(int M, int N, int K) {
  using C = Fp8Cfg<BM, BN, NS>;
  char cfg[96];
  std::snprintf(cfg, sizeof cfg, "fp8 %dx%d ring %d, %dx%dx%d", BM, BN, NS, M, N, K);
  const int nk = (K + 127) / 128;
  const bool hs = NS == 2 && K % 128 == 0;
  for (int tm : edge_tiles(M, BM))
    for (int tn : edge_tiles(N, BN)) {
      const int rows_x = std::min(BM, M - tm * BM), rows_w = std::min(BN, N - tn * BN);
      const int last = hs ? nk : nk + NS;
      for (int kt = 0; kt < last; ++kt) {
        const int kb = kt * 128, slot = (kt % NS) * C::STAGE;
        audit_region<typename C::RA>(cfg, slot, C::LDS, slot, slot + C::STAGE, (uint32_t)(rows_w * K), rows_w, K, K,
                                     K, kb, kb, K, 16, true);
        audit_region<typename C::RB>(cfg, slot + C::A_BYTES, C::LDS, slot, slot + C::STAGE, (uint32_t)(rows_x * K),
                                     rows_x, K, K, K, kb, kb, K, 16, true);
        if (hs) {  // the hoisted lane offsets: those of stage 0 with this stage's soffset
          for (int wave = 0; wave < 4; ++wave)
            for (int i = 0; i < C::LOADS_MIN; ++i) {
              const int LA = C::RA::MIN_PER_WAVE;
              const int ld = wave + 4 * (i < LA ? i : i - LA);
              for (int lane = 0; lane < 64; ++lane) {
                DmaAddr d = i < LA ? region_load<typename C::RA>(ld, lane, K, 0, 0, K)
                                   : region_load<typename C::RB>(ld, lane, K, 0, 0, K);
                d.soff = (i < LA ? region_load<typename C::RA>(ld, lane, K, kb, kb, K)
                                 : region_load<typename C::RB>(ld, lane, K, kb, kb, K)).soff;
                const int rows = i < LA ? rows_w : rows_x;
                check_lane(cfg, d, slot + (i < LA ? 0 : C::A_BYTES), 16, C::LDS, slot, slot + C::STAGE,
                           (uint32_t)(rows * K), rows, K, K, true);
              }
            }
        }
      }
    }
  std::printf("ok %s\n", cfg);
}

// ---- nvfp4 W4A4 (gemm_w4a4.hip): K % 256 == 0, stages 0 .. nk + 1
template <int BM, int BN>
void audit_w4a4(int M, int N, int K) {
  using C = W4Cfg<BM, BN>;
  char cfg[96];
  std::snprintf(cfg, sizeof cfg, "w4a4 %dx%d, %dx%dx%d", BM, BN, M, N, K);
  const int nk = K / 256, kp = K / 2, ks = K / 16;
  for (int tm : edge_tiles(M, BM))
    for (int tn : edge_tiles(N, BN)) {
      const int rows_x = std::min(BM, M - tm * BM), rows_w = std::min(BN, N - tn * BN);
      for (int kt = 0; kt < nk + 2; ++kt) {
        const int kb = kt * 256, slot = (kt & 1) * C::STAGE;
        audit_region<typename C::RA>(cfg, slot + C::A_OFF, C::LDS, slot, slot + C::STAGE, (uint32_t)(rows_w * kp),
                                     rows_w, kp, kp, kp, kb >> 1, kb, K, 32, true);
        audit_region<typename C::RB>(cfg, slot + C::B_OFF, C::LDS, slot, slot + C::STAGE, (uint32_t)(rows_x * kp),
                                     rows_x, kp, kp, kp, kb >> 1, kb, K, 32, true);
        audit_region<typename C::SA>(cfg, slot + C::SA_OFF, C::LDS, slot, slot + C::STAGE, (uint32_t)(rows_w * ks),
                                     rows_w, ks, ks, ks, kb >> 4, kb, K, 256, true);
        audit_region<typename C::SB>(cfg, slot + C::SB_OFF, C::LDS, slot, slot + C::STAGE, (uint32_t)(rows_x * ks),
                                     rows_x, ks, ks, ks, kb >> 4, kb, K, 256, true);
      }
    }
  std::printf("ok %s\n", cfg);
}

// ---- weight-only W4A16 / W8A16 (gemm_a16.hip): stages 0 .. nk + 1, X with row pitch ldx
template <int BM, int BN, bool FP4>
void audit_a16(int M, int N, int K, int ldx) {
  using C = ACfg<BM, BN, FP4>;
  char cfg[96];
  std::snprintf(cfg, sizeof cfg, "a16 %s %dx%d, %dx%dx%d ldx %d", FP4 ? "nvfp4" : "e4m3", BM, BN, M, N, K, ldx);
  const int nk = (K + 127) / 128, xpitch = ldx * 2, wpitch = FP4 ? K / 2 : K, ks = K / 16;
  for (int tm : edge_tiles(M, BM))
    for (int tn : edge_tiles(N, BN)) {
      const int rows_x = std::min(BM, M - tm * BM), rows_w = std::min(BN, N - tn * BN);
      for (int kt = 0; kt < nk + 2; ++kt) {
        const int kb = kt * 128, slot = (kt & 1) * C::STAGE;
        audit_region<typename C::RX>(cfg, slot + C::X_OFF, C::LDS, slot, slot + C::STAGE,
                                     (uint32_t)(rows_x * xpitch), rows_x, xpitch, 2L * K, xpitch, 2 * kb, kb, K, 8,
                                     true);
        audit_region<typename C::RW>(cfg, slot + C::W_OFF, C::LDS, slot, slot + C::STAGE,
                                     (uint32_t)(rows_w * wpitch), rows_w, wpitch, wpitch, wpitch,
                                     FP4 ? kb / 2 : kb, kb, K, FP4 ? 32 : 16, true);
        if (FP4) {
          for (int wave = 0; wave < 4; ++wave)
            for (int i = 0; i < (Scales8<BN>::LOADS + 3) / 4; ++i) {
              const int ld = wave + 4 * i;
              if (ld >= Scales8<BN>::LOADS) break;
              for (int lane = 0; lane < 64; ++lane)
                check_lane(cfg, scales8_load(ld, lane, ks, kb, K), slot + C::S_OFF, 4, C::LDS, slot,
                           slot + C::STAGE, (uint32_t)(rows_w * ks), rows_w, ks, ks, kb + 64 * (lane & 1) < K);
            }
        }
      }
    }
  std::printf("ok %s\n", cfg);
}

// ---- few-token LDS-DMA kernel (gemm_skinny.hip, E4M3 weights): every stage of K, per wave
template <int MODE, int MB, int NW>
void audit_skinny(int M, int N, int K, int ldx) {
  using SC = SkCfg<MODE, MB, NW, false>;
  using L = SkLayout<MODE>;
  char cfg[96];
  std::snprintf(cfg, sizeof cfg, "skinny %s MB %d, %dx%dx%d ldx %d", L::XBF ? "w8a16" : "w8a8", MB, M, N, K, ldx);
  const int nk = (K + kSkK - 1) / kSkK, xpitch = L::XBF ? ldx * 2 : K;
  for (int tm : edge_tiles(M, 32 * MB))
    for (int tn : edge_tiles(N, 32)) {
      const int n0 = tn * 32, m0 = tm * 32 * MB, rows_w = std::min(32, N - n0);
      for (int wave = 0; wave < NW; ++wave)
        for (int i = 0; i < 2; ++i)
          for (int s = 0; s < nk; ++s) {
            const int kv = s * kSkK, slot = wave * SC::WAVE + (i & 1) * SC::STAGE;
            for (int j = 0; j < MB; ++j) {
              const int mj = m0 + 32 * j, rows = M - mj <= 0 ? 0 : std::min(32, M - mj);
              const uint32_t rec = L::XBF ? (rows ? (uint32_t)((rows - 1) * xpitch + 2 * K) : 0u) : (uint32_t)(rows * K);
              for (int ld = 0; ld < L::XC::LOADS; ++ld) {
                if (ld * L::XC::RPL >= rows) break;
                for (int lane = 0; lane < 64; ++lane) {
                  const int row = ld * L::XC::RPL + lane / L::XC::C;
                  const int c = swz_chunk<L::XC::C * 16>(row, lane % L::XC::C);
                  const DmaAddr d = L::XBF ? code_load<256>(ld, lane, xpitch, 2 * kv, kv, 8, K)
                                           : code_load<128>(ld, lane, xpitch, kv, kv, 16, K);
                  check_lane(cfg, d, slot + L::W_BYTES + j * L::X_BYTES, 16, SC::LDS, slot, slot + SC::STAGE, rec,
                             rows, xpitch, L::XBF ? 2L * K : K, kv + c * (L::XBF ? 8 : 16) < K);
                }
              }
            }
            for (int ld = 0; ld < L::WC::LOADS; ++ld)
              for (int lane = 0; lane < 64; ++lane) {
                const int row = ld * L::WC::RPL + lane / L::WC::C;
                const int c = swz_chunk<128>(row, lane % L::WC::C);
                check_lane(cfg, code_load<128>(ld, lane, K, kv, kv, 16, K), slot, 16, SC::LDS, slot,
                           slot + SC::STAGE, (uint32_t)(rows_w * K), rows_w, K, K, kv + c * 16 < K);
              }
          }
    }
  std::printf("ok %s\n", cfg);
}

}  // namespace

int main() {
  // shapes: ragged M and N, K with and without a partial last stage, the largest K the
  // 32-bit offsets are sized for in each family
  const int fp8_shapes[][3] = {{64, 64, 128}, {77, 100, 96}, {300, 520, 1056}, {4096, 3072, 3072},
                               {3100, 4000, 768}, {1000, 4960, 512}, {513, 257, 12288}, {256, 256, 32}};
  for (auto& s : fp8_shapes) {
    audit_fp8<64, 64, 4>(s[0], s[1], s[2]);
    audit_fp8<64, 128, 4>(s[0], s[1], s[2]);
    audit_fp8<128, 128, 4>(s[0], s[1], s[2]);
    audit_fp8<128, 128, 2>(s[0], s[1], s[2]);  // two workgroups a compute unit, hand-ordered loop
    audit_fp8<256, 192, 2>(s[0], s[1], s[2]);
    audit_fp8<256, 256, 2>(s[0], s[1], s[2]);
  }
  for (auto& s : {std::pair<int, int>{4096, 3072}, {300, 520}, {77, 100}, {513, 257}}) {
    audit_fp8_scales(64, 64, s.first, s.second);
    audit_fp8_scales(64, 128, s.first, s.second);
    audit_fp8_scales(128, 128, s.first, s.second);
    audit_fp8_scales(256, 192, s.first, s.second);
    audit_fp8_scales(256, 256, s.first, s.second);
  }
  const int lora_shapes[][2] = {{64, 64}, {300, 520}, {4096, 3072}, {77, 100}, {513, 257}};
  for (auto& s : lora_shapes)
    for (int rank : {8, 16, 24, 32}) {
      audit_lora_rows<64, 64>(s[0], s[1], rank);
      audit_lora_rows<64, 128>(s[0], s[1], rank);
      audit_lora_rows<128, 128>(s[0], s[1], rank);
      audit_lora_rows<256, 192>(s[0], s[1], rank);
    }
  for (auto& s : lora_shapes)
    for (int rank : {40, 48, 56, 64})
      for (int buf : {0, 1}) audit_lora_late<256, 192>(s[0], s[1], rank, buf);
  for (auto& s : lora_shapes)
    for (int rank : {72, 96, 120, 128})
      for (int buf : {0, 1})
        for (int k_lo : {0, 64}) audit_lora_late<256, 192>(s[0], s[1], rank, buf, k_lo);
  const int w4_shapes[][3] = {{64, 128, 256}, {300, 520, 512}, {4096, 12288, 3072}, {3100, 4000, 768},
                              {513, 257, 12288}};
  for (auto& s : w4_shapes) {
    audit_w4a4<64, 64>(s[0], s[1], s[2]);
    audit_w4a4<64, 128>(s[0], s[1], s[2]);
    audit_w4a4<128, 128>(s[0], s[1], s[2]);
    audit_w4a4<256, 192>(s[0], s[1], s[2]);
    audit_w4a4<256, 256>(s[0], s[1], s[2]);
  }
  const int a16_shapes[][4] = {{64, 128, 256, 256}, {300, 520, 1088, 1096}, {4096, 12288, 3072, 3072},
                               {77, 100, 192, 200}, {513, 257, 12288, 16384}};
  for (auto& s : a16_shapes) {
    audit_a16<64, 64, true>(s[0], s[1], s[2], s[3]);
    audit_a16<64, 128, true>(s[0], s[1], s[2], s[3]);
    audit_a16<128, 128, true>(s[0], s[1], s[2], s[3]);
    audit_a16<256, 128, true>(s[0], s[1], s[2], s[3]);
    audit_a16<256, 192, true>(s[0], s[1], s[2], s[3]);
    audit_a16<64, 64, false>(s[0], s[1], s[2], s[3]);
    audit_a16<64, 128, false>(s[0], s[1], s[2], s[3]);
    audit_a16<128, 128, false>(s[0], s[1], s[2], s[3]);
    audit_a16<128, 192, false>(s[0], s[1], s[2], s[3]);
    audit_a16<128, 256, false>(s[0], s[1], s[2], s[3]);
  }
  const int sk_shapes[][4] = {{16, 3072, 3072, 3072}, {20, 1024, 512, 520}, {64, 128, 256, 256}, {1, 8, 32, 32},
                              {48, 12288, 3104, 3112}, {128, 100, 96, 128}};
  for (auto& s : sk_shapes) {
    audit_skinny<kW8A8, 1, 4>(s[0], s[1], s[2], s[3]);
    audit_skinny<kW8A8, 2, 4>(s[0], s[1], s[2], s[3]);
    audit_skinny<kW8A16, 1, 4>(s[0], s[1], s[2], s[3]);
    audit_skinny<kW8A8, 1, 8>(s[0], s[1], s[2], s[3]);
    audit_skinny<kW8A16, 1, 2>(s[0], s[1], s[2], s[3]);
  }
  std::printf("all LDS-DMA loads in bounds: %ld lanes checked\n", g_lanes);
  return 0;
}
