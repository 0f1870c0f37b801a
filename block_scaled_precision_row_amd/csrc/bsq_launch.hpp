// Internal launch interface between the C ABI (bsq_api.cpp) and the kernels.
// Arguments are already validated by the caller; each function enqueues its
// kernels on `s` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bsq {

// Device scratch owned by the library (scratch.hip): kScratchBytes per GPU, 256-byte aligned,
// held until the process ends. scratch_buffer() returns the current device's copy (looked up
// once per device). Every user on one GPU shares it.
constexpr size_t kScratchBytes = (size_t)64 << 20;
hipError_t scratch_buffer(void** out);

hipError_t launch_quant_fp8r(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* xq,
                             float* sx, hipStream_t s);
hipError_t launch_quant_nvfp4(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const float* g,
                              uint8_t* xq, uint8_t* xs, hipStream_t s);
int calibrate_partials(int64_t M);
hipError_t launch_calibrate(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, float* out,
                            float* partials, hipStream_t s);
hipError_t launch_dequant_nvfp4(const uint8_t* w, const uint8_t* sf, const float* g, int64_t N,
                                int64_t K, uint16_t* out, hipStream_t s);
hipError_t launch_dequant_fp8r(const uint8_t* w, const float* sw, int64_t N, int64_t K,
                               uint16_t* out, hipStream_t s);

// Whether a tiled GEMM writes Y with non-temporal stores: when its operands and output
// together overflow the 256 MiB last-level (Infinity) cache by a margin, cached output
// writes evict operand panels that later tiles read again. Measured on the fp8 GEMM: 9-11 %
// faster with streaming stores at 16384 x {9216, 12288} x 3072 and 16384 x 3072 x 12288,
// 4 % at 4096 x 12288 x 12288, but 3-6 % slower at 8192 x 12288 x 3072 (264 MB) and no
// different at 160 MB; the W4A4 GEMM moves by 1.5 % at most either way.
inline bool stream_output(int64_t operand_bytes, int64_t M, int64_t N) {
  const double bytes = (double)operand_bytes + 2.0 * (double)M * (double)N;
  return bytes > 1.1 * 256.0 * 1024.0 * 1024.0;
}

// Expected time of a grid of BM x BN tiles, in units of `tile_cost` (one tile's run time):
// the tiles run in ceil(tiles / 256) rounds on the 256 compute units (one workgroup of a
// large tile per unit), and a partial last round takes as long as a full one -- the 264
// tiles of 256 x 192 at 3072 x 4096 take twice the time of 256 tiles.
inline int64_t rounds_cost(int64_t M, int64_t N, int BM, int BN, int tile_cost) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  return (tiles + 255) / 256 * tile_cost;
}

// Optional quantized form of a tiled GEMM's output for the next linear (N % 32 == 0):
//   nvfp4: yq [M][N/2] packed E2M1 and ys [M][N/16] E4M3 with global scale *gy, encoded in the
//          epilogue (the 16-blocks along N lie inside a tile);
//   fp8r:  pmax [M][ceil(N/64)], each row's maximum |y| over each 64-column segment, for
//          launch_encode_fp8r_rows to finish once every tile of the row has written its part.
struct YQuant {
  uint8_t* yq = nullptr;
  uint8_t* ys = nullptr;
  const float* gy = nullptr;
  float* pmax = nullptr;
};
inline int64_t ypmax_segments(int64_t N) { return (N + 63) / 64; }

// W8A8: y = bf16((sum e4m3(xq) e4m3(w)) * sx[m] * sw[n])
// (with lt != nullptr, plus the adapter term T B^T; see DecArgs). y may be null when q asks
// for the nvfp4 encoding.
hipError_t launch_gemm_fp8(const uint8_t* xq, const float* sx, const uint8_t* w, const float* sw,
                           uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, const uint16_t* lt,
                           const uint16_t* lb, int rank, hipStream_t s, const YQuant* q = nullptr);
// fp8r encoding of a bf16 Y [M][ldy] (N % 32 == 0) whose row maxima per 64-column segment are
// in pmax [M][ceil(N/64)]: with a = the row's maximum, d = fp32(a / 448), r = fp32(1 / d),
// yq[m][n] = E4M3(fp32(y * r)), yd[m] = d -- what launch_quant_fp8r computes for the same Y.
hipError_t launch_encode_fp8r_rows(const uint16_t* y, int64_t M, int64_t N, int64_t ldy, const float* pmax,
                                   uint8_t* yq, float* yd, hipStream_t s);
// LoRA down projection: t [M][rank] = bf16(f * X A^T), X bf16 [M][ldx], A bf16 [rank][K], with
// f = scale, or scale / (*ga * *gb) when ga != nullptr (T for a GEMM that scales its
// accumulators by *ga * *gb). K is cut into lora_down_slices(M, K, rank) slices; with more than
// one, `part` holds their fp32 partial products [slices][M][rank]. With xq != nullptr the same
// kernel also writes X's nvfp4 encoding with global scale *gq (as launch_quant_nvfp4 does).
int lora_down_slices(int64_t M, int64_t K, int rank);
int64_t lora_down_slice_k(int64_t K, int slices);
hipError_t launch_lora_down(const uint16_t* x, int64_t ldx, const uint16_t* a, int64_t M, int64_t K, int rank,
                            float scale, const float* ga, const float* gb, float* part, uint16_t* t, hipStream_t s,
                            const float* gq = nullptr, uint8_t* xq = nullptr, uint8_t* xs = nullptr);

// The same down projection (same f) from whole rows of X, K <= 6144 (lora_down_rows_fits, else
// hipErrorInvalidValue), optionally writing X's encoding for the GEMM in the same pass, bit
// for bit what the activation quantizers write: fp8r (xq [M][K], sx [M]) or nvfp4 (xq
// [M][K/2], xs [M][K/16], global scale *gq). lora_down_rows_pick: whether it beats the sliced
// kernel (with the encoding, the sliced kernel plus the quantizer for fp8r) at this shape.
enum DownEnc : int { kDownPlain = 0, kDownFp8r = 1, kDownNvfp4 = 2 };
struct RowsEncode {
  DownEnc enc = kDownPlain;
  uint8_t* xq = nullptr;
  float* sx = nullptr;
  uint8_t* xs = nullptr;
  const float* gq = nullptr;
};
bool lora_down_rows_fits(int64_t K);
bool lora_down_rows_pick(int64_t M, int64_t K, int rank, DownEnc enc);
hipError_t launch_lora_down_rows(const uint16_t* x, int64_t ldx, const uint16_t* a, int64_t M, int64_t K, int rank,
                                 float scale, const float* ga, const float* gb, uint16_t* t, const RowsEncode& en,
                                 hipStream_t s);

// Decode-to-16-bit GEMMs on the bf16 / f16 matrix cores.
enum DecMode : int {
  kW4A4 = 0,   // X nvfp4 (xq, xs, *gx), W nvfp4 (w, ws, *gw); f16 MFMA; alpha = gx * gw
  kW4A16 = 1,  // X bf16, W nvfp4; bf16 MFMA; alpha = gw
  kW8A16 = 2,  // X bf16, W E4M3 with per-row scale sw[n]; bf16 MFMA
  kW8A8 = 3,   // X E4M3 (xq) with per-row scale sx[m], W E4M3 with sw[n]; fp8 MFMA (skinny kernel only)
};
struct DecArgs {
  const uint16_t* x;   // bf16 activations (A16 modes)
  int64_t ldx;
  const uint8_t* xq;   // packed E2M1 activations [M][K/2] (W4A4)
  const uint8_t* xs;   // E4M3 activation block scales [M][K/16] (W4A4)
  const float* gx;     // activation global scale (W4A4)
  const uint8_t* w;    // packed E2M1 [N][K/2] or E4M3 [N][K]
  const uint8_t* ws;   // E4M3 weight block scales [N][K/16] (nvfp4)
  const float* gw;     // weight global scale (nvfp4)
  const float* sw;     // per-row weight scales [N] (W8A16, W8A8)
  const float* sx;     // per-row activation scales [M] (W8A8)
  uint16_t* y;         // bf16 output [M][ldy]; may be null when yq is set (W4A4 only)
  int64_t ldy;
  int64_t M, N, K;
  uint8_t* yq;         // optional nvfp4 copy of Y for the next linear: packed E2M1 [M][N/2] (W4A4)
  uint8_t* ys;         // its E4M3 block scales [M][N/16]
  const float* gy;     // its global scale (the next linear's input_scale)
  float* ypmax;        // optional row maxima of |Y| per 64-column segment [M][ceil(N/64)], for an
                       // fp8r encoding of Y (tiled W4A4 kernel)
  // optional low-rank adapter: y += T B^T with T = s X A^T [M][rank] (bf16, scaled) and
  // B [N][rank] (bf16); lt == nullptr means none. The tiled W4A4 kernel instead takes
  // T / (gx gw) and adds T B^T to its accumulators before the K loop.
  const uint16_t* lt;
  const uint16_t* lb;
  int rank;
  int stream_y;        // write Y with non-temporal stores (set by the tiled launchers)
};
// whether the adapter's T must be divided by gx * gw for this W4A4 launch (tiled kernel)
bool lora_pre_scaled_w4a4(const DecArgs& a);
hipError_t launch_gemm_dec(DecMode mode, const DecArgs& a, hipStream_t s);
// W4A16 / W8A16 on the LDS-DMA pipeline with in-register weight decode (tiled shapes)
bool gemm_a16_supported(DecMode mode, const DecArgs& a);
hipError_t launch_gemm_a16(DecMode mode, const DecArgs& a, hipStream_t s);
// W4A4 on the LDS-DMA pipeline with in-register decode; needs K % 256 == 0
bool gemm_w4a4_supported(const DecArgs& a);
hipError_t launch_gemm_w4a4(const DecArgs& a, hipStream_t s);
// Grouped launches: the tiles of up to kMaxGroup independent GEMMs of one scheme in one grid
// (every problem with K % 256 == 0 for W4A4, K % 128 == 0 for fp8r). Problems are taken in the
// order given; callers put the longest K first so that the last round holds the short tiles.
constexpr int kMaxGroup = 8;
struct Fp8Problem {
  const uint8_t* xq;  // E4M3 activations [M][K]
  const float* sx;    // per-row activation scales [M]
  const uint8_t* w;   // E4M3 weights [N][K]
  const float* sw;    // per-row weight scales [N]
  uint16_t* y;        // bf16 output [M][ldy]
  int64_t ldy;
  int M, N, K;
  int stream_y;       // set by the launcher
};
bool gemm_fp8_grouped_supported(const Fp8Problem* p, int count);
hipError_t launch_gemm_fp8_grouped(const Fp8Problem* p, int count, hipStream_t s);
bool gemm_w4a4_grouped_supported(const DecArgs* p, int count);
hipError_t launch_gemm_w4a4_grouped(const DecArgs* p, int count, hipStream_t s);

// Few-token GEMMs: 32 weight rows per workgroup, K split over its 8 waves
bool gemm_skinny_supported(DecMode mode, const DecArgs& a);
hipError_t launch_gemm_skinny(DecMode mode, const DecArgs& a, hipStream_t s);
// Several few-token W4A4 or W8A8 GEMMs (no adapter, bf16 output) in one grid
bool gemm_skinny_grouped_supported(DecMode mode, const DecArgs* p, int count);
hipError_t launch_gemm_skinny_grouped(DecMode mode, const DecArgs* p, int count, hipStream_t s);

}  // namespace bsq

#include <atomic>

namespace bsq {
// Raise a kernel's dynamic-LDS limit once per device (the GEMMs use more than
// the 64 KB default; gfx950 has 160 KB per workgroup).
inline hipError_t ensure_lds_limit(const void* fn, int bytes, std::atomic<unsigned long long>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = 1ull << (dev & 63);
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}
}  // namespace bsq
