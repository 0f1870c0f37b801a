// C ABI of the block-scaled quantized linear layer (declared in include/bsq.h).
//
// Every entry point validates all of its arguments on the host before any
// HIP call, then checks (once per device) that the current device is gfx950,
// then enqueues its kernels on the caller's stream. Nothing here allocates,
// frees or synchronizes device memory.
#include "bsq.h"

#include <atomic>
#include <cmath>
#include <cstring>
#include <string>
#include <utility>

#include "bsq_launch.hpp"

namespace {

constexpr int64_t kMaxThreads = (int64_t)1 << 31;  // bound on work-items of any single launch
constexpr int kMaxDevices = 64;

thread_local std::string g_last_hip;

bsq_status hip_fail(hipError_t e) {
  g_last_hip = hipGetErrorString(e);
  return BSQ_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t pad256(size_t n) { return (n + 255) & ~(size_t)255; }

bsq_status check_device() {
  static std::atomic<int> state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return BSQ_ERR_DEVICE;
  }
  int st = state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) {
      (void)hipGetLastError();
      return BSQ_ERR_DEVICE;
    }
    st = std::strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? BSQ_OK : BSQ_ERR_DEVICE;
}

// shape rules shared by every entry point: K > 0, K % 32 == 0, rows >= 0,
// ld >= K and ld % 8 == 0
bsq_status check_rows(int64_t rows, int64_t K, int64_t ld) {
  if (rows < 0 || K <= 0 || K % 32 != 0 || K > (int64_t)1 << 20) return BSQ_ERR_SHAPE;
  if (ld < K || ld % 8 != 0) return BSQ_ERR_SHAPE;
  if (rows > 0 && rows > ((int64_t)1 << 62) / ld) return BSQ_ERR_SHAPE;
  return BSQ_OK;
}

size_t ws_fp8r(int64_t M, int64_t K) { return pad256((size_t)(M * K)) + pad256((size_t)(4 * M)); }
size_t ws_nvfp4(int64_t M, int64_t K) { return pad256((size_t)(M * K / 2)) + pad256((size_t)(M * K / 16)); }

bsq_status check_gemm_common(const uint16_t* x, int64_t ldx, const void* w, uint16_t* y, int64_t ldy,
                             int64_t M, int64_t N, int64_t K, uint32_t flags) {
  if (flags & ~BSQ_WEIGHT_ONLY) return BSQ_ERR_ARG;
  bsq_status st = check_rows(M, K, ldx);
  if (st != BSQ_OK) return st;
  if (N < 0 || N > ((int64_t)1 << 30) || M > ((int64_t)1 << 30)) return BSQ_ERR_SHAPE;
  if (ldy < N || (M > 0 && M > ((int64_t)1 << 62) / (ldy > 0 ? ldy : 1))) return BSQ_ERR_SHAPE;
  if (M == 0 || N == 0) return BSQ_OK;
  if (!x || !w || !y) return BSQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16)) return BSQ_ERR_ALIGN;
  if (M * (K / 16) >= kMaxThreads || N * (K / 16) >= kMaxThreads) return BSQ_ERR_SHAPE;
  return BSQ_OK;
}

// Few tokens: the skinny kernel (32 weight rows per workgroup, K split over its waves) keeps
// every compute unit streaming weights where the tiled kernels would leave most of them idle
// and walk K serially; with more rows the tiled kernels' operand reuse wins. Per scheme: the
// skinny kernel always runs up to `always` rows, and up to `most` rows while the tiled
// kernel would have fewer than 64 tiles of 128 x 128 (crossovers measured on MI355X with
// cold weights, K = 3072, N = 3072 and 12288, against the tiled kernels' small-grid tiles:
// at N = 12288 those win from 32 tokens (W4A4, W8A8) or 48 (W4A16, W8A16), at N = 3072 from
// 192 tokens).
struct SkinnyRule {
  int64_t always, most;
};
SkinnyRule skinny_rule(bsq::DecMode mode) {
  switch (mode) {
    case bsq::kW4A4: return {16, 128};
    case bsq::kW4A16: return {32, 128};
    case bsq::kW8A8: return {16, 128};
    default: return {32, 128};  // W8A16
  }
}
bool route_skinny(bsq::DecMode mode, const bsq::DecArgs& a) {
  const SkinnyRule r = skinny_rule(mode);
  const int64_t tiles = ((a.M + 127) / 128) * ((a.N + 127) / 128);
  const bool pick = a.M <= r.always || (a.M <= r.most && tiles < 64);
  return pick && bsq::gemm_skinny_supported(mode, a);
}
hipError_t launch_dec_or_skinny(bsq::DecMode mode, const bsq::DecArgs& a, hipStream_t s) {
  return route_skinny(mode, a) ? bsq::launch_gemm_skinny(mode, a, s) : bsq::launch_gemm_dec(mode, a, s);
}
hipError_t launch_w8a8(const uint8_t* xq, const float* sx, const uint8_t* w, const float* sw, uint16_t* y,
                       int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t s, const uint16_t* lt = nullptr,
                       const uint16_t* lb = nullptr, int rank = 0) {
  bsq::DecArgs a{};
  a.xq = xq; a.sx = sx; a.w = w; a.sw = sw; a.y = y; a.ldy = ldy; a.M = M; a.N = N; a.K = K;
  a.lt = lt; a.lb = lb; a.rank = rank;
  if (route_skinny(bsq::kW8A8, a)) return bsq::launch_gemm_skinny(bsq::kW8A8, a, s);
  return bsq::launch_gemm_fp8(xq, sx, w, sw, y, ldy, M, N, K, lt, lb, rank, s);
}

// ---- low-rank adapter ----------------------------------------------------------------
constexpr int64_t kMaxRank = 128;
// the down projection's output T [M][rank] bf16, then its fp32 partial products when K is sliced
size_t ws_lora_down(int64_t M, int64_t K, int64_t rank) {
  const int slices = bsq::lora_down_slices(M, K, (int)rank);
  return pad256((size_t)(M * rank * 2)) + (slices > 1 ? pad256((size_t)slices * (size_t)(M * rank * 4)) : 0);
}
float* lora_part(void* ws, int64_t M, int64_t rank) {
  return reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + pad256((size_t)(M * rank * 2)));
}
// T = bf16(s X A^T) alone (no encoding of X), by whichever kernel is faster at this shape
hipError_t lora_down_plain(const uint16_t* x, int64_t ldx, const uint16_t* a, int64_t M, int64_t K, int64_t rank,
                           float scale, uint16_t* t, float* part, hipStream_t s) {
  if (bsq::lora_down_rows_pick(M, K, (int)rank, bsq::kDownPlain))
    return bsq::launch_lora_down_rows(x, ldx, a, M, K, (int)rank, scale, nullptr, nullptr, t, bsq::RowsEncode{}, s);
  return bsq::launch_lora_down(x, ldx, a, M, K, (int)rank, scale, nullptr, nullptr, part, t, s);
}

// adapter rules on top of the linear's: rank, scale, pointers, and the 32-bit buffer offsets
// of the down-projection (32 rows of x) and up-projection (T and B rows) kernels
// (an empty call, M == 0 or N == 0, passes the shape and scale rules and touches no pointer)
bsq_status check_lora(int64_t ldx, const uint16_t* a, const uint16_t* b, int64_t rank, float scale, int64_t M,
                      int64_t N) {
  if (rank < 1 || rank > kMaxRank) return BSQ_ERR_SHAPE;
  if (ldx >= ((int64_t)1 << 24)) return BSQ_ERR_SHAPE;
  if (M * rank >= ((int64_t)1 << 29) || N * rank >= ((int64_t)1 << 29)) return BSQ_ERR_SHAPE;
  if (!std::isfinite(scale)) return BSQ_ERR_ARG;
  if (M == 0 || N == 0) return BSQ_OK;
  if (!a || !b) return BSQ_ERR_NULL;
  if (!aligned(a, 16) || !aligned(b, 16)) return BSQ_ERR_ALIGN;
  return BSQ_OK;
}

}  // namespace

extern "C" {

int bsq_abi_version(void) { return BSQ_ABI_VERSION; }

const char* bsq_status_string(bsq_status s) {
  switch (s) {
    case BSQ_OK: return "ok";
    case BSQ_ERR_NULL: return "null pointer";
    case BSQ_ERR_SHAPE: return "invalid shape or leading dimension";
    case BSQ_ERR_ALIGN: return "misaligned pointer";
    case BSQ_ERR_WORKSPACE: return "workspace missing or too small";
    case BSQ_ERR_DEVICE: return "no gfx950 device is current";
    case BSQ_ERR_HIP: return "HIP launch failed";
    case BSQ_ERR_ARG: return "invalid format or flags";
  }
  return "unknown status";
}

const char* bsq_last_hip_error(void) { return g_last_hip.c_str(); }

bsq_status bsq_quantize_act_fp8r(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* xq,
                                 float* x_scale, hipStream_t stream) {
  bsq_status st = check_rows(M, K, ldx);
  if (st != BSQ_OK) return st;
  if (M == 0) return BSQ_OK;
  if (!x || !xq || !x_scale) return BSQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(x_scale, 4)) return BSQ_ERR_ALIGN;
  if (M * 64 >= kMaxThreads) return BSQ_ERR_SHAPE;
  if ((st = check_device()) != BSQ_OK) return st;
  hipError_t e = bsq::launch_quant_fp8r(x, M, K, ldx, xq, x_scale, stream);
  return e == hipSuccess ? BSQ_OK : hip_fail(e);
}

bsq_status bsq_quantize_act_nvfp4(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                  const float* global_scale, uint8_t* xq, uint8_t* x_bscale,
                                  hipStream_t stream) {
  bsq_status st = check_rows(M, K, ldx);
  if (st != BSQ_OK) return st;
  if (M == 0) return BSQ_OK;
  if (!x || !global_scale || !xq || !x_bscale) return BSQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(global_scale, 4) || !aligned(xq, 16) || !aligned(x_bscale, 4))
    return BSQ_ERR_ALIGN;
  if (M * (K / 16) >= kMaxThreads) return BSQ_ERR_SHAPE;
  if ((st = check_device()) != BSQ_OK) return st;
  hipError_t e = bsq::launch_quant_nvfp4(x, M, K, ldx, global_scale, xq, x_bscale, stream);
  return e == hipSuccess ? BSQ_OK : hip_fail(e);
}

size_t bsq_calibrate_workspace_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0) return 0;
  return pad256(4 * (size_t)bsq::calibrate_partials(M));
}

bsq_status bsq_calibrate_global_scale(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, float* out_scale,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  bsq_status st = check_rows(M, K, ldx);
  if (st != BSQ_OK) return st;
  if (M == 0) return BSQ_ERR_SHAPE;
  if (!x || !out_scale) return BSQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(out_scale, 4)) return BSQ_ERR_ALIGN;
  if (!workspace || workspace_bytes < bsq_calibrate_workspace_bytes(M, K) || !aligned(workspace, 4))
    return BSQ_ERR_WORKSPACE;
  if ((st = check_device()) != BSQ_OK) return st;
  hipError_t e = bsq::launch_calibrate(x, M, K, ldx, out_scale, static_cast<float*>(workspace), stream);
  return e == hipSuccess ? BSQ_OK : hip_fail(e);
}

size_t bsq_gemm_workspace_bytes(bsq_format f, int64_t M, int64_t N, int64_t K, uint32_t flags) {
  (void)N;
  if ((flags & BSQ_WEIGHT_ONLY) || M <= 0 || K <= 0) return 0;
  if (f == BSQ_FMT_FP8R) return ws_fp8r(M, K);
  if (f == BSQ_FMT_NVFP4) return ws_nvfp4(M, K);
  return 0;
}

bsq_status bsq_gemm_fp8r(const uint16_t* x, int64_t ldx, const uint8_t* w, const float* w_scale, uint16_t* y,
                         int64_t ldy, int64_t M, int64_t N, int64_t K, uint32_t flags, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  bsq_status st = check_gemm_common(x, ldx, w, y, ldy, M, N, K, flags);
  if (st != BSQ_OK || M == 0 || N == 0) return st;
  if (!w_scale) return BSQ_ERR_NULL;
  if (!aligned(w_scale, 4)) return BSQ_ERR_ALIGN;
  const bool weight_only = flags & BSQ_WEIGHT_ONLY;
  if (!weight_only) {
    if (!workspace || workspace_bytes < ws_fp8r(M, K)) return BSQ_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return BSQ_ERR_ALIGN;
  }
  if ((st = check_device()) != BSQ_OK) return st;
  hipError_t e;
  if (weight_only) {
    bsq::DecArgs a{};
    a.x = x; a.ldx = ldx; a.w = w; a.sw = w_scale; a.y = y; a.ldy = ldy; a.M = M; a.N = N; a.K = K;
    e = launch_dec_or_skinny(bsq::kW8A16, a, stream);
  } else {
    uint8_t* xq = static_cast<uint8_t*>(workspace);
    float* sx = reinterpret_cast<float*>(xq + pad256((size_t)(M * K)));
    e = bsq::launch_quant_fp8r(x, M, K, ldx, xq, sx, stream);
    if (e == hipSuccess) e = launch_w8a8(xq, sx, w, w_scale, y, ldy, M, N, K, stream);
  }
  return e == hipSuccess ? BSQ_OK : hip_fail(e);
}

static_assert(BSQ_NOALLOC_MAX_BYTES == bsq::kScratchBytes, "the header states the scratch size");

bsq_status bsq_gemm_fp8r_noalloc(const uint16_t* x, int64_t ldx, const uint8_t* w, const float* w_scale,
                                 uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, uint32_t flags,
                                 hipStream_t stream) {
  bsq_status st = check_gemm_common(x, ldx, w, y, ldy, M, N, K, flags);
  if (st != BSQ_OK || M == 0 || N == 0) return st;
  if (!w_scale) return BSQ_ERR_NULL;
  if (!aligned(w_scale, 4)) return BSQ_ERR_ALIGN;
  const bool weight_only = flags & BSQ_WEIGHT_ONLY;
  if (!weight_only && ws_fp8r(M, K) > bsq::kScratchBytes) return BSQ_ERR_WORKSPACE;
  if ((st = check_device()) != BSQ_OK) return st;
  if (weight_only)  // no scratch needed: the plain entry point allocates nothing either
    return bsq_gemm_fp8r(x, ldx, w, w_scale, y, ldy, M, N, K, flags, nullptr, 0, stream);
  void* ws = nullptr;
  hipError_t e = bsq::scratch_buffer(&ws);
  if (e != hipSuccess) return hip_fail(e);
  // the same launches as bsq_gemm_fp8r with the library's scratch as its workspace: the
  // quantizer overwrites every byte the GEMM reads, so nothing needs clearing
  uint8_t* xq = static_cast<uint8_t*>(ws);
  float* sx = reinterpret_cast<float*>(xq + pad256((size_t)(M * K)));
  e = bsq::launch_quant_fp8r(x, M, K, ldx, xq, sx, stream);
  if (e == hipSuccess) e = launch_w8a8(xq, sx, w, w_scale, y, ldy, M, N, K, stream);
  return e == hipSuccess ? BSQ_OK : hip_fail(e);
}

bsq_status bsq_gemm_nvfp4(const uint16_t* x, int64_t ldx, const uint8_t* w, const uint8_t* w_bscale,
                          const float* w_scale2, const float* input_scale, uint16_t* y, int64_t ldy, int64_t M,
                          int64_t N, int64_t K, uint32_t flags, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  bsq_status st = check_gemm_common(x, ldx, w, y, ldy, M, N, K, flags);
  if (st != BSQ_OK || M == 0 || N == 0) return st;
  const bool weight_only = flags & BSQ_WEIGHT_ONLY;
  if (!w_bscale || !w_scale2 || (!weight_only && !input_scale)) return BSQ_ERR_NULL;
  if (!aligned(w_bscale, 4) || !aligned(w_scale2, 4) || (input_scale && !aligned(input_scale, 4)))
    return BSQ_ERR_ALIGN;
  if (!weight_only) {
    if (!workspace || workspace_bytes < ws_nvfp4(M, K)) return BSQ_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return BSQ_ERR_ALIGN;
  }
  if ((st = check_device()) != BSQ_OK) return st;
  bsq::DecArgs a{};
  a.x = x; a.ldx = ldx; a.w = w; a.ws = w_bscale; a.gw = w_scale2; a.y = y; a.ldy = ldy;
  a.M = M; a.N = N; a.K = K;
  hipError_t e;
  if (weight_only) {
    e = launch_dec_or_skinny(bsq::kW4A16, a, stream);
  } else {
    uint8_t* xq = static_cast<uint8_t*>(workspace);
    uint8_t* xs = xq + pad256((size_t)(M * K / 2));
    a.xq = xq; a.xs = xs; a.gx = input_scale;
    e = bsq::launch_quant_nvfp4(x, M, K, ldx, input_scale, xq, xs, stream);
    if (e == hipSuccess) e = launch_dec_or_skinny(bsq::kW4A4, a, stream);
  }
  return e == hipSuccess ? BSQ_OK : hip_fail(e);
}

namespace {
// argument checks of the pre-quantized W8A8 and W4A4 linears (also per problem of a grouped
// launch); empty shapes pass without looking at any pointer
bsq_status check_fp8r_q(const uint8_t* xq, const float* x_scale, const uint8_t* w, const float* w_scale,
                        uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K) {
  // xq rows are dense (ld = K); reuse the common checks with ldx = K
  bsq_status st = check_gemm_common(reinterpret_cast<const uint16_t*>(xq), K, w, y, ldy, M, N, K, 0);
  if (st != BSQ_OK || M == 0 || N == 0) return st;
  if (!x_scale || !w_scale) return BSQ_ERR_NULL;
  if (!aligned(x_scale, 4) || !aligned(w_scale, 4)) return BSQ_ERR_ALIGN;
  return BSQ_OK;
}
bsq_status check_nvfp4_q(const uint8_t* xq, const uint8_t* x_bscale, const float* input_scale, const uint8_t* w,
                         const uint8_t* w_bscale, const float* w_scale2, uint16_t* y, int64_t ldy, int64_t M,
                         int64_t N, int64_t K) {
  bsq_status st = check_gemm_common(reinterpret_cast<const uint16_t*>(xq), K, w, y, ldy, M, N, K, 0);
  if (st != BSQ_OK || M == 0 || N == 0) return st;
  if (!x_bscale || !input_scale || !w_bscale || !w_scale2) return BSQ_ERR_NULL;
  if (!aligned(x_bscale, 4) || !aligned(input_scale, 4) || !aligned(w_bscale, 4) || !aligned(w_scale2, 4))
    return BSQ_ERR_ALIGN;
  return BSQ_OK;
}
}  // namespace

bsq_status bsq_gemm_fp8r_q(const uint8_t* xq, const float* x_scale, const uint8_t* w, const float* w_scale,
                           uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  bsq_status st = check_fp8r_q(xq, x_scale, w, w_scale, y, ldy, M, N, K);
  if (st != BSQ_OK || M == 0 || N == 0) return st;
  if ((st = check_device()) != BSQ_OK) return st;
  hipError_t e = launch_w8a8(xq, x_scale, w, w_scale, y, ldy, M, N, K, stream);
  return e == hipSuccess ? BSQ_OK : hip_fail(e);
}

bsq_status bsq_gemm_nvfp4_q(const uint8_t* xq, const uint8_t* x_bscale, const float* input_scale,
                            const uint8_t* w, const uint8_t* w_bscale, const float* w_scale2, uint16_t* y,
                            int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  bsq_status st = check_nvfp4_q(xq, x_bscale, input_scale, w, w_bscale, w_scale2, y, ldy, M, N, K);
  if (st != BSQ_OK || M == 0 || N == 0) return st;
  if ((st = check_device()) != BSQ_OK) return st;
  bsq::DecArgs a{};
  a.xq = xq; a.xs = x_bscale; a.gx = input_scale; a.w = w; a.ws = w_bscale; a.gw = w_scale2;
  a.y = y; a.ldy = ldy; a.M = M; a.N = N; a.K = K;
  hipError_t e = launch_dec_or_skinny(bsq::kW4A4, a, stream);
  return e == hipSuccess ? BSQ_OK : hip_fail(e);
}

static_assert(BSQ_MAX_GROUP == bsq::kMaxGroup, "the header states the group limit");

bsq_status bsq_gemm_grouped_weight_only(bsq_format format, const bsq_weight_only_problem* problems, int count,
                                        hipStream_t stream) {
  if (format != BSQ_FMT_FP8R && format != BSQ_FMT_NVFP4) return BSQ_ERR_ARG;
  if (count < 0 || count > BSQ_MAX_GROUP) return BSQ_ERR_ARG;
  if (count == 0) return BSQ_OK;
  if (!problems) return BSQ_ERR_NULL;
  const bool fp8 = format == BSQ_FMT_FP8R;
  // every problem is checked (as the single weight-only calls check it) before anything is enqueued
  int order[BSQ_MAX_GROUP], n = 0;
  for (int i = 0; i < count; ++i) {
    const bsq_weight_only_problem& p = problems[i];
    if (fp8 && p.w_scale2) return BSQ_ERR_ARG;
    bsq_status st = check_gemm_common(p.x, p.ldx, p.w, p.y, p.ldy, p.M, p.N, p.K, BSQ_WEIGHT_ONLY);
    if (st != BSQ_OK) return st;
    if (p.M == 0 || p.N == 0) continue;
    if (!p.w_scale || (!fp8 && !p.w_scale2)) return BSQ_ERR_NULL;
    if (!aligned(p.w_scale, 4) || (p.w_scale2 && !aligned(p.w_scale2, 4))) return BSQ_ERR_ALIGN;
    order[n++] = i;
  }
  if (n == 0) return BSQ_OK;
  bsq_status st = check_device();
  if (st != BSQ_OK) return st;
  for (int i = 1; i < n; ++i)  // longest K first (stable)
    for (int j = i; j > 0 && problems[order[j]].K > problems[order[j - 1]].K; --j) std::swap(order[j], order[j - 1]);
  const bsq::DecMode mode = fp8 ? bsq::kW8A16 : bsq::kW4A16;
  auto args = [&](const bsq_weight_only_problem& p) {
    bsq::DecArgs a{};
    a.x = p.x; a.ldx = p.ldx; a.w = p.w; a.y = p.y; a.ldy = p.ldy; a.M = p.M; a.N = p.N; a.K = p.K;
    if (fp8) {
      a.sw = static_cast<const float*>(p.w_scale);
    } else {
      a.ws = static_cast<const uint8_t*>(p.w_scale); a.gw = p.w_scale2;
    }
    return a;
  };
  bsq::DecArgs q[BSQ_MAX_GROUP];
  int few = 0;
  for (int i = 0; i < n; ++i) {
    q[i] = args(problems[order[i]]);
    few += route_skinny(mode, q[i]) ? 1 : 0;
  }
  hipError_t e = hipSuccess;
  if (few == n && bsq::gemm_skinny_grouped_supported(mode, q, n)) {
    e = bsq::launch_gemm_skinny_grouped(mode, q, n, stream);
  } else {
    for (int i = 0; i < count && e == hipSuccess; ++i)
      if (problems[i].M > 0 && problems[i].N > 0) e = launch_dec_or_skinny(mode, args(problems[i]), stream);
  }
  return e == hipSuccess ? BSQ_OK : hip_fail(e);
}

bsq_status bsq_gemm_grouped_q(bsq_format format, const bsq_gemm_problem* problems, int count, hipStream_t stream) {
  if (format != BSQ_FMT_FP8R && format != BSQ_FMT_NVFP4) return BSQ_ERR_ARG;
  if (count < 0 || count > BSQ_MAX_GROUP) return BSQ_ERR_ARG;
  if (count == 0) return BSQ_OK;
  if (!problems) return BSQ_ERR_NULL;
  const bool fp8 = format == BSQ_FMT_FP8R;
  // every problem is checked before anything is enqueued; empty ones are dropped
  int order[BSQ_MAX_GROUP], n = 0;
  for (int i = 0; i < count; ++i) {
    const bsq_gemm_problem& p = problems[i];
    bsq_status st;
    if (fp8) {
      if (p.input_scale || p.w_scale2) return BSQ_ERR_ARG;
      st = check_fp8r_q(p.xq, static_cast<const float*>(p.x_scale), p.w, static_cast<const float*>(p.w_scale), p.y,
                        p.ldy, p.M, p.N, p.K);
    } else {
      st = check_nvfp4_q(p.xq, static_cast<const uint8_t*>(p.x_scale), p.input_scale, p.w,
                         static_cast<const uint8_t*>(p.w_scale), p.w_scale2, p.y, p.ldy, p.M, p.N, p.K);
    }
    if (st != BSQ_OK) return st;
    if (p.M > 0 && p.N > 0) order[n++] = i;
  }
  if (n == 0) return BSQ_OK;
  bsq_status st = check_device();
  if (st != BSQ_OK) return st;
  // longest K first (stable), so the grid's last round holds the shortest tiles
  for (int i = 1; i < n; ++i)
    for (int j = i; j > 0 && problems[order[j]].K > problems[order[j - 1]].K; --j) std::swap(order[j], order[j - 1]);
  // the problems as the single entry points see them
  const bsq::DecMode mode = fp8 ? bsq::kW8A8 : bsq::kW4A4;
  auto args = [&](const bsq_gemm_problem& p) {
    bsq::DecArgs a{};
    a.xq = p.xq; a.w = p.w; a.y = p.y; a.ldy = p.ldy; a.M = p.M; a.N = p.N; a.K = p.K;
    if (fp8) {
      a.sx = static_cast<const float*>(p.x_scale); a.sw = static_cast<const float*>(p.w_scale);
    } else {
      a.xs = static_cast<const uint8_t*>(p.x_scale); a.gx = p.input_scale;
      a.ws = static_cast<const uint8_t*>(p.w_scale); a.gw = p.w_scale2;
    }
    return a;
  };
  bsq::DecArgs q[BSQ_MAX_GROUP];
  int few = 0;  // problems on the few-token route
  for (int i = 0; i < n; ++i) {
    q[i] = args(problems[order[i]]);
    few += route_skinny(mode, q[i]) ? 1 : 0;
  }
  // one grid when every problem takes the same route and the grouped kernels cover the group
  hipError_t e = hipSuccess;
  bool done = false;
  // Up to 64 tokens the few-token grid also serves a group whose larger problems alone would take
  // the tiled kernels: a joint block's four linears (cold weights) at 32 / 64 tokens as one
  // few-token grid against four launches, nvfp4 33.0 / 50.0 vs 71.8 / 60.2 us, fp8r 32.6 / 46.8
  // vs 49.3 / 50.4 us (at 96 and 128 tokens the launches win: 83 / 85 vs 96 / 106 us nvfp4).
  int64_t mmax = 0;
  for (int i = 0; i < n; ++i) mmax = q[i].M > mmax ? q[i].M : mmax;
  if ((few == n || (few > 0 && mmax <= 64)) && bsq::gemm_skinny_grouped_supported(mode, q, n)) {
    e = bsq::launch_gemm_skinny_grouped(mode, q, n, stream);
    done = true;
  } else if (few == 0 && fp8) {
    bsq::Fp8Problem f[BSQ_MAX_GROUP];
    for (int i = 0; i < n; ++i)
      f[i] = bsq::Fp8Problem{q[i].xq, q[i].sx, q[i].w, q[i].sw, q[i].y, q[i].ldy, (int)q[i].M, (int)q[i].N,
                             (int)q[i].K, 0};
    if (bsq::gemm_fp8_grouped_supported(f, n)) {
      e = bsq::launch_gemm_fp8_grouped(f, n, stream);
      done = true;
    }
  } else if (few == 0 && bsq::gemm_w4a4_grouped_supported(q, n)) {
    e = bsq::launch_gemm_w4a4_grouped(q, n, stream);
    done = true;
  }
  // otherwise one launch per problem, in the order given
  for (int i = 0; i < count && !done && e == hipSuccess; ++i) {
    const bsq_gemm_problem& p = problems[i];
    if (p.M == 0 || p.N == 0) continue;
    if (fp8)
      e = launch_w8a8(p.xq, static_cast<const float*>(p.x_scale), p.w, static_cast<const float*>(p.w_scale), p.y,
                      p.ldy, p.M, p.N, p.K, stream);
    else
      e = launch_dec_or_skinny(bsq::kW4A4, args(p), stream);
  }
  return e == hipSuccess ? BSQ_OK : hip_fail(e);
}

size_t bsq_gemm_nvfp4_quantize_y_workspace_bytes(int64_t M, int64_t N, int64_t K, int with_y) {
  if (with_y || M <= 0 || N <= 0 || K <= 0) return 0;
  bsq::DecArgs a{};
  a.M = M; a.N = N; a.K = K;
  if (route_skinny(bsq::kW4A4, a) || bsq::gemm_w4a4_supported(a)) return 0;
  return pad256((size_t)M * (size_t)N * 2);
}

bsq_status bsq_gemm_nvfp4_q_quantize_y(const uint8_t* xq, const uint8_t* x_bscale, const float* input_scale,
                                       const uint8_t* w, const uint8_t* w_bscale, const float* w_scale2,
                                       const float* y_scale, uint8_t* yq, uint8_t* y_bscale, uint16_t* y,
                                       int64_t ldy, int64_t M, int64_t N, int64_t K, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  // without a bf16 output the shape is checked as for a dense [M][N] one, with yq standing in
  bsq_status st = check_gemm_common(reinterpret_cast<const uint16_t*>(xq), K, w,
                                    y ? y : reinterpret_cast<uint16_t*>(yq), y ? ldy : N, M, N, K, 0);
  if (st != BSQ_OK) return st;
  if (N % 32 != 0 || (y && ldy % 8 != 0)) return BSQ_ERR_SHAPE;
  if (M == 0 || N == 0) return BSQ_OK;
  if (!x_bscale || !input_scale || !w_bscale || !w_scale2 || !y_scale || !yq || !y_bscale) return BSQ_ERR_NULL;
  if (!aligned(x_bscale, 4) || !aligned(input_scale, 4) || !aligned(w_bscale, 4) || !aligned(w_scale2, 4) ||
      !aligned(y_scale, 4) || !aligned(yq, 16))
    return BSQ_ERR_ALIGN;
  if (M * (N / 16) >= kMaxThreads) return BSQ_ERR_SHAPE;
  bsq::DecArgs a{};
  a.xq = xq; a.xs = x_bscale; a.gx = input_scale; a.w = w; a.ws = w_bscale; a.gw = w_scale2;
  a.y = y; a.ldy = ldy; a.M = M; a.N = N; a.K = K;
  a.yq = yq; a.ys = y_bscale; a.gy = y_scale;
  const bool fused = route_skinny(bsq::kW4A4, a) || bsq::gemm_w4a4_supported(a);
  uint16_t* ybuf = y;
  int64_t ldb = ldy;
  if (!fused && !y) {
    if (!workspace || workspace_bytes < bsq_gemm_nvfp4_quantize_y_workspace_bytes(M, N, K, 0) ||
        !aligned(workspace, 16))
      return BSQ_ERR_WORKSPACE;
    ybuf = static_cast<uint16_t*>(workspace);
    ldb = N;
  }
  if ((st = check_device()) != BSQ_OK) return st;
  hipError_t e;
  if (route_skinny(bsq::kW4A4, a)) {
    e = bsq::launch_gemm_skinny(bsq::kW4A4, a, stream);
  } else if (fused) {
    e = bsq::launch_gemm_w4a4(a, stream);
  } else {
    // unfused: bf16 Y (into y or the workspace), then the activation quantizer over it
    a.y = ybuf; a.ldy = ldb; a.yq = nullptr; a.ys = nullptr; a.gy = nullptr;
    e = bsq::launch_gemm_dec(bsq::kW4A4, a, stream);
    if (e == hipSuccess) e = bsq::launch_quant_nvfp4(ybuf, M, N, ldb, y_scale, yq, y_bscale, stream);
  }
  return e == hipSuccess ? BSQ_OK : hip_fail(e);
}

size_t bsq_gemm_quantize_y_workspace_bytes(bsq_format out_format, int64_t M, int64_t N, int with_y) {
  if ((out_format != BSQ_FMT_FP8R && out_format != BSQ_FMT_NVFP4) || M <= 0 || N <= 0) return 0;
  size_t n = with_y ? 0 : pad256((size_t)M * (size_t)N * 2);  // bf16 Y when the caller takes none
  if (out_format == BSQ_FMT_FP8R) n += pad256((size_t)bsq::ypmax_segments(N) * (size_t)M * 4);
  return n;
}

namespace {
// shared checks of the quantized-output entry points; on success *ybuf / *ldb / *pmax point at
// where the bf16 Y and the fp8r row maxima go
bsq_status check_quantize_y(bsq_format out_format, const float* y_global, uint8_t* yq, void* yq_scale, uint16_t* y,
                            int64_t ldy, int64_t M, int64_t N, void* workspace, size_t workspace_bytes,
                            uint16_t** ybuf, int64_t* ldb, float** pmax) {
  if (out_format != BSQ_FMT_FP8R && out_format != BSQ_FMT_NVFP4) return BSQ_ERR_ARG;
  if (out_format == BSQ_FMT_FP8R && y_global) return BSQ_ERR_ARG;
  if (N % 32 != 0 || (y && ldy % 8 != 0)) return BSQ_ERR_SHAPE;
  if (M == 0 || N == 0) return BSQ_OK;
  if (!yq || !yq_scale || (out_format == BSQ_FMT_NVFP4 && !y_global)) return BSQ_ERR_NULL;
  if (!aligned(yq, 16) || !aligned(yq_scale, 4) || (y_global && !aligned(y_global, 4))) return BSQ_ERR_ALIGN;
  if (M * (N / 16) >= kMaxThreads) return BSQ_ERR_SHAPE;
  const size_t need = bsq_gemm_quantize_y_workspace_bytes(out_format, M, N, y != nullptr);
  if (need && (!workspace || workspace_bytes < need)) return BSQ_ERR_WORKSPACE;
  if (need && !aligned(workspace, 256)) return BSQ_ERR_ALIGN;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  *ybuf = y;
  *ldb = ldy;
  if (!y) {
    *ybuf = reinterpret_cast<uint16_t*>(ws);
    *ldb = N;
    ws += pad256((size_t)M * (size_t)N * 2);
  }
  *pmax = out_format == BSQ_FMT_FP8R ? reinterpret_cast<float*>(ws) : nullptr;
  return BSQ_OK;
}

// the next linear's encoding of a bf16 Y already in memory (routes without a fused epilogue)
hipError_t quantize_y_after(bsq_format out_format, const uint16_t* ybuf, int64_t ldb, int64_t M, int64_t N,
                            const float* y_global, uint8_t* yq, void* yq_scale, hipStream_t stream) {
  if (out_format == BSQ_FMT_NVFP4)
    return bsq::launch_quant_nvfp4(ybuf, M, N, ldb, y_global, yq, static_cast<uint8_t*>(yq_scale), stream);
  return bsq::launch_quant_fp8r(ybuf, M, N, ldb, yq, static_cast<float*>(yq_scale), stream);
}
}  // namespace

bsq_status bsq_gemm_fp8r_q_quantize_y(const uint8_t* xq, const float* x_scale, const uint8_t* w, const float* w_scale,
                                      bsq_format out_format, const float* y_global, uint8_t* yq, void* yq_scale,
                                      uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  // without a bf16 output the shape is checked as for a dense [M][N] one, with yq standing in
  bsq_status st = check_gemm_common(reinterpret_cast<const uint16_t*>(xq), K, w,
                                    y ? y : reinterpret_cast<uint16_t*>(yq), y ? ldy : N, M, N, K, 0);
  if (st != BSQ_OK) return st;
  uint16_t* ybuf = nullptr;
  int64_t ldb = 0;
  float* pmax = nullptr;
  st = check_quantize_y(out_format, y_global, yq, yq_scale, y, ldy, M, N, workspace, workspace_bytes, &ybuf, &ldb,
                        &pmax);
  if (st != BSQ_OK || M == 0 || N == 0) return st;
  if (!x_scale || !w_scale) return BSQ_ERR_NULL;
  if (!aligned(x_scale, 4) || !aligned(w_scale, 4)) return BSQ_ERR_ALIGN;
  if ((st = check_device()) != BSQ_OK) return st;
  bsq::DecArgs a{};
  a.xq = xq; a.sx = x_scale; a.w = w; a.sw = w_scale; a.M = M; a.N = N; a.K = K;
  hipError_t e;
  if (route_skinny(bsq::kW8A8, a)) {  // few tokens: the GEMM, then the quantizer over its Y
    a.y = ybuf; a.ldy = ldb;
    e = bsq::launch_gemm_skinny(bsq::kW8A8, a, stream);
    if (e == hipSuccess) e = quantize_y_after(out_format, ybuf, ldb, M, N, y_global, yq, yq_scale, stream);
  } else if (out_format == BSQ_FMT_NVFP4) {  // encoded in the epilogue; bf16 Y only if asked for
    bsq::YQuant q;
    q.yq = yq; q.ys = static_cast<uint8_t*>(yq_scale); q.gy = y_global;
    e = bsq::launch_gemm_fp8(xq, x_scale, w, w_scale, y, ldy, M, N, K, nullptr, nullptr, 0, stream, &q);
  } else {  // row maxima in the epilogue, then the encoding pass over Y
    bsq::YQuant q;
    q.pmax = pmax;
    e = bsq::launch_gemm_fp8(xq, x_scale, w, w_scale, ybuf, ldb, M, N, K, nullptr, nullptr, 0, stream, &q);
    if (e == hipSuccess)
      e = bsq::launch_encode_fp8r_rows(ybuf, M, N, ldb, pmax, yq, static_cast<float*>(yq_scale), stream);
  }
  return e == hipSuccess ? BSQ_OK : hip_fail(e);
}

bsq_status bsq_gemm_nvfp4_q_quantize_y_fp8r(const uint8_t* xq, const uint8_t* x_bscale, const float* input_scale,
                                            const uint8_t* w, const uint8_t* w_bscale, const float* w_scale2,
                                            uint8_t* yq, float* y_rowscale, uint16_t* y, int64_t ldy, int64_t M,
                                            int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                                            hipStream_t stream) {
  bsq_status st = check_gemm_common(reinterpret_cast<const uint16_t*>(xq), K, w,
                                    y ? y : reinterpret_cast<uint16_t*>(yq), y ? ldy : N, M, N, K, 0);
  if (st != BSQ_OK) return st;
  uint16_t* ybuf = nullptr;
  int64_t ldb = 0;
  float* pmax = nullptr;
  st = check_quantize_y(BSQ_FMT_FP8R, nullptr, yq, y_rowscale, y, ldy, M, N, workspace, workspace_bytes, &ybuf, &ldb,
                        &pmax);
  if (st != BSQ_OK || M == 0 || N == 0) return st;
  if (!x_bscale || !input_scale || !w_bscale || !w_scale2) return BSQ_ERR_NULL;
  if (!aligned(x_bscale, 4) || !aligned(input_scale, 4) || !aligned(w_bscale, 4) || !aligned(w_scale2, 4))
    return BSQ_ERR_ALIGN;
  if ((st = check_device()) != BSQ_OK) return st;
  bsq::DecArgs a{};
  a.xq = xq; a.xs = x_bscale; a.gx = input_scale; a.w = w; a.ws = w_bscale; a.gw = w_scale2;
  a.y = ybuf; a.ldy = ldb; a.M = M; a.N = N; a.K = K;
  hipError_t e;
  if (!route_skinny(bsq::kW4A4, a) && bsq::gemm_w4a4_supported(a)) {  // row maxima in the epilogue
    a.ypmax = pmax;
    e = bsq::launch_gemm_w4a4(a, stream);
    if (e == hipSuccess) e = bsq::launch_encode_fp8r_rows(ybuf, M, N, ldb, pmax, yq, y_rowscale, stream);
  } else {
    e = launch_dec_or_skinny(bsq::kW4A4, a, stream);
    if (e == hipSuccess) e = quantize_y_after(BSQ_FMT_FP8R, ybuf, ldb, M, N, nullptr, yq, y_rowscale, stream);
  }
  return e == hipSuccess ? BSQ_OK : hip_fail(e);
}

bsq_status bsq_gemm_weight_only_quantize_y(bsq_format w_format, const uint16_t* x, int64_t ldx, const uint8_t* w,
                                           const void* w_scale, const float* w_scale2, bsq_format out_format,
                                           const float* y_global, uint8_t* yq, void* yq_scale, uint16_t* y,
                                           int64_t ldy, int64_t M, int64_t N, int64_t K, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream) {
  if (w_format != BSQ_FMT_FP8R && w_format != BSQ_FMT_NVFP4) return BSQ_ERR_ARG;
  if (w_format == BSQ_FMT_FP8R && w_scale2) return BSQ_ERR_ARG;
  // without a bf16 output the shape is checked as for a dense [M][N] one, with yq standing in
  bsq_status st = check_gemm_common(x, ldx, w, y ? y : reinterpret_cast<uint16_t*>(yq), y ? ldy : N, M, N, K, 0);
  if (st != BSQ_OK) return st;
  uint16_t* ybuf = nullptr;
  int64_t ldb = 0;
  float* pmax = nullptr;
  st = check_quantize_y(out_format, y_global, yq, yq_scale, y, ldy, M, N, workspace, workspace_bytes, &ybuf, &ldb,
                        &pmax);
  if (st != BSQ_OK || M == 0 || N == 0) return st;
  if (!w_scale || (w_format == BSQ_FMT_NVFP4 && !w_scale2)) return BSQ_ERR_NULL;
  if (!aligned(w_scale, 4) || (w_scale2 && !aligned(w_scale2, 4))) return BSQ_ERR_ALIGN;
  if ((st = check_device()) != BSQ_OK) return st;
  const bsq::DecMode mode = w_format == BSQ_FMT_NVFP4 ? bsq::kW4A16 : bsq::kW8A16;
  bsq::DecArgs a{};
  a.x = x; a.ldx = ldx; a.w = w; a.M = M; a.N = N; a.K = K;
  if (mode == bsq::kW4A16) {
    a.ws = static_cast<const uint8_t*>(w_scale);
    a.gw = w_scale2;
  } else {
    a.sw = static_cast<const float*>(w_scale);
  }
  hipError_t e;
  if (!route_skinny(mode, a) && bsq::gemm_a16_supported(mode, a)) {
    if (out_format == BSQ_FMT_NVFP4) {  // encoded in the tiled epilogue; bf16 Y only if asked for
      a.y = y; a.ldy = ldy;
      a.yq = yq; a.ys = static_cast<uint8_t*>(yq_scale); a.gy = y_global;
      e = bsq::launch_gemm_a16(mode, a, stream);
    } else {  // row maxima in the epilogue, then the encoding pass over Y
      a.y = ybuf; a.ldy = ldb; a.ypmax = pmax;
      e = bsq::launch_gemm_a16(mode, a, stream);
      if (e == hipSuccess)
        e = bsq::launch_encode_fp8r_rows(ybuf, M, N, ldb, pmax, yq, static_cast<float*>(yq_scale), stream);
    }
  } else {  // few tokens or the decode GEMM: bf16 Y, then the quantizer over it
    a.y = ybuf; a.ldy = ldb;
    e = launch_dec_or_skinny(mode, a, stream);
    if (e == hipSuccess) e = quantize_y_after(out_format, ybuf, ldb, M, N, y_global, yq, yq_scale, stream);
  }
  return e == hipSuccess ? BSQ_OK : hip_fail(e);
}

size_t bsq_lora_workspace_bytes(bsq_format f, int64_t M, int64_t N, int64_t K, int64_t rank, uint32_t flags) {
  if ((f != BSQ_FMT_FP8R && f != BSQ_FMT_NVFP4) || M <= 0 || K <= 0 || rank <= 0) return 0;
  return bsq_gemm_workspace_bytes(f, M, N, K, flags) + ws_lora_down(M, K, rank);
}

size_t bsq_lora_down_workspace_bytes(int64_t M, int64_t K, int64_t rank) {
  if (M <= 0 || K <= 0 || rank <= 0) return 0;
  const int slices = bsq::lora_down_slices(M, K, (int)rank);
  return slices > 1 ? pad256((size_t)slices * (size_t)(M * rank * 4)) : 0;
}

bsq_status bsq_lora_down(const uint16_t* x, int64_t ldx, const uint16_t* lora_a, int64_t M, int64_t K,
                         int64_t rank, float lora_scale, uint16_t* t, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  bsq_status st = check_rows(M, K, ldx);
  if (st != BSQ_OK) return st;
  if (rank < 1 || rank > kMaxRank || ldx >= ((int64_t)1 << 24) || M * rank >= ((int64_t)1 << 29))
    return BSQ_ERR_SHAPE;
  if (!std::isfinite(lora_scale)) return BSQ_ERR_ARG;
  if (M == 0) return BSQ_OK;
  if (!x || !lora_a || !t) return BSQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(lora_a, 16) || !aligned(t, 16)) return BSQ_ERR_ALIGN;
  const size_t need = bsq_lora_down_workspace_bytes(M, K, rank);
  if (need && (!workspace || workspace_bytes < need)) return BSQ_ERR_WORKSPACE;
  if (need && !aligned(workspace, 16)) return BSQ_ERR_ALIGN;
  if ((st = check_device()) != BSQ_OK) return st;
  hipError_t e = lora_down_plain(x, ldx, lora_a, M, K, rank, lora_scale, t, static_cast<float*>(workspace), stream);
  return e == hipSuccess ? BSQ_OK : hip_fail(e);
}

bsq_status bsq_gemm_fp8r_lora(const uint16_t* x, int64_t ldx, const uint8_t* w, const float* w_scale,
                              const uint16_t* lora_a, const uint16_t* lora_b, int64_t rank, float lora_scale,
                              uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, uint32_t flags,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  bsq_status st = check_gemm_common(x, ldx, w, y, ldy, M, N, K, flags);
  if (st != BSQ_OK) return st;
  if ((st = check_lora(ldx, lora_a, lora_b, rank, lora_scale, M, N)) != BSQ_OK) return st;
  if (M == 0 || N == 0) return BSQ_OK;
  if (!w_scale) return BSQ_ERR_NULL;
  if (!aligned(w_scale, 4)) return BSQ_ERR_ALIGN;
  if (!workspace || workspace_bytes < bsq_lora_workspace_bytes(BSQ_FMT_FP8R, M, N, K, rank, flags))
    return BSQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return BSQ_ERR_ALIGN;
  if ((st = check_device()) != BSQ_OK) return st;
  const bool weight_only = flags & BSQ_WEIGHT_ONLY;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* t = reinterpret_cast<uint16_t*>(ws + bsq_gemm_workspace_bytes(BSQ_FMT_FP8R, M, N, K, flags));
  if (!weight_only && bsq::lora_down_rows_pick(M, K, (int)rank, bsq::kDownFp8r)) {
    // one kernel encodes X to fp8r (into the workspace, as the quantizer would) and computes T
    bsq::RowsEncode en;
    en.enc = bsq::kDownFp8r;
    en.xq = ws;
    en.sx = reinterpret_cast<float*>(ws + pad256((size_t)(M * K)));
    hipError_t e = bsq::launch_lora_down_rows(x, ldx, lora_a, M, K, (int)rank, lora_scale, nullptr, nullptr, t, en,
                                              stream);
    if (e == hipSuccess) e = launch_w8a8(ws, en.sx, w, w_scale, y, ldy, M, N, K, stream, t, lora_b, (int)rank);
    return e == hipSuccess ? BSQ_OK : hip_fail(e);
  }
  hipError_t e = lora_down_plain(x, ldx, lora_a, M, K, rank, lora_scale, t, lora_part(t, M, rank), stream);
  if (e == hipSuccess) {
    if (weight_only) {
      bsq::DecArgs a{};
      a.x = x; a.ldx = ldx; a.w = w; a.sw = w_scale; a.y = y; a.ldy = ldy; a.M = M; a.N = N; a.K = K;
      a.lt = t; a.lb = lora_b; a.rank = (int)rank;
      e = launch_dec_or_skinny(bsq::kW8A16, a, stream);
    } else {
      float* sx = reinterpret_cast<float*>(ws + pad256((size_t)(M * K)));
      e = bsq::launch_quant_fp8r(x, M, K, ldx, ws, sx, stream);
      if (e == hipSuccess) e = launch_w8a8(ws, sx, w, w_scale, y, ldy, M, N, K, stream, t, lora_b, (int)rank);
    }
  }
  return e == hipSuccess ? BSQ_OK : hip_fail(e);
}

bsq_status bsq_gemm_nvfp4_lora(const uint16_t* x, int64_t ldx, const uint8_t* w, const uint8_t* w_bscale,
                               const float* w_scale2, const float* input_scale, const uint16_t* lora_a,
                               const uint16_t* lora_b, int64_t rank, float lora_scale, uint16_t* y, int64_t ldy,
                               int64_t M, int64_t N, int64_t K, uint32_t flags, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  bsq_status st = check_gemm_common(x, ldx, w, y, ldy, M, N, K, flags);
  if (st != BSQ_OK) return st;
  if ((st = check_lora(ldx, lora_a, lora_b, rank, lora_scale, M, N)) != BSQ_OK) return st;
  if (M == 0 || N == 0) return BSQ_OK;
  const bool weight_only = flags & BSQ_WEIGHT_ONLY;
  if (!w_bscale || !w_scale2 || (!weight_only && !input_scale)) return BSQ_ERR_NULL;
  if (!aligned(w_bscale, 4) || !aligned(w_scale2, 4) || (input_scale && !aligned(input_scale, 4)))
    return BSQ_ERR_ALIGN;
  if (!workspace || workspace_bytes < bsq_lora_workspace_bytes(BSQ_FMT_NVFP4, M, N, K, rank, flags))
    return BSQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return BSQ_ERR_ALIGN;
  if ((st = check_device()) != BSQ_OK) return st;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* t = reinterpret_cast<uint16_t*>(ws + bsq_gemm_workspace_bytes(BSQ_FMT_NVFP4, M, N, K, flags));
  bsq::DecArgs a{};
  a.x = x; a.ldx = ldx; a.w = w; a.ws = w_bscale; a.gw = w_scale2; a.y = y; a.ldy = ldy;
  a.M = M; a.N = N; a.K = K;
  a.lt = t; a.lb = lora_b; a.rank = (int)rank;
  // the tiled W4A4 kernel adds the adapter before its K loop and takes T / (gx gw)
  const bool pre = !weight_only && !route_skinny(bsq::kW4A4, a) && bsq::lora_pre_scaled_w4a4(a);
  hipError_t e;
  if (weight_only) {
    e = lora_down_plain(x, ldx, lora_a, M, K, rank, lora_scale, t, lora_part(t, M, rank), stream);
    if (e == hipSuccess) e = launch_dec_or_skinny(bsq::kW4A16, a, stream);
  } else {
    // one pass over X: the down projection also writes X's nvfp4 encoding for the GEMM
    uint8_t* xs = ws + pad256((size_t)(M * K / 2));
    a.xq = ws; a.xs = xs; a.gx = input_scale;
    const float* ga = pre ? input_scale : nullptr;
    const float* gb = pre ? w_scale2 : nullptr;
    if (bsq::lora_down_rows_pick(M, K, (int)rank, bsq::kDownNvfp4)) {
      bsq::RowsEncode en;
      en.enc = bsq::kDownNvfp4;
      en.xq = ws;
      en.xs = xs;
      en.gq = input_scale;
      e = bsq::launch_lora_down_rows(x, ldx, lora_a, M, K, (int)rank, lora_scale, ga, gb, t, en, stream);
    } else {
      e = bsq::launch_lora_down(x, ldx, lora_a, M, K, (int)rank, lora_scale, ga, gb, lora_part(t, M, rank), t, stream,
                                input_scale, ws, xs);
    }
    if (e == hipSuccess) e = launch_dec_or_skinny(bsq::kW4A4, a, stream);
  }
  return e == hipSuccess ? BSQ_OK : hip_fail(e);
}

bsq_status bsq_dequant_to_bf16(bsq_format f, const uint8_t* w, const void* w_scale, const float* w_scale2,
                               int64_t N, int64_t K, uint16_t* w_bf16, hipStream_t stream) {
  if (f != BSQ_FMT_FP8R && f != BSQ_FMT_NVFP4) return BSQ_ERR_ARG;
  if (f == BSQ_FMT_FP8R && w_scale2) return BSQ_ERR_ARG;
  bsq_status st = check_rows(N, K, K);
  if (st != BSQ_OK) return st;
  if (N == 0) return BSQ_OK;
  if (!w || !w_scale || !w_bf16 || (f == BSQ_FMT_NVFP4 && !w_scale2)) return BSQ_ERR_NULL;
  if (!aligned(w, 16) || !aligned(w_scale, 4) || !aligned(w_bf16, 16) || (w_scale2 && !aligned(w_scale2, 4)))
    return BSQ_ERR_ALIGN;
  if (N * (K / 16) >= kMaxThreads) return BSQ_ERR_SHAPE;
  if ((st = check_device()) != BSQ_OK) return st;
  hipError_t e = f == BSQ_FMT_NVFP4
                     ? bsq::launch_dequant_nvfp4(w, static_cast<const uint8_t*>(w_scale), w_scale2, N, K, w_bf16,
                                                 stream)
                     : bsq::launch_dequant_fp8r(w, static_cast<const float*>(w_scale), N, K, w_bf16, stream);
  return e == hipSuccess ? BSQ_OK : hip_fail(e);
}

}  // extern "C"
