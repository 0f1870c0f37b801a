// Device-side helpers shared by the bsq kernels (gfx950 / CDNA4 only).
//
// Number formats ("BFL (fp8r / nvfp4)", scheme list): E4M3 (OCP "FN": bias 7,
// max 448, S.1111.111 = NaN, no Inf) for fp8r values and nvfp4 block scales;
// E2M1 (bias 1, magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6) for nvfp4 values,
// packed two per byte with the even element in the low nibble.
//
// Conversions use the gfx950 hardware instructions. Their behaviour was
// checked on MI355X against bit-level round-to-nearest-even encoders over
// every finite fp32 input:
//   v_cvt_pk_fp8_f32          : RNE to E4M3FN, subnormals kept, sign of zero
//                               kept; inputs above 448 must be clamped first
//                               (the clamp gives the saturating encoding).
//   v_cvt_scalef32_pk_fp4_f32 : RNE to E2M1 with saturation at +-6 (scale 1).
//   v_cvt_pk_bf16_f32         : RNE to bf16.
//   v_cvt_f32_fp8             : exact E4M3 decode.
//   v_cvt_scalef32_pk_*_fp4   : exact E2M1 decode times 2^exponent(scale) --
//                               only the scale's exponent is applied, so an
//                               E4M3 block scale (4 significant bits) is
//                               multiplied in separately.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.0f;
constexpr float kE2M1Max = 6.0f;

// ---- bf16 ---------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// two fp32 -> packed bf16 pair (round to nearest even), lo in bits 15:0
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  union { v2bf v; uint32_t u; } r;
  r.v = v2bf{(__bf16)lo, (__bf16)hi};
  return r.u;
}

// ---- E4M3 ---------------------------------------------------------------------
// Encode into byte `byte_sel` (0..3) of `old`: two values at a time go into a
// 16-bit half; callers build whole words with enc_e4m3x4.
__device__ __forceinline__ uint32_t enc_e4m3x4(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
  b = __builtin_amdgcn_fmed3f(b, -kE4M3Max, kE4M3Max);
  c = __builtin_amdgcn_fmed3f(c, -kE4M3Max, kE4M3Max);
  d = __builtin_amdgcn_fmed3f(d, -kE4M3Max, kE4M3Max);
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0u, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}
__device__ __forceinline__ uint32_t enc_e4m3(float a) {
  a = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, 0.0f, 0u, false) & 0xFFu;
}
// fp8r per-chunk steps on 8 bf16 values (one 16-byte chunk of a row): the largest magnitude,
// and the E4M3 codes of fp32(x * r) for the row's reciprocal scale r
__device__ __forceinline__ float absmax8(uint4 v) {
  return fmaxf(fmaxf(fmaxf(fabsf(bf16_lo(v.x)), fabsf(bf16_hi(v.x))),
                     fmaxf(fabsf(bf16_lo(v.y)), fabsf(bf16_hi(v.y)))),
               fmaxf(fmaxf(fabsf(bf16_lo(v.z)), fabsf(bf16_hi(v.z))),
                     fmaxf(fabsf(bf16_lo(v.w)), fabsf(bf16_hi(v.w)))));
}
__device__ __forceinline__ uint2 encode8_fp8(uint4 v, float r) {
  uint2 o;
  o.x = enc_e4m3x4(bf16_lo(v.x) * r, bf16_hi(v.x) * r, bf16_lo(v.y) * r, bf16_hi(v.y) * r);
  o.y = enc_e4m3x4(bf16_lo(v.z) * r, bf16_hi(v.z) * r, bf16_lo(v.w) * r, bf16_hi(v.w) * r);
  return o;
}
// decode byte `sel` of w
template <int sel>
__device__ __forceinline__ float dec_e4m3(uint32_t w) { return __builtin_amdgcn_cvt_f32_fp8((int)w, sel); }
// decode two E4M3 bytes (word half `hi`) to two fp32
template <bool hi>
__device__ __forceinline__ v2f dec_e4m3x2(uint32_t w) { return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, hi); }

// ---- E2M1 ---------------------------------------------------------------------
// Encode eight fp32 values into one word of packed E2M1 (element 0 in the low
// nibble). Hardware saturates at +-6; scale 1.0 applies no exponent shift.
__device__ __forceinline__ uint32_t enc_e2m1x8(const float* v) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
  return w;
}
// byte `sel` of w -> two fp32 E2M1 values (exact)
template <int sel>
__device__ __forceinline__ v2f dec_e2m1x2_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, sel);
}
template <int sel>
__device__ __forceinline__ v2h dec_e2m1x2_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, sel);
}

// ---- nvfp4 block quantizer ---------------------------------------------------------
// One 16-element block ("BFL (fp8r / nvfp4)", nvfp4 bullet; every step one IEEE-rounded fp32
// operation): a = max |f|, sf = E4M3(fp32(fp32(a / 6) * G)), r = fp32(G / sf) (0 when sf
// is 0), q = E2M1(fp32(f * r)); G = fp32(1 / g) is passed in. Returns the scale byte and
// the 16 codes packed in `codes` (element 0 in the low nibble). Used by the activation
// quantizer and by the GEMM epilogue that quantizes its own output, so both give identical
// bits for the same inputs.
__device__ __forceinline__ uint32_t quant_block16_nvfp4(float (&f)[16], float G, uint2& codes) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(f[i]));
  const float u = (a / kE2M1Max) * G;
  const uint32_t sf = enc_e4m3(u);
  const float sfv = dec_e4m3<0>(sf);
  const float r = sfv > 0.0f ? G / sfv : 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) f[i] = f[i] * r;
  codes.x = enc_e2m1x8(f);
  codes.y = enc_e2m1x8(f + 8);
  return sf;
}
// the 16 bf16 values of two 16-byte chunks as fp32
__device__ __forceinline__ void bf16x16_to_f32(uint4 v0, uint4 v1, float (&f)[16]) {
  const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
}

// ---- streaming stores ----------------------------------------------------------
// 16-byte store with the non-temporal hint, for outputs that this kernel does
// not read back (dequantized weights, GEMM results)
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_stream(uint4* p, uint4 v) {
  __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(p));
}

// ---- wave reductions ----------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// ---- launch geometry ----------------------------------------------------------
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2). Remap the linear id so that each XCD receives a contiguous range of
// tiles; the range is then walked in groups of `group_m` tile-rows so that
// concurrently running tiles share operand rows in that XCD's L2.
constexpr int kNumXcd = 8;
__device__ __forceinline__ int xcd_contiguous_id(int pid, int total) {
  const int xcd = pid % kNumXcd, slot = pid / kNumXcd;
  const int base = total / kNumXcd, rem = total % kNumXcd;
  return xcd * base + (xcd < rem ? xcd : rem) + slot;
}
__device__ __forceinline__ void grouped_tile(int id, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
  const int per_group = group_m * tiles_n;
  const int g = id / per_group, first_m = g * group_m;
  const int gm = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
  const int in = id - g * per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

}  // namespace bsq

namespace bsq {

// ---- LDS staging ----------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_ptr_t;
// word 3 of a raw buffer resource on gfx9-family parts (32-bit data format,
// no swizzle); out-of-range loads return zeros
constexpr int kBufferConfig = 0x00020000;

typedef int v4i __attribute__((ext_vector_type(4)));

// Raw buffer resource for `bytes` bytes at `base` (stride 0); reads at or
// past `bytes` return zeros.
__device__ __forceinline__ v4i buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return v4i{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)bytes, kBufferConfig};
}

// The same resource as the compiler's buffer-resource type, for the raw
// buffer-load builtins (the compiler keeps it in scalar registers)
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kBufOut = 0x40000000u;  // an offset past the records of every resource built here

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferConfig);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t off) {
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t bload2(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

// LDS byte offset of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((lds_ptr_t)(p));
}

// global -> LDS copy of 16 bytes per lane: lane l's bytes at rsrc + voff + soff
// land at LDS [lds + 16 l, lds + 16 l + 16). Written as inline asm so that the
// compiler does not serialize unrelated LDS reads behind it; the caller
// waits for completion (wait_vmem) before the barrier that publishes the data.
// The compiler inserts no wait states in front of inline asm: an SGPR operand
// written by a VALU instruction (e.g. a spill reload by v_readlane) less than
// five wait states before would be read stale. tests/test_asm_hazards.py checks
// the kernels' assembly for that pattern.
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t lds, int voff, int soff) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds));
}

// 128-byte LDS rows, 16-byte chunks XOR-swizzled by ((row >> 1) & 7): a
// ds_read_b128 serves 16 lanes per 256-byte window of the 64-bank LDS, and
// 16 consecutive rows reading the same logical chunk then touch 16 distinct
// 16-byte slots
__device__ __forceinline__ int lds_swz(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

// s_waitcnt encodings (gfx9): vmcnt[3:0]+[15:14], expcnt[6:4], lgkmcnt[11:8]
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// wait until at most n (< 16) vector-memory operations are outstanding
template <int n>
__device__ __forceinline__ void wait_vmem_upto_c() { __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15)); }
#define wait_vmem_upto(n) wait_vmem_upto_c<((n) < 15 ? (n) : 15)>()
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

}  // namespace bsq
