// common.hpp -- device helpers shared by the gfx950 selective-scan kernels.
//
// Element I/O for fp32 and bf16 storage, the softplus and SiLU used around the
// recurrence, and the fp32 -> bf16 store (round to nearest even, done by the
// hardware v_cvt_pk_bf16_f32 on gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;  // 1 / ln 2
constexpr float kLn2 = 0.6931471805599453f;

// Storage tags.
struct F32 {};
struct BF16 {};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values -> two bf16 (round to nearest even) packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t to_bf16(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// Raw storage of VW consecutive elements, loaded with one vector access.
template <class IO, int VW> struct Raw;
template <> struct Raw<F32, 4> { float4 v; };
template <> struct Raw<F32, 2> { float2 v; };
template <> struct Raw<F32, 1> { float v; };
template <> struct Raw<BF16, 4> { uint2 v; };
template <> struct Raw<BF16, 2> { uint32_t v; };
template <> struct Raw<BF16, 1> { uint16_t v; };

template <class IO, int VW> __device__ __forceinline__ Raw<IO, VW> raw_zero() {
  Raw<IO, VW> r;
  __builtin_memset(&r, 0, sizeof(r));
  return r;
}

// Load elements [idx, idx + VW) of a row-major tensor.  idx must be a
// multiple of VW and the base suitably aligned (checked on the host).
template <class IO, int VW> __device__ __forceinline__ Raw<IO, VW> raw_load(const void* base, int64_t idx);
template <> __device__ __forceinline__ Raw<F32, 4> raw_load<F32, 4>(const void* base, int64_t idx) {
  return {*reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx)};
}
template <> __device__ __forceinline__ Raw<F32, 2> raw_load<F32, 2>(const void* base, int64_t idx) {
  return {*reinterpret_cast<const float2*>(static_cast<const float*>(base) + idx)};
}
template <> __device__ __forceinline__ Raw<F32, 1> raw_load<F32, 1>(const void* base, int64_t idx) {
  return {static_cast<const float*>(base)[idx]};
}
template <> __device__ __forceinline__ Raw<BF16, 4> raw_load<BF16, 4>(const void* base, int64_t idx) {
  return {*reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx)};
}
template <> __device__ __forceinline__ Raw<BF16, 2> raw_load<BF16, 2>(const void* base, int64_t idx) {
  return {*reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(base) + idx)};
}
template <> __device__ __forceinline__ Raw<BF16, 1> raw_load<BF16, 1>(const void* base, int64_t idx) {
  return {static_cast<const uint16_t*>(base)[idx]};
}

template <class IO, int VW> __device__ __forceinline__ void unpack(const Raw<IO, VW>& r, float* out);
template <> __device__ __forceinline__ void unpack<F32, 4>(const Raw<F32, 4>& r, float* o) {
  o[0] = r.v.x; o[1] = r.v.y; o[2] = r.v.z; o[3] = r.v.w;
}
template <> __device__ __forceinline__ void unpack<F32, 2>(const Raw<F32, 2>& r, float* o) {
  o[0] = r.v.x; o[1] = r.v.y;
}
template <> __device__ __forceinline__ void unpack<F32, 1>(const Raw<F32, 1>& r, float* o) { o[0] = r.v; }
template <> __device__ __forceinline__ void unpack<BF16, 4>(const Raw<BF16, 4>& r, float* o) {
  o[0] = bf16_lo(r.v.x); o[1] = bf16_hi(r.v.x); o[2] = bf16_lo(r.v.y); o[3] = bf16_hi(r.v.y);
}
template <> __device__ __forceinline__ void unpack<BF16, 2>(const Raw<BF16, 2>& r, float* o) {
  o[0] = bf16_lo(r.v); o[1] = bf16_hi(r.v);
}
template <> __device__ __forceinline__ void unpack<BF16, 1>(const Raw<BF16, 1>& r, float* o) {
  o[0] = __uint_as_float(static_cast<uint32_t>(r.v) << 16);
}

template <class IO, int VW> __device__ __forceinline__ void store_vals(void* base, int64_t idx, const float* v);
template <> __device__ __forceinline__ void store_vals<F32, 4>(void* base, int64_t idx, const float* v) {
  *reinterpret_cast<float4*>(static_cast<float*>(base) + idx) = make_float4(v[0], v[1], v[2], v[3]);
}
template <> __device__ __forceinline__ void store_vals<F32, 2>(void* base, int64_t idx, const float* v) {
  *reinterpret_cast<float2*>(static_cast<float*>(base) + idx) = make_float2(v[0], v[1]);
}
template <> __device__ __forceinline__ void store_vals<F32, 1>(void* base, int64_t idx, const float* v) {
  static_cast<float*>(base)[idx] = v[0];
}
template <> __device__ __forceinline__ void store_vals<BF16, 4>(void* base, int64_t idx, const float* v) {
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + idx) =
      make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}
template <> __device__ __forceinline__ void store_vals<BF16, 2>(void* base, int64_t idx, const float* v) {
  *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(base) + idx) = pack_bf16x2(v[0], v[1]);
}
template <> __device__ __forceinline__ void store_vals<BF16, 1>(void* base, int64_t idx, const float* v) {
  static_cast<uint16_t*>(base)[idx] = to_bf16(v[0]);
}

// Buffer (V#) access.  A raw buffer resource covers [base, base + bytes);
// loads at offsets outside it return zero and stores there are dropped by the
// hardware, so a ragged tail needs no branch.  Offsets are 32-bit bytes.  The
// range check takes the whole offset, the scalar (soff) part included (as
// measured on gfx950), so a wave-uniform part of an offset (a block's start)
// goes in soff: one scalar value for every lane instead of a vector add per
// lane, with the same zero reads and dropped stores past the range.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufWord3 = 0x00020000;  // gfx9 descriptor word 3: 32-bit data format, raw (unswizzled) addressing

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0xffffffffLL ? 0xffffffffLL : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(static_cast<uint32_t>(n)),
                                           kBufWord3);
}

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <class IO, int VW> __device__ __forceinline__ Raw<IO, VW> buf_load(rsrc_t r, int voff, int soff);
template <> __device__ __forceinline__ Raw<F32, 4> buf_load<F32, 4>(rsrc_t r, int voff, int soff) {
  return {__builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0))};
}
template <> __device__ __forceinline__ Raw<F32, 2> buf_load<F32, 2>(rsrc_t r, int voff, int soff) {
  return {__builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0))};
}
template <> __device__ __forceinline__ Raw<F32, 1> buf_load<F32, 1>(rsrc_t r, int voff, int soff) {
  return {__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0))};
}
template <> __device__ __forceinline__ Raw<BF16, 4> buf_load<BF16, 4>(rsrc_t r, int voff, int soff) {
  return {__builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0))};
}
template <> __device__ __forceinline__ Raw<BF16, 2> buf_load<BF16, 2>(rsrc_t r, int voff, int soff) {
  return {__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0)};
}
template <> __device__ __forceinline__ Raw<BF16, 1> buf_load<BF16, 1>(rsrc_t r, int voff, int soff) {
  return {__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0)};
}

template <class IO, int VW> __device__ __forceinline__ void buf_store(rsrc_t r, int voff, int soff, const float* v);
template <> __device__ __forceinline__ void buf_store<F32, 4>(rsrc_t r, int voff, int soff, const float* v) {
  const u32x4_t x = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
  __builtin_amdgcn_raw_buffer_store_b128(x, r, voff, soff, 0);
}
template <> __device__ __forceinline__ void buf_store<F32, 2>(rsrc_t r, int voff, int soff, const float* v) {
  const u32x2_t x = {__float_as_uint(v[0]), __float_as_uint(v[1])};
  __builtin_amdgcn_raw_buffer_store_b64(x, r, voff, soff, 0);
}
template <> __device__ __forceinline__ void buf_store<F32, 1>(rsrc_t r, int voff, int soff, const float* v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[0]), r, voff, soff, 0);
}
template <> __device__ __forceinline__ void buf_store<BF16, 4>(rsrc_t r, int voff, int soff, const float* v) {
  const u32x2_t x = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  __builtin_amdgcn_raw_buffer_store_b64(x, r, voff, soff, 0);
}
template <> __device__ __forceinline__ void buf_store<BF16, 2>(rsrc_t r, int voff, int soff, const float* v) {
  __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(v[0], v[1]), r, voff, soff, 0);
}
template <> __device__ __forceinline__ void buf_store<BF16, 1>(rsrc_t r, int voff, int soff, const float* v) {
  __builtin_amdgcn_raw_buffer_store_b16(to_bf16(v[0]), r, voff, soff, 0);
}

// Loads of wave-uniform fp32 data through the constant address space, so the
// compiler issues scalar (s_load) loads into SGPRs, which the VALU then takes
// as operands directly.
typedef const __attribute__((address_space(4))) float* cfloat_p;
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef const __attribute__((address_space(4))) f32x16_t* cf32x16_p;

// Element idx of a bf16 or fp32 tensor, widened to fp32.
template <class IO> __device__ __forceinline__ float load_elem(const void* base, int64_t idx);
template <> __device__ __forceinline__ float load_elem<F32>(const void* base, int64_t idx) {
  return static_cast<const float*>(base)[idx];
}
template <> __device__ __forceinline__ float load_elem<BF16>(const void* base, int64_t idx) {
  return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[idx]) << 16);
}

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^-|x|).  With e = e^-|x|
// and u = 1 + e rounded to fp32, log1p(e) = ln 2 * log2(u) + (e - (u - 1)):
// the second term is the rounding error of u (exact, since u - 1 is), which
// keeps the sum accurate where e is tiny.  The hardware log2 is accurate to
// ~1 ulp relative also next to 1, so no series or branch is needed; measured
// on [-30, 30] the result is within 2e-6 relative of the exact value (the
// rounding of the exp argument dominates).
__device__ __forceinline__ float log1p_exp_neg_abs(float x) {
  const float e = __builtin_amdgcn_exp2f(-__builtin_fabsf(x) * kLog2e);
  const float u = 1.0f + e;
  const float c = e - (u - 1.0f);
  return __builtin_fmaf(__builtin_amdgcn_logf(u), kLn2, c);
}
__device__ __forceinline__ float softplus_f(float x) { return __builtin_fmaxf(x, 0.0f) + log1p_exp_neg_abs(x); }

// The step from x = delta_raw + bias: softplus(x) with (sp_k, sp_lo) = (1, 0),
// x itself with (0, -inf); one expression either way, so no branch.
__device__ __forceinline__ float step_of(float x, float sp_k, float sp_lo) {
  return __builtin_fmaf(sp_k, log1p_exp_neg_abs(x), __builtin_fmaxf(x, sp_lo));
}

// Chained launches hand a state (or an adjoint) from one piece of a sequence
// to the next through the workspace: a ready flag per piece, set by the
// workgroup that finished the piece before it.  A waiting workgroup's thread 0
// polls the flag at most `limit` times, each after a short sleep; the default
// limit (kSpinLimit polls of ~256 clocks) is about a third of a second.  On a
// time-out the kernel sets kStatusHandoffTimeout in the workspace's status word
// (word 0, which the host reads back with ssm_workspace_status) and the piece
// goes on from NaN, so every kernel ends and the outputs that depend on the
// lost hand-off show the failure.
// Discretisation rules of the scan kernels (forward and backward).
constexpr int kRuleEuler = 0;    // h_t = exp(delta_t A) h_{t-1} + delta_t B_t u_t
constexpr int kRuleTrap = 1;     // the trapezoidal three-term recurrence (Mamba-3), see scan_kernel

constexpr unsigned kSpinLimit = 1u << 18;
constexpr unsigned kStatusHandoffTimeout = 1u;

// True once *flag is non-zero, false after `limit` polls without it.
__device__ __forceinline__ bool poll_ready(const unsigned* flag, unsigned limit) {
  unsigned polls = 0;
  while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
    if (++polls > limit) return false;
    __builtin_amdgcn_s_sleep(4);
  }
  return true;
}

// The backward over packed sequences: sequence s's checkpoints (the state
// entering each of its 16-token blocks) start at block cu[s] / 16 +
// kPackedCkptSlack * s of its tile column, which leaves room for the whole
// trips of blocks the checkpoint pass writes (up to 3 past the last).
constexpr int kPackedCkptSlack = 5;

// A compile-time int as a type (for unrolled steps written as lambdas).
template <int I> struct IC { static constexpr int value = I; };

// Lane K (0..15) of each 16-lane row of v, broadcast across the row (DPP
// row_newbcast; the compiler folds it into a multiply's first operand).
template <int K> __device__ __forceinline__ float row_bcast(float v) {
  static_assert(K >= 0 && K < 16, "row lane");
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + K, 0xf, 0xf, true));
}

// acc + row_bcast<K>(v) * x as one v_fmac_f32_dpp: the compiler does not fold
// a broadcast into an FMA that accumulates in place.  A DPP read of a VGPR
// that a VALU instruction wrote in the two wait states before it is a hazard
// the compiler cannot see inside asm.  Here v is only ever written by buffer
// loads; the library build scans the generated assembly for the hazard and
// fails if it finds one (build.py).
template <int K> __device__ __forceinline__ float fmac_row_bcast(float acc, float v, float x) {
  static_assert(K >= 0 && K < 16, "row lane");
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "+v"(acc) : "v"(v), "v"(x), "n"(K));
  return acc;
}

// SiLU(z) = z * sigmoid(z) = z / (1 + e^-z); e^-z = inf for very negative z gives -0.
__device__ __forceinline__ float silu_f(float z) {
  const float e = __builtin_amdgcn_exp2f(-z * kLog2e);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace ssm
