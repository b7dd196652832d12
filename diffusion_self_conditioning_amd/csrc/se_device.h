// se_device.h -- device-side helpers shared by the libsoftembed kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace se {

constexpr float kLog2e = 1.4426950408889634f;   // log2(e)
constexpr float kLn2 = 0.6931471805599453f;     // ln(2)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Streaming 16-byte loads for data read once (nontemporal hint: no reuse expected,
// keeps the stream from displacing data other workgroups re-read from L2).
__device__ __forceinline__ uint4 load_stream_u4(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 load_stream_f4(const void* p) {
  const f32x4_t v = __builtin_nontemporal_load(static_cast<const f32x4_t*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// Streaming stores of bf16 probabilities (nontemporal hint): they are read back only by
// the contraction that follows, so they are written past the caches instead of leaving
// dirty lines in L2 that the contraction's table stream would then have to evict
// (measured on MI355X: the whole-vocabulary step 4-5% faster).
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_stream_u2(void* p, uint32_t lo, uint32_t hi) {
  const u32x2_t v = {lo, hi};
  __builtin_nontemporal_store(v, static_cast<u32x2_t*>(p));
}
__device__ __forceinline__ void store_stream_u4(void* p, const uint4& o) {
  const u32x4_t v = {o.x, o.y, o.z, o.w};
  __builtin_nontemporal_store(v, static_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void store_stream_u16(uint16_t* p, uint16_t v) {
  __builtin_nontemporal_store(v, p);
}

// Buffer resource over [base, base + bytes) for raw (unstructured) buffer loads:
// the base sits in scalar registers, each load adds a 32-bit per-lane offset and a
// 32-bit wave-uniform offset.  Dword 3 selects 32-bit raw access on gfx950.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// 16-byte raw buffer loads (LLVM's raw buffer-load intrinsic, bound by name: the
// clang builtin of the same width drops all but one lane of the vector here).
// `aux` 2 = nontemporal (streamed once).
__device__ u32x4_t se_raw_buffer_load_u4(__amdgpu_buffer_rsrc_t rsrc, int voff, int soff,
                                         int aux) __asm("llvm.amdgcn.raw.ptr.buffer.load.v4i32");
__device__ f32x4_t se_raw_buffer_load_f4(__amdgpu_buffer_rsrc_t rsrc, int voff, int soff,
                                         int aux) __asm("llvm.amdgcn.raw.ptr.buffer.load.v4f32");
__device__ __forceinline__ uint4 buffer_load_u4(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                uint32_t soff) {
  const u32x4_t v = se_raw_buffer_load_u4(r, (int)voff, (int)soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 buffer_load_u4_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                   uint32_t soff) {
  const u32x4_t v = se_raw_buffer_load_u4(r, (int)voff, (int)soff, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 buffer_load_f4(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                 uint32_t soff) {
  const f32x4_t v = se_raw_buffer_load_f4(r, (int)voff, (int)soff, 0);
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 buffer_load_f4_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                    uint32_t soff) {
  const f32x4_t v = se_raw_buffer_load_f4(r, (int)voff, (int)soff, 2);
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ float se_raw_buffer_load_f1(__amdgpu_buffer_rsrc_t rsrc, int voff, int soff,
                                      int aux) __asm("llvm.amdgcn.raw.ptr.buffer.load.f32");
__device__ __forceinline__ float buffer_load_f1(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                uint32_t soff) {
  return se_raw_buffer_load_f1(r, (int)voff, (int)soff, 0);
}

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// p = e^(l - lse) as 2^(l*log2e - lse*log2e); `nl` = -(lse * log2e) is computed
// once per row by the caller.  Both the materialising kernel and the fused
// prologue use exactly this sequence so their bf16 probabilities are equal.
__device__ __forceinline__ float prob_from_logit(float l, float nl) {
  return exp2_hw(__builtin_fmaf(l, kLog2e, nl));
}

__device__ __forceinline__ float neg_lse_log2(float lse) { return -(lse * kLog2e); }

// Two fp32 -> packed bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32.
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// ---- reductions over each half (32 lanes) of a wave ------------------------------------
// Lanes 0-31 and 32-63 reduce separately and every lane ends with its half's result:
// four DPP exchanges inside each 16-lane row (xor 1, xor 2, half-row mirror, row
// mirror), then one swizzle that swaps the two rows of a half (xor 16).
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl,
                                                            0xF, 0xF, true));
}
template <int kCtrl>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, kCtrl, 0xF, 0xF, true);
}
__device__ __forceinline__ float swz16_f(float v) {     // lane ^ 16 within 32 lanes
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}
__device__ __forceinline__ int swz16_i(int v) { return __builtin_amdgcn_ds_swizzle(v, 0x401F); }

__device__ __forceinline__ float half_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return v + swz16_f(v);
}
__device__ __forceinline__ float half_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return fmaxf(v, swz16_f(v));
}
// (value, index) maximum, ties to the lower index
__device__ __forceinline__ void argmax_step(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
}
__device__ __forceinline__ void half_argmax(float& v, int& i) {
  argmax_step(v, i, dpp_f<0xB1>(v), dpp_i<0xB1>(i));
  argmax_step(v, i, dpp_f<0x4E>(v), dpp_i<0x4E>(i));
  argmax_step(v, i, dpp_f<0x141>(v), dpp_i<0x141>(i));
  argmax_step(v, i, dpp_f<0x140>(v), dpp_i<0x140>(i));
  argmax_step(v, i, swz16_f(v), swz16_i(i));
}

// whole-wave reductions (64 lanes) on top of the half-wave ones
__device__ __forceinline__ float wave_sum(float v) {
  v = half_sum(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  half_argmax(v, i);
  const float v1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const int i1 = __builtin_amdgcn_readlane(i, 32);
  v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  i = __builtin_amdgcn_readlane(i, 0);
  argmax_step(v, i, v1, i1);
}

// The merge of one row's range statistics, by one whole wavefront (the one-read step; the
// partition identity of calvarado04.com, "The fix", on softmax numerators).  Range r of the
// row holds stats[r * n_rows + row] = {m_r, Z_r, S1_r (nats), m_r} and the vocabulary id of
// its first maximum.  At the overall maximum M:
//   Z = sum_r e^(m_r - M) Z_r,  S1 = sum_r e^(m_r - M) (S1_r + (m_r - M) Z_r),
//   lse = M + ln Z,  H = ln Z - S1 / Z,  argmax = the smallest id reaching M,
// and split range r0 + j gets the factor gamma e^(m - M) / Z (factors[j * n_rows + row]).
// Lane l takes ranges l, l + 64, ... in order; the lanes then combine in the fixed
// butterfly order, so the result is bitwise repeatable wherever it runs.
__device__ __forceinline__ void merge_ranges_row(const float4* __restrict__ stats,
                                                 const int32_t* __restrict__ stat_arg,
                                                 int64_t n_rows, int n_ranges, int r0, int splits,
                                                 float gamma, float* __restrict__ factors,
                                                 float* __restrict__ row_max,
                                                 float* __restrict__ row_lse,
                                                 float* __restrict__ row_entropy,
                                                 int32_t* __restrict__ row_argmax, int64_t row) {
  const int lane = threadIdx.x & 63;
  float mx = -INFINITY;
  int arg = 0x7fffffff;
  for (int r = lane; r < n_ranges; r += 64)
    argmax_step(mx, arg, stats[(int64_t)r * n_rows + row].x, stat_arg[(int64_t)r * n_rows + row]);
  wave_argmax(mx, arg);
  float z = 0.f, s1 = 0.f;
  for (int r = lane; r < n_ranges; r += 64) {
    const float4 st = stats[(int64_t)r * n_rows + row];
    const float d = st.x - mx;
    const float f = exp2_hw(d * kLog2e);
    z = __builtin_fmaf(f, st.y, z);
    s1 = __builtin_fmaf(f, __builtin_fmaf(d, st.y, st.z), s1);
  }
  z = wave_sum(z);
  s1 = wave_sum(s1);
  const float lz = logf(z);
  if (lane == 0) {
    row_max[row] = mx;
    row_lse[row] = mx + lz;
    row_entropy[row] = lz - s1 / z;
    row_argmax[row] = arg;
  }
  const float gz = gamma / z;
  for (int j = lane; j < splits; j += 64)
    factors[(int64_t)j * n_rows + row] =
        gz * exp2_hw((stats[(int64_t)(r0 + j) * n_rows + row].x - mx) * kLog2e);
}

// 16 OCP e4m3 codes (byte j of `c` = element j) times a power-of-two `scale`, as 16
// bf16 values: elements 0..7 in `lo`, 8..15 in `hi`.  Every e4m3 value times a power
// of two in the normal range is a bf16 value, so the conversion is exact.
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t c, float scale, bool high) {
  return high ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, scale, true))
              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, scale, false));
}
__device__ __forceinline__ void fp8x16_to_bf16(const uint4& c, float scale, uint4& lo, uint4& hi) {
  lo = make_uint4(fp8x2_to_bf16x2(c.x, scale, false), fp8x2_to_bf16x2(c.x, scale, true),
                  fp8x2_to_bf16x2(c.y, scale, false), fp8x2_to_bf16x2(c.y, scale, true));
  hi = make_uint4(fp8x2_to_bf16x2(c.z, scale, false), fp8x2_to_bf16x2(c.z, scale, true),
                  fp8x2_to_bf16x2(c.w, scale, false), fp8x2_to_bf16x2(c.w, scale, true));
}

}  // namespace se
