// soft_embed.hip -- the slice contraction  out = gamma * P[:, s:e] W_shard[0:e-s, :]
// on bf16 MFMA with fp32 accumulation, split-K over the vocabulary axis.
//
// The expected token embedding (calvarado04.com, "Where the shapes stop
// agreeing") restricted to one rank's vocab slice is that rank's partial S^(r);
// the normaliser gamma scales it ("The fix").  Split-K is the partition identity
// of the same section applied inside one GPU: each workgroup contracts one range
// of vocabulary steps, and the partial tiles are summed in a fixed order.
//
// Tiling (512 threads = 8 wave64s, one workgroup per CU):
//   workgroup tile 256 (rows) x 256 (hidden) x 32 (vocab per step), double
//   buffered in LDS (2 x 32 KiB).  Waves form a 2 x 4 grid; each owns a
//   128 x 64 sub-tile = 4 x 2 blocks of v_mfma_f32_32x32x16_bf16.
// Global loads run kStages steps ahead through registers: the loads of step
//   k + kStages are issued right after step k + 1 has been written to LDS, in the
//   order in which they will be consumed, so each wait names exactly the loads
//   it needs and the later ones stay in flight.
// A operand (probabilities, vocab-contiguous rows) in LDS as [row][vocab]:
//   fused   -- fp32 logits are loaded, turned into 2^(l log2e - lse log2e),
//              rounded to bf16 and written to LDS; P never reaches memory.
//   unfused -- bf16 probabilities are copied global -> LDS.
//   A fragments are single ds_read_b128s.
// B operand (embedding shard) in LDS as loaded, [vocab][hidden]: 16-byte
//   chunks, no register shuffles.  The MFMA wants 8 vocab-consecutive values of
//   one hidden column per lane; ds_read_b64_tr_b16 delivers them: in each group
//   of 16 lanes, lane i names the 4-element piece (row kb + i/4, columns
//   nb + 4 (i%4) .. +3) and lane j receives rows kb .. kb+3 of column nb + j.
// Both LDS tiles XOR-swizzle their 16-byte chunk index by the row so that every
//   write and every fragment read of a 16-lane group touches 64 distinct banks.
// Rows past M, vocab positions past K and hidden columns past N are never read;
// they enter the tile as exact zeros.
#include "se_device.h"
#include "se_launch.h"

namespace se {
namespace {

constexpr int kXcds = 8;
constexpr int kAStageBytes = kBM * kBK * 2;      // [256][kBK] bf16
constexpr int kWStageBytes = kBK * kBN * 2;      // [kBK][256] bf16
constexpr int kARowBytes = 2 * kBK;
constexpr int kARowsPerBankLine = 256 / kARowBytes;   // rows sharing one 64-bank line
constexpr int kAChunks = kBK / 8;                      // 16-byte chunks per A row
// A fused: float4 per thread, kBK / 4 threads per row; A bf16 and W: 16 B per thread
constexpr int kAFusedTpr = kBK / 4;
constexpr int kAFusedPasses = kBM / (kGemmThreads / kAFusedTpr);
constexpr int kABf16Tpr = kBK / 8;
constexpr int kABf16Passes = kBM / (kGemmThreads / kABf16Tpr);
constexpr int kWPasses = kBK / (kGemmThreads / 32);
constexpr int kBufBytes = kAStageBytes + kWStageBytes;
constexpr int kLdsBytes = 2 * kBufBytes;         // 64 KiB

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;

// Workgroups are dealt to the 8 XCDs round-robin (block b runs on XCD b % 8).
// Renumber them so that each XCD owns a contiguous run of logical ids: the tiles
// of one split are then mostly on one XCD and read the same probability columns
// through that XCD's L2 instead of once per XCD.
__device__ __forceinline__ int xcd_local_order(int b, int g) {
  const int x = b % kXcds, slot = b / kXcds;
  const int q = g / kXcds, r = g % kXcds;
  return x * q + (x < r ? x : r) + slot;
}

// byte offset of A element (m, k): rows of 2 kBK bytes, 16-byte chunk index
// (k / 8) XOR ((m / rows-per-bank-line) mod chunks-per-row)
__device__ __forceinline__ int a_off(int m, int k) {
  return m * kARowBytes + 16 * ((k >> 3) ^ ((m / kARowsPerBankLine) % kAChunks)) + 2 * (k & 7);
}
// byte offset of W element (k, n): rows of 512 bytes, chunk (n / 8) ^ (4 (k & 3))
__device__ __forceinline__ int w_off(int k, int n) {
  return k * 512 + 16 * ((n >> 3) ^ (4 * (k & 3))) + 2 * (n & 7);
}

template <bool FUSED>
struct AStage;
template <>
struct AStage<true> {
  float4 v[kAFusedPasses];   // fp32 logits, one float4 per pass
};
template <>
struct AStage<false> {
  uint4 v[kABf16Passes];     // bf16 probabilities, 8 per pass
};

struct WStage {
  uint4 v[kWPasses];         // bf16 table rows w_r + 16 i, columns 8 w_j .. +7
};

template <bool FUSED>
__global__ void __launch_bounds__(kGemmThreads)
soft_embed_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 2;          // 0..1 : 128-row half
  const int wn = wave & 3;           // 0..3 : 64-column quarter

  const int b = xcd_local_order((int)blockIdx.x, (int)gridDim.x);
  const int t = b % p.tiles;
  const int s = b / p.tiles;
  const int64_t m0 = (int64_t)(t / p.tiles_n) * kBM;
  const int64_t n0 = (int64_t)(t % p.tiles_n) * kBN;
  const int ks0 = (int)(((int64_t)s * p.ksteps) / p.splits);
  const int ks1 = (int)(((int64_t)(s + 1) * p.ksteps) / p.splits);

  // ---- per-thread load coordinates --------------------------------------------
  // A fused: kBK/4 threads x float4 per row; A bf16: kBK/8 threads x 16 B per row;
  // W: 32 threads x 16 B per row (256 bf16), 16 rows per pass.
  constexpr int kATpr = FUSED ? kAFusedTpr : kABf16Tpr;
  constexpr int kAPasses = FUSED ? kAFusedPasses : kABf16Passes;
  constexpr int kARowsPerPass = kGemmThreads / kATpr;
  const int a_c = tid % kATpr;
  const int a_m = tid / kATpr;
  const int w_j = tid & 31;
  const int w_r = tid >> 5;

  // Rows past M and columns past N only feed output rows / columns that are never
  // written, so their loads are clamped to the last valid row / column instead of
  // being guarded: the pipelined loads stay branch-free.
  float nl[kAFusedPasses];
  if constexpr (FUSED) {
#pragma unroll
    for (int i = 0; i < kAFusedPasses; ++i) {
      const int64_t row = min(m0 + a_m + kARowsPerPass * i, p.M - 1);
      nl[i] = neg_lse_log2(p.lse[row]);
    }
  }
  const int64_t w_col = min(n0 + 8 * w_j, p.N - 8);

  // Full step: every vocab position of the step is inside the slice.
  auto load_full = [&](int ks, AStage<FUSED>& ra, WStage& rw) {
    const int64_t kb = (int64_t)ks * kBK;
    if constexpr (FUSED) {
      const float* a = static_cast<const float*>(p.a) + p.col0 + kb + 4 * a_c;
#pragma unroll
      for (int i = 0; i < kAPasses; ++i) {
        const int64_t row = min(m0 + a_m + kARowsPerPass * i, p.M - 1);
        ra.v[i] = *reinterpret_cast<const float4*>(a + row * p.lda);
      }
    } else {
      const uint16_t* a = static_cast<const uint16_t*>(p.a) + p.col0 + kb + 8 * a_c;
#pragma unroll
      for (int i = 0; i < kAPasses; ++i) {
        const int64_t row = min(m0 + a_m + kARowsPerPass * i, p.M - 1);
        ra.v[i] = *reinterpret_cast<const uint4*>(a + row * p.lda);
      }
    }
#pragma unroll
    for (int i = 0; i < kWPasses; ++i)
      rw.v[i] = *reinterpret_cast<const uint4*>(p.w + (kb + w_r + 16 * i) * p.ldw + w_col);
  };

  // Last, partial step: vocab positions past K enter as exact zeros (probability
  // 0 from a -inf logit, or a zero bf16) and table rows past K are never read.
  auto load_tail = [&](int ks, AStage<FUSED>& ra, WStage& rw) {
    const int64_t kb = (int64_t)ks * kBK;
    if constexpr (FUSED) {
      const float* a = static_cast<const float*>(p.a);
      const int64_t kk = kb + 4 * a_c;
#pragma unroll
      for (int i = 0; i < kAPasses; ++i) {
        const int64_t row = min(m0 + a_m + kARowsPerPass * i, p.M - 1);
        const float* src = a + row * p.lda + p.col0 + kk;
        float4 v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        if (kk + 4 <= p.K) {
          v = *reinterpret_cast<const float4*>(src);
        } else {
          if (kk + 0 < p.K) v.x = src[0];
          if (kk + 1 < p.K) v.y = src[1];
          if (kk + 2 < p.K) v.z = src[2];
        }
        ra.v[i] = v;
      }
    } else {
      const uint16_t* a = static_cast<const uint16_t*>(p.a);
      const int64_t kk = kb + 8 * a_c;
#pragma unroll
      for (int i = 0; i < kAPasses; ++i) {
        const int64_t row = min(m0 + a_m + kARowsPerPass * i, p.M - 1);
        const uint16_t* src = a + row * p.lda + p.col0 + kk;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (kk + 8 <= p.K) {
          v = *reinterpret_cast<const uint4*>(src);
        } else if (kk < p.K) {
          uint32_t h[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) h[j] = (kk + j < p.K) ? (uint32_t)src[j] : 0u;
          v = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                         h[6] | (h[7] << 16));
        }
        ra.v[i] = v;
      }
    }
#pragma unroll
    for (int i = 0; i < kWPasses; ++i) {
      const int64_t kr = kb + w_r + 16 * i;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (kr < p.K) v = *reinterpret_cast<const uint4*>(p.w + kr * p.ldw + w_col);
      rw.v[i] = v;
    }
  };

  auto store = [&](int buf, const AStage<FUSED>& ra, const WStage& rw) {
    unsigned char* A = lds + buf * kBufBytes;
    unsigned char* W = A + kAStageBytes;
    if constexpr (FUSED) {
#pragma unroll
      for (int i = 0; i < kAPasses; ++i) {
        const float4 v = ra.v[i];
        uint2 o;
        o.x = pack_bf16x2(prob_from_logit(v.x, nl[i]), prob_from_logit(v.y, nl[i]));
        o.y = pack_bf16x2(prob_from_logit(v.z, nl[i]), prob_from_logit(v.w, nl[i]));
        *reinterpret_cast<uint2*>(A + a_off(a_m + kARowsPerPass * i, 4 * a_c)) = o;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kAPasses; ++i)
        *reinterpret_cast<uint4*>(A + a_off(a_m + kARowsPerPass * i, 8 * a_c)) = ra.v[i];
    }
#pragma unroll
    for (int i = 0; i < kWPasses; ++i)
      *reinterpret_cast<uint4*>(W + w_off(w_r + 16 * i, 8 * w_j)) = rw.v[i];
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  // per-lane fragment coordinates
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int grp = lane >> 4;              // 16-lane group
  const int gi = lane & 15;
  // transpose-read piece of this lane: row offset gi / 4, column offset 4 (gi % 4)
  const int tr_k = 8 * (grp >> 1) + (gi >> 2);
  const int tr_n = 16 * (grp & 1) + 4 * (gi & 3);

  auto compute = [&](int buf) {
    const unsigned char* A = lds + buf * kBufBytes;
    const unsigned char* W = A + kAStageBytes;
#pragma unroll
    for (int q = 0; q < kBK / 16; ++q) {
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int m = 128 * wm + 32 * mi + l32;
        af[mi] = *reinterpret_cast<const bf16x8*>(A + a_off(m, 16 * q + 8 * half));
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int nb = 64 * wn + 32 * ni + tr_n;
        const int kb = 16 * q + tr_k;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_ptr)(W + w_off(kb, nb)));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_ptr)(W + w_off(kb + 4, nb)));
        bfr[ni] = __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo),
                                          __builtin_bit_cast(bf16x4_t, hi), 0, 1, 2, 3, 4, 5,
                                          6, 7);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni],
                                                                0, 0, 0);
    }
  };

  // ---- main loop: kStages register stages in flight, LDS double buffer ----------
  // Steps [ks0, kf) are full.  Their loads are issued kStages steps ahead in
  // consumption order; past the end the step index is clamped, so the loop body
  // has no load branches (a few redundant in-bounds loads at the very end).
  const int kf = min(ks1, (int)(p.K / kBK));
  AStage<FUSED> ra[kStages];
  WStage rw[kStages];
  if (ks0 < kf) {
    const int klast = kf - 1;
#pragma unroll
    for (int j = 0; j < kStages; ++j) load_full(min(ks0 + j, klast), ra[j], rw[j]);
    store(0, ra[0], rw[0]);
    load_full(min(ks0 + kStages, klast), ra[0], rw[0]);
    __syncthreads();
    for (int base = ks0; base < kf; base += kStages) {
#pragma unroll
      for (int j = 0; j < kStages; ++j) {
        const int ks = base + j;
        if (ks < kf) {
          const int buf = (ks - ks0) & 1;
          compute(buf);
          const int nj = (j + 1) % kStages;
          if (ks + 1 < kf) store(buf ^ 1, ra[nj], rw[nj]);
          load_full(min(ks + 1 + kStages, klast), ra[nj], rw[nj]);
          __syncthreads();
        }
      }
    }
  }
  if (kf < ks1) {
    // the slice's last, partial step (only the final split has one)
    load_tail(kf, ra[0], rw[0]);
    store(0, ra[0], rw[0]);
    __syncthreads();
    compute(0);
  }

  // ---- epilogue ---------------------------------------------------------------
  // 32x32 MFMA accumulator layout: register r of lane l holds
  //   row 8 (r / 4) + 4 (l / 32) + (r % 4),  column l % 32  of the block.
  if (p.splits == 1) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int64_t col = n0 + 64 * wn + 32 * ni + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + 128 * wm + 32 * mi + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < p.M && col < p.N) p.out[row * p.ldo + col] = p.gamma * acc[mi][ni][r];
        }
      }
  } else {
    // partial tile in register order: fully coalesced 256-byte stores
    float* dst = p.ws + ((int64_t)s * p.tiles + t) * kTileFloats;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dst[((wave * 8 + mi * 2 + ni) * 16 + r) * 64 + lane] = acc[mi][ni][r];
  }
}

// Sum the split partials of every tile in split order, scale by gamma, scatter
// to the row-major output.  Each thread owns 4 consecutive partial elements
// (4 consecutive output columns of one row).
constexpr int kReduceThreads = 256;

__global__ void __launch_bounds__(kReduceThreads)
splitk_reduce_kernel(const float* __restrict__ ws, int tiles, int tiles_n, int splits,
                     int64_t M, int64_t N, float gamma, float* __restrict__ out, int64_t ldo) {
  constexpr int kBlocksPerTile = (int)(kTileFloats / (4 * kReduceThreads));
  const int t = blockIdx.x / kBlocksPerTile;
  const int e0 = ((blockIdx.x % kBlocksPerTile) * kReduceThreads + threadIdx.x) * 4;
  const int l0 = e0 & 63;
  const int r = (e0 >> 6) & 15;
  const int blk = e0 >> 10;
  const int wave = blk >> 3, mi = (blk >> 1) & 3, ni = blk & 1;
  const int wm = wave >> 2, wn = wave & 3;
  const int64_t row = (int64_t)(t / tiles_n) * kBM + 128 * wm + 32 * mi + 8 * (r >> 2) +
                      4 * (l0 >> 5) + (r & 3);
  const int64_t col = (int64_t)(t % tiles_n) * kBN + 64 * wn + 32 * ni + (l0 & 31);
  if (row >= M || col >= N) return;
  const float* src = ws + (int64_t)t * kTileFloats + e0;
  float4 a = *reinterpret_cast<const float4*>(src);
  for (int s = 1; s < splits; ++s) {
    const float4 v = *reinterpret_cast<const float4*>(src + (int64_t)s * tiles * kTileFloats);
    a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
  }
  *reinterpret_cast<float4*>(out + row * ldo + col) =
      make_float4(gamma * a.x, gamma * a.y, gamma * a.z, gamma * a.w);
}

__global__ void zero_rows_kernel(float* __restrict__ out, int64_t ldo, int64_t N) {
  const int64_t row = blockIdx.y;
  const int64_t c = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (c < N) *reinterpret_cast<float4*>(out + row * ldo + c) = make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace

hipError_t launch_soft_embed(const GemmParams& p, bool fused, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.tiles * p.splits));
  if (fused)
    hipLaunchKernelGGL(soft_embed_kernel<true>, grid, dim3(kGemmThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(soft_embed_kernel<false>, grid, dim3(kGemmThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const int blocks = p.tiles * (int)(kTileFloats / (4 * kReduceThreads));
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(kReduceThreads), 0, stream, p.ws,
                     p.tiles, p.tiles_n, p.splits, p.M, p.N, p.gamma, p.out, p.ldo);
  return hipGetLastError();
}

hipError_t launch_zero_rows(float* out, int64_t ldo, int64_t M, int64_t N, hipStream_t stream) {
  const int64_t groups = (N + 3) / 4;
  const dim3 grid((unsigned)((groups + 255) / 256), (unsigned)M);
  hipLaunchKernelGGL(zero_rows_kernel, grid, dim3(256), 0, stream, out, ldo, N);
  return hipGetLastError();
}

}  // namespace se
