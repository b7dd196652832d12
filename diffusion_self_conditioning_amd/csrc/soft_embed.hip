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
//   workgroup tile 256 (rows) x 256 (hidden) x 64 (vocab per step), double
//   buffered in LDS (2 x 72 KiB).  Waves form a 2 x 4 grid; each owns a
//   128 x 64 sub-tile = 4 x 2 blocks of v_mfma_f32_32x32x16_bf16.
// A operand (probabilities, K-contiguous rows):
//   fused   -- fp32 logits are loaded, turned into 2^(l log2e - lse log2e),
//              rounded to bf16 and written to LDS; P never reaches memory.
//   unfused -- bf16 probabilities are copied global -> LDS.
// B operand (embedding shard, hidden-contiguous rows): every thread loads an
//   8 (vocab) x 4 (hidden) block with 8-byte loads that coalesce into 512-byte
//   row segments, transposes it in registers (16 byte permutes) and writes four
//   16-byte vocab-contiguous chunks, so each MFMA B fragment is one ds_read_b128.
//   The chunk index is XOR-swizzled with bits 4..5 of the hidden index, which
//   keeps both the transposing writes and the fragment reads free of LDS bank
//   conflicts.
// Rows past M, vocab positions past K and hidden columns past N are never read;
// they enter the tile as exact zeros.
#include "se_device.h"
#include "se_launch.h"

namespace se {
namespace {

constexpr int kPitch = kBK + 8;                  // bf16 per LDS row (144 bytes)
constexpr int kStageRows = kBM + kBN;            // A rows then B rows
constexpr int kStageElems = kStageRows * kPitch;
constexpr int kLdsElems = 2 * kStageElems;       // 147456 bytes

__device__ __forceinline__ int bswz(int n) { return (n >> 4) & 3; }

template <bool FUSED>
struct ARegs;
template <>
struct ARegs<true> {
  float4 v[8];      // rows ar0 + 32 i, columns 4 c4 .. +3
  float nl[8];      // -(lse * log2e) of those rows
};
template <>
struct ARegs<false> {
  uint4 v[4];       // rows ar0 + 64 i, columns 8 c8 .. +7 (bf16)
};

template <bool FUSED>
__global__ void __launch_bounds__(kGemmThreads)
soft_embed_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[kLdsElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 2;          // 0..1 : 128-row half
  const int wn = wave & 3;           // 0..3 : 64-column quarter

  const int b = blockIdx.x;
  const int t = b % p.tiles;
  const int s = b / p.tiles;
  const int64_t m0 = (int64_t)(t / p.tiles_n) * kBM;
  const int64_t n0 = (int64_t)(t % p.tiles_n) * kBN;
  const int ks0 = (int)(((int64_t)s * p.ksteps) / p.splits);
  const int ks1 = (int)(((int64_t)(s + 1) * p.ksteps) / p.splits);

  // ---- operand load mappings -------------------------------------------------
  // A fused: 16 threads per row (16 x float4 = 64 fp32), 32 rows per pass, 8 passes.
  // A bf16 : 8 threads per row (8 x 16 B = 64 bf16), 64 rows per pass, 4 passes.
  const int a_c = FUSED ? (tid & 15) : (tid & 7);
  const int a_r0 = FUSED ? (tid >> 4) : (tid >> 3);
  // B: wave = 8-row vocab group, lane = 4-column hidden group.
  const int b_kg = wave;
  const int b_ng = lane;

  ARegs<FUSED> ra;
  uint2 rb[8];

  if constexpr (FUSED) {
    const float* lse = p.lse;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t row = m0 + a_r0 + 32 * i;
      ra.nl[i] = row < p.M ? neg_lse_log2(lse[row]) : 0.f;
    }
  }

  auto load_global = [&](int ks) {
    const int64_t kb = (int64_t)ks * kBK;
    if constexpr (FUSED) {
      const float* a = static_cast<const float*>(p.a);
      const int64_t kk = kb + 4 * a_c;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t row = m0 + a_r0 + 32 * i;
        float4 v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        if (row < p.M) {
          const float* src = a + row * p.lda + p.col0 + kk;
          if (kk + 4 <= p.K) {
            v = *reinterpret_cast<const float4*>(src);
          } else {
            if (kk + 0 < p.K) v.x = src[0];
            if (kk + 1 < p.K) v.y = src[1];
            if (kk + 2 < p.K) v.z = src[2];
          }
        }
        ra.v[i] = v;
      }
    } else {
      const uint16_t* a = static_cast<const uint16_t*>(p.a);
      const int64_t kk = kb + 8 * a_c;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + a_r0 + 64 * i;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (row < p.M) {
          const uint16_t* src = a + row * p.lda + p.col0 + kk;
          if (kk + 8 <= p.K) {
            v = *reinterpret_cast<const uint4*>(src);
          } else if (kk < p.K) {
            uint32_t h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) h[j] = (kk + j < p.K) ? (uint32_t)src[j] : 0u;
            v = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                           h[6] | (h[7] << 16));
          }
        }
        ra.v[i] = v;
      }
    }
    const int64_t col = n0 + 4 * b_ng;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t kr = kb + 8 * b_kg + i;
      uint2 v = make_uint2(0u, 0u);
      if (kr < p.K && col < p.N) v = *reinterpret_cast<const uint2*>(p.w + kr * p.ldw + col);
      rb[i] = v;
    }
  };

  auto store_lds = [&](int buf) {
    uint16_t* A = lds + buf * kStageElems;
    uint16_t* B = A + kBM * kPitch;
    if constexpr (FUSED) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 v = ra.v[i];
        const float nl = ra.nl[i];
        uint2 o;
        o.x = pack_bf16x2(prob_from_logit(v.x, nl), prob_from_logit(v.y, nl));
        o.y = pack_bf16x2(prob_from_logit(v.z, nl), prob_from_logit(v.w, nl));
        *reinterpret_cast<uint2*>(A + (a_r0 + 32 * i) * kPitch + 4 * a_c) = o;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(A + (a_r0 + 64 * i) * kPitch + 8 * a_c) = ra.v[i];
    }
    // transpose the 8 (vocab) x 4 (hidden) block: column j becomes a 16-byte
    // vocab-contiguous chunk of hidden row 4 ng + j.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = (j < 2) ? rb[2 * q].x : rb[2 * q].y;
        const uint32_t hi = (j < 2) ? rb[2 * q + 1].x : rb[2 * q + 1].y;
        w[q] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      const int n = 4 * b_ng + j;
      *reinterpret_cast<uint4*>(B + n * kPitch + 8 * (b_kg ^ bswz(n))) =
          make_uint4(w[0], w[1], w[2], w[3]);
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  auto compute = [&](int buf) {
    const uint16_t* A = lds + buf * kStageElems;
    const uint16_t* B = A + kBM * kPitch;
    const int half = lane >> 5;
    const int l32 = lane & 31;
#pragma unroll
    for (int q = 0; q < kBK / 16; ++q) {
      const int chunk = 2 * q + half;
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int r = 128 * wm + 32 * mi + l32;
        af[mi] = *reinterpret_cast<const bf16x8*>(A + r * kPitch + 8 * chunk);
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int n = 64 * wn + 32 * ni + l32;
        bfr[ni] = *reinterpret_cast<const bf16x8*>(B + n * kPitch + 8 * (chunk ^ bswz(n)));
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
  };

  if (ks0 < ks1) {
    load_global(ks0);
    store_lds(0);
    __syncthreads();
    for (int ks = ks0; ks < ks1; ++ks) {
      const int buf = (ks - ks0) & 1;
      const bool more = ks + 1 < ks1;
      if (more) load_global(ks + 1);
      compute(buf);
      if (more) store_lds(buf ^ 1);
      __syncthreads();
    }
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
