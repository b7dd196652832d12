// soft_embed.hip -- the slice contraction  out = gamma * P[:, s:e] W_shard[0:e-s, :]
// on bf16 MFMA with fp32 accumulation, split-K over the vocabulary axis.
//
// The expected token embedding (calvarado04.com, "Where the shapes stop
// agreeing") restricted to one rank's vocab slice is that rank's partial S^(r);
// the normaliser gamma scales it ("The fix").  Split-K is the partition identity
// of the same section applied inside one GPU: each workgroup contracts one range
// of vocabulary positions, and the partial tiles are summed in a fixed order.
//
// Tiling (512 threads = 8 wave64s, one workgroup per CU): a 256 (rows) x 256
// (hidden) output tile, walked along the vocabulary in steps of BK (32 for the
// fused variant, 64 for the bf16 one).  Waves form a 2 x 4 grid; each owns a
// 128 x 64 sub-tile = 4 x 2 blocks of v_mfma_f32_32x32x16_bf16.
//
// LDS holds two buffers, each an A tile [256][BK] and a table tile [BK][256]:
//   A (probabilities, vocab-contiguous rows): fused -- fp32 logits are loaded,
//     turned into 2^(l log2e - lse log2e), rounded to bf16 and written to LDS, so
//     P never reaches memory; unfused -- bf16 probabilities are copied.  A
//     fragments are single ds_read_b128s.
//   W (embedding shard) is stored as loaded, [vocab][hidden]: the MFMA wants 8
//     vocab-consecutive values of one hidden column per lane and
//     ds_read_b64_tr_b16 delivers them: in each group of 16 lanes, lane i names
//     the 4-element piece (row kb + i/4, columns nb + 4 (i%4) .. +3) and lane j
//     receives rows kb .. kb+3 of column nb + j; two such reads form a fragment.
//   Both tiles XOR-swizzle their 16-byte chunk index with the row, so every write
//   and every fragment read of a 16-lane group touches 64 distinct banks.
//
// Pipeline: two register stages of global loads.  While the waves multiply step
// k out of one LDS buffer, piece by piece between the MFMAs they write step k + 1
// from registers into the other buffer and refill those registers with step
// k + 3; loads are issued in the order they are consumed, so every wait names
// exactly the piece it needs.  The table is streamed with nontemporal loads.  The
// main loop covers only full steps and has no load branches: rows past M and
// columns past N are clamped (they only feed output rows / columns that are never
// written).  A slice's last, partial step runs after the loop with guarded loads:
// vocab positions past K enter as exact zeros and table rows past K are never read.
#include "se_device.h"
#include "se_launch.h"

namespace se {
namespace {

constexpr int kXcds = 8;

// Workgroups are dealt to the 8 XCDs round-robin (block b runs on XCD b % 8).
// Renumber them so that each XCD owns a contiguous run of logical ids: the tiles
// of one split are then mostly on one XCD and read the same probability columns
// through that XCD's L2 instead of once per XCD.
__device__ __forceinline__ int xcd_local_order(int b, int g) {
  const int x = b % kXcds, slot = b / kXcds;
  const int q = g / kXcds, r = g % kXcds;
  return x * q + (x < r ? x : r) + slot;
}

// byte offset of table element (k, n) in a [BK][256] LDS tile: rows of 512 bytes,
// 16-byte chunk index (n / 8) XOR 4 (k % 4)
__device__ __forceinline__ int w_off(int k, int n) {
  return k * 512 + 16 * ((n >> 3) ^ (4 * (k & 3))) + 2 * (n & 7);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;

template <bool FUSED, int BK>
struct Cfg {
  static constexpr int kKSub = BK / 16;                        // MFMA k-steps per step
  static constexpr int kAStage = kBM * BK * 2;                 // bytes of the A tile
  static constexpr int kWStage = BK * kBN * 2;                 // bytes of the table tile
  static constexpr int kBuf = kAStage + kWStage;
  static constexpr int kARowBytes = 2 * BK;
  static constexpr int kARowsPerLine = 256 / kARowBytes;       // rows per 64-bank line
  static constexpr int kAChunks = BK / 8;                      // 16-byte chunks per A row
  // A loads: fused float4 per thread (BK/4 threads per row), bf16 16 B (BK/8 per row)
  static constexpr int kATpr = FUSED ? BK / 4 : BK / 8;
  static constexpr int kARowsPerPass = kGemmThreads / kATpr;
  static constexpr int kAPasses = kBM / kARowsPerPass;
  static constexpr int kWPasses = BK / (kGemmThreads / 32);    // 32 threads per table row
  static constexpr int kAPiece = kAPasses / kKSub;
  static constexpr int kWPiece = kWPasses / kKSub;
  static_assert(kAPiece * kKSub == kAPasses && kWPiece * kKSub == kWPasses, "pieces");
  static_assert(kSplitQuantum % BK == 0, "steps must tile the split quantum");

  // byte offset of A element (m, k): 16-byte chunk index (k / 8) XOR a row function
  __device__ static __forceinline__ int a_off(int m, int k) {
    return m * kARowBytes + 16 * ((k >> 3) ^ ((m / kARowsPerLine) % kAChunks)) + 2 * (k & 7);
  }
};

template <bool FUSED, int BK>
struct ARegs;
template <int BK>
struct ARegs<true, BK> {
  float4 v[Cfg<true, BK>::kAPasses];      // fp32 logits
};
template <int BK>
struct ARegs<false, BK> {
  uint4 v[Cfg<false, BK>::kAPasses];      // bf16 probabilities
};
template <int BK>
struct WRegs {
  uint4 v[Cfg<true, BK>::kWPasses];       // bf16 table chunks
};

template <bool FUSED, int BK>
__global__ void __launch_bounds__(kGemmThreads)
soft_embed_kernel(const GemmParams p) {
  using C = Cfg<FUSED, BK>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * C::kBuf];

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
  // this split's vocab range [k_lo, k_hi), in steps of BK: [s0, s1), full below sf
  const int64_t k_lo = (((int64_t)s * p.kblocks) / p.splits) * kSplitQuantum;
  const int64_t k_hi = min((((int64_t)(s + 1) * p.kblocks) / p.splits) * kSplitQuantum, p.K);
  const int s0 = (int)(k_lo / BK);
  const int s1 = (int)((k_hi + BK - 1) / BK);
  const int sf = min(s1, (int)(p.K / BK));

  // ---- per-thread load coordinates ----------------------------------------------
  const int a_c = tid % C::kATpr;
  const int a_m = tid / C::kATpr;
  const int w_j = tid & 31;
  const int w_r = tid >> 5;

  // Rows past M and columns past N only feed output rows / columns that are never
  // written, so their loads are clamped to the last valid row / column.
  auto a_row = [&](int i) -> int64_t { return min(m0 + a_m + C::kARowsPerPass * i, p.M - 1); };
  float nl[C::kAPasses];
  if constexpr (FUSED) {
#pragma unroll
    for (int i = 0; i < C::kAPasses; ++i) nl[i] = neg_lse_log2(p.lse[a_row(i)]);
  }
  const int64_t w_col = min(n0 + 8 * w_j, p.N - 8);

  // piece `pc` (of kKSub) of a full step
  auto load_piece = [&](int ks, int pc, ARegs<FUSED, BK>& ra, WRegs<BK>& rw) {
    const int64_t kb = (int64_t)ks * BK;
#pragma unroll
    for (int i = pc * C::kAPiece; i < (pc + 1) * C::kAPiece; ++i) {
      if constexpr (FUSED) {
        const float* a = static_cast<const float*>(p.a) + p.col0 + kb + 4 * a_c;
        ra.v[i] = *reinterpret_cast<const float4*>(a + a_row(i) * p.lda);
      } else {
        const uint16_t* a = static_cast<const uint16_t*>(p.a) + p.col0 + kb + 8 * a_c;
        ra.v[i] = *reinterpret_cast<const uint4*>(a + a_row(i) * p.lda);
      }
    }
#pragma unroll
    for (int i = pc * C::kWPiece; i < (pc + 1) * C::kWPiece; ++i)
      rw.v[i] = load_stream_u4(p.w + (kb + w_r + 16 * i) * p.ldw + w_col);
  };
  auto store_piece = [&](int buf, int pc, const ARegs<FUSED, BK>& ra, const WRegs<BK>& rw) {
    unsigned char* A = lds + buf * C::kBuf;
    unsigned char* W = A + C::kAStage;
#pragma unroll
    for (int i = pc * C::kAPiece; i < (pc + 1) * C::kAPiece; ++i) {
      const int m = a_m + C::kARowsPerPass * i;
      if constexpr (FUSED) {
        const float4 v = ra.v[i];
        uint2 o;
        o.x = pack_bf16x2(prob_from_logit(v.x, nl[i]), prob_from_logit(v.y, nl[i]));
        o.y = pack_bf16x2(prob_from_logit(v.z, nl[i]), prob_from_logit(v.w, nl[i]));
        *reinterpret_cast<uint2*>(A + C::a_off(m, 4 * a_c)) = o;
      } else {
        *reinterpret_cast<uint4*>(A + C::a_off(m, 8 * a_c)) = ra.v[i];
      }
    }
#pragma unroll
    for (int i = pc * C::kWPiece; i < (pc + 1) * C::kWPiece; ++i)
      *reinterpret_cast<uint4*>(W + w_off(w_r + 16 * i, 8 * w_j)) = rw.v[i];
  };
  // the slice's last, partial step: positions past K are exact zeros (probability 0
  // from a -inf logit, or a zero bf16); table rows past K are never read
  auto load_tail = [&](int ks, ARegs<FUSED, BK>& ra, WRegs<BK>& rw) {
    const int64_t kb = (int64_t)ks * BK;
#pragma unroll
    for (int i = 0; i < C::kAPasses; ++i) {
      if constexpr (FUSED) {
        const int64_t kk = kb + 4 * a_c;
        const float* src = static_cast<const float*>(p.a) + a_row(i) * p.lda + p.col0 + kk;
        float4 v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        if (kk + 4 <= p.K) {
          v = *reinterpret_cast<const float4*>(src);
        } else {
          if (kk + 0 < p.K) v.x = src[0];
          if (kk + 1 < p.K) v.y = src[1];
          if (kk + 2 < p.K) v.z = src[2];
        }
        ra.v[i] = v;
      } else {
        const int64_t kk = kb + 8 * a_c;
        const uint16_t* src = static_cast<const uint16_t*>(p.a) + a_row(i) * p.lda + p.col0 + kk;
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
    for (int i = 0; i < C::kWPasses; ++i) {
      const int64_t kr = kb + w_r + 16 * i;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (kr < p.K) v = *reinterpret_cast<const uint4*>(p.w + kr * p.ldw + w_col);
      rw.v[i] = v;
    }
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
  const int tr_k = 8 * (grp >> 1) + (gi >> 2);
  const int tr_n = 16 * (grp & 1) + 4 * (gi & 3);

  // MFMAs of one step out of LDS buffer `buf`; `side(q)` runs after substep q
  auto compute = [&](int buf, auto&& side) {
    const unsigned char* A = lds + buf * C::kBuf;
    const unsigned char* W = A + C::kAStage;
#pragma unroll
    for (int q = 0; q < C::kKSub; ++q) {
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8*>(A + C::a_off(128 * wm + 32 * mi + l32,
                                                               16 * q + 8 * half));
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int nb = 64 * wn + 32 * ni + tr_n;
        const int kb = 16 * q + tr_k;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(W + w_off(kb, nb)));
        const v4i16 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(W + w_off(kb + 4, nb)));
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
      side(q);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- main loop over the full steps [s0, sf) --------------------------------------
  ARegs<FUSED, BK> ra[2];
  WRegs<BK> rw[2];
  if (s0 < sf) {
    const int slast = sf - 1;
#pragma unroll
    for (int pc = 0; pc < C::kKSub; ++pc) load_piece(s0, pc, ra[0], rw[0]);
#pragma unroll
    for (int pc = 0; pc < C::kKSub; ++pc) load_piece(min(s0 + 1, slast), pc, ra[1], rw[1]);
#pragma unroll
    for (int pc = 0; pc < C::kKSub; ++pc) {
      store_piece(0, pc, ra[0], rw[0]);
      load_piece(min(s0 + 2, slast), pc, ra[0], rw[0]);
    }
    __syncthreads();
    for (int base = s0; base < sf; base += 2) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ks = base + j;
        if (ks < sf) {
          const int buf = (ks - s0) & 1;
          const int nj = (j + 1) & 1;             // register stage holding step ks + 1
          const bool more = ks + 1 < sf;
          const int knext = min(ks + 3, slast);
          compute(buf, [&](int q) {
            if (more) store_piece(buf ^ 1, q, ra[nj], rw[nj]);
            load_piece(knext, q, ra[nj], rw[nj]);
          });
          __syncthreads();
        }
      }
    }
  }
  if (sf < s1) {
    load_tail(sf, ra[0], rw[0]);
#pragma unroll
    for (int pc = 0; pc < C::kKSub; ++pc) store_piece(0, pc, ra[0], rw[0]);
    __syncthreads();
    compute(0, [](int) {});
  }

  // ---- epilogue ---------------------------------------------------------------------
  // 32x32 MFMA accumulator layout: register r of lane l holds
  //   row 8 (r / 4) + 4 (l / 32) + (r % 4),  column l % 32  of the block.
  if (p.splits == 1) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int64_t col = n0 + 64 * wn + 32 * ni + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + 128 * wm + 32 * mi + 8 * (r >> 2) + 4 * half + (r & 3);
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
  // fused: 32 vocab positions per step (fp32 logits staging); bf16: 64
  if (fused)
    hipLaunchKernelGGL((soft_embed_kernel<true, 32>), grid, dim3(kGemmThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((soft_embed_kernel<false, 64>), grid, dim3(kGemmThreads), 0, stream, p);
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
