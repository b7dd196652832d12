// soft_embed.hip -- the slice contraction  out = gamma * P[:, s:e] W_shard[0:e-s, :]
// on bf16 MFMA with fp32 accumulation, split-K over the vocabulary axis.
//
// The expected token embedding (calvarado04.com, "Where the shapes stop
// agreeing") restricted to one rank's vocab slice is that rank's partial S^(r);
// the normaliser gamma scales it ("The fix").  Split-K is the partition identity
// of the same section applied inside one GPU: each workgroup contracts one range
// of vocabulary positions, and the partial tiles are summed in a fixed order.
//
// Tiling: one workgroup per CU, a 256 (rows) x 256 (hidden) output tile, in
// 8 wave64s (default; two per SIMD, so one wave's MFMAs run while the other waits
// on memory) forming a 2 x 4 grid of 128 x 64 wave tiles (4 x 2 blocks of
// v_mfma_f32_32x32x16_bf16, 128 fp32 accumulators per lane), or 4 waves in a 2 x 2
// grid of 128 x 128 tiles (256 accumulators in AGPRs).  Both give bitwise equal
// results: every output element adds the same products in the same order.
//
// The vocabulary is walked in steps of 32 positions grouped into super-steps of
// 128.  LDS holds (160 KB):
//   two probability tiles P [256][128] bf16, one per super-step (current / next).
//     A fragment (8 consecutive positions of one row) is one ds_read_b128.
//     fused: fp32 logits become 2^(l log2e - lse log2e) rounded to bf16 and are
//     written here, so P never reaches memory; unfused: bf16 probabilities are
//     copied.  The probability rows are loaded 512 (fused) or 256 (unfused) bytes
//     at a time -- each load instruction covers 2 (4) rows, not 8 (16): the vector
//     memory path serves few long runs much faster than many short ones.
//   two table tiles W [32][256] bf16, one per step (current / next).  W is stored
//     as loaded, [vocab][hidden]; the MFMA wants 8 vocab-consecutive values of one
//     hidden column per lane, which ds_read_b64_tr_b16 delivers: in each group of
//     16 lanes, lane i names the 4-element piece (row kb + i/4, columns
//     nb + 4 (i%4) .. +3) and lane j receives rows kb .. kb+3 of column nb + j;
//     two such reads form a fragment.
//   Both tiles XOR-swizzle their 16-byte chunk index with the row, so the writes
//   and the fragment reads of every 16-lane group hit distinct banks.
//
// Pipeline.  Table: two register stages; while step k is multiplied, step k + 1
// goes from registers to LDS and the registers are refilled with step k + 3.
// Probabilities: two register sets of one quarter super-step each; during step q
// of super-step S, quarter q of super-step S + 1 is converted into the other P tile
// and its registers are refilled two quarters ahead.  All of it is interleaved
// with the MFMAs.  Per-lane addresses are 32-bit offsets from wave-uniform buffer
// bases, so advancing a step costs only scalar arithmetic.  The main loop covers
// whole super-steps and has no load branches: loads past the split's end are
// clamped to its last super-step (the data lands in a tile that is never read).
// A slice's last, partial super-step runs after the loop with guarded loads:
// positions past K enter as exact zeros, table rows past K are never read.  Rows
// past M are clamped (they only feed output rows that are never written); that
// path computes addresses per load and is used only when M is not a multiple of
// 256.
//
// e4m3 table (W8): the shard arrives as OCP FP8 E4M3 codes with one power-of-two
// scale per vocabulary row (the FP8 weights of the agentlenshq overview, section on
// performance and quantization).  Each lane loads 16 codes of one row per step and
// that row's scale; v_cvt_scalef32_pk_bf16_fp8 turns them into bf16 (exactly: code x
// power of two is a bf16 value) on the way into the same LDS tile, so everything after
// the LDS write is the bf16 kernel and the two agree bit for bit on the dequantized
// table.
#include "se_device.h"
#include "se_dispatch.h"
#include "se_launch.h"

#ifndef SE_W_LOAD
#define SE_W_LOAD buffer_load_u4_nt   // the table is streamed once: nontemporal loads
#endif

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

constexpr int kBK = 32;                          // vocab positions per step
constexpr int kQ = 4;                            // steps per super-step
constexpr int kSS = kBK * kQ;                    // vocab positions per super-step
static_assert(kSS == kSuperStep, "the host's view of a super-step");
constexpr int kPBuf = kBM * kSS * 2;             // bf16 probability tile of a super-step
constexpr int kWBuf = kBK * kBN * 2;             // bf16 table tile of a step
constexpr int kWBase = 2 * kPBuf;                // LDS: [P0][P1][W0][W1]
constexpr int kLds = 2 * kPBuf + 2 * kWBuf;
static_assert(kLds <= 160 * 1024, "LDS budget of one CU");
static_assert(kSplitQuantum % kSS == 0, "super-steps must tile the split quantum");
// Waves: 2 rows x kWN columns of wave tiles, each 128 x kTN (kMI x kNI MFMA blocks)
constexpr int kWaves = kGemmThreads / 64;
static_assert(kWaves == 4 || kWaves == 8, "4 (2 x 2) or 8 (2 x 4) waves");
constexpr int kWN = kWaves / 2;
constexpr int kTN = kBN / kWN;
constexpr int kMI = 4;
constexpr int kNI = kTN / 32;
constexpr int kArows = kBM / kWaves;             // probability rows produced per wave
constexpr int kWrows = kBK / kWaves;             // table rows per wave and step

// byte offset of P element (m, k) in a [256][128] tile: 256-byte rows, 16-byte
// chunk index (k / 8) XOR (m % 16)
__device__ __forceinline__ int p_off(int m, int k) {
  return m * 256 + 16 * ((k >> 3) ^ (m & 15)) + 2 * (k & 7);
}
// byte offset of W element (k, n) in a [32][256] tile: 512-byte rows, 16-byte
// chunk index (n / 8) XOR 4 (k % 4)
__device__ __forceinline__ int w_off(int k, int n) {
  return k * 512 + 16 * ((n >> 3) ^ (4 * (k & 3))) + 2 * (n & 7);
}

// Probability producer geometry, per wave and super-step (the wave's kArows rows).
//   fused: loads of 4 fp32; load i covers rows kArows wave + 2 i + lane/32,
//          positions 4 (lane % 32) .. +3.
//   unfused: loads of 8 bf16; load i covers rows kArows wave + 4 i + lane/16,
//          positions 8 (lane % 16) .. +7.
// A quarter (one step's share) is a quarter of the loads; two register sets of a
// quarter.
template <bool FUSED>
struct AGeo;
template <>
struct AGeo<true> {
  static constexpr int kRowsPerLoad = 2, kEsz = 4, kLoads = kArows / 2, kPerQ = kLoads / 4;
  typedef float4 reg_t;
  __device__ static int row(int i, int lane) { return 2 * i + (lane >> 5); }
  __device__ static int pos(int lane) { return 4 * (lane & 31); }
};
template <>
struct AGeo<false> {
  static constexpr int kRowsPerLoad = 4, kEsz = 2, kLoads = kArows / 4, kPerQ = kLoads / 4;
  typedef uint4 reg_t;
  __device__ static int row(int i, int lane) { return 4 * i + (lane >> 4); }
  __device__ static int pos(int lane) { return 8 * (lane & 15); }
};

// Table producer geometry, per wave and step (the wave's kWrows rows of the step).
//   bf16: loads of 8 values; load j covers rows 2 j + lane/32, columns 8 (lane % 32) ..
//   e4m3: loads of 16 codes; load j covers rows 4 j + lane/16, columns 16 (lane % 16) ..;
//         they become bf16 (times the row's scale) on the way into LDS, so the LDS
//         tile, the fragment reads and the MFMAs are the same for both tables.
template <bool W8>
struct WGeo;
template <>
struct WGeo<false> {
  static constexpr int kRowsPerLoad = 2, kEsz = 2, kCols = 8, kLoads = kWrows / 2;
  __device__ static int row(int lane) { return lane >> 5; }
  __device__ static int col(int lane) { return 8 * (lane & 31); }
};
template <>
struct WGeo<true> {
  static constexpr int kRowsPerLoad = 4, kEsz = 1, kCols = 16, kLoads = kWrows / 4;
  __device__ static int row(int lane) { return lane >> 4; }
  __device__ static int col(int lane) { return 16 * (lane & 15); }
};
static_assert(WGeo<true>::kLoads >= 1, "an e4m3 load covers 4 table rows");

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;

template <bool FUSED, bool FULL, bool W8>
__global__ void __launch_bounds__(kGemmThreads)
__attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
soft_embed_kernel(const GemmParams p) {
  using G = AGeo<FUSED>;
  using WG = WGeo<W8>;
  constexpr int kWJ = WG::kLoads;                // table loads per wave and step
  using AReg = typename G::reg_t;
  constexpr int kEsz = G::kEsz;
  constexpr int kPerQ = G::kPerQ;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / kWN;         // 128-row half
  const int wn = wave % kWN;         // kTN-column slice

  const int b = xcd_local_order((int)blockIdx.x, (int)gridDim.x);
  const int t = b % p.tiles;
  const int s = b / p.tiles;
  const int m0 = (t / p.tiles_n) * kBM;
  const int n0 = (t % p.tiles_n) * kBN;
  // this split's vocab range [k_lo, k_hi): full super-steps [S0, Sf), then (last
  // split only) the partial super-step Sf, whose steps end at ks_end
  const int64_t k_lo = (((int64_t)s * p.kblocks) / p.splits) * kSplitQuantum;
  const int64_t k_hi = min((((int64_t)(s + 1) * p.kblocks) / p.splits) * kSplitQuantum, p.K);
  const int S0 = (int)(k_lo / kSS);
  const int Sf = (int)(min(k_hi, (p.K / kSS) * kSS) / kSS);
  const int ks_end = (int)((k_hi + kBK - 1) / kBK);
  const int M = (int)p.M, N = (int)p.N;
  const int tile_rows = min(kBM, M - m0);

  // ---- probability producer: buffer resource at (row m0, column col0) -----------------
  // Super-step S of a row starts p.a_ss bytes after super-step S - 1: 128 positions for
  // a row-major matrix, or a whole [rows][128] block for the super-step-tiled layout
  // of the staged probabilities (then every 4-row load is one contiguous 1 KB run).
  const int64_t a_ld = p.lda * kEsz;
  const bool a_rowmajor = p.a_ss == (int64_t)kSS * kEsz;
  const int64_t a_span = a_rowmajor ? p.K * kEsz
                                    : ((p.K + kSS - 1) / kSS - 1) * p.a_ss + (int64_t)kSS * kEsz;
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(
      static_cast<const unsigned char*>(p.a) + ((int64_t)m0 * p.lda + p.col0) * kEsz,
      (uint32_t)min((int64_t)(tile_rows - 1) * a_ld + a_span, (int64_t)UINT32_MAX));
  const int a_row0 = kArows * wave;
  const uint32_t a_lo = (uint32_t)((a_row0 + G::row(0, lane)) * a_ld) + kEsz * G::pos(lane);
  // -(lse log2e) of row kArows wave + lane; load i fetches its rows' values with a
  // cross-lane permute (no LDS storage)
  float nl_lane = 0.f;
  if constexpr (FUSED) nl_lane = neg_lse_log2(p.lse[m0 + min(a_row0 + lane, tile_rows - 1)]);
  auto nl_of = [&](int i) -> float {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                         4 * G::row(i, lane), __builtin_bit_cast(int, nl_lane)));
  };
  // LDS store offset of load i (within a P tile).  Row kArows wave + R i + r (r = this
  // lane's row within the load) has swizzle (R i + r) % 16 = (R (i % (16 / R))) ^ r,
  // so the offset is a per-lane base with the chunk bits XORed by 16 R (i % (16 / R)).
  constexpr int kR = G::kRowsPerLoad;
  const int a_r = G::row(0, lane);
  const uint32_t a_st_row = (uint32_t)(a_row0 + a_r) * 256;
  const uint32_t a_st_chk = 16u * (uint32_t)((G::pos(lane) >> 3) ^ a_r) + 2u * (G::pos(lane) & 7);

  // load i of super-step S (clamped by the caller)
  auto load_a = [&](int S, int i) -> AReg {
    uint32_t voff, soff = (uint32_t)S * (uint32_t)p.a_ss;
    if constexpr (FULL) {
      voff = a_lo;
      soff += (uint32_t)(i * G::kRowsPerLoad * a_ld);
    } else {
      const int row = min(a_row0 + G::row(i, lane), tile_rows - 1);
      voff = (uint32_t)(row * a_ld) + kEsz * G::pos(lane);
    }
    if constexpr (FUSED) return buffer_load_f4(a_rsrc, voff, soff);
    else return buffer_load_u4(a_rsrc, voff, soff);
  };
  // convert / copy load i (register r) into P tile `pbuf`
  auto store_a = [&](int pbuf, int i, const AReg& r, float nl) {
    unsigned char* dst = lds + pbuf * kPBuf + a_st_row + i * kR * 256 +
                         (a_st_chk ^ (uint32_t)(16 * kR * (i % (16 / kR))));
    if constexpr (FUSED) {
      uint2 o;
      o.x = pack_bf16x2(prob_from_logit(r.x, nl), prob_from_logit(r.y, nl));
      o.y = pack_bf16x2(prob_from_logit(r.z, nl), prob_from_logit(r.w, nl));
      *reinterpret_cast<uint2*>(dst) = o;
    } else {
      *reinterpret_cast<uint4*>(dst) = r;
    }
  };

  // ---- table producer: buffer resources at shard row k_lo ------------------------------
  // step ks, load j (< kWJ): rows kWrows wave + WG::kRowsPerLoad j + WG::row(lane)
  const int64_t w_ld = p.ldw * WG::kEsz;
  const __amdgpu_buffer_rsrc_t w_rsrc =
      make_rsrc(static_cast<const unsigned char*>(p.w) + k_lo * w_ld,
                (uint32_t)min((k_hi - k_lo) * w_ld, (int64_t)UINT32_MAX));
  const int w_r = kWrows * wave + WG::row(lane);   // this lane's row in load 0 of a step
  const uint32_t w_lo =
      (uint32_t)(w_r * w_ld) + WG::kEsz * (uint32_t)min(n0 + WG::col(lane), N - WG::kCols);
  // LDS store offsets.  bf16: the rows of loads j and j + 1 differ in swizzle phase
  // (row % 4); e4m3: every load of a lane has the same phase and fills two chunks.
  uint32_t w_st[2];
  if constexpr (W8) {
    w_st[0] = kWBase + w_off(w_r, WG::col(lane));
    w_st[1] = kWBase + w_off(w_r, WG::col(lane) + 8);
  } else {
#pragma unroll
    for (int e = 0; e < 2; ++e) w_st[e] = kWBase + w_off(w_r + 2 * e, WG::col(lane)) - 1024 * e;
  }
  // e4m3 row scales of the split, one fp32 per lane and load
  const __amdgpu_buffer_rsrc_t s_rsrc =
      make_rsrc(W8 ? static_cast<const void*>(p.wscale + k_lo) : p.w,
                W8 ? (uint32_t)min((k_hi - k_lo) * 4, (int64_t)UINT32_MAX) : 0u);
  auto load_w = [&](int ks, int j) -> uint4 {
    return SE_W_LOAD(w_rsrc, w_lo,
                     (uint32_t)(((int64_t)ks * kBK - k_lo + WG::kRowsPerLoad * j) * w_ld));
  };
  auto load_s = [&](int ks, int j) -> float {
    return buffer_load_f1(s_rsrc, 4u * (uint32_t)w_r,
                          (uint32_t)(((int64_t)ks * kBK - k_lo + WG::kRowsPerLoad * j) * 4));
  };
  auto store_w = [&](int wbuf, int j, const uint4& r, float sc) {
    unsigned char* base = lds + wbuf * kWBuf;
    if constexpr (W8) {
      uint4 lo, hi;
      fp8x16_to_bf16(r, sc, lo, hi);
      *reinterpret_cast<uint4*>(base + w_st[0] + 512 * WG::kRowsPerLoad * j) = lo;
      *reinterpret_cast<uint4*>(base + w_st[1] + 512 * WG::kRowsPerLoad * j) = hi;
    } else {
      *reinterpret_cast<uint4*>(base + w_st[j & 1] + 1024 * j) = r;
    }
  };

  f32x16 acc[kMI][kNI];
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  // ---- fragments ---------------------------------------------------------------------
  // A, substep u (0..7) of a super-step: row 128 wm + 32 mi + lane % 32, positions
  // 16 u + 8 (lane / 32) .. +7
  // p_off(row, 16 u + 8 h) with row % 16 = lane % 16 is rd_row + (rd_chk ^ 32 u)
  const uint32_t rd_row = (uint32_t)(128 * wm + (lane & 31)) * 256;
  const uint32_t rd_chk = 16u * (uint32_t)((lane >> 5) ^ (lane & 15));
  // W: 16-lane group g, lane i: piece (row 8 (g/2) + i/4, columns 32 ni + 16 (g%2) + 4 (i%4))
  uint32_t b_rd[kNI];
  {
    const int g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
      b_rd[ni] = kWBase + w_off(8 * (g >> 1) + (i >> 2), kTN * wn + 32 * ni + 16 * (g & 1) + 4 * (i & 3));
  }
  auto frag_read = [&](int pbuf, int wbuf, int u, int q, bf16x8 (&af)[kMI], bf16x8 (&bf)[kNI]) {
    const unsigned char* pa = lds + pbuf * kPBuf + rd_row + (rd_chk ^ (uint32_t)(32 * u));
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi) af[mi] = *reinterpret_cast<const bf16x8*>(pa + 8192 * mi);
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      const unsigned char* wp = lds + wbuf * kWBuf + b_rd[ni] + 8192 * q;
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(wp));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(wp + 2048));
      bf[ni] = __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo),
                                       __builtin_bit_cast(bf16x4_t, hi), 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  auto mfmas = [&](const bf16x8 (&af)[kMI], const bf16x8 (&bf)[kNI]) {
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
  };

  // One step: the 2 substeps' fragments are read up front; side(q) is interleaved
  // with substep q's MFMAs (in the compiler's order; explicit interleaves measured no
  // faster).
  constexpr int kMF = kMI * kNI;                     // MFMAs per substep
  auto compute = [&](int pbuf, int wbuf, int qstep, auto&& side) {
    bf16x8 a0[kMI], b0[kNI], a1[kMI], b1[kNI];
    frag_read(pbuf, wbuf, 2 * qstep, 0, a0, b0);
    frag_read(pbuf, wbuf, 2 * qstep + 1, 1, a1, b1);
    mfmas(a0, b0);
    side(0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(a1, b1);
    side(1);
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- main loop over the full super-steps [S0, Sf) ------------------------------------
  AReg ra[2][kPerQ];                 // quarter registers: set q % 2
  uint4 rw[2][kWJ];                  // table register stages
  float rs[2][kWJ];                  // e4m3 row scales of those stages
  if (S0 < Sf) {
    const int Slast = Sf - 1;
    const int kslast = 4 * Sf - 1;
    const int ks0 = 4 * S0;
    // prologue: P tile of S0 complete, quarters 0 / 1 of S0 + 1 in flight; table
    // step ks0 in LDS, ks0 + 1 / ks0 + 2 in flight
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
#pragma unroll
      for (int i = 0; i < kPerQ; ++i) ra[q & 1][i] = load_a(S0, q * kPerQ + i);
#pragma unroll
      for (int i = 0; i < kPerQ; ++i) store_a(S0 & 1, q * kPerQ + i, ra[q & 1][i], nl_of(q * kPerQ + i));
    }
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < kPerQ; ++i) ra[q][i] = load_a(min(S0 + 1, Slast), q * kPerQ + i);
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int j = 0; j < kWJ; ++j) {
        rw[st][j] = load_w(min(ks0 + st, kslast), j);
        rs[st][j] = W8 ? load_s(min(ks0 + st, kslast), j) : 0.f;
      }
#pragma unroll
    for (int j = 0; j < kWJ; ++j) store_w(0, j, rw[0][j], rs[0][j]);
#pragma unroll
    for (int j = 0; j < kWJ; ++j) {
      rw[0][j] = load_w(min(ks0 + 2, kslast), j);
      rs[0][j] = W8 ? load_s(min(ks0 + 2, kslast), j) : 0.f;
    }
    __syncthreads();

    for (int S = S0; S < Sf; ++S) {
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        const int ks = 4 * S + q;
        uint4 (&rwn)[kWJ] = rw[(q + 1) & 1];          // table step ks + 1
        float (&rsn)[kWJ] = rs[(q + 1) & 1];
        AReg (&rq)[kPerQ] = ra[q & 1];                // quarter q of super-step S + 1
        // refill: quarter q + 2 of S + 1, or quarter q - 2 of S + 2
        const int Sr = min(q < 2 ? S + 1 : S + 2, Slast);
        const int qr = (q + 2) & 3;
        const int kn = min(ks + 3, kslast);
        float nlq[FUSED ? kPerQ : 1];
        if constexpr (FUSED) {
#pragma unroll
          for (int i = 0; i < kPerQ; ++i) nlq[i] = nl_of(q * kPerQ + i);
        }
        __builtin_amdgcn_sched_barrier(0);
        auto side = [&](int h) {
          // table loads j in [ceil(h kWJ / 2), ceil((h + 1) kWJ / 2)): a single load
          // goes with the first half
#pragma unroll
          for (int j = (h * kWJ + 1) / 2; j < ((h + 1) * kWJ + 1) / 2; ++j)
            store_w((q + 1) & 1, j, rwn[j], rsn[j]);
#pragma unroll
          for (int i = h * kPerQ / 2; i < (h + 1) * kPerQ / 2; ++i)
            store_a((S + 1) & 1, q * kPerQ + i, rq[i], nlq[FUSED ? i : 0]);
#pragma unroll
          for (int j = (h * kWJ + 1) / 2; j < ((h + 1) * kWJ + 1) / 2; ++j) {
            rwn[j] = load_w(kn, j);
            if constexpr (W8) rsn[j] = load_s(kn, j);
          }
#pragma unroll
          for (int i = h * kPerQ / 2; i < (h + 1) * kPerQ / 2; ++i) rq[i] = load_a(Sr, qr * kPerQ + i);
        };
        compute(S & 1, q & 1, q, side);
        __syncthreads();
      }
    }
  }

  // ---- the partial last super-step (last split only) -------------------------------------
  if (4 * Sf < ks_end) {
    const int64_t kb = (int64_t)Sf * kSS;
    const unsigned char* abase = static_cast<const unsigned char*>(p.a) +
                                 ((int64_t)m0 * p.lda + p.col0) * kEsz + (int64_t)Sf * p.a_ss;
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) {
      const int row = min(a_row0 + G::row(i, lane), tile_rows - 1);
      const int64_t kk = kb + G::pos(lane);
      const unsigned char* src = abase + (int64_t)row * a_ld + kEsz * G::pos(lane);
      AReg v;
      if constexpr (FUSED) {
        const float* f = reinterpret_cast<const float*>(src);
        v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        if (kk + 4 <= p.K) {
          v = *reinterpret_cast<const float4*>(f);
        } else {
          if (kk + 0 < p.K) v.x = f[0];
          if (kk + 1 < p.K) v.y = f[1];
          if (kk + 2 < p.K) v.z = f[2];
        }
      } else {
        const uint16_t* h = reinterpret_cast<const uint16_t*>(src);
        v = make_uint4(0u, 0u, 0u, 0u);
        if (kk + 8 <= p.K) {
          v = *reinterpret_cast<const uint4*>(h);
        } else if (kk < p.K) {
          uint32_t e[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) e[j] = (kk + j < p.K) ? (uint32_t)h[j] : 0u;
          v = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                         e[6] | (e[7] << 16));
        }
      }
      store_a(0, i, v, nl_of(i));
    }
    for (int ks = 4 * Sf; ks < ks_end; ++ks) {
      const int64_t kr0 = (int64_t)ks * kBK;
      const unsigned char* wb = reinterpret_cast<const unsigned char*>(p.w) + kr0 * w_ld;
#pragma unroll
      for (int j = 0; j < kWJ; ++j) {
        const int64_t kr = kr0 + w_r + WG::kRowsPerLoad * j;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        float sc = 0.f;
        if (kr < p.K) {
          v = *reinterpret_cast<const uint4*>(wb + (int64_t)(WG::kRowsPerLoad * j) * w_ld + w_lo);
          if constexpr (W8) sc = p.wscale[kr];
        }
        store_w(0, j, v, sc);
      }
      __syncthreads();
      compute(0, 0, ks - 4 * Sf, [](int) {});
      __syncthreads();
    }
  }

  // ---- epilogue ---------------------------------------------------------------------
  // 32x32 MFMA accumulator layout: register r of lane l holds
  //   row 8 (r / 4) + 4 (l / 32) + (r % 4),  column l % 32  of the block.
  if (p.splits == 1 && !p.keep_partials) {
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni) {
        const int col = n0 + kTN * wn + 32 * ni + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + 128 * wm + 32 * mi + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < M && col < N) p.out[(int64_t)row * p.ldo + col] = p.gamma * acc[mi][ni][r];
        }
      }
  } else {
    // partial tile in register order: fully coalesced 256-byte stores
    float* dst = p.ws + ((int64_t)s * p.tiles + t) * kTileFloats;
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dst[((wave * kMF + mi * kNI + ni) * 16 + r) * 64 + lane] = acc[mi][ni][r];
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
  const int blk = e0 >> 10;                       // (wave * kMI + mi) * kNI + ni
  const int wave = blk / (kMI * kNI), mi = (blk / kNI) % kMI, ni = blk % kNI;
  const int wm = wave / kWN, wn = wave % kWN;
  const int64_t row = (int64_t)(t / tiles_n) * kBM + 128 * wm + 32 * mi + 8 * (r >> 2) +
                      4 * (l0 >> 5) + (r & 3);
  const int64_t col = (int64_t)(t % tiles_n) * kBN + kTN * wn + 32 * ni + (l0 & 31);
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

// Split reduction with a factor per (split, row): out = sum_s f[s][row] U_s in split
// order (the whole-step sweep's rescaling, f = gamma e^(m_s - lse)).
__global__ void __launch_bounds__(kReduceThreads)
scaled_reduce_kernel(const float* __restrict__ ws, const float* __restrict__ factors,
                     int64_t rows_pad, int tiles, int tiles_n, int splits, int64_t M, int64_t N,
                     float* __restrict__ out, int64_t ldo) {
  constexpr int kBlocksPerTile = (int)(kTileFloats / (4 * kReduceThreads));
  const int t = blockIdx.x / kBlocksPerTile;
  const int e0 = ((blockIdx.x % kBlocksPerTile) * kReduceThreads + threadIdx.x) * 4;
  const int l0 = e0 & 63;
  const int r = (e0 >> 6) & 15;
  const int blk = e0 >> 10;
  const int wave = blk / (kMI * kNI), mi = (blk / kNI) % kMI, ni = blk % kNI;
  const int wm = wave / kWN, wn = wave % kWN;
  const int64_t row = (int64_t)(t / tiles_n) * kBM + 128 * wm + 32 * mi + 8 * (r >> 2) +
                      4 * (l0 >> 5) + (r & 3);
  const int64_t col = (int64_t)(t % tiles_n) * kBN + kTN * wn + 32 * ni + (l0 & 31);
  if (row >= M || col >= N) return;
  const float* src = ws + (int64_t)t * kTileFloats + e0;
  float f = factors[row];
  float4 v = *reinterpret_cast<const float4*>(src);
  float4 a = make_float4(f * v.x, f * v.y, f * v.z, f * v.w);
  for (int s = 1; s < splits; ++s) {
    f = factors[(int64_t)s * rows_pad + row];
    v = *reinterpret_cast<const float4*>(src + (int64_t)s * tiles * kTileFloats);
    a.x = __builtin_fmaf(f, v.x, a.x);
    a.y = __builtin_fmaf(f, v.y, a.y);
    a.z = __builtin_fmaf(f, v.z, a.z);
    a.w = __builtin_fmaf(f, v.w, a.w);
  }
  *reinterpret_cast<float4*>(out + row * ldo + col) = a;
}

// One-pass reduction.  Split s holds the partial U_s of probabilities taken against a
// reference m_s, with Z_s and S1_s against the same reference and its maximum M_s
// (stats[s][row] = {m_s, Z_s, S1_s, M_s}).  At the overall maximum M = max_s M_s:
//   f_s = e^(m_s - M),  Z = sum_s f_s Z_s,  out = gamma sum_s f_s U_s / Z,
//   lse = M + ln Z,  H = ln Z - sum_s f_s (S1_s + (m_s - M) Z_s) / Z,
//   argmax = the position of the first split reaching M (splits are in vocabulary
// order).  The splits are visited in order, so the result is bitwise repeatable.
__global__ void __launch_bounds__(256)
onepass_reduce_kernel(const float* __restrict__ ws, const float4* __restrict__ stats,
                      const int32_t* __restrict__ stat_arg, int64_t rows_pad, int tiles,
                      int tiles_n, int splits, int64_t M, int64_t N, float gamma, int64_t col0,
                      float* __restrict__ out, int64_t ldo, float* __restrict__ row_max,
                      float* __restrict__ row_lse, float* __restrict__ row_entropy,
                      int32_t* __restrict__ row_argmax) {
  constexpr int kBlocksPerTile = (int)(kTileFloats / (4 * 256));
  const int t = blockIdx.x / kBlocksPerTile;
  const int e0 = ((blockIdx.x % kBlocksPerTile) * 256 + threadIdx.x) * 4;
  const int l0 = e0 & 63;
  const int r = (e0 >> 6) & 15;
  const int blk = e0 >> 10;
  const int wave = blk / (kMI * kNI), mi = (blk / kNI) % kMI, ni = blk % kNI;
  const int wm = wave / kWN, wn = wave % kWN;
  const int64_t row = (int64_t)(t / tiles_n) * kBM + 128 * wm + 32 * mi + 8 * (r >> 2) +
                      4 * (l0 >> 5) + (r & 3);
  const int64_t col = (int64_t)(t % tiles_n) * kBN + kTN * wn + 32 * ni + (l0 & 31);
  if (row >= M || col >= N) return;
  float mx = -INFINITY;
  int arg = 0;
  for (int sp = 0; sp < splits; ++sp) {
    const float ms = stats[sp * rows_pad + row].w;
    if (ms > mx) { mx = ms; arg = stat_arg[sp * rows_pad + row]; }
  }
  float z = 0.f, s1 = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* src = ws + (int64_t)t * kTileFloats + e0;
  for (int sp = 0; sp < splits; ++sp) {
    const float4 st = stats[sp * rows_pad + row];
    const float d = st.x - mx;
    const float f = exp2_hw(d * kLog2e);
    z = fmaf(f, st.y, z);
    s1 = fmaf(f, fmaf(d, st.y, st.z), s1);
    const float4 v = *reinterpret_cast<const float4*>(src + (int64_t)sp * tiles * kTileFloats);
    a.x = fmaf(f, v.x, a.x); a.y = fmaf(f, v.y, a.y);
    a.z = fmaf(f, v.z, a.z); a.w = fmaf(f, v.w, a.w);
  }
  const float g = gamma / z;
  *reinterpret_cast<float4*>(out + row * ldo + col) = make_float4(g * a.x, g * a.y, g * a.z, g * a.w);
  if (col == 0) {
    const float lz = logf(z);
    row_max[row] = mx;
    row_lse[row] = mx + lz;
    row_entropy[row] = lz - s1 / z;
    row_argmax[row] = (int32_t)(col0 + arg);
  }
}


__global__ void zero_rows_kernel(float* __restrict__ out, int64_t ldo, int64_t N) {
  const int64_t row = blockIdx.y;
  const int64_t c = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (c < N) *reinterpret_cast<float4*>(out + row * ldo + c) = make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace

namespace {

// ---- contraction of bf16 probabilities: ping-pong waves, operands straight into LDS -----
// For bf16 probabilities, super-step-tiled (the staged, whole-step and one-pass calls) or
// row-major (se_soft_embed); bf16 table, or e4m3 table (W8) with one row tile.  Same 8
// waves, wave tiles, MFMAs, k order and partial layout as soft_embed_kernel, so the results
// are bit for bit the same; the schedule differs:
//   - Waves 0-3 (group 0) and 4-7 (group 1), one of each per SIMD, run a phase apart.  A
//     32-position step is two phases per wave: M (the step's fragments read from LDS, loads
//     for later steps issued) and C (its 16 MFMAs, at raised wave priority).  While one
//     group is in C the other is in M, so each SIMD's matrix core has a wave to feed it
//     while the other wave waits on LDS and memory.  Every phase ends with a workgroup
//     barrier; group 1 takes one extra barrier before its loop and group 0 one after it.
//   - Operands go from memory to LDS with buffer_load ... lds: no staging registers and no
//     LDS writes in the loop.  Group 0 loads the probability stages (64 positions, 32 KB,
//     two buffers, a whole stage in the M phase of every other step); group 1 the table
//     steps (32 positions, 16 KB, ring of four, three steps ahead).
//   - Every buffer is its own LDS array and the barriers are plain s_barrier with the wait
//     counts written out (empty asm memory clobbers keep LDS accesses on their side), so a
//     wave waits only for the loads the next phases read.
// When a step's data lands, for step s (group 0's M(s) follows barrier 2 s, group 1's one
// barrier later):
//   - group 0 loads stage t + 1 in M(2 t) into the buffer stage t - 1 held (released by
//     group 1's M(2 t - 1)) and waits for it at the end of C(2 t + 1);
//   - group 1 loads table step s + 3 in M(s) into the buffer of step s - 1 (released by its
//     own M(s - 1)) and, keeping its last 8 loads in flight, has step s + 1 in LDS at the
//     end of M(s).
// Splits of at least kThreeStageMin super-steps (bf16 table) take a third probability
// stage buffer, in the 32 KB the e4m3 code ring uses otherwise: group 0 then loads stage
// t + 2 in two halves, in M(2 t) and M(2 t + 1), into the buffer stage t - 1 held, and waits
// for stage t + 1 at the end of C(2 t + 1) with stage t + 2's 8 loads still in flight.  Half
// a stage per M phase instead of a whole one every other phase keeps group 0's M phases
// short of the other group's MFMAs, and the stage arrives a step earlier.  The loop is
// unrolled over the three-buffer cycle so that every buffer is a distinct LDS array at
// compile time (with run-time buffer offsets the compiler cannot tell the stage loads from
// the fragment reads and serialises them).  Same MFMAs in the same order: bitwise equal.
// Short splits (the one-rank slice) keep two buffers: there the longer prologue and the
// extra tail loads cost more than the schedule gains (measured).
constexpr int kPPStage = 64;                      // positions per probability stage
constexpr int kPPStageBytes = kBM * kPPStage * 2; // [256 rows][64 positions] bf16
constexpr int kPPStepBytes = kBK * kBN * 2;       // [32 rows][256 columns] bf16
constexpr int kThreeStageMin = 32;                // super-steps of a split for three stages
static_assert(3 * kPPStageBytes + 4 * kPPStepBytes <= 160 * 1024, "LDS budget of one CU");
// probability stage: row m at 128 m bytes, 16-byte chunk c (8 positions) at c ^ pp_swz(m).
// A fragment read takes one chunk of 32 consecutive rows; the swizzle gives every 8 (and
// every 16) consecutive rows distinct 16-byte slots of a 128-byte (256-byte) bank line.
__device__ __forceinline__ int pp_swz(int m) { return ((m >> 1) ^ ((m & 1) << 2)) & 7; }
__device__ __forceinline__ int pp_off(int m, int c) { return m * 128 + 16 * (c ^ pp_swz(m)); }
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// An LDS array of its own for each tag.  Loads into one and reads of another stay apart: the
// compiler tells LDS objects apart, but not two ranges of one object that a buffer load
// fills, and it would wait for such loads before every read.
template <int Tag, int Bytes>
__device__ __forceinline__ unsigned char* lds_array() {
  __shared__ __attribute__((aligned(16))) unsigned char a[Bytes];
  return a;
}

// s_waitcnt with vmcnt(n) and lgkmcnt(0) (expcnt not waited on)
template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | ((n >> 4) << 14));
}
// Workgroup barrier once this wave's LDS reads are complete and all but its n most recent
// memory loads have landed.  The scheduling barriers keep every instruction on its side of
// the phase boundary; the asm clobbers keep memory accesses there (s_barrier is no fence).
template <int n>
__device__ __forceinline__ void phase_end() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  wait_vm_lgkm0<n>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
constexpr int kNoVmWait = 63;
constexpr int kPP8RawBytes = kBK * kBN;           // [32 rows][256 columns] e4m3 codes
static_assert(4 * kPP8RawBytes == kPPStageBytes, "the e4m3 code ring fills the third stage buffer");
static_assert(3 * kPPStageBytes + 4 * kPP8RawBytes <= 160 * 1024, "LDS budget of the D8 form");
// codes read in place (D8): step row k at 256 k bytes, 16-byte chunk c (16 columns) at
// c ^ d8_swz(k).  A transpose read of 16 lanes takes 8 consecutive rows (k = 8 j .. 8 j + 7)
// of one chunk; the swizzle puts those rows in 8 chunks distinct modulo 8, and the rows of
// the neighbouring chunk (c ^ 1) in the 8 other chunks of the 256-byte line.
__device__ __forceinline__ int d8_swz(int k) { return (k & 7) | ((k & 1) << 3); }
typedef int v2i32_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i32_t* lds_v2i32_ptr;
// s_waitcnt with vmcnt(n) only
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// TABLE_NT: the table loads carry the nontemporal hint.  Right when one row tile reads each
// table row once; with several row tiles the others re-read it, and cached loads let them
// find it in L2.
// W8: the table is e4m3 codes with a power-of-two scale per row.  Group 1 loads a step's
// codes into a raw buffer (ring of four, three steps ahead) and the scales of its rows into
// registers; two M phases later each wave converts the rows it loaded itself (so a wait on
// its own loads suffices) to bf16, exactly as soft_embed_kernel's e4m3 producer does, into
// the step's table buffer, one step before anyone reads it.
// D8: e4m3 codes again, with the probabilities already multiplied by the row scales (the
// product P[m, k] s_k is exact in bf16, as s_k is a power of two).  Group 1 loads a step's
// codes like a bf16 step, and the M phases read the fragments from the codes themselves
// with transpose reads of 8 codes, turned into bf16 by unscaled conversions in registers:
// no conversion pass and half the table bytes in LDS.
template <bool TABLE_NT, bool W8, bool D8>
__global__ void __launch_bounds__(kGemmThreads)
__attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
soft_embed_pp_kernel(const GemmParams p) {
  static_assert(kWaves == 8 && kMI == 4 && kNI == 2 && kWN == 4, "the 8-wave layout");
  static_assert(!(W8 && D8), "one e4m3 form");
  constexpr bool RAW = W8 || D8;                  // the table as e4m3 codes
  __shared__ __attribute__((aligned(16))) unsigned char P0[kPPStageBytes], P1[kPPStageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char W0[kPPStepBytes], W1[kPPStepBytes];
  __shared__ __attribute__((aligned(16))) unsigned char W2[kPPStepBytes], W3[kPPStepBytes];
  // the third probability stage (bf16 table and D8, long splits), and the e4m3 codes of
  // four steps ([32 rows][256 codes]; W8: row r at 256 r as loaded, D8: swizzled): each its
  // own LDS array, declared only in the forms that use it
  unsigned char *P2 = nullptr, *R0 = nullptr, *R1 = nullptr, *R2 = nullptr, *R3 = nullptr;
  if constexpr (RAW) {
    R0 = lds_array<10, kPP8RawBytes>();
    R1 = lds_array<11, kPP8RawBytes>();
    R2 = lds_array<12, kPP8RawBytes>();
    R3 = lds_array<13, kPP8RawBytes>();
  }
  if constexpr (!W8) P2 = lds_array<2, kPPStageBytes>();
  // the table buffers the fragments read: bf16 steps (W8: converted), or D8's codes
  unsigned char* const T0 = D8 ? R0 : W0;
  unsigned char* const T1 = D8 ? R1 : W1;
  unsigned char* const T2 = D8 ? R2 : W2;
  unsigned char* const T3 = D8 ? R3 : W3;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = wave >> 2, q = wave & 3;
  const int wm = wave / kWN, wn = wave % kWN;
  const int b = xcd_local_order((int)blockIdx.x, (int)gridDim.x);
  const int t = b % p.tiles;
  const int s = b / p.tiles;
  const int m0 = (t / p.tiles_n) * kBM;
  const int n0 = (t % p.tiles_n) * kBN;
  const int N = (int)p.N;
  // this split's vocab range [k_lo, k_hi): nq whole super-steps, then (last split only)
  // the remaining positions
  const int64_t k_lo = (((int64_t)s * p.kblocks) / p.splits) * kSplitQuantum;
  const int64_t k_hi = min((((int64_t)(s + 1) * p.kblocks) / p.splits) * kSplitQuantum, p.K);
  const int nq = (int)((min(k_hi, (p.K / kSS) * kSS) - k_lo) / kSS);
  const int nsteps = kQ * nq;
  const bool three = !W8 && nq >= kThreeStageMin;   // the same for every wave of the workgroup
  // rows of this tile that exist; rows past them load row tile_rows - 1 again (finite data,
  // every load in bounds) and are never written out
  const int tile_rows = min(kBM, (int)p.M - m0);

  // probabilities: position k of the tile's row m at (k / 128) a_blk + m a_rs + 2 (k % 128)
  // bytes from a_base; super-step-tiled (a_blk = rows * 256, a_rs = 256) or row-major
  // (a_blk = 256, a_rs = 2 lda, a_base at column col0).  The main loop reads whole
  // super-steps only, so no load reaches past the slice.
  const bool a_tiled = p.a_ss != (int64_t)kSuperStep * 2;
  const int64_t a_blk = a_tiled ? p.M * (int64_t)kSuperStep * 2 : (int64_t)kSuperStep * 2;
  const int64_t a_rs = a_tiled ? (int64_t)kSuperStep * 2 : p.lda * 2;
  const unsigned char* a_base =
      static_cast<const unsigned char*>(p.a) +
      (a_tiled ? (int64_t)m0 * kSuperStep * 2 : ((int64_t)m0 * p.lda + p.col0) * 2);
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(
      a_base, (uint32_t)min(a_tiled ? ((p.K + kSuperStep - 1) / kSuperStep - 1) * a_blk +
                                          (int64_t)kBM * kSuperStep * 2
                                    : (kBM - 1) * a_rs + p.K * 2,
                            (int64_t)UINT32_MAX));
  const int64_t w_ld = p.ldw * (RAW ? 1 : 2);
  const __amdgpu_buffer_rsrc_t w_rsrc =
      make_rsrc(static_cast<const unsigned char*>(p.w) + k_lo * w_ld,
                (uint32_t)min((k_hi - k_lo) * w_ld, (int64_t)UINT32_MAX));
  // e4m3 table: one fp32 (power-of-two) scale per shard row
  const __amdgpu_buffer_rsrc_t s_rsrc =
      make_rsrc(W8 ? static_cast<const void*>(p.wscale + k_lo) : p.w,
                W8 ? (uint32_t)min((k_hi - k_lo) * 4, (int64_t)UINT32_MAX) : 0u);
  // Each load moves 64 lanes x 16 bytes into 1 KB of LDS, lane l at byte 16 l.
  //   group 0, wave q: stage rows 64 q .. + 63, 8 rows per load; lane l of load i writes row
  //     64 q + 8 i + l / 8, stored chunk l % 8, which holds logical chunk (l % 8) ^ pp_swz(row)
  //   group 1, wave q: step rows 8 q .. + 7, 2 rows per load; lane l of load i writes row
  //     8 q + 2 i + l / 32, stored chunk l % 32, which holds column chunk (l % 32) ^ 4 (row % 4)
  uint32_t voff[8];
  if (grp == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 64 * q + 8 * i + (lane >> 3);
      voff[i] = (uint32_t)(min(r, tile_rows - 1) * a_rs) + 16u * (uint32_t)((lane & 7) ^ pp_swz(r));
    }
  } else if constexpr (!RAW) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = 8 * q + 2 * i + (lane >> 5);
      const int col = n0 + 8 * ((lane & 31) ^ (4 * (k & 3)));
      voff[i] = (uint32_t)(k * w_ld) + 2u * (uint32_t)min(col, N - 8);
    }
#pragma unroll
    for (int i = 4; i < 8; ++i) voff[i] = 0u;
  } else if constexpr (D8) {
    // wave q loads step rows 8 q .. + 7, 4 rows per load: lane l of load i writes row
    // k = 8 q + 4 i + l / 16, stored chunk l % 16, which holds column chunk (l % 16) ^ d8_swz(k)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int k = 8 * q + 4 * i + (lane >> 4);
      const int col = n0 + 16 * ((lane & 15) ^ d8_swz(k));
      voff[i] = (uint32_t)(k * w_ld) + (uint32_t)min(col, N - 16);
    }
#pragma unroll
    for (int i = 2; i < 8; ++i) voff[i] = 0u;
  } else {
    // e4m3: wave q loads step rows 8 q .. + 7 as codes, 4 rows per load (lane l of load i:
    // row 8 q + 4 i + l / 16, columns 16 (l % 16) .. + 15), and the scales of its rows
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int k = 8 * q + 4 * i + (lane >> 4);
      voff[i] = (uint32_t)(k * w_ld) + (uint32_t)min(n0 + 16 * (lane & 15), N - 16);
      voff[2 + i] = 4u * (uint32_t)k;
    }
#pragma unroll
    for (int i = 4; i < 8; ++i) voff[i] = 0u;
  }
  // loads past the last stage or step repeat the last one (into a buffer no later phase reads)
  auto load_stage = [&](unsigned char* buf, int ps) {
    const int64_t k0 = k_lo + (int64_t)kPPStage * min(ps, 2 * nq - 1);
    const uint32_t soff = (uint32_t)((k0 / kSuperStep) * a_blk + 2 * (k0 % kSuperStep));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_void_ptr)(buf + 1024 * (8 * q + i)),
                                               16, voff[i], soff, 0, 0);
  };
  // half h of that stage: each wave's rows 64 q + 32 h .. + 31
  auto load_half = [&](unsigned char* buf, int ps, int h) {
    const int64_t k0 = k_lo + (int64_t)kPPStage * min(ps, 2 * nq - 1);
    const uint32_t soff = (uint32_t)((k0 / kSuperStep) * a_blk + 2 * (k0 % kSuperStep));
#pragma unroll
    for (int i = 4 * h; i < 4 * h + 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_void_ptr)(buf + 1024 * (8 * q + i)),
                                               16, voff[i], soff, 0, 0);
  };
  auto load_step = [&](unsigned char* buf, int st) {
    const uint32_t soff = (uint32_t)((int64_t)kBK * min(st, nsteps - 1) * w_ld);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, (lds_void_ptr)(buf + 1024 * (4 * q + i)),
                                               16, voff[i], soff, 0, TABLE_NT ? 2 : 0);
  };
  // D8: codes of step st, 2 loads per wave
  auto load_step_d8 = [&](unsigned char* raw, int st) {
    const uint32_t soff = (uint32_t)((int64_t)kBK * min(st, nsteps - 1) * w_ld);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, (lds_void_ptr)(raw + 1024 * (2 * q + i)),
                                               16, voff[i], soff, 0, TABLE_NT ? 2 : 0);
  };
  // a table step into its buffer (bf16 or D8); group 1's wait for the step after the one in
  // use leaves the two later steps' loads in flight
  auto load_tab = [&](unsigned char* buf, int st) {
    if constexpr (D8) load_step_d8(buf, st);
    else load_step(buf, st);
  };
  constexpr int kTabWait = D8 ? 4 : 8;
  // e4m3: codes of step st into a raw buffer, the scales of the wave's rows into sc
  auto load_step8 = [&](unsigned char* raw, int st, float (&sc)[2]) {
    const int64_t k0 = (int64_t)kBK * min(st, nsteps - 1);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, (lds_void_ptr)(raw + 1024 * (2 * q + i)), 16,
                                               voff[i], (uint32_t)(k0 * w_ld), 0, TABLE_NT ? 2 : 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) sc[i] = buffer_load_f1(s_rsrc, voff[2 + i], (uint32_t)(4 * k0));
  };
  // e4m3: the wave's own rows of a raw step, times their scales, as bf16 into a table buffer
  // (the layout soft_embed_kernel's e4m3 producer writes)
  auto convert8 = [&](const unsigned char* raw, unsigned char* wb, const float (&sc)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 c = *reinterpret_cast<const uint4*>(raw + 1024 * (2 * q + i) + 16 * lane);
      const int k = 8 * q + 4 * i + (lane >> 4), col = 16 * (lane & 15);
      uint4 lo, hi;
      fp8x16_to_bf16(c, sc[i], lo, hi);
      *reinterpret_cast<uint4*>(wb + w_off(k, col)) = lo;
      *reinterpret_cast<uint4*>(wb + w_off(k, col + 8)) = hi;
    }
  };
  float sc0[2], sc1[2], sc2[2], sc3[2];

  f32x16 acc[kMI][kNI];
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  // fragments of substep u (16 positions) of a step held in half h of a stage: A row
  // 128 wm + 32 mi + lane % 32, positions 32 h + 16 u + 8 (lane / 32) .. +7; B as in
  // soft_embed_kernel
  const int a_row = 128 * wm + (lane & 31);
  uint32_t b_rd[kNI];
  {
    const int g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      if constexpr (D8) {
        // 16 lanes read rows 8 (g / 2) + i / 2 (8 codes each, half i % 2 of the chunk);
        // lane 16 g + j receives column j of the chunk's 8 rows
        const int k = 8 * (g >> 1) + (i >> 1);
        const int c = (kTN * wn + 32 * ni) / 16 + (g & 1);
        b_rd[ni] = (uint32_t)(256 * k + 16 * (c ^ d8_swz(k)) + 8 * (i & 1));
      } else {
        b_rd[ni] = (uint32_t)w_off(8 * (g >> 1) + (i >> 2), kTN * wn + 32 * ni + 16 * (g & 1) + 4 * (i & 3));
      }
    }
  }
  bf16x8 a0[kMI], b0[kNI], a1[kMI], b1[kNI];
  auto frag = [&](const unsigned char* pb, const unsigned char* wb, int h, int u, bf16x8 (&af)[kMI],
                  bf16x8 (&bf)[kNI]) {
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
      af[mi] = *reinterpret_cast<const bf16x8*>(pb + pp_off(a_row + 32 * mi, 4 * h + 2 * u + (lane >> 5)));
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      if constexpr (D8) {
        // 8 codes (rows 16 u + 8 (lane / 32) .. + 7 of one column), exact in bf16
        const v2i32_t c = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (lds_v2i32_ptr)(wb + b_rd[ni] + 4096 * u));
        const uint4 v = make_uint4(fp8x2_to_bf16x2((uint32_t)c.x, 1.f, false),
                                   fp8x2_to_bf16x2((uint32_t)c.x, 1.f, true),
                                   fp8x2_to_bf16x2((uint32_t)c.y, 1.f, false),
                                   fp8x2_to_bf16x2((uint32_t)c.y, 1.f, true));
        bf[ni] = __builtin_bit_cast(bf16x8, v);
      } else {
        const unsigned char* wp = wb + b_rd[ni] + 8192 * u;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(wp));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(wp + 2048));
        bf[ni] = __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo),
                                         __builtin_bit_cast(bf16x4_t, hi), 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
  };
  auto mfmas = [&](const bf16x8 (&af)[kMI], const bf16x8 (&bf)[kNI]) {
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
  };
  auto m_phase = [&](const unsigned char* pb, const unsigned char* wb, int h) {
    frag(pb, wb, h, 0, a0, b0);
    frag(pb, wb, h, 1, a1, b1);
  };
  auto c_phase = [&]() {
    __builtin_amdgcn_s_setprio(1);
    mfmas(a0, b0);
    mfmas(a1, b1);
    __builtin_amdgcn_s_setprio(0);
  };

  // three stages: super-step qd with stage 2 qd in pa, 2 qd + 1 in pb, and stage 2 qd + 2
  // loaded into pc (the buffer stage 2 qd - 1 held), stage 2 qd + 3 into pa
  auto g0_super = [&](int qd, unsigned char* pa, unsigned char* pb, unsigned char* pc) {
    load_half(pc, 2 * qd + 2, 0);
    m_phase(pa, T0, 0);
    phase_end<kNoVmWait>();
    c_phase();
    phase_end<kNoVmWait>();
    load_half(pc, 2 * qd + 2, 1);
    m_phase(pa, T1, 1);
    phase_end<kNoVmWait>();
    c_phase();
    phase_end<8>();                             // stage 2 qd + 1 in LDS
    load_half(pa, 2 * qd + 3, 0);
    m_phase(pb, T2, 0);
    phase_end<kNoVmWait>();
    c_phase();
    phase_end<kNoVmWait>();
    load_half(pa, 2 * qd + 3, 1);
    m_phase(pb, T3, 1);
    phase_end<kNoVmWait>();
    c_phase();
    phase_end<8>();                             // stage 2 qd + 2 in LDS
  };
  auto g1_super = [&](int qd, unsigned char* pa, unsigned char* pb) {
    const int s0 = kQ * qd;
    load_tab(T3, s0 + 3);
    m_phase(pa, T0, 0);
    phase_end<kTabWait>();                      // table step s0 + 1 in LDS
    c_phase();
    phase_end<kNoVmWait>();
    load_tab(T0, s0 + 4);
    m_phase(pa, T1, 1);
    phase_end<kTabWait>();
    c_phase();
    phase_end<kNoVmWait>();
    load_tab(T1, s0 + 5);
    m_phase(pb, T2, 0);
    phase_end<kTabWait>();
    c_phase();
    phase_end<kNoVmWait>();
    load_tab(T2, s0 + 6);
    m_phase(pb, T3, 1);
    phase_end<kTabWait>();
    c_phase();
    phase_end<kNoVmWait>();
  };

  if (nq > 0) {
    if (grp == 0) {
      load_stage(P0, 0);
      if (three) load_stage(P1, 1);
    } else if constexpr (!W8) {
      load_tab(T0, 0);
      load_tab(T1, 1);
      load_tab(T2, 2);
    } else {
      load_step8(R0, 0, sc0);
      load_step8(R1, 1, sc1);
      load_step8(R2, 2, sc2);
    }
    if (three && grp == 0)
      phase_end<8>();                           // stage 0 in LDS; stage 1 may be in flight
    else
      phase_end<0>();
    if constexpr (W8) {                         // table step 0 as bf16 before anyone reads it
      if (grp == 1) convert8(R0, W0, sc0);
      phase_end<0>();
    }
    if (three) {
      // buffers of stages 2 qd, 2 qd + 1, 2 qd + 2 for qd = 0, 1, 2 (mod 3)
      int qd = 0;
      if (grp == 0) {
        for (; qd + 3 <= nq; qd += 3) {
          g0_super(qd, P0, P1, P2);
          g0_super(qd + 1, P2, P0, P1);
          g0_super(qd + 2, P1, P2, P0);
        }
        if (qd < nq) g0_super(qd, P0, P1, P2);
        if (qd + 1 < nq) g0_super(qd + 1, P2, P0, P1);
        phase_end<kNoVmWait>();                 // pairs with group 1's first barrier
      } else {
        phase_end<kNoVmWait>();                 // one phase behind group 0
        for (; qd + 3 <= nq; qd += 3) {
          g1_super(qd, P0, P1);
          g1_super(qd + 1, P2, P0);
          g1_super(qd + 2, P1, P2);
        }
        if (qd < nq) g1_super(qd, P0, P1);
        if (qd + 1 < nq) g1_super(qd + 1, P2, P0);
      }
    } else if (grp == 0) {
      for (int qd = 0; qd < nq; ++qd) {         // steps 4 qd .. 4 qd + 3: stages 2 qd, 2 qd + 1
        load_stage(P1, 2 * qd + 1);
        m_phase(P0, T0, 0);
        phase_end<kNoVmWait>();
        c_phase();
        phase_end<kNoVmWait>();
        m_phase(P0, T1, 1);
        phase_end<kNoVmWait>();
        c_phase();
        phase_end<0>();                         // stage 2 qd + 1 in LDS
        load_stage(P0, 2 * qd + 2);
        m_phase(P1, T2, 0);
        phase_end<kNoVmWait>();
        c_phase();
        phase_end<kNoVmWait>();
        m_phase(P1, T3, 1);
        phase_end<kNoVmWait>();
        c_phase();
        phase_end<0>();                         // stage 2 qd + 2 in LDS
      }
      phase_end<kNoVmWait>();                   // pairs with group 1's first barrier
    } else {
      phase_end<kNoVmWait>();                   // one phase behind group 0
      for (int qd = 0; qd < nq; ++qd) {
        const int s0 = kQ * qd;
        if constexpr (!W8) {
          load_tab(T3, s0 + 3);
          m_phase(P0, T0, 0);
          phase_end<kTabWait>();                // table step s0 + 1 in LDS
          c_phase();
          phase_end<kNoVmWait>();
          load_tab(T0, s0 + 4);
          m_phase(P0, T1, 1);
          phase_end<kTabWait>();
          c_phase();
          phase_end<kNoVmWait>();
          load_tab(T1, s0 + 5);
          m_phase(P1, T2, 0);
          phase_end<kTabWait>();
          c_phase();
          phase_end<kNoVmWait>();
          load_tab(T2, s0 + 6);
          m_phase(P1, T3, 1);
          phase_end<kTabWait>();
          c_phase();
          phase_end<kNoVmWait>();
        } else {
          // step s: codes of step s + 3 requested; step s + 1's (requested two M phases
          // ago: at most the 8 later loads may be in flight) converted into its buffer
          load_step8(R3, s0 + 3, sc3);
          m_phase(P0, W0, 0);
          wait_vm<8>();
          convert8(R1, W1, sc1);
          phase_end<kNoVmWait>();
          c_phase();
          phase_end<kNoVmWait>();
          load_step8(R0, s0 + 4, sc0);
          m_phase(P0, W1, 1);
          wait_vm<8>();
          convert8(R2, W2, sc2);
          phase_end<kNoVmWait>();
          c_phase();
          phase_end<kNoVmWait>();
          load_step8(R1, s0 + 5, sc1);
          m_phase(P1, W2, 0);
          wait_vm<8>();
          convert8(R3, W3, sc3);
          phase_end<kNoVmWait>();
          c_phase();
          phase_end<kNoVmWait>();
          load_step8(R2, s0 + 6, sc2);
          m_phase(P1, W3, 1);
          wait_vm<8>();
          convert8(R0, W0, sc0);
          phase_end<kNoVmWait>();
          c_phase();
          phase_end<kNoVmWait>();
        }
      }
    }
  }
  // no load may still be writing LDS when the tail reuses the buffers or the waves end
  phase_end<0>();

  // ---- the last split's remaining positions, 32 at a time, with guarded loads ---------
  for (int64_t k0 = k_lo + (int64_t)kSS * nq; k0 < k_hi; k0 += kBK) {
    // probabilities: 256 rows x 4 chunks of 8 positions, 2 per thread
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = tid + kGemmThreads * j;
      const int row = e >> 2, c = e & 3;
      const int64_t kk = k0 + 8 * c;
      const uint16_t* hp = reinterpret_cast<const uint16_t*>(
          a_base + (kk / kSuperStep) * a_blk + min(row, tile_rows - 1) * a_rs + 2 * (kk % kSuperStep));
      uint32_t v[8];
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) v[e8] = (kk + e8 < p.K) ? (uint32_t)hp[e8] : 0u;
      *reinterpret_cast<uint4*>(P0 + pp_off(row, c)) =
          make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
    }
    if constexpr (D8) {
      // codes: 32 rows x 16 chunks of 16 columns, one per thread, in the swizzled layout
      // (rows past the slice: zero codes)
      const int k = tid >> 4, c = tid & 15;
      const int64_t kr = k0 + k;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (kr < p.K)
        v = *reinterpret_cast<const uint4*>(static_cast<const unsigned char*>(p.w) + kr * w_ld +
                                            min(n0 + 16 * c, N - 16));
      *reinterpret_cast<uint4*>(R0 + 256 * k + 16 * (c ^ d8_swz(k))) = v;
    } else if constexpr (!W8) {
      // table: 32 rows x 32 chunks of 8 columns, 2 per thread
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = tid + kGemmThreads * j;
        const int k = e >> 5, c = e & 31;
        const int64_t kr = k0 + k;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (kr < p.K)
          v = *reinterpret_cast<const uint4*>(static_cast<const unsigned char*>(p.w) + kr * w_ld +
                                              2 * (int64_t)min(n0 + 8 * c, N - 8));
        *reinterpret_cast<uint4*>(W0 + w_off(k, 8 * c)) = v;
      }
    } else {
      // e4m3 table: 32 rows x 16 pieces of 16 codes, one per thread, converted with the
      // row's scale (rows past the slice: zeros)
      const int k = tid >> 4, col = 16 * (tid & 15);
      const int64_t kr = k0 + k;
      uint4 lo = make_uint4(0u, 0u, 0u, 0u), hi = lo;
      if (kr < p.K) {
        const uint4 c = *reinterpret_cast<const uint4*>(static_cast<const unsigned char*>(p.w) +
                                                        kr * w_ld + min(n0 + col, N - 16));
        fp8x16_to_bf16(c, p.wscale[kr], lo, hi);
      }
      *reinterpret_cast<uint4*>(W0 + w_off(k, col)) = lo;
      *reinterpret_cast<uint4*>(W0 + w_off(k, col + 8)) = hi;
    }
    __syncthreads();
    m_phase(P0, T0, 0);
    mfmas(a0, b0);
    mfmas(a1, b1);
    __syncthreads();
  }

  // ---- epilogue, as soft_embed_kernel's ------------------------------------------------
  if (p.splits == 1 && !p.keep_partials) {
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni) {
        const int col = n0 + kTN * wn + 32 * ni + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + 128 * wm + 32 * mi + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (col < N && row < (int)p.M) p.out[(int64_t)row * p.ldo + col] = p.gamma * acc[mi][ni][r];
        }
      }
  } else {
    float* dst = p.ws + ((int64_t)s * p.tiles + t) * kTileFloats;
    constexpr int kMF = kMI * kNI;
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dst[((wave * kMF + mi * kNI + ni) * 16 + r) * 64 + lane] = acc[mi][ni][r];
  }

  // ---- the one-read calls' range merge, in the workgroups of the shorter splits -----------
  // Their main loop ends a 128-position block before the longest split's, so the merge of
  // kWaves rows (one per wave) fits in time the launch would otherwise idle; rows are dealt
  // to those workgroups in (split, tile) order.
  if (p.merge_rows) {
    const int64_t longest = (p.kblocks + p.splits - 1) / p.splits;
    auto blocks_of = [&](int q) -> int64_t {
      return ((int64_t)(q + 1) * p.kblocks) / p.splits - ((int64_t)q * p.kblocks) / p.splits;
    };
    if (blocks_of(s) < longest) {
      int before = 0;
      for (int q = 0; q < s; ++q) before += blocks_of(q) < longest ? 1 : 0;
      const int64_t row = ((int64_t)before * p.tiles + t) * kWaves + wave;
      if (row < p.M)
        merge_ranges_row(reinterpret_cast<const float4*>(p.stats), p.stat_arg, p.M,
                         p.merge_ranges, p.merge_r0, p.splits, p.gamma, p.factors, p.row_max,
                         p.row_lse, p.row_entropy, p.row_argmax, row);
    }
  }
}

template <bool FUSED, bool W8>
hipError_t launch_contraction(const GemmParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.tiles * p.splits));
  // bf16 probabilities (staged super-step-tiled, or row-major): the ping-pong kernel (bit
  // for bit the same result).  Probabilities that carry the row scales: its form that reads
  // the codes in place, at any number of row tiles.  An e4m3 table with unscaled
  // probabilities: one row tile only (with several, the conversion, all in group 1's M
  // phase, outlasts the other group's MFMAs and the register-staged kernel is faster)
  const bool staged = p.a_ss == p.M * (int64_t)kSuperStep * 2 || p.a_ss == (int64_t)kSuperStep * 2;
  if (p.w8_direct) {                            // pre-scaled probabilities, codes read in place
    if (FUSED || !W8 || !staged) return hipErrorInvalidValue;
    if (p.tiles == p.tiles_n)
      SE_LAUNCH((soft_embed_pp_kernel<true, false, true>), grid, dim3(kGemmThreads), 0, stream, p);
    else
      SE_LAUNCH((soft_embed_pp_kernel<false, false, true>), grid, dim3(kGemmThreads), 0, stream, p);
    return hipSuccess;
  }
  if (!FUSED && staged && (!W8 || p.tiles == p.tiles_n)) {
    if (p.tiles == p.tiles_n)                   // one row tile
      SE_LAUNCH((soft_embed_pp_kernel<true, W8, false>), grid, dim3(kGemmThreads), 0, stream, p);
    else
      SE_LAUNCH((soft_embed_pp_kernel<false, W8, false>), grid, dim3(kGemmThreads), 0, stream, p);
    return hipSuccess;
  }
  if (p.merge_rows) return hipErrorInvalidValue;   // only the ping-pong kernel merges ranges
  // whole 256-row tiles take the path with per-lane addresses fixed for the kernel
  if (p.M % kBM == 0)
    SE_LAUNCH((soft_embed_kernel<FUSED, true, W8>), grid, dim3(kGemmThreads), 0, stream, p);
  else
    SE_LAUNCH((soft_embed_kernel<FUSED, false, W8>), grid, dim3(kGemmThreads), 0, stream, p);
  return hipSuccess;
}

}  // namespace

hipError_t launch_soft_embed(const GemmParams& p, bool fused, bool w8, hipStream_t stream) {
  hipError_t e;
  if (fused && w8) e = launch_contraction<true, true>(p, stream);
  else if (fused) e = launch_contraction<true, false>(p, stream);
  else if (w8) e = launch_contraction<false, true>(p, stream);
  else e = launch_contraction<false, false>(p, stream);
  if (e != hipSuccess) return e;
  e = launched(stream);
  if (e != hipSuccess || p.splits == 1 || p.keep_partials) return e;
  const int blocks = p.tiles * (int)(kTileFloats / (4 * kReduceThreads));
  SE_LAUNCH(splitk_reduce_kernel, dim3(blocks), dim3(kReduceThreads), 0, stream, p.ws,
                     p.tiles, p.tiles_n, p.splits, p.M, p.N, p.gamma, p.out, p.ldo);
  return launched(stream);
}

hipError_t launch_onepass_reduce(const GemmParams& p, float* row_max, float* row_lse,
                                 float* row_entropy, int32_t* row_argmax, int64_t col0,
                                 hipStream_t stream) {
  const int blocks = p.tiles * (int)(kTileFloats / (4 * 256));
  SE_LAUNCH(onepass_reduce_kernel, dim3(blocks), dim3(256), 0, stream, p.ws,
                     reinterpret_cast<const float4*>(p.stats), p.stat_arg, p.rows_pad, p.tiles,
                     p.tiles_n, p.splits, p.M, p.N, p.gamma, col0, p.out, p.ldo, row_max,
                     row_lse, row_entropy, row_argmax);
  return launched(stream);
}

hipError_t launch_scaled_reduce(const GemmParams& p, const float* factors, hipStream_t stream) {
  const int blocks = p.tiles * (int)(kTileFloats / (4 * kReduceThreads));
  SE_LAUNCH(scaled_reduce_kernel, dim3(blocks), dim3(kReduceThreads), 0, stream, p.ws,
                     factors, p.rows_pad, p.tiles, p.tiles_n, p.splits, p.M, p.N, p.out, p.ldo);
  return launched(stream);
}

hipError_t launch_zero_rows(float* out, int64_t ldo, int64_t M, int64_t N, hipStream_t stream) {
  const int64_t groups = (N + 3) / 4;
  const dim3 grid((unsigned)((groups + 255) / 256), (unsigned)M);
  SE_LAUNCH(zero_rows_kernel, grid, dim3(256), 0, stream, out, ldo, N);
  return launched(stream);
}

}  // namespace se
