// Paged prefill attention for 16-bit caches (gfx950): the step before decode.
//
// A chunk of a sequence's new tokens attends causally over the sequence's
// whole context -- its earlier tokens and the chunk itself, whose keys and
// values were written through the slots first -- read through the block
// table like decode ("Paged Attention as a Memory Manager", §How the Kernel
// Executes Paged Attention: at prefill each new sequence gets its logical
// blocks in order; "Paged Attention: Virtual Memory for the KV Cache", §The
// fix borrowed from operating systems).  Query token t of a chunk of L tokens
// in a context of P sits at position P - L + t and sees positions 0 .. its
// own: textbook causal attention (the pages give no formula), i.e. for each
// token exactly the decode result at that length.
//
// Work decomposition.  One workgroup per (sequence, kv head, block of
// 64 CB / group query tokens); its four waves each own CB blocks of 16
// matrix-core columns, the (query token, query head) pairs of 16 / group
// tokens of the kv head's group per block.  The workgroup streams the
// 16-token K/V tiles of the positions its tokens can see through an 8-slot
// LDS ring filled by direct global->LDS loads, each wave loading a quarter of
// every tile, so every K/V byte read serves 64 CB columns (CB = 2 or 3 for
// long chunks: more flops per byte streamed; CB = 1 keeps short chunks
// spread over many workgroups).  Per tile, wave and column block:
// S^T = K Q^T with v_mfma_f32_16x16x32 (the K operand read once for all
// blocks), a causal limit per column (skipped where every key of the tiles
// is visible to every column of the block), an online softmax over a lazy
// reference maximum (the exponent folds the scale in as one fma; the
// reference is raised to the column's exact maximum only when a lane's
// weights of a step sum past 2^15, which leaves no maximum on the common
// path), P rounded to fp16 for one P V product into O^T; a block none of
// whose columns sees the tiles skips them.  A workgroup covers its tokens'
// whole prefix, and many workgroups run at once (but for the context split
// below).
//
// P V in fp16.  The weights are at most 2^15 and keep 11 significant bits
// (bf16 would keep 8, too few for the 2e-3 bound); the values are converted
// to fp16 once per workgroup, in LDS, by the wave that loaded them, while the
// pair before them computes.  bf16 values fp16 cannot hold as they are (a
// group of 32 dims whose largest magnitude so far is 2^16 or more, or below
// 2^-10) are held as v 2^frame with a power-of-two frame per group; the
// group's accumulators follow its frame, which never grows once a nonzero
// value was seen, so they only ever shrink (exactly, but for what falls below
// fp32's range).
//
// Context split.  A launch of few workgroups (short chunks of few sequences)
// may cut each sequence's prefix into pieces streamed by workgroups of their
// own (grid z, the last piece first); each piece leaves its columns' partial
// states (reference maximum, weight sum, unnormalised output) in a
// workspace, and prefill_merge_kernel combines them by log-sum-exp.  The
// pieces end before the chunk's first position, so every column sees at
// least the first key of every piece.
//
// Tiles go in pairs: one softmax step covers 32 keys (one cross-lane
// reduction and one rescale check per 32 keys), and P V is one
// v_mfma_f32_16x16x32 per 16 value dims over both tiles (on gfx950 twice the
// rate of the 16x16x16 form over one tile): key k = 8 q + i of the product
// is key 4 q + i of the first tile for i < 4, of the second for i >= 4, in
// both operands.  Registers are held to two waves per SIMD.
#include <type_traits>

#include "pa_device.h"
#include "pa_kernels.h"
#include "prefill_split.h"

namespace pa {

namespace {

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// LDS reads of the ring and the block ids.  As volatile LDS accesses the
// compiler keeps them where they are (after the explicit waits and the
// barrier) and does not add a wait for every direct load still in flight.
template <class V>
__device__ __forceinline__ V ring_read(const uint8_t* p) {
  return *(const volatile __attribute__((address_space(3))) V*)(p);
}
template <class V>
__device__ __forceinline__ void ring_write(uint8_t* p, const V& v) {
  *(volatile __attribute__((address_space(3))) V*)(p) = v;
}

// Sum of the eight fp16 values of h in fp32 (products by one are exact).
// The pairs are taken with shuffles: reading them as the 32-bit words of a
// bit cast of h made this compiler (ROCm 7.2) use the first word four times.
__device__ __forceinline__ float sum8_f16(const f16x8& h) {
  const f16x2 one = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
  float a = __builtin_amdgcn_fdot2(__builtin_shufflevector(h, h, 0, 1), one, 0.f, false);
  float b = __builtin_amdgcn_fdot2(__builtin_shufflevector(h, h, 2, 3), one, 0.f, false);
  a = __builtin_amdgcn_fdot2(__builtin_shufflevector(h, h, 4, 5), one, a, false);
  b = __builtin_amdgcn_fdot2(__builtin_shufflevector(h, h, 6, 7), one, b, false);
  return a + b;
}

// Power-of-two frame of a half of the values, from the largest exponent e
// (the unbiased exponent field) of its values so far: values are held in
// fp16 as v 2^frame.  0 while e is in [-10, 15] (every bf16 value converts
// exactly or, below 2^-14, within 2^-25 of an absolute error) or no nonzero
// value was seen (e = kNoExp), else the frame that puts 2^e at 2^14.  The
// frame never grows once a nonzero value was seen, so the accumulators only
// ever shrink when it changes.
constexpr int kNoExp = -(1 << 20);
__device__ __forceinline__ int fp16_frame(int e) {
  return (e == kNoExp || (e >= -10 && e <= 15)) ? 0 : 14 - e;
}

// The bf16 magnitude (bits, sign cleared) from which a value can change the
// frame of a group whose largest exponent so far is e: any nonzero value
// while none was seen, 2^16 while e is in [-10, 15], else 2^(e + 1) (the
// infinity bits at most, so that infinities and NaN always take the exact
// path).
__device__ __forceinline__ uint32_t fp16_frame_threshold(int e) {
  if (e == kNoExp) return 1u;
  if (e >= -10 && e <= 15) return 0x4780u;
  return uint32_t(min(e + 128, 255)) << 7;
}

// Wait until this wave's loads of the oldest tiles in flight have landed,
// when k newer tiles (LPW loads each) may stay in flight (k uniform, at most
// KMAX).
template <int LPW, int KMAX>
__device__ __forceinline__ void wait_oldest_tile(int k) {
  if constexpr (KMAX > 0) {
    if (k >= KMAX) {
      vm_wait<KMAX * LPW>();
      return;
    }
    wait_oldest_tile<LPW, KMAX - 1>(k);
  } else {
    vm_wait<0>();
  }
}

template <class T, int D, int BS, int G, int CB, bool SPLITK, bool ONCE = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(PrefillArgs a, PrefillSplitArgs sp) {
  using bits = typename T::bits;
  using MF = MfmaOps<T>;
  using PV = MfmaOps<F16>;             // P V in fp16 whatever the cache type
  constexpr bool kBf16 = std::is_same_v<T, BF16>;
  // bf16 values with three column blocks are converted to fp16 in LDS for
  // one P V product (the conversion pays off over that many columns); other
  // bf16 shapes split P into a bf16 high part and the rounded remainder for
  // two products; fp16 values take one fp16 product as they are
  constexpr bool CONV = kBf16 && CB == 3;
  constexpr bool SPLIT = kBf16 && !CONV;
  constexpr int TB = 16 / G;           // query tokens per column block
  constexpr int TQ = CB * TB;          // per wave
  constexpr int TQW = 4 * TQ;          // per workgroup
  constexpr int NS = D / 32;           // QK slices of 32 dims
  constexpr int NT = D / 16;           // PV row tiles of 16 dims
  constexpr int KI = D / 32;           // 1 KiB loads per K (and per V) tile
  constexpr int LPW = 2 * KI / 4;      // loads per wave per tile
  // ring slots: four pairs of tiles (the split variant, whose launches hold
  // about 2048 workgroups, three: 6 slots keep three workgroups per compute
  // unit where 8 allow two)
  constexpr int NSL = SPLITK ? 6 : 8;
  constexpr int IDCAP = 512;           // tiles whose block ids are staged at once
  static_assert(kPrefillRankMax % 4 == 0 && kPrefillRankMax <= 256 && 2 * IDCAP - 1 >= kPrefillRankMax, "rank scratch");
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  static_assert(LPW >= 1 && LPW * (NSL - 1) < 64, "loads per wave");
  // the ring is the dynamic LDS array, a separate object from the block ids,
  // so the compiler can tell that its direct loads never write s_ids; reads
  // of a landed slot are ordered by the explicit waits below
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  constexpr int SLOT = 2 * KI * 1024;
  __shared__ __attribute__((aligned(16))) int2 s_ids[IDCAP];   // (16-byte reads of the ranked lengths)
  __shared__ __attribute__((aligned(16))) int s_frame[2][4];   // per pair parity and group of 32 dims: the values' frame

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int c = lane & 15;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  // Sequences go in order of decreasing context (ties by index): grid y
  // counts (rank, kv head), so the workgroups of the longest contexts are
  // dispatched first and the launch's tail holds short ones (with the index
  // order a long sequence dispatched last left most compute units idle).
  // Each workgroup ranks the lengths itself, in the block-id array before
  // it is staged: one comparison per sequence and thread, up to
  // kPrefillRankMax sequences (more keep the index order).
  const int h = blockIdx.y % Hkv;
  int s = blockIdx.y / Hkv;
  if (a.num_seqs <= kPrefillRankMax) {
    // [0, B): lengths (-1 past B, up to a multiple of 4), [2 IDCAP - 1]: the
    // sequence of rank s
    int* rk = reinterpret_cast<int*>(s_ids);
    const int B = a.num_seqs;
    const int t = threadIdx.x;
    if (t < ((B + 3) & ~3)) rk[t] = t < B ? min(max(a.ctx[t], 0), a.max_ctx) : -1;
    __syncthreads();
    if (t < B) {
      const int pt = rk[t];
      int rank = 0;
      for (int u = 0; u < B; u += 4) {
        const int4 pu = *reinterpret_cast<const int4*>(rk + u);
        rank += (pu.x > pt || (pu.x == pt && u + 0 < t)) ? 1 : 0;
        rank += (pu.y > pt || (pu.y == pt && u + 1 < t)) ? 1 : 0;
        rank += (pu.z > pt || (pu.z == pt && u + 2 < t)) ? 1 : 0;
        rank += (pu.w > pt || (pu.w == pt && u + 3 < t)) ? 1 : 0;
      }
      if (rank == s) rk[2 * IDCAP - 1] = t;
    }
    __syncthreads();
    s = uniform(rk[2 * IDCAP - 1]);
    __syncthreads();                             // (the array is the block ids' next)
  }
  const int qs = a.query_start[s];
  const int P = min(max(a.ctx[s], 0), a.max_ctx);
  const int L = min(max(a.query_start[s + 1] - qs, 0), P);
  const int tq0 = blockIdx.x * TQW;
  if (tq0 >= L) return;                          // (whole workgroup)
  const int p0 = P - L;                          // position of the chunk's first token
  const int kmax = p0 + min(L, tq0 + TQW);       // positions the workgroup's tokens see
  const int nt = (kmax + 15) / 16;
  // Context split (SPLITK, launches with few workgroups, which take one
  // column block): piece z of S streams tiles [z SPL, (z + 1) SPL) and the
  // last one every tile from (S - 1) SPL on.  The pieces but the last end
  // before the chunk's first position, so every column sees every key of
  // those and the first key of the last one.  A split sequence leaves each
  // piece's partial state in the workspace for the merge.  (Without SPLITK
  // the bounds are the constants 0 and nt: runtime bounds cost the
  // three-block kernel 2%.)
  const int S = SPLITK ? p0 / (16 * sp.split_tiles) + 1 : 1;
  if (SPLITK && int(blockIdx.z) >= S) return;       // (whole workgroup)
  const int zp = SPLITK ? S - 1 - int(blockIdx.z) : 0;   // the longest piece first
  const int tb = SPLITK ? zp * sp.split_tiles : 0;       // tiles [tb, te) (tb even)
  const int te = SPLITK && zp < S - 1 ? tb + sp.split_tiles : nt;

  // this lane's column in block cb: token cb TB + j of the wave, head gc of
  // the group
  const int tw0 = tq0 + wave * TQ;
  const int j = c / G, gc = c % G;
  bool col_valid[CB];
  int lim[CB];                                   // causal limit of the column (exclusive)
  int64_t qrow[CB];
  u32x4 qop[CB][NS];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    col_valid[cb] = tw0 + cb * TB + j < L;
    const int tok = min(tw0 + cb * TB + j, L - 1);  // (a spare column repeats the last token)
    lim[cb] = p0 + tok + 1;
    qrow[cb] = (int64_t(qs) + tok) * Hq + int64_t(h) * G + gc;
    const bits* qp = static_cast<const bits*>(a.q) + qrow[cb] * D;
#pragma unroll
    for (int m = 0; m < NS; ++m) qop[cb][m] = *reinterpret_cast<const u32x4*>(qp + (4 * m + q) * 8);
  }
  // the last position any column of block cb sees, and the causal limit of
  // its first column, below which no key of the block is masked (both
  // uniform over the wave)
  int blk_last[CB], blk_open[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    blk_last[cb] = uniform(p0 + min(L, tw0 + (cb + 1) * TB) - 1);
    blk_open[cb] = uniform(p0 + min(tw0 + cb * TB, L - 1) + 1);
  }
  // scores are taken raw and scaled inside the exponent, which needs a
  // positive factor: a negative scale flips the sign of q (exact), a zero
  // one zeroes q and scales by 1 (every score is 0 either way)
  const float sraw = a.scale_log2;
  const uint32_t qflip = sraw < 0.f ? 0x80008000u : 0u;
  const uint32_t qkeep = sraw == 0.f ? 0u : 0xFFFFFFFFu;
  const float sf = sraw == 0.f ? 1.f : fabsf(sraw);
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int m = 0; m < NS; ++m)
#pragma unroll
      for (int w = 0; w < 4; ++w) qop[cb][m][w] = (qop[cb][m][w] & qkeep) ^ qflip;
  // the query loads complete here, in a wait the compiler knows about
  // (vmcnt 0; expcnt and lgkmcnt at their maxima): otherwise it waits for
  // every load in flight before each tile's first product
  __builtin_amdgcn_s_waitcnt(0x0F70);

  const int32_t* row = a.tables + int64_t(s) * a.table_stride;
  const bits* kpool = static_cast<const bits*>(a.k);
  const bits* vpool = static_cast<const bits*>(a.v);
  // block ids of tiles [from, from + IDCAP) (the whole workgroup)
  int id_base = 0;
  auto stage_ids = [&](int from) {
    const int n = min(IDCAP, te - from);
    for (int i = threadIdx.x; i < n; i += 256) {
      const int t = from + i;
      int2 ids;
      if constexpr (BS == 16) {
        ids.x = ids.y = row[t];
      } else if constexpr (BS == 32) {
        ids.x = ids.y = row[t >> 1];
      } else {
        ids.x = row[2 * t];
        ids.y = 16 * t + 8 < kmax ? row[2 * t + 1] : ids.x;
      }
      s_ids[i] = ids;
    }
    id_base = from;
  };
  // this wave's share of the loads of tile t into its slot: with D = 128
  // K load w and V load w (its own group of 32 value dims), with D = 64 load
  // w (waves 2 and 3 the values)
  auto issue = [&](int t) {
    uint8_t* sl = ring + (t % NSL) * SLOT;
    const int b0 = uniform(ring_read<int32_t>(reinterpret_cast<const uint8_t*>(&s_ids[t - id_base].x)));
    const int b1 = uniform(ring_read<int32_t>(reinterpret_cast<const uint8_t*>(&s_ids[t - id_base].y)));
#pragma unroll
    for (int ii = 0; ii < LPW; ++ii) {
      const int i = LPW == 1 ? wave : ii * KI + wave;   // load i of the tile's 2 KI
      if (i < KI) {
        const int u = i * 64 + lane;
        const int jj = u >> 4, tt = u & 15;
        int blk, tk;
        if constexpr (BS == 16) {
          blk = b0;
          tk = tt;
        } else if constexpr (BS == 32) {
          blk = b0;
          tk = 16 * (t & 1) + tt;
        } else {
          blk = tt < 8 ? b0 : b1;
          tk = tt & 7;
        }
        const int64_t e = ((int64_t(blk) * Hkv + h) * (D / 8) + jj) * (BS * 8) + tk * 8;
        if constexpr (ONCE) dma16_once(kpool + e, sl + i * 1024);
        else dma16(kpool + e, sl + i * 1024);
      } else {
        const int u = (i - KI) * 64 + lane;
        const int d = u >> 1, hh = u & 1;
        int blk, tk0;
        if constexpr (BS == 16) {
          blk = b0;
          tk0 = 8 * hh;
        } else if constexpr (BS == 32) {
          blk = b0;
          tk0 = 16 * (t & 1) + 8 * hh;
        } else {
          blk = hh ? b1 : b0;
          tk0 = 0;
        }
        const int64_t e = ((int64_t(blk) * Hkv + h) * D + d) * BS + tk0;
        if constexpr (ONCE) dma16_once(vpool + e, sl + i * 1024);
        else dma16(vpool + e, sl + i * 1024);
      }
    }
  };

  f32x4 acc[CB][NT];
  float m_ref[CB], l_lane[CB];                   // (reference maximum: scaled, log2 units)
  // one column block's weights of a pair for P V
  struct Weights {
    f16x8 h;                                     // rounded to fp16
    float p[SPLIT ? 8 : 1];                      // (SPLIT) in fp32
  };
  int frame[KI];                                 // accumulators of each group of 32 dims hold O 2^frame
#pragma unroll
  for (int g = 0; g < KI; ++g) frame[g] = 0;
  int vexp = kNoExp;                             // (value loaders) largest exponent of their group so far
  uint32_t vthr = 1u;                            // and the magnitude bits from which it can change
  int vfr = 0;                                   // and its frame
  const int vgrp = LPW == 1 ? wave - 2 : wave;   // the group of 32 value dims this wave loads (if in [0, KI))
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[cb][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_ref[cb] = kNegInf;
    l_lane[cb] = 0.f;
  }

  // The values of pair t in fp16, 16-dim tile n (1 KiB, laid out as the P V
  // operand: [key quad q][dim c of the tile] x 16 bytes, keys 4 q .. 4 q + 3
  // of tile t, then of tile t + 1), where the raw values of its group of 32
  // dims were: tile 2 g of group g in the value part of tile t's slot, tile
  // 2 g + 1 in that of tile t + 1.
  auto cv_tile = [&](int t, int n) __attribute__((always_inline)) {
    return ring + ((t + (n & 1)) % NSL) * SLOT + KI * 1024 + (n >> 1) * 1024;
  };

  // Every wave that loads values converts its group of 32 dims of pair t to
  // fp16 in place once its loads of the pair have landed (it reads all of
  // its bytes before it writes), zeros past the workgroup's last position
  // (which may hold anything, NaN poison included); bf16 values are held as
  // v 2^frame, the group's frame (see fp16_frame) published with the pair.
  constexpr int NH = 2;                          // 16-dim tiles per group
  auto convert_read = [&](int t, u32x4 (&w)[NH]) __attribute__((always_inline)) {
    const uint8_t* sa = ring + (t % NSL) * SLOT + KI * 1024 + vgrp * 1024;
    const uint8_t* sb = ring + ((t + 1) % NSL) * SLOT + KI * 1024 + vgrp * 1024;
#pragma unroll
    for (int n2 = 0; n2 < NH; ++n2) {
      const int d = 16 * n2 + c;                 // dim in the group
      const u32x2 va = ring_read<u32x2>(sa + d * 32 + 8 * q);
      const u32x2 vb = ring_read<u32x2>(sb + d * 32 + 8 * q);
      w[n2] = u32x4{va[0], va[1], vb[0], vb[1]};
    }
  };
  auto convert_finish = [&](int t, u32x4 (&w)[NH]) __attribute__((always_inline)) {
    if (16 * t + 32 > kmax) {
      const int kp0 = 16 * t + 4 * q;
#pragma unroll
      for (int n2 = 0; n2 < NH; ++n2) {
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
          const int k0 = kp0 + (w2 >> 1) * 16 + 2 * (w2 & 1);   // the two keys of 32-bit word w2
          uint32_t x = w[n2][w2];
          if (k0 >= kmax) x &= 0xFFFF0000u;
          if (k0 + 1 >= kmax) x &= 0x0000FFFFu;
          w[n2][w2] = x;
        }
      }
    }
    if constexpr (kBf16) {
      // the frame can change only if a magnitude reaches the group's
      // threshold (16-bit integer maxima of the bits); then the exact
      // largest magnitude of the pair updates the group's exponent
      u16x2 m16 = {0, 0};
#pragma unroll
      for (int n2 = 0; n2 < NH; ++n2)
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2)
          m16 = __builtin_elementwise_max(m16, __builtin_bit_cast(u16x2, w[n2][w2] & 0x7FFF7FFFu));
      const uint32_t mlane = max(uint32_t(m16[0]), uint32_t(m16[1]));
      if (__builtin_amdgcn_ballot_w64(mlane >= vthr)) {
        float mx = 0.f;
#pragma unroll
        for (int n2 = 0; n2 < NH; ++n2)
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2)
            mx = fmaxf(mx, fmaxf(fabsf(BF16::lo(w[n2][w2])), fabsf(BF16::hi(w[n2][w2]))));
        mx = reduce_low_bits<OpMax, 6>(mx);
        const uint32_t mb = uniform(__float_as_uint(mx));
        if (mb != 0u) vexp = uniform(max(vexp, int(mb >> 23) - 127));
        vthr = uniform(fp16_frame_threshold(vexp));
        vfr = uniform(fp16_frame(vexp));
      }
      const int fr = vfr;
      if (fr == 0) {
#pragma unroll
        for (int n2 = 0; n2 < NH; ++n2)
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2)
            w[n2][w2] = __builtin_bit_cast(
                uint32_t, f16x2{static_cast<_Float16>(BF16::lo(w[n2][w2])), static_cast<_Float16>(BF16::hi(w[n2][w2]))});
      } else {
#pragma unroll
        for (int n2 = 0; n2 < NH; ++n2)
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2)
            w[n2][w2] = __builtin_bit_cast(
                uint32_t, f16x2{static_cast<_Float16>(__builtin_amdgcn_ldexpf(BF16::lo(w[n2][w2]), fr)),
                                static_cast<_Float16>(__builtin_amdgcn_ldexpf(BF16::hi(w[n2][w2]), fr))});
      }
      if (lane == 0) ring_write<int>(reinterpret_cast<uint8_t*>(&s_frame[(t >> 1) & 1][vgrp]), fr);
    }
#pragma unroll
    for (int n2 = 0; n2 < NH; ++n2) ring_write<u32x4>(cv_tile(t, 2 * vgrp + n2) + (q * 16 + c) * 16, w[n2]);
  };
  auto convert = [&](int t) __attribute__((always_inline)) {
    u32x4 w[NH];
    convert_read(t, w);
    convert_finish(t, w);
  };

  // P V of one column block over the pair: P rounded to fp16 against fp16
  // values in one product, or (SPLIT) its bf16 high part and remainder in two
  auto pv_pair = [&](int cb, const Weights& wt, const u32x4 (&vr)[NT]) __attribute__((always_inline)) {
    if constexpr (SPLIT) {
      typename MF::v8 phi, plo;
      MF::split(wt.p, phi, plo);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        acc[cb][n] = MF::pv32(vr[n], phi, acc[cb][n]);
        acc[cb][n] = MF::pv32(vr[n], plo, acc[cb][n]);
      }
    } else {
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[cb][n] = PV::pv32(vr[n], wt.h, acc[cb][n]);
    }
  };

  // raise column block cb's reference maximum to the exact maximum of its
  // column over the pair (sv: its raw scores, masked ones -inf), rescaling
  // what was summed against the old one
  auto raise_reference = [&](int cb, const float (&sv)[8]) __attribute__((always_inline)) {
    float cm = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    cm = xor16<OpMax>(cm);
    cm = xor32<OpMax>(cm);
    const float mn = cm * sf;
    const bool up = mn > m_ref[cb];
    const float alpha = up ? (m_ref[cb] == kNegInf ? 0.f : fast_exp2(m_ref[cb] - mn)) : 1.f;
    m_ref[cb] = up ? mn : m_ref[cb];
    l_lane[cb] *= alpha;
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[cb][n] *= alpha;
  };

  // exponents of the raw scores sv against block cb's reference, rounded to
  // fp16 (SPLIT: kept in fp32) with their sum (ps)
  auto weights = [&](int cb, const float (&sv)[8], Weights& wt, float& ps) __attribute__((always_inline)) {
    if constexpr (SPLIT) {
#pragma unroll
      for (int i = 0; i < 8; ++i) wt.p[i] = fast_exp2(__builtin_fmaf(sv[i], sf, -m_ref[cb]));
      ps = ((wt.p[0] + wt.p[1]) + (wt.p[2] + wt.p[3])) + ((wt.p[4] + wt.p[5]) + (wt.p[6] + wt.p[7]));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) wt.h[i] = static_cast<_Float16>(fast_exp2(__builtin_fmaf(sv[i], sf, -m_ref[cb])));
      ps = sum8_f16(wt.h);
    }
  };

  // one softmax step over tiles t, t + 1 (OPEN: every key of the pair is
  // visible to every column of the wave, and the reference maxima are finite)
  auto pair_step = [&](int t, auto open_tag) __attribute__((always_inline)) {
    constexpr bool OPEN = decltype(open_tag)::value;
    const uint8_t* sa = ring + (t % NSL) * SLOT;
    const uint8_t* sb = ring + ((t + 1) % NSL) * SLOT;
    const int kp0 = 16 * t + 4 * q;              // keys kp0 .. + 3 (tile t), kp0 + 16 .. + 19 (tile t + 1)
    f32x4 sc[CB][2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const uint8_t* sl = h2 ? sb : sa;
      u32x4 kr[NS];
#pragma unroll
      for (int m = 0; m < NS; ++m) kr[m] = ring_read<u32x4>(sl + ((4 * m + q) * 16 + c) * 16);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        sc[cb][h2] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (!OPEN) {
          if (16 * t > blk_last[cb]) continue;
        }
#pragma unroll
        for (int m = 0; m < NS; ++m) sc[cb][h2] = MF::qk(kr[m], qop[cb][m], sc[cb][h2]);
      }
    }
    if constexpr (CONV) {
      // the accumulators follow the frames of the values (a change, rare,
      // only ever shrinks them, exactly but for what falls below fp32's
      // range)
      const u32x4 f4 = ring_read<u32x4>(reinterpret_cast<const uint8_t*>(&s_frame[(t >> 1) & 1][0]));
      int fr[KI];
      bool moved = false;
#pragma unroll
      for (int g = 0; g < KI; ++g) {
        fr[g] = uniform(int(f4[g]));
        moved = moved || fr[g] != frame[g];
      }
      if (moved) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[cb][n][i] = __builtin_amdgcn_ldexpf(acc[cb][n][i], fr[n >> 1] - frame[n >> 1]);
#pragma unroll
        for (int g = 0; g < KI; ++g) frame[g] = fr[g];
      }
    }
    // the next pair: once this wave's loads of it have landed (those of the
    // two pairs after it may stay in flight), its values are converted, the
    // vector work overlapping this pair's matrix products
    if constexpr (CONV) {
      if (t + 2 < te) {
        wait_oldest_tile<LPW, 4>(min(te, t + 8) - min(te, t + 4));
        if (vgrp >= 0 && vgrp < KI) convert(t + 2);
      }
    }
    // the pair's values, 8 keys per lane (k = 8 q + i: key kp0 + i of tile t
    // for i < 4, of tile t + 1 for i >= 4): converted, or as the slots hold
    // them with zeros past the workgroup's last position (which may hold
    // anything, NaN poison included)
    u32x4 vr[NT];
    if constexpr (CONV) {
#pragma unroll
      for (int n = 0; n < NT; ++n) vr[n] = ring_read<u32x4>(cv_tile(t, n) + (q * 16 + c) * 16);
    } else {
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const u32x2 va = ring_read<u32x2>(sa + KI * 1024 + (16 * n + c) * 32 + 8 * q);
        const u32x2 vb = ring_read<u32x2>(sb + KI * 1024 + (16 * n + c) * 32 + 8 * q);
        vr[n] = u32x4{va[0], va[1], vb[0], vb[1]};
      }
      if (!OPEN && 16 * t + 32 > kmax) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2) {
            const int k0 = kp0 + (w2 >> 1) * 16 + 2 * (w2 & 1);   // the two keys of 32-bit word w2
            uint32_t x = vr[n][w2];
            if (k0 >= kmax) x &= 0xFFFF0000u;
            if (k0 + 1 >= kmax) x &= 0x0000FFFFu;
            vr[n][w2] = x;
          }
        }
      }
    }
    if constexpr (OPEN) {
      // weights against the reference maxima as they stand; a column's
      // reference is raised to its exact maximum only when a lane's eight
      // weights sum past 2^15 (or are not a number), so that every weight
      // fits fp16; one check per block, so that the P V products of a block
      // overlap the vector work of the next
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const float sv[8] = {sc[cb][0][0], sc[cb][0][1], sc[cb][0][2], sc[cb][0][3],
                             sc[cb][1][0], sc[cb][1][1], sc[cb][1][2], sc[cb][1][3]};
        Weights wt;
        float ps;
        weights(cb, sv, wt, ps);
        if (__builtin_amdgcn_ballot_w64(!(ps <= 32768.f))) {
          raise_reference(cb, sv);
          weights(cb, sv, wt, ps);
        }
        l_lane[cb] += ps;
        pv_pair(cb, wt, vr);
      }
    } else {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        // (tile 0 holds position 0, which every column sees, so no block
        // skips the first pair: m_ref is finite from then on and masked terms
        // give exp2(-inf) = 0)
        if (16 * t > blk_last[cb]) continue;
        float sv[8];
        if (16 * t + 32 <= blk_open[cb]) {
          // every key of the pair is visible to every column of the block
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sv[i] = sc[cb][0][i];
            sv[4 + i] = sc[cb][1][i];
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sv[i] = kp0 + i < lim[cb] ? sc[cb][0][i] : kNegInf;
            sv[4 + i] = kp0 + 16 + i < lim[cb] ? sc[cb][1][i] : kNegInf;
          }
        }
        // weights against the column's reference maximum as it stands; it is
        // raised (to the column's exact maximum, over its four lanes) only
        // when a lane's eight weights sum past 2^15 or are not finite (the
        // first step, whose reference is -inf): no maximum at all on the
        // common path
        Weights wt;
        float ps;
        weights(cb, sv, wt, ps);
        if (__builtin_amdgcn_ballot_w64(!(ps <= 32768.f))) {
          raise_reference(cb, sv);
          weights(cb, sv, wt, ps);
        }
        l_lane[cb] += ps;
        pv_pair(cb, wt, vr);
      }
    }
  };

  stage_ids(tb);
  __syncthreads();
  // refill the slots of tiles t + i, i in [I0, I0 + 2) (the pair before
  // the one computing)
  auto refill = [&](int t, auto i0_tag) __attribute__((always_inline)) {
    constexpr int I0 = decltype(i0_tag)::value;
#pragma unroll
    for (int i = I0; i < I0 + 2; ++i) {
      const int tn = t + i;
      if (tn < te) {
        if (tn >= id_base + IDCAP) {
          // next window of block ids (every slot's loads have landed: the
          // compiler waits for the table reads before the LDS writes)
          stage_ids(tn);
          lgkm_wait0();
          wg_barrier();
        }
        issue(tn);
      }
    }
  };
  // Tiles go in pairs (32 keys per softmax step).  CONV: pair p computes from
  // slots 2p, 2p + 1 (mod 8), its values converted while pair p - 1
  // computed; pair p + 1 lands and is converted during pair p, pair p + 2 is
  // in flight and pair p + 3 fills the slots of pair p - 1.  Otherwise pair p
  // computes from slots 2p, 2p + 1 (mod NSL) while the next NSL / 2 - 2 pairs
  // are in flight and the one after them fills the slots of pair p - 1.
#pragma unroll
  for (int i = 0; i < NSL - 2; ++i)
    if (tb + i < te) issue(tb + i);
  if constexpr (CONV) {
    // the first pair's values, before any math
    wait_oldest_tile<LPW, 4>(min(te, tb + 6) - min(te, tb + 2));
    if (vgrp >= 0 && vgrp < KI) convert(tb);
    lgkm_wait0();
    wg_barrier();
  }
  auto advance = [&](int t, auto open_tag) __attribute__((always_inline)) {
    if constexpr (CONV) {
      // refill, compute (converting the next pair), then finish this wave's
      // LDS writes and meet the others: past the barrier every wave is done
      // with this pair and the next one is landed and converted
      refill(t, std::integral_constant<int, 6>{});
      pair_step(t, open_tag);
      lgkm_wait0();
      wg_barrier();
    } else {
      // this wave's loads of tiles t and t + 1 have landed once at most its
      // loads of the newer tiles are outstanding; the barrier then covers
      // every wave's share (and every wave is done with the previous pair,
      // whose slots are refilled next)
      wait_oldest_tile<LPW, NSL - 4>(min(te - 1, t + NSL - 3) - min(te - 1, t + 1));
      wg_barrier();
      refill(t, std::integral_constant<int, NSL - 2>{});
      pair_step(t, open_tag);
    }
  };
  // Pairs past the first whose keys every column of the wave sees (those
  // before the wave's first causal limit) take the open path: no causal
  // mask, no skipped block, no zeroed values, and one rescale check for all
  // blocks, so that each phase is one straight run of code in which the
  // matrix products of one block overlap the vector work of the next.  The
  // first pair (where the reference maxima are set) and those from the
  // diagonal on take the general path: a causal limit per column, blocks
  // past their last position skipped, and a missing tile t + 1 read from a
  // stale slot with every score masked and every value selected to zero.
  // first t (even or odd) not open (no later than the end: (blk_open - 32) / 16 + 1 < nt)
  const int open_end = SPLITK ? min(te, max(tb + 2, (blk_open[0] - 32) / 16 + 1)) : max(2, (blk_open[0] - 32) / 16 + 1);
  int t = tb;
  advance(t, std::false_type{});
  for (t = tb + 2; t < open_end; t += 2) advance(t, std::true_type{});
  for (; t < te; t += 2) advance(t, std::false_type{});

#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    float l = xor16<OpSum>(l_lane[cb]);
    l = xor32<OpSum>(l);
    if (col_valid[cb] && S > 1) {
      // this piece's partial state: reference maximum and sum of the column,
      // and its unnormalised output (the frames taken out)
      const int64_t prow =
          ((int64_t(zp) * a.num_seqs + s) * sp.rows_per_seq + tw0 + cb * TB + j) * Hq + int64_t(h) * G + gc;
      if (q == 0) *reinterpret_cast<float2*>(sp.ws_ml + 2 * prow) = float2{m_ref[cb], l};
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        f32x4 v = acc[cb][n];
        if constexpr (CONV) {
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = __builtin_amdgcn_ldexpf(v[i], -frame[n >> 1]);
        }
        *reinterpret_cast<f32x4*>(sp.ws_acc + prow * D + 16 * n + 4 * q) = v;
      }
    } else if (col_valid[cb]) {
      const float inv = 1.f / l;
      const int64_t o = qrow[cb] * D + 4 * q;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        f32x4 v = acc[cb][n] * inv;
        if constexpr (CONV) {
          const int fr = frame[n >> 1];
          if (fr != 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = __builtin_amdgcn_ldexpf(acc[cb][n][i], -fr) * inv;
          }
        }
        if (a.out_f32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + o + 16 * n) = v;
        } else {
          const uint32_t lo = T::from_f32(v[0]) | (T::from_f32(v[1]) << 16);
          const uint32_t hi = T::from_f32(v[2]) | (T::from_f32(v[3]) << 16);
          *reinterpret_cast<u32x2*>(static_cast<bits*>(a.out) + o + 16 * n) = u32x2{lo, hi};
        }
      }
    }
  }
}

// Log-sum-exp merge of the pieces of each split sequence: for every query
// token and head
//     M = max_z m_z,  out = sum_z 2^(m_z - M) acc_z / sum_z 2^(m_z - M) l_z
// over its pieces in order (the same pieces as the prefill kernel's, from the
// same lengths).  One thread per 4 output columns; grid y = sequences.
template <class T, int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillArgs a, PrefillSplitArgs sp) {
  using bits = typename T::bits;
  const int s = blockIdx.y;
  const int Hq = a.num_q_heads;
  const int qs = a.query_start[s];
  const int P = min(max(a.ctx[s], 0), a.max_ctx);
  const int L = min(max(a.query_start[s + 1] - qs, 0), P);
  const int S = (P - L) / (16 * sp.split_tiles) + 1;
  if (S == 1) return;                            // written by the prefill kernel
  constexpr int U = D / 4;
  const int64_t u = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int tok = int(u / (int64_t(Hq) * U));
  if (tok >= L || tok >= sp.rows_per_seq) return;
  const int r = int(u % (int64_t(Hq) * U));
  const int hd = r / U, d4 = r % U;
  float M = kNegInf, l = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < S; ++z) {
    const int64_t prow = ((int64_t(z) * a.num_seqs + s) * sp.rows_per_seq + tok) * Hq + hd;
    const float2 ml = *reinterpret_cast<const float2*>(sp.ws_ml + 2 * prow);
    const f32x4 v = *reinterpret_cast<const f32x4*>(sp.ws_acc + prow * D + 4 * d4);
    if (ml.x == kNegInf) continue;               // (no key: cannot happen, every piece has one)
    const float mn = fmaxf(M, ml.x);
    const float c0 = M == kNegInf ? 0.f : fast_exp2(M - mn);
    const float c1 = fast_exp2(ml.x - mn);
    l = l * c0 + ml.y * c1;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = o[i] * c0 + v[i] * c1;
    M = mn;
  }
  const float inv = 1.f / l;
  const int64_t off = (int64_t(qs + tok) * Hq + hd) * D + 4 * d4;
  if (a.out_f32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + off) = o * inv;
  } else {
    // (the fp32 output rounded: see opaque_f32)
    const uint32_t lo = T::from_f32(opaque_f32(o[0] * inv)) | (T::from_f32(opaque_f32(o[1] * inv)) << 16);
    const uint32_t hi = T::from_f32(opaque_f32(o[2] * inv)) | (T::from_f32(opaque_f32(o[3] * inv)) << 16);
    *reinterpret_cast<u32x2*>(static_cast<bits*>(a.out) + off) = u32x2{lo, hi};
  }
}

template <class T, int D, int BS, int G>
hipError_t launch_g(const PrefillArgs& a, const PrefillSplitArgs& sp, int32_t max_query_len, hipStream_t stream) {
  const int cb = prefill_column_blocks(G, max_query_len, a.num_seqs, a.num_kv_heads);
  const int tpw = 4 * cb * (16 / G);
  // the tile ring: 8 slots of K and V (6 for a split launch)
  const size_t lds = size_t(sp.split_tiles ? 6 : 8) * 2 * (D / 32) * 1024;
  // (pieces of a split context along z, the longest first)
  dim3 grid((max_query_len + tpw - 1) / tpw, a.num_seqs * a.num_kv_heads, sp.split_tiles ? sp.split_max : 1),
      block(256);
  // (a split launch has fewer workgroups than two or three column blocks
  // are chosen for: it always takes one)
  if (sp.split_tiles && cb != 1) return hipErrorInvalidValue;
  // (with one query block per sequence, no two workgroups of a sequence
  // read the same tile: the loads take the streaming policy of the decode
  // pass; a block that sequences share is still read once per sharer)
  const bool once = max_query_len <= tpw;
  if (sp.split_tiles && once) hipLaunchKernelGGL((prefill_kernel<T, D, BS, G, 1, true, true>), grid, block, lds, stream, a, sp);
  else if (sp.split_tiles) hipLaunchKernelGGL((prefill_kernel<T, D, BS, G, 1, true>), grid, block, lds, stream, a, sp);
  else if (cb == 3) hipLaunchKernelGGL((prefill_kernel<T, D, BS, G, 3, false>), grid, block, lds, stream, a, sp);
  else if (cb == 2) hipLaunchKernelGGL((prefill_kernel<T, D, BS, G, 2, false>), grid, block, lds, stream, a, sp);
  else if (once) hipLaunchKernelGGL((prefill_kernel<T, D, BS, G, 1, false, true>), grid, block, lds, stream, a, sp);
  else hipLaunchKernelGGL((prefill_kernel<T, D, BS, G, 1, false>), grid, block, lds, stream, a, sp);
  if (hipError_t e = hipGetLastError()) return e;
  if (!sp.split_tiles) return hipSuccess;
  const int64_t units = int64_t(sp.rows_per_seq) * a.num_q_heads * (D / 4);
  hipLaunchKernelGGL((prefill_merge_kernel<T, D>), dim3(static_cast<uint32_t>((units + 255) / 256), a.num_seqs),
                     dim3(256), 0, stream, a, sp);
  return hipGetLastError();
}

template <class T, int D, int BS>
hipError_t launch_b(const PrefillArgs& a, const PrefillSplitArgs& sp, int32_t group, int32_t max_query_len,
                    hipStream_t stream) {
  switch (group) {
    case 1: return launch_g<T, D, BS, 1>(a, sp, max_query_len, stream);
    case 2: return launch_g<T, D, BS, 2>(a, sp, max_query_len, stream);
    case 4: return launch_g<T, D, BS, 4>(a, sp, max_query_len, stream);
    case 8: return launch_g<T, D, BS, 8>(a, sp, max_query_len, stream);
    case 16: return launch_g<T, D, BS, 16>(a, sp, max_query_len, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class T, int D>
hipError_t launch_d(const PrefillArgs& a, const PrefillSplitArgs& sp, int32_t bs, int32_t group, int32_t max_query_len,
                    hipStream_t stream) {
  switch (bs) {
    case 8: return launch_b<T, D, 8>(a, sp, group, max_query_len, stream);
    case 16: return launch_b<T, D, 16>(a, sp, group, max_query_len, stream);
    case 32: return launch_b<T, D, 32>(a, sp, group, max_query_len, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class T>
hipError_t launch_t(const PrefillArgs& a, const PrefillSplitArgs& sp, int32_t d, int32_t bs, int32_t group,
                    int32_t max_query_len, hipStream_t stream) {
  switch (d) {
    case 64: return launch_d<T, 64>(a, sp, bs, group, max_query_len, stream);
    case 128: return launch_d<T, 128>(a, sp, bs, group, max_query_len, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill_split(const PrefillArgs& a, const PrefillSplitArgs& sp, int32_t dtype, int32_t d,
                                int32_t bs, int32_t group, int32_t max_query_len, hipStream_t stream) {
  if (max_query_len <= 0 || a.num_seqs <= 0) return hipSuccess;
  switch (dtype) {
    case 1: return launch_t<F16>(a, sp, d, bs, group, max_query_len, stream);
    case 2: return launch_t<BF16>(a, sp, d, bs, group, max_query_len, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill(const PrefillArgs& a, int32_t dtype, int32_t d, int32_t bs, int32_t group,
                          int32_t max_query_len, hipStream_t stream) {
  return launch_prefill_split(a, PrefillSplitArgs{}, dtype, d, bs, group, max_query_len, stream);
}

}  // namespace pa
