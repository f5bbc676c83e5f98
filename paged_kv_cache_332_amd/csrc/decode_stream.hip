// Paged decode attention, stream kernel for 16-bit caches (gfx950).
//
// The kernel follows each sequence's block table instead of assuming the
// sequence is contiguous ("Paged Attention: Virtual Memory for the KV Cache",
// §The fix borrowed from operating systems; glossary "What is Paged
// Attention?") and computes plain softmax attention of one query per head;
// the query heads of one grouped-query group share each K/V byte (§What it
// does not fix).
//
// Work decomposition.  An item is one (sequence, kv head) pair; its tiles are
// the 16-token slices of the sequence.  All tiles of all items are laid end to
// end (sequence-major, then kv head, then tile) and every workgroup of the
// grid -- one per compute unit, four waves each -- takes a contiguous share of
// that list, split evenly over its waves.  Shares are equal, or proportional
// to per-workgroup weights the caller derives from the busy times the kernel
// reports (compute units do not all stream at the same rate, and an even
// split leaves the fast ones idle at the end).  A wave streams across item
// boundaries without draining.  An item cut between waves leaves a partial state
// (running max, sum, unnormalised output) per wave in the workspace, written
// with plain stores; a second, small kernel merges the partial states of each
// cut item by log-sum-exp in worker order.  The kernel boundary orders the
// two, so the stream kernel needs no atomics or device-wide fences (on gfx950
// a device-scope fence writes back and invalidates the whole L2 of the XCD,
// which stalls every wave behind it).
//
// Memory pipeline.  Each wave owns a ring of NSLOT tile slots in LDS and
// fills them with direct global->LDS loads (global_load_lds_dwordx4: lane l
// writes its 16 bytes at slot + 16 l), NSLOT - 1 tiles ahead of the tile it
// computes.  The loads never occupy registers, so a wave keeps up to
// NSLOT - 1 tiles (8 KiB each for bf16, D = 128) in flight.  The compiler
// does not order these loads against later LDS reads: every wait is an
// explicit s_waitcnt on the vector-memory counter, which counts loads in
// issue order.  Per tile a wave issues DPT = 2 D / 32 loads (K then V), plus
// the query rows when the tile starts an item for that wave; waiting until at
// most DPT (NSLOT - 1) loads are outstanding therefore guarantees the oldest
// tile has landed (extra query loads only make the wait stricter).  The K/V
// loads carry the non-temporal cache policy where a tile covers whole 128-byte
// lines, which no later tile of the pass reads again (with the default policy
// the pass ran about 12% slower); at block size 32 the V lines are shared by
// two tiles and keep the default policy.
//
// Slot layout (bf16/f16, 16-byte units):
//   K  [D/8][16 tokens][8]   the MFMA A operand of S^T = K Q^T reads chunk
//                            4m + q of token c with one ds_read_b128
//   V  [D][16 tokens]        the MFMA A operand of O^T += V^T P^T reads row
//                            16n + c, tokens 4q..4q+3 with one ds_read_b64
//   Q  [GMAX][D]             the query rows of the item (when it starts)
// Both gathers work for any block size: each lane computes the physical
// address of its 16 bytes from the block ids of the tile.
//
// Math per tile (lane l = 16 q + c): as the partition kernel --
// v_mfma_f32_16x16x32 for S^T (head c, tokens 4q..4q+3 per lane), a running
// reference maximum per head refreshed only when it grows by more than 2^8,
// P split into a 16-bit high part and the rounded remainder for two
// v_mfma_f32_16x16x16 products into O^T, fp32 accumulation, tokens past the
// context masked by select.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

namespace {

// Position in the tile list: item (seq, kvh), tile t of nt, global index g.
struct Cursor {
  int64_t g;
  int seq, kvh, t, nt, ctx;
};

}  // namespace

// First tile of wave w (0..4 grid) when the T tiles are split evenly over
// the grid's workgroups and each workgroup's share evenly over its four
// waves (the split when no plan is given).
__device__ __forceinline__ int64_t stream_wave_start(int64_t T, int64_t w, int grid) {
  const int64_t b = w >> 2;
  const int64_t a0 = T * b / grid;
  const int64_t a1 = T * (b + 1) / grid;
  return a0 + (a1 - a0) * (w & 3) / 4;
}

template <class T, int D, int BS, int GMAX, int NSLOT>
__global__ __launch_bounds__(256) void decode_stream_kernel(StreamArgs sa) {
  // The tile ring is the dynamic LDS array; block ids, lengths and prefix
  // sums live in separate static arrays, so the compiler can tell that their
  // reads never alias the ring's direct loads and adds no waits for them.
  __shared__ int2 s_tbl[4][kStreamTcap];
  __shared__ int32_t s_ctx[kStreamMaxSeqs + 1];     // entry B is scratch
  __shared__ int32_t s_pre[kStreamMaxSeqs + 1];
  using bits = typename T::bits;
  using MF = MfmaOps<T>;
  using v4 = typename MF::v4;
  using el = typename MF::e;
  constexpr int NS = D / 32;                         // QK slices of 32 dims
  constexpr int NT = D / 16;                         // PV row tiles of 16 dims
  constexpr int KI = D / 32;                         // 1 KiB loads per K (and per V) tile
  constexpr int DPT = 2 * KI;                        // loads per tile
  constexpr int QI = (GMAX * D * 2 + 1023) / 1024;   // 1 KiB loads for the query rows
  constexpr int SB = (2 * KI + QI) * 1024;           // slot bytes
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  static_assert(DPT * (NSLOT - 1) < 64, "vmcnt range");

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const uint64_t t_begin = __builtin_amdgcn_s_memrealtime();
  const DecodeArgs& a = sa.d;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int c = lane & 15;
  const int B = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int G = Hq / Hkv;
  constexpr int tcap = kStreamTcap;

  uint8_t* slots = smem + wave * (NSLOT * SB);
  int2* tbl = s_tbl[wave];
  int32_t* ctxs = s_ctx;
  int32_t* pre = s_pre;                              // [B + 1] exclusive prefix of tiles

  const bits* kpool = static_cast<const bits*>(a.k);
  const bits* vpool = static_cast<const bits*>(a.v);
  const bits* qbase = static_cast<const bits*>(a.q);

  // issue the loads of one tile into slot s (ids = its block ids, the second
  // one's complement when the tile's blocks are shared and stay cached; with
  // qload the item's query rows too: the tile starts the item or the wave)
  auto issue = [&](const Cursor& cu, int s, int2 ids, bool qload) {
    uint8_t* sl = slots + s * SB;
    const bool once = ids.y >= 0;
    ids.y = once ? ids.y : ~ids.y;
    if (qload) {
      // query rows of the item; lanes past G * D read row 0 again
      const int64_t qrow = (int64_t(cu.seq) * Hq + int64_t(cu.kvh) * G) * D;
#pragma unroll
      for (int i = 0; i < QI; ++i) {
        const int u = i * 64 + lane;
        const int uu = u < G * D / 8 ? u : 0;
        dma16(qbase + qrow + int64_t(uu) * 8, sl + 2 * KI * 1024 + i * 1024);
      }
    }
    int64_t ek[KI], ev[KI];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int u = i * 64 + lane;
      const int j = u >> 4, t = u & 15;
      int blk, tok;
      if constexpr (BS == 16) {
        blk = ids.x;
        tok = t;
      } else if constexpr (BS == 32) {
        blk = ids.x;
        tok = 16 * (cu.t & 1) + t;
      } else {
        blk = t < 8 ? ids.x : ids.y;
        tok = t & 7;
      }
      ek[i] = ((int64_t(blk) * Hkv + cu.kvh) * (D / 8) + j) * (BS * 8) + tok * 8;
    }
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int u = i * 64 + lane;
      const int d = u >> 1, h = u & 1;
      int blk, tok0;
      if constexpr (BS == 16) {
        blk = ids.x;
        tok0 = 8 * h;
      } else if constexpr (BS == 32) {
        blk = ids.x;
        tok0 = 16 * (cu.t & 1) + 8 * h;
      } else {
        blk = h ? ids.y : ids.x;
        tok0 = 0;
      }
      ev[i] = ((int64_t(blk) * Hkv + cu.kvh) * D + d) * BS + tok0;
    }
    // one uniform branch per tile around the loads alone
    if (once) {
#pragma unroll
      for (int i = 0; i < KI; ++i) dma16_once(kpool + ek[i], sl + i * 1024);
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        // at block size 32 a tile holds half of each 64-byte V row and the
        // next tile reads the other half of the same lines: those stay cached
        if constexpr (BS == 32) dma16(vpool + ev[i], sl + KI * 1024 + i * 1024);
        else dma16_once(vpool + ev[i], sl + KI * 1024 + i * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < KI; ++i) dma16(kpool + ek[i], sl + i * 1024);
#pragma unroll
      for (int i = 0; i < KI; ++i) dma16(vpool + ev[i], sl + KI * 1024 + i * 1024);
    }
  };


  // This wave's share of a host plan, read with no branch around it (a
  // harmless read of the workspace without a plan) so that its latency
  // overlaps the loads of the lengths and prefix sums below: the start-up
  // is one round trip for all of them, not one per load.
  const int64_t w = int64_t(blockIdx.x) * 4 + wave;
  const int32_t* plan_src = sa.wave_start ? sa.wave_start + w : reinterpret_cast<const int32_t*>(sa.rec_ml);
  const int32_t plan_a = plan_src[0];
  const int32_t plan_b = plan_src[1];

  // ---- tiles per sequence and their prefix sums (whole workgroup) --------
  if (sa.pre_in) {
    for (int i = threadIdx.x; i <= B; i += 256) {
      // both loads issue before either is used (entry B of ctxs takes a
      // copy of length 0 and is never read; B >= 1)
      const int32_t pv = sa.pre_in[i];
      const int32_t cv = a.ctx[i < B ? i : 0];
      pre[i] = pv;
      ctxs[i] = min(max(cv, 0), a.max_ctx);
    }
    // the writes are done once lgkmcnt drains; a bare barrier does not wait
    // for other loads in flight
    lgkm_wait0();
    wg_barrier();
  } else {
    int32_t* part = reinterpret_cast<int32_t*>(&s_tbl[0][0]);  // 512 ints of scratch
    const int per = (B + 255) / 256;
    const int i0 = threadIdx.x * per;
    int sum = 0;
    for (int i = i0; i < min(B, i0 + per); ++i) {
      const int n = min(max(a.ctx[i], 0), a.max_ctx);
      ctxs[i] = n;
      sum += (n + 15) / 16;
    }
    part[threadIdx.x] = sum;
    __syncthreads();
    int* src = part;
    int* dst = part + 256;
    for (int off = 1; off < 256; off <<= 1) {
      const int v = src[threadIdx.x] + (threadIdx.x >= off ? src[threadIdx.x - off] : 0);
      dst[threadIdx.x] = v;
      __syncthreads();
      int* t = src;
      src = dst;
      dst = t;
    }
    int run = src[threadIdx.x] - sum;                  // exclusive prefix of this thread's chunk
    for (int i = i0; i < min(B, i0 + per); ++i) {
      pre[i] = run;
      run += (ctxs[i] + 15) / 16;
    }
    if (threadIdx.x == 255) pre[B] = src[255];
    __syncthreads();
  }
  const int64_t ntot = int64_t(Hkv) * pre[B];

  // sequences with no context get zero rows
  for (int s = blockIdx.x; s < B; s += gridDim.x) {
    if (ctxs[s] == 0) {
      for (int i = threadIdx.x; i < Hq * D; i += 256) {
        const int64_t o = int64_t(s) * Hq * D + i;
        if (a.out_f32) static_cast<float*>(a.out)[o] = 0.f;
        else static_cast<bits*>(a.out)[o] = 0;
      }
    }
  }

  const int64_t ga = sa.wave_start ? int64_t(plan_a) : stream_wave_start(ntot, w, gridDim.x);
  const int64_t gb = sa.wave_start ? int64_t(plan_b) : stream_wave_start(ntot, w + 1, gridDim.x);
  if (ga >= gb) {  // no workgroup barrier below this point
    if (sa.wave_time && lane == 0) {
      const int32_t t0 = static_cast<int32_t>(t_begin);
      *reinterpret_cast<int2*>(sa.wave_time + 2 * w) = make_int2(t0, t0);
    }
    return;
  }

  // ---- cursors over the tile list -----------------------------------------
  auto locate = [&](int64_t g) {
    // largest sequence whose first tile (of kv head 0) is at or before g
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (int64_t(Hkv) * pre[mid] <= g) lo = mid;
      else hi = mid - 1;
    }
    Cursor cu;
    cu.g = g;
    cu.seq = lo;
    cu.nt = pre[lo + 1] - pre[lo];
    cu.ctx = ctxs[lo];
    const int r = int(g - int64_t(Hkv) * pre[lo]);  // < Hkv * nt
    cu.kvh = r / cu.nt;
    cu.t = r - cu.kvh * cu.nt;
    return cu;
  };
  auto advance = [&](Cursor& cu) {
    ++cu.g;
    if (++cu.t < cu.nt) return;
    cu.t = 0;
    if (++cu.kvh < Hkv) return;
    cu.kvh = 0;
    do {
      ++cu.seq;
    } while (cu.seq < B && ctxs[cu.seq] == 0);
    if (cu.seq < B) {
      cu.nt = uniform(pre[cu.seq + 1] - pre[cu.seq]);
      cu.ctx = uniform(ctxs[cu.seq]);
    }
  };
  auto make_uniform = [&](Cursor& cu) {
    cu.seq = uniform(cu.seq);
    cu.kvh = uniform(cu.kvh);
    cu.t = uniform(cu.t);
    cu.nt = uniform(cu.nt);
    cu.ctx = uniform(cu.ctx);
  };

  // ---- per-item state -----------------------------------------------------
  u32x4 qop[NS];
  f32x4 acc[NT];
  float m_ref = kNegInf, l_lane = 0.f;
  Cursor item;  // item being accumulated (valid once started)
  bool have_item = false;

  auto flush = [&]() {
    float l = xor16<OpSum>(l_lane);
    l = xor32<OpSum>(l);
    const int64_t gs = int64_t(Hkv) * pre[item.seq] + int64_t(item.kvh) * item.nt;
    const int64_t ge = gs + item.nt;
    const int64_t row0 = int64_t(item.seq) * Hq + int64_t(item.kvh) * G;
    if (gs >= ga && ge <= gb) {
      if (c < G) {
        const float inv = 1.f / l;
        const int64_t o = (row0 + c) * D + 4 * q;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const f32x4 v = acc[n] * inv;
          if (a.out_f32) {
            *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + o + 16 * n) = v;
          } else {
            const uint32_t lo = T::from_f32(v[0]) | (T::from_f32(v[1]) << 16);
            const uint32_t hi = T::from_f32(v[2]) | (T::from_f32(v[3]) << 16);
            *reinterpret_cast<u32x2*>(static_cast<bits*>(a.out) + o + 16 * n) = u32x2{lo, hi};
          }
        }
      }
      return;
    }
    // partial state of a cut item: record slot 0 for the item holding this
    // wave's first tile, 1 for its last
    const int rs = (gs <= ga) ? 0 : 1;
    const int64_t rec = (w * 2 + rs) * GMAX;
    if (c < G) {
#pragma unroll
      for (int n = 0; n < NT; ++n)
        *reinterpret_cast<f32x4*>(sa.rec_acc + (rec + c) * D + 16 * n + 4 * q) = acc[n];
      if (q == 0) *reinterpret_cast<float2*>(sa.rec_ml + (rec + c) * 2) = float2{m_ref, l};
    }
  };

  // compute the tile in slot s at cursor cu
  auto compute = [&](const Cursor& cu, int s) {
    const uint8_t* sl = slots + s * SB;
    if (cu.t == 0 || cu.g == ga) {
      if (have_item) flush();
      item = cu;
      have_item = true;
      m_ref = kNegInf;
      l_lane = 0.f;
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      // B operand Q^T: head c, d-chunk 4m + q
#pragma unroll
      for (int m = 0; m < NS; ++m) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(sl + 2 * KI * 1024 + (min(c, G - 1) * (D / 8) + 4 * m + q) * 16);
        qop[m] = c < G ? v : u32x4{0u, 0u, 0u, 0u};
      }
    }
    u32x4 kr[NS];
    u32x2 vr[NT];
#pragma unroll
    for (int m = 0; m < NS; ++m) kr[m] = *reinterpret_cast<const u32x4*>(sl + ((4 * m + q) * 16 + c) * 16);
#pragma unroll
    for (int n = 0; n < NT; ++n) vr[n] = *reinterpret_cast<const u32x2*>(sl + KI * 1024 + (16 * n + c) * 32 + 8 * q);

    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NS; ++m) sc = MF::qk(kr[m], qop[m], sc);
    const int tok0 = 16 * cu.t + 4 * q;
    const bool partial = 16 * cu.t + 16 > cu.ctx;
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = (!partial || tok0 + i < cu.ctx) ? sc[i] * a.scale_log2 : kNegInf;
    float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mt = xor16<OpMax>(mt);
    mt = xor32<OpMax>(mt);
    const bool need = mt > m_ref + 8.f;
    if (__builtin_amdgcn_ballot_w64(need)) {
      // a new reference maximum for the heads that need it; one within 2^8
      // of the stale reference is kept (every term of a head scales alike)
      const float alpha = need ? (m_ref == kNegInf ? 0.f : fast_exp2(m_ref - mt)) : 1.f;
      m_ref = need ? mt : m_ref;
      l_lane *= alpha;
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sv[i] - m_ref);
    l_lane += (p[0] + p[1]) + (p[2] + p[3]);
    v4 phi, plo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const el h = static_cast<el>(p[i]);
      phi[i] = h;
      plo[i] = static_cast<el>(p[i] - static_cast<float>(h));
    }
    if (partial) {
      // tokens past the context may hold anything (NaN poison included):
      // select zeros instead of multiplying by a zero weight
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        uint32_t w0 = vr[n][0], w1 = vr[n][1];
        if (tok0 + 0 >= cu.ctx) w0 &= 0xFFFF0000u;
        if (tok0 + 1 >= cu.ctx) w0 &= 0x0000FFFFu;
        if (tok0 + 2 >= cu.ctx) w1 &= 0xFFFF0000u;
        if (tok0 + 3 >= cu.ctx) w1 &= 0x0000FFFFu;
        vr[n] = u32x2{w0, w1};
      }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      acc[n] = MF::pv(vr[n], phi, acc[n]);
      acc[n] = MF::pv(vr[n], plo, acc[n]);
    }
  };

  // ---- passes of at most tcap tiles: stage block ids, then stream ---------
  const int32_t* tables = a.tables;
  // (without shared counts the lengths are read instead and not used, so
  // that no branch stands around the load)
  const int32_t* shr_src = sa.shared ? sa.shared : a.ctx;
  for (int64_t pa0 = ga; pa0 < gb; pa0 += tcap) {
    const int n = int(min(int64_t(tcap), gb - pa0));
    // block ids of each tile of the pass (BS 8: two blocks per tile; the
    // second is the first again when it holds no context token)
    // all table reads of the pass are issued before the first is used (one
    // round trip, not one per 64 tiles)
    // (the values are only combined at the LDS writes, so no load waits for
    // another)
    // (the positions are found first and the loads issued after them: a
    // load in flight across the search loop makes the compiler wait for it)
    constexpr int kIdIters = (tcap + 63) / 64;
    int32_t idx[kIdIters], idy[kIdIters], shr[kIdIters], bi[kIdIters], sq[kIdIters], tt[kIdIters];
    bool two[kIdIters];
#pragma unroll
    for (int j = 0; j < kIdIters; ++j) {
      const int i = lane + 64 * j;
      two[j] = false;
      sq[j] = 0;
      tt[j] = 0;
      if (i < n) {
        const Cursor cu = locate(pa0 + i);
        sq[j] = cu.seq;
        tt[j] = cu.t;
        // the second block of a tile at block size 8 only when it holds a
        // context token (else an in-range entry is read and not used)
        two[j] = BS == 8 && 16 * cu.t + 8 < cu.ctx;
      }
      // first block of the tile, against the sequence's shared blocks
      bi[j] = BS == 16 ? tt[j] : BS == 32 ? tt[j] >> 1 : 2 * tt[j];
    }
#pragma unroll
    for (int j = 0; j < kIdIters; ++j) {
      const int i = lane + 64 * j;
      shr[j] = 0;
      if (i < n) {
        const int32_t* row = tables + int64_t(sq[j]) * a.table_stride;
        shr[j] = shr_src[sq[j]];
        idx[j] = row[bi[j]];
        if constexpr (BS == 8) idy[j] = row[two[j] ? bi[j] + 1 : bi[j]];
      }
    }
#pragma unroll
    for (int j = 0; j < kIdIters; ++j) {
      const int i = lane + 64 * j;
      if (i < n) {
        const int32_t y = BS == 8 && two[j] ? idy[j] : idx[j];
        tbl[i] = int2{idx[j], sa.shared && bi[j] < shr[j] ? ~y : y};
      }
    }
    lgkm_wait0();
    __builtin_amdgcn_wave_barrier();

    Cursor ic = locate(pa0);
    make_uniform(ic);
    Cursor cc = ic;
#pragma unroll
    for (int i = 0; i < NSLOT - 1; ++i) {
      if (i < n) {
        const int2 ids = tbl[i];
        issue(ic, i, int2{uniform(ids.x), uniform(ids.y)}, ic.t == 0 || ic.g == ga);
        advance(ic);
      }
    }
    for (int k = 0; k < n; ++k) {
      const int kn = k + NSLOT - 1;
      if (kn < n) {
        // the slot of tile k - 1: its LDS reads finished before its math ran
        lgkm_wait0();
        const int2 ids = tbl[kn];
        issue(ic, kn % NSLOT, int2{uniform(ids.x), uniform(ids.y)}, ic.t == 0 || ic.g == ga);
        advance(ic);
        vm_wait<DPT*(NSLOT - 1)>();
      } else {
        vm_wait<0>();
      }
      compute(cc, k % NSLOT);
      advance(cc);
    }
  }
  if (have_item) flush();
  if (sa.wave_time && lane == 0)
    *reinterpret_cast<int2*>(sa.wave_time + 2 * w) =
        make_int2(static_cast<int32_t>(t_begin), static_cast<int32_t>(__builtin_amdgcn_s_memrealtime()));
}

// Log-sum-exp merge of one item (sequence seq, kv head kvh) that the stream
// kernel cut between waves, from the partial states the waves recorded:
//     M = max_w m_w,  out = sum_w 2^(m_w - M) acc_w / sum_w 2^(m_w - M) l_w
// taken in wave order (so the result does not depend on timing), a batch of
// R waves at a time with the running maximum carried between batches.
// next(w) yields the item's waves in order, starting with w0, and returns
// false after the last; w0 holds its state in record slot r0 (1 when the item
// starts inside its range), every later wave in slot 0.
template <class T, int D, int GMAX, class Next>
__device__ __forceinline__ void merge_item(const StreamArgs& sa, int seq, int kvh, int64_t w0, int r0, Next next) {
  using bits = typename T::bits;
  const DecodeArgs& a = sa.d;
  const int lane = threadIdx.x;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int G = Hq / Hkv;
  const int64_t row0 = int64_t(seq) * Hq + int64_t(kvh) * G;
  // each lane merges units idx = lane + 64 u (4 output columns each) of the
  // G x D item; a batch's loads are in flight together
  constexpr int NU = (GMAX * D / 4 + 63) / 64;
  constexpr int R = 4;
  const int units = G * (D / 4);
  float M[NU], L[NU];
  f32x4 O[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    M[u] = kNegInf;
    L[u] = 0.f;
    O[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto rec_of = [&](int64_t wi, int j) { return (wi * 2 + (wi == w0 ? r0 : 0)) * GMAX + j; };
  bool more = true;
  while (more) {
    int64_t wr[R];       // the next R waves (w0 again past the last, unused)
    bool live[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int64_t x = w0;
      live[r] = more && next(x);
      more = live[r];
      wr[r] = live[r] ? x : w0;
    }
    // one round trip per batch: every record's (max, sum) and partial output
    float2 ml[R][NU];
    f32x4 v[R][NU];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int idx = lane + 64 * u;
        const int64_t rj = rec_of(wr[r], idx < units ? idx / (D / 4) : 0);
        ml[r][u] = *reinterpret_cast<const float2*>(sa.rec_ml + rj * 2);
        v[r][u] = *reinterpret_cast<const f32x4*>(sa.rec_acc + rj * D + 4 * (idx < units ? idx % (D / 4) : 0));
      }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      float mb = M[u];
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (live[r]) mb = fmaxf(mb, ml[r][u].x);
      const float c0 = M[u] == kNegInf ? 0.f : fast_exp2(M[u] - mb);
      L[u] *= c0;
      O[u] *= c0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (live[r]) {
          const float e = fast_exp2(ml[r][u].x - mb);
          L[u] = __builtin_fmaf(e, ml[r][u].y, L[u]);
#pragma unroll
          for (int i = 0; i < 4; ++i) O[u][i] = __builtin_fmaf(e, v[r][u][i], O[u][i]);
        }
      }
      M[u] = mb;
    }
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int idx = lane + 64 * u;
    if (idx >= units) continue;
    const int j = idx / (D / 4), d4 = idx % (D / 4);
    const float inv = 1.f / L[u];
    const int64_t o = (row0 + j) * D + 4 * d4;
    if (a.out_f32) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + o) = O[u] * inv;
    } else {
      // (the fp32 output rounded: see opaque_f32)
      const uint32_t lo = T::from_f32(opaque_f32(O[u][0] * inv)) | (T::from_f32(opaque_f32(O[u][1] * inv)) << 16);
      const uint32_t hi = T::from_f32(opaque_f32(O[u][2] * inv)) | (T::from_f32(opaque_f32(O[u][3] * inv)) << 16);
      *reinterpret_cast<u32x2*>(static_cast<bits*>(a.out) + o) = u32x2{lo, hi};
    }
  }
}

// Merge without a plan: one wave per item (sequence, kv head).  It recomputes
// the item's place in the tile list from the context lengths and the even
// split of the grid, and merges when the item spans more than one wave.
template <class T, int D, int GMAX>
__global__ __launch_bounds__(64) void stream_merge_kernel(StreamArgs sa, int32_t grid) {
  const DecodeArgs& a = sa.d;
  const int lane = threadIdx.x;
  const int B = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  const int seq = blockIdx.x / Hkv;
  const int kvh = blockIdx.x % Hkv;
  // tiles of earlier sequences and of all sequences
  int64_t before = 0, all = 0;
  int own = 0;
  for (int i = lane; i < B; i += 64) {
    const int n = (min(max(a.ctx[i], 0), a.max_ctx) + 15) / 16;
    all += n;
    if (i < seq) before += n;
    if (i == seq) own = n;
  }
  for (int off = 32; off; off >>= 1) {
    all += __shfl_xor(all, off);
    before += __shfl_xor(before, off);
    own += __shfl_xor(own, off);
  }
  if (own == 0) return;
  const int64_t ntot = int64_t(Hkv) * all;
  const int64_t nw = int64_t(grid) * 4;
  auto start = [&](int64_t w) { return w >= nw ? ntot : stream_wave_start(ntot, w, grid); };
  // last wave whose range starts at or before g (its range holds g)
  auto owner = [&](int64_t g) {
    int64_t lo = 0, hi = nw - 1;
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) >> 1;
      if (start(mid) <= g) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  const int64_t gs = int64_t(Hkv) * before + int64_t(kvh) * own;
  const int64_t wlo = owner(gs);
  const int64_t whi = owner(gs + own - 1);
  if (wlo == whi) return;  // written whole by its wave
  // the waves with tiles from wlo to whi (skipping empty ranges)
  int64_t cur = wlo;
  merge_item<T, D, GMAX>(sa, seq, kvh, wlo, start(wlo) < gs ? 1 : 0, [&](int64_t& x) {
    while (cur <= whi && start(cur) >= start(cur + 1)) ++cur;
    if (cur > whi) return false;
    x = cur++;
    return true;
  });
}

// Merge with the host plan: one wave per cut item.  Its plan entry (one
// 32-byte load) holds the item, its wave count, the offset of its waves in
// the full list and the first four of them, so an item cut over at most
// four waves needs one round trip for the entry and one for the records.
template <class T, int D, int GMAX>
__global__ __launch_bounds__(64) void stream_merge_planned_kernel(StreamArgs sa) {
  const int4* e = reinterpret_cast<const int4*>(sa.cut_entry + 8 * int64_t(blockIdx.x));
  const int4 e0 = e[0], e1 = e[1];            // {code, count, off, w0}, {w1, w2, w3, -}
  const int code = e0.x, count = e0.y, off = e0.z;
  const int item = code >> 1;
  const int Hkv = sa.d.num_kv_heads;
  int i = 0;
  merge_item<T, D, GMAX>(sa, item / Hkv, item % Hkv, e0.w, code & 1, [&](int64_t& x) {
    if (i >= count) return false;
    x = i == 0 ? e0.w : i == 1 ? e1.x : i == 2 ? e1.y : i == 3 ? e1.z : sa.cut_workers[off + i];
    ++i;
    return true;
  });
}

// ------------------------------------------------------------------ launch
namespace {

template <int D, int GMAX, int NSLOT>
constexpr int stream_slot_bytes() {
  return (2 * (D / 32) + (GMAX * D * 2 + 1023) / 1024) * 1024;
}

}  // namespace

// ==== host side: launch configuration (no device code below this line) ====

size_t stream_lds_bytes(int d, int gmax, int nslot) {
  const int qi = (gmax * d * 2 + 1023) / 1024;
  const size_t sb = size_t(2 * (d / 32) + qi) * 1024;
  return 4 * nslot * sb;
}

template <class T, int D, int BS, int GMAX, int NSLOT>
static hipError_t launch_s(const StreamArgs& sa, size_t lds, int grid, int phases, hipStream_t stream) {
  auto kern = decode_stream_kernel<T, D, BS, GMAX, NSLOT>;
  // the dynamic size of an instantiation depends only on its template
  // arguments; allow it once per device
  static std::atomic<uint64_t> allowed{0};
  if (hipError_t e = allow_dynamic_lds(kern, lds, allowed)) return e;
  if (phases & 1) {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, stream, sa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(phases & 2)) return hipSuccess;
  if (sa.cut_entry) {
    if (sa.num_cut <= 0) return hipSuccess;
    hipLaunchKernelGGL((stream_merge_planned_kernel<T, D, GMAX>), dim3(static_cast<uint32_t>(sa.num_cut)), dim3(64),
                       0, stream, sa);
    return hipGetLastError();
  }
  const int64_t items = int64_t(sa.d.num_seqs) * sa.d.num_kv_heads;
  hipLaunchKernelGGL((stream_merge_kernel<T, D, GMAX>), dim3(static_cast<uint32_t>(items)), dim3(64), 0, stream, sa,
                     grid);
  return hipGetLastError();
}

template <class T, int D, int BS, int GMAX>
static hipError_t launch_n(const StreamArgs& sa, int nslot, size_t lds, int grid, int phases, hipStream_t stream) {
  switch (nslot) {
    case 2: return launch_s<T, D, BS, GMAX, 2>(sa, lds, grid, phases, stream);
    case 3: return launch_s<T, D, BS, GMAX, 3>(sa, lds, grid, phases, stream);
    case 4: return launch_s<T, D, BS, GMAX, 4>(sa, lds, grid, phases, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class T, int D, int BS>
static hipError_t launch_g(const StreamArgs& sa, int gmax, int nslot, size_t lds, int grid, int phases,
                           hipStream_t stream) {
  switch (gmax) {
    case 4: return launch_n<T, D, BS, 4>(sa, nslot, lds, grid, phases, stream);
    case 8: return launch_n<T, D, BS, 8>(sa, nslot, lds, grid, phases, stream);
    case 16: return launch_n<T, D, BS, 16>(sa, nslot, lds, grid, phases, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class T, int D>
static hipError_t launch_b(const StreamArgs& sa, int bs, int gmax, int nslot, size_t lds, int grid, int phases,
                           hipStream_t stream) {
  switch (bs) {
    case 8: return launch_g<T, D, 8>(sa, gmax, nslot, lds, grid, phases, stream);
    case 16: return launch_g<T, D, 16>(sa, gmax, nslot, lds, grid, phases, stream);
    case 32: return launch_g<T, D, 32>(sa, gmax, nslot, lds, grid, phases, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class T>
static hipError_t launch_d(const StreamArgs& sa, int d, int bs, int gmax, int nslot, size_t lds, int grid,
                           int phases, hipStream_t stream) {
  switch (d) {
    case 64: return launch_b<T, 64>(sa, bs, gmax, nslot, lds, grid, phases, stream);
    case 128: return launch_b<T, 128>(sa, bs, gmax, nslot, lds, grid, phases, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_stream(const StreamArgs& sa, int32_t dtype, int32_t d, int32_t bs, int32_t gmax,
                                int32_t nslot, size_t lds, int32_t grid, int32_t phases, hipStream_t stream) {
  switch (dtype) {
    case 1: return launch_d<F16>(sa, d, bs, gmax, nslot, lds, grid, phases, stream);
    case 2: return launch_d<BF16>(sa, d, bs, gmax, nslot, lds, grid, phases, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
