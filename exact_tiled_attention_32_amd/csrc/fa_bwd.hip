// Backward kernels: recompute-based gradients of exact attention (gfx950).
//
// The pages give the principle, not the formulas: the backward recomputes the attention
// tile on chip from Q, K and the saved softmax statistics instead of storing P
// (sendsoonai.com "FlashAttention: IO-aware explained", section "Recomputation and IO
// complexity"; cochat.ai audit of "FlashAttention: Fast and Memory-Efficient Exact
// Attention with IO-Awareness", quoted App. B.2/B.4). The gradients are the chain rule of
// O = softmax(scale Q K^T) V:
//     P = exp(scale S - lse),  dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),
//     dK = scale dS^T Q,       dQ = scale dS K,     with D_i = sum_j P_ij dP_ij = dO_i . O_i.
// Loop order for dK, dV follows the quoted Theorem 5 proof (App. C): each key/value tile
// is loaded once and its dK, dV accumulate on chip while query tiles stream past. The
// proof's dQ updates (one read/write pass over dQ per key tile) would be fp32 atomics
// here; on MI355X those are performed past the per-XCD L2 and run at ~1.3 TB/s, which
// bounded the whole backward. dQ is therefore computed by its own query-major kernel that
// recomputes the score tile (two more products per tile, no atomics).
//
// Two launches on the caller's stream (three with a block mask):
//   (1. bwd_order: block-sparse only, the order of the dK/dV key tiles)
//   2. bwd_dq:    one workgroup per (b, h, 128-query tile); 4 waves, one query per lane.
//                 Its prologue is the D pre-pass: each lane forms D = rowsum(dO o O) of its
//                 query in fp32 from the dO and O rows and writes it to the workspace.
//   3. bwd_dkdv:  one workgroup per (b, h, 128-key tile); 4 waves, two workgroups per CU;
//                 reads D (so it runs after the dQ kernel)
// As in the forward, packed sequences, causal and windowed masks, dropout (the mask
// regenerated from the same Philox4x32-10 counters) and a head dimension of 16 are
// variants of the same kernels.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = kBwdKeyTile;  // keys per dK/dV workgroup (32 per wave)

// ---------------------------------------------------------------------------------------
// 1. Block-sparse only: the order in which the dK/dV workgroups take their key tiles, most
//     kept mask blocks first. The work of a key tile is proportional to the kept blocks of
//     its mask column; a column kept for every query block (a "global" column) can take
//     far longer than the rest, and started last it would set the end of the launch.
//     One workgroup of 1024 threads: column counts into LDS (several 16-byte row loads in
//     flight per thread), then a bitonic sort of (count, tile) keys.
// ---------------------------------------------------------------------------------------
constexpr int kOrderThreads = 1024;

__global__ __launch_bounds__(kOrderThreads) void bwd_order_kernel(const uint8_t* __restrict__ mask, int nb, int mb,
                                                             int ntk, uint32_t* __restrict__ order) {
  __shared__ uint32_t cnt[kMaxKeyTiles];   // kept blocks per mask column (nb <= ntk)
  __shared__ uint32_t keys[kMaxKeyTiles];
  const int tid = threadIdx.x;
  for (int c = tid; c < nb; c += kOrderThreads) cnt[c] = 0;
  __syncthreads();
  if (nb % 16 == 0 && (reinterpret_cast<uintptr_t>(mask) & 15) == 0) {
    // 16 columns per thread and 16-byte loads: column group g = tid % G, every R-th row
    const int G = nb / 16, R = kOrderThreads / G;
    if (tid < G * R) {
      const int g = tid % G;
      uint32_t n[16] = {};
#pragma unroll 4
      for (int r = tid / G; r < nb; r += R) {
        const u32x4 v = gload16(mask + (size_t)r * nb + 16 * g);
#pragma unroll
        for (int i = 0; i < 16; ++i) n[i] += ((v[i >> 2] >> (8 * (i & 3))) & 0xFFu) != 0;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) atomicAdd(&cnt[16 * g + i], n[i]);
    }
  } else {
    // any width: each thread sums its columns down the rows
    for (int c = tid; c < nb; c += kOrderThreads) {
      uint32_t n = 0;
      for (int r = 0; r < nb; ++r) n += mask[(size_t)r * nb + c] != 0;
      cnt[c] = n;
    }
  }
  __syncthreads();
  int P = 1;
  while (P < ntk) P <<= 1;
  // ascending order of (0xFFFF - count) << 16 | tile: most blocks first, ties by tile
  for (int j = tid; j < P; j += kOrderThreads)
    keys[j] = j < ntk ? ((0xFFFFu - min(cnt[(j * kBwdKeyTile) / mb], 0xFFFFu)) << 16) | (uint32_t)j : 0xFFFFFFFFu;
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += kOrderThreads) {
        const int x = i ^ j;
        if (x > i) {
          const uint32_t a = keys[i], b = keys[x];
          const bool up = (i & k) == 0;
          if ((a > b) == up) {
            keys[i] = b;
            keys[x] = a;
          }
        }
      }
      __syncthreads();
    }
  for (int i = tid; i < ntk; i += kOrderThreads) order[i] = keys[i] & 0xFFFFu;
}

// ---------------------------------------------------------------------------------------
// 3. dK / dV kernel: one workgroup per (b, h, 128-key tile). Wave w owns key group
//    kg = w % 4 (keys 32 kg .. 32 kg + 31 of the tile) and takes QBW 32-row query blocks
//    per step (1 at d = 128, 2 below). Normally the workgroup is those 4 waves and two
//    workgroups share a CU (two waves per SIMD from different workgroups); the dropout
//    variant at d = 128 has 8 waves, the second four taking the other half (qh = w / 4) of
//    each 64-row query step, one workgroup per CU. Orientation (v_mfma_f32_32x32x16_bf16):
//   S, dP   = Q K^T, dO V^T   (M = the wave's queries, N = its 32 keys): Q/dO rows and K/V
//             rows are 16-byte LDS reads (K fragments held in registers at d = 128).
//   dV^T   += dO^T P          (M = d, N = keys): dO^T from transpose reads, P straight
//   dK^T   += Q^T dS           from the accumulator (same layout trick as the forward).
//   With two query halves, their dK^T, dV^T partials are summed through LDS at the end.
// ---------------------------------------------------------------------------------------
// s_waitcnt immediate for vmcnt(0), expcnt and lgkmcnt left free (gfx9 encoding).
constexpr int kWaitVmcnt0 = 0x0F70;

// Waves of a key group (32 keys) that split each query step between them (QH). With one,
// a workgroup is 4 waves and two workgroups share a CU, so the two waves of a SIMD belong
// to different workgroups and drift apart instead of meeting at every barrier. With two,
// a workgroup is 8 waves, one per CU, and a key tile's query steps are shared by twice
// as many waves: the block-sparse path uses it, where the kept blocks of a few "global"
// key columns make some key tiles far longer than the rest and their duration sets the
// end of the launch; so does the dropout variant at d = 128, which cannot hold K in
// registers next to its generator state and so needs K in LDS.
template <int D, bool DROP>
constexpr int dkdv_halves() { return D == 128 && DROP ? 2 : 1; }
constexpr int dkdv_threads(int qh) { return 256 * qh; }
// 32-query blocks per wave and step
template <int D>
constexpr int dkdv_query_blocks() { return D == 128 ? 1 : 2; }

// Query tiles [i0, ntq) whose mask block in column `cb` is nonzero (block-sparse path).
template <int NT>
__device__ int build_qtile_list(uint16_t* list, int* wcount, const uint8_t* mask, int cb, int nb, int mb, int i0,
                                int ntq, int bq) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  int count = 0;
  for (int base = i0; base < ntq; base += NT) {
    const int i = base + tid;
    const bool keep = i < ntq && mask[(size_t)((i * bq) / mb) * nb + cb] != 0;
    const uint64_t bal = __ballot(keep);
    const int pre = __popcll(bal & ((1ull << l) - 1ull));
    if (l == 0) wcount[w] = __popcll(bal);
    __syncthreads();
    int off = count, tot = 0;
    for (int k = 0; k < NT / 64; ++k) {
      off += k < w ? wcount[k] : 0;
      tot += wcount[k];
    }
    if (keep) list[off + pre] = (uint16_t)i;
    count += tot;
    __syncthreads();
  }
  return count;
}

// DG: head dimension in memory; D: tile width (16 runs on 32-wide tiles, upper half zero).
// QBWO: 32-query blocks per wave and step when not the default (0). Short sequences at
// d = 64 (dense, no dropout) take one instead of two, without the block-sparse tile list:
// 48 KB of LDS and 168 registers, so that three workgroups share a CU instead of two and a
// launch of up to three workgroups per CU is resident at once.
template <int D, bool DROP, int DG = D, int QH = dkdv_halves<D, DROP>(), int QBWO = 0>
__global__ __launch_bounds__(dkdv_threads(QH), QH == 1 ? 2 : 1) void bwd_dkdv_kernel(BwdArgs a) {
  static_assert(DG == D || (D == 32 && DG == 16), "narrow heads run on 32-wide tiles");
  static_assert(QH == 1 || QH == 2, "one or two query halves");
  static_assert(QH == 2 || dkdv_halves<D, DROP>() == 1, "this variant needs the 8-wave layout");
  constexpr bool LIST = QBWO == 0;  // block-sparse query-tile list
  constexpr int kMainThreads = dkdv_threads(QH);
  constexpr int NW = 4 * QH;                  // waves per workgroup
  constexpr int KSG = (DG + 15) / 16;  // k-steps that carry data
  constexpr int QBW = QBWO ? QBWO : dkdv_query_blocks<D>();  // 32-query blocks per wave per step
  constexpr int BQ = 32 * QBW * QH;            // query rows per step
  // At d = 128 without dropout the wave's K fragments (the A operand of S, the same in
  // every step) are loaded once into registers and K is not kept in LDS.
  constexpr bool KREG = D == 128 && !DROP && QH == 1;
  constexpr int MD = D / 32;           // 32-row blocks of dK^T / dV^T
  constexpr int QT = BQ * D * 2;       // bytes of a Q or dO tile
  constexpr int KT = kBK * D * 2;      // bytes of the K or V tile
  constexpr int KVT = KREG ? KT : 2 * KT;  // the K | V tile in LDS (V alone when K is in registers)
  constexpr int NDMA = QT / (kMainThreads * 16);     // DMA instructions per wave per Q/dO tile
  constexpr int RPB = 1024 / (2 * D);                 // rows per 1 KB DMA block
  constexpr int KCH = kBK * (D / 8) / kMainThreads;  // 16-byte chunks per thread per K/V tile
  // LDS: the two Q | dO staging buffers and the K | V tile are separate arrays. The
  // compiler can then tell that the direct global -> LDS loads into one buffer do not
  // touch the other, and does not wait for them before reading it.
  __shared__ __attribute__((aligned(16))) char qd0[2 * QT];
  __shared__ __attribute__((aligned(16))) char qd1[2 * QT];
  __shared__ __attribute__((aligned(16))) char kvt[KVT];
  __shared__ __attribute__((aligned(16))) float stats[2][2][BQ];  // [buf][lse2 | D][row]
  __shared__ uint16_t qlist[LIST ? kMaxTileList : 1];
  __shared__ int wcount[8];
  FA_LDS char* const kt = (FA_LDS char*)kvt;  // (unused when K is in registers)
  FA_LDS char* const vt = KREG ? kt : kt + KT;
  // With two query halves, after the loop the upper half hands its partials over through
  // LDS: dK^T of key group kg in kvt, dV^T in the Q | dO buffer kg / 2.
  constexpr int RED = MD * 16 * 64;  // floats per key group and tensor
  static_assert(QH == 1 || (4 * RED * 4 <= KVT && 2 * RED * 4 <= 2 * QT), "dK/dV reduction fits in LDS");

  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  // key tile: small j (most causal work) first, or the block-sparse order (most kept
  // blocks first)
  const int jt = a.order ? (int)a.order[blockIdx.x / BH] : (int)(blockIdx.x / BH);
  const int b = bh / a.H;
  const int k0 = jt * kBK;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, h = l >> 5, kl = l & 31;
  const int kg = w & 3, qh = w >> 2;
  const int key = k0 + 32 * kg + kl;    // the key this lane's accumulator columns refer to
  const int qw0 = 32 * QBW * qh;        // the wave's first query row inside a step
  const HeadSlice sl = head_slice<DG>(a, bh);
  const int N = sl.N;
  if (k0 >= N) return;  // a key tile past the end of a shorter sequence (uniform)
  const size_t hoff = sl.hoff, rs = (size_t)a.rs;
  const __bf16* __restrict__ Q = reinterpret_cast<const __bf16*>(a.q) + hoff;
  const __bf16* __restrict__ K = reinterpret_cast<const __bf16*>(a.k) + hoff;
  const __bf16* __restrict__ V = reinterpret_cast<const __bf16*>(a.v) + hoff;
  const __bf16* __restrict__ dO = reinterpret_cast<const __bf16*>(a.dout) + hoff;
  const float* __restrict__ lse = a.lse + sl.loff;
  const float* __restrict__ dsum = a.dsum + sl.loff;

  int kv_end = N;
  if (a.kv_len) kv_end = min(max(a.kv_len[b], 0), N);
  // Query tiles [i0, i1) that may attend to a key of this tile: query i sees key j iff
  // i - wl <= j <= i + wr, i.e. j - wr <= i <= j + wl.
  const int ntq = (N + BQ - 1) / BQ;
  const int i0 = a.wr >= 0 ? max(k0 - a.wr, 0) / BQ : 0;
  const int i1 = a.wl >= 0 ? min((min(k0 + kBK - 1 + a.wl, N - 1)) / BQ + 1, ntq) : ntq;
  int nq = k0 < kv_end ? max(i1 - i0, 0) : 0;  // key tile entirely padded: zero dK/dV
  if constexpr (LIST) {
    if (a.mask && nq > 0)
      nq = __builtin_amdgcn_readfirstlane(
          build_qtile_list<kMainThreads>(qlist, wcount, a.mask, k0 / a.mb, a.nb, a.mb, i0, ntq, BQ));
  }

  // Per-lane LDS byte offsets, fixed for the whole kernel. Within a swizzled row the
  // offsets of chunk c and of chunk c ^ m differ by an XOR with 16 m, so one base register
  // per operand family serves every k-step and d-block (the XOR only touches bits below
  // the row stride).
  // Adding a multiple of 32 rows (8 KB at d = 128, 4 KB at d = 64) leaves the XOR-ed bits
  // alone, so the wave's row shifts are folded into the bases.
  const int row_off0 = tile_off<D>(qw0 + kl, 8 * h);  // Q / dO row operand, k-step 0
  // The K / V row operand (row 32 kg + kl) has the same swizzle (both rows agree mod 16),
  // so it is the Q / dO offset moved by whole rows, into the K tile.
  const int kv_off0 = row_off0 + (32 * kg - qw0) * 2 * D;
  int tr_lo0, tr_hi0;        // Q^T / dO^T transpose reads of d-block 0 (+16 s4 rows)
  tr8_offsets<D>(0, tr_lo0, tr_hi0);
  tr_lo0 += qw0 * 2 * D;
  tr_hi0 += qw0 * 2 * D;
  int ro0 = row_off0, ko0 = kv_off0, tl0 = tr_lo0, th0 = tr_hi0;
  // Q / dO staging by raw buffer -> LDS loads: each wave instruction fills 1 KB, lane i
  // the 16 bytes at offset 16 i, so lane i fetches the chunk whose swizzled slot that is.
  // A query tile's buffer range ends at row N, so rows past it (last query tile only)
  // arrive as zeros; they also get P = 0 through the staged lse (+inf). The per-lane byte
  // offsets inside a tile are fixed; only the tile's base (scalar) changes per step.
  // Lane l of DMA block c covers row (NW c + w) RPB + l / (D/8); the block rows are a
  // multiple of 16 apart, so the swizzled column is the same for every block.
  const int dma_row0 = w * RPB + l / (D / 8);
  const int dma_col = ((l % (D / 8)) ^ swz<D>(dma_row0)) * 8;
  static_assert((NW * RPB) % 16 == 0, "DMA block step must keep the swizzle");
  static_assert(NDMA >= 1 && NDMA * kMainThreads * 16 == QT, "Q / dO tile staging covers the tile");
  int qdma_off[NDMA];
#pragma unroll
  for (int c = 0; c < NDMA; ++c)
    qdma_off[c] = (DG == D || dma_col < DG) ? ((dma_row0 + c * NW * RPB) * a.rs + dma_col) * 2
                                            : (int)0xFFFFFFF0u;  // past any range: reads zero

  f32x16 dkt[MD], dvt[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) {
    dkt[md] = f32x16{};
    dvt[md] = f32x16{};
  }

  float sr = 0.f;
  bool svalid = false;
  auto stage_q = [&](int it, auto bufc) {
    const int q0 = it * BQ;
    FA_LDS char* qb = (FA_LDS char*)(decltype(bufc)::value ? qd1 : qd0);
    // rows of the tile inside the slice (uniform: kept scalar, like the descriptors)
    const int rows = __builtin_amdgcn_readfirstlane(min(max(N - q0, 0), BQ));
    const uint32_t bytes = (uint32_t)rows * (uint32_t)(a.rs * 2);
    const auto rq = make_rsrc(Q + (size_t)q0 * rs, bytes);
    const auto rd = make_rsrc(dO + (size_t)q0 * rs, bytes);
#pragma unroll
    for (int c = 0; c < NDMA; ++c) {
      FA_LDS char* blk = qb + (c * NW + w) * 1024;
      const int voff = qdma_off[c];  // (a local copy: see the forward's staging)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (FA_LDS void*)blk, 16, voff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (FA_LDS void*)(blk + QT), 16, voff, 0, 0, 0);
    }
    // threads [0, BQ) stage lse, threads [BQ, 2 BQ) stage D (whole waves: 2 BQ is a
    // multiple of 64, so the other waves skip this by a scalar branch)
    if (w * 64 < 2 * BQ) {
      const int qq = q0 + (tid % BQ);
      svalid = qq < N;
      const float* src = tid < BQ ? lse : dsum;
      sr = src[min(qq, N - 1)];
    }
  };
  auto store_stats = [&](int buf) {
    if (tid < 2 * BQ) {
      float v;
      if (tid < BQ) {
        // an empty row (lse = -inf) and a row past N map to +inf so that P = 0 there
        v = (!svalid || sr == kNegInf) ? __builtin_inff() : sr * kLog2e;
      } else {
        v = svalid ? sr : 0.f;
      }
      stats[buf][tid / BQ][tid % BQ] = v;
    }
  };
  // Wait for this wave's staging loads before the barrier that publishes the staged tile.
  auto wait_loads = [&]() { __builtin_amdgcn_s_waitcnt(kWaitVmcnt0); };
  // Query tiles are visited last-first.
  auto tile_at = [&](int t) {
    if constexpr (LIST) return a.mask ? __builtin_amdgcn_readfirstlane((int)qlist[nq - 1 - t]) : i0 + nq - 1 - t;
    else return i0 + nq - 1 - t;
  };

  // K fragments in registers: lane (kl, h) holds K[key][16 ks + 8 h .. + 7] (zero past N)
  bf16x8 kf[KREG ? KSG : 1];
  if constexpr (KREG) {
    const __bf16* krow = K + (size_t)min(key, N - 1) * rs + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KSG; ++ks)
      kf[ks] = key < N ? __builtin_bit_cast(bf16x8, gload16(krow + 16 * ks)) : bf16x8{};
  }
  stage_q(nq > 0 ? tile_at(0) : 0, std::integral_constant<int, 0>{});
  // The V tile, and the K tile unless K is held in registers, stay in LDS for the whole
  // kernel (rows past N are zero). Requested after the first query tile's staging, so that
  // the prologue waits for one memory latency, not two.
#pragma unroll
  for (int c = 0; c < KCH; ++c) {
    const int id = tid + kMainThreads * c;
    const int row = id / (D / 8), col = (id % (D / 8)) * 8;
    const int kk = min(k0 + row, N - 1);
    const bool ok = k0 + row < N && col < DG;
    const int cc = col < DG ? col : 0;  // (a column in range; the value is dropped)
    if constexpr (!KREG) {
      const u32x4 kv = gload16(K + (size_t)kk * rs + cc);
      lds_store16(kt + tile_off<D>(row, col), ok ? kv : u32x4{});
    }
    const u32x4 vv = gload16(V + (size_t)kk * rs + cc);
    lds_store16(vt + tile_off<D>(row, col), ok ? vv : u32x4{});
  }
  wait_loads();
  store_stats(0);
  __syncthreads();
  asm volatile("" ::: "memory");

  auto step = [&](auto bufc, int t) {
    constexpr int BUF = decltype(bufc)::value;
    const int it = tile_at(t);
    const int q0 = it * BQ;
    // buffer BUF ^ 1 was last read in step t - 1: stream the next query tile into it
    stage_q(tile_at(min(t + 1, nq - 1)), std::integral_constant<int, BUF ^ 1>{});
    // Offset bases made opaque once per step (no copy; the value is unchanged): keeps the
    // compiler from hoisting every derived offset out of the loop into its own register.
    asm volatile("" : "+v"(ro0), "+v"(ko0), "+v"(tl0), "+v"(th0));
    const FA_LDS char* qb = (const FA_LDS char*)(BUF ? qd1 : qd0);
    const FA_LDS char* db = qb + QT;

    // S = Q K^T and dP = dO V^T: the wave's QBW query blocks x its 32 keys.
    f32x16 s[QBW], dp[QBW];
#pragma unroll
    for (int b2 = 0; b2 < QBW; ++b2) {
      s[b2] = f32x16{};
      dp[b2] = f32x16{};
    }
    // Software-pipelined: the operands of k-step ks + 1 are requested before the products
    // of k-step ks are issued (the scheduling barrier keeps that order).
    struct SOps {
      bf16x8 k, v, q[QBW], d[QBW];
    };
    auto load_s = [&](int ks, SOps& o) {
      const int qo = ro0 ^ (32 * ks), ko = ko0 ^ (32 * ks);
      if constexpr (!KREG) o.k = lds_ld8(kt + ko);
      o.v = lds_ld8(vt + ko);
#pragma unroll
      for (int b2 = 0; b2 < QBW; ++b2) {
        o.q[b2] = lds_ld8(qb + qo + b2 * 32 * 2 * D);
        o.d[b2] = lds_ld8(db + qo + b2 * 32 * 2 * D);
      }
    };
    SOps so[2];
    load_s(0, so[0]);
    // At d = 128 (dense, no dropout) the wave raises its issue priority over the other wave
    // of its SIMD for the score products: 2.7 % faster kernel in a same-box A/B; at d = 64,
    // or around the dV / dK products, it measured no gain or a loss.
    constexpr bool kPrioS = D == 128 && !DROP && QH == 1;
    if constexpr (kPrioS) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < KSG; ++ks) {
      if (ks + 1 < KSG) load_s(ks + 1, so[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      const SOps& o = so[ks & 1];
#pragma unroll
      for (int b2 = 0; b2 < QBW; ++b2) {
        s[b2] = mfma32(o.q[b2], KREG ? kf[ks] : o.k, s[b2]);
        dp[b2] = mfma32(o.d[b2], o.v, dp[b2]);
      }
    }
    if constexpr (kPrioS) __builtin_amdgcn_s_setprio(0);
    // P = exp2(S * scale * log2e - lse * log2e), dS = P (dP - D); with dropout the value
    // products see P o Z and dS = P (Z dP / (1 - p) - D), Z the keep mask of the pair: bit
    // 4 g + e of zbits[b2] for query e of register group g (dropout_bits_klane, one call
    // per lane per pair of groups).
    uint32_t zbits[QBW];
#pragma unroll
    for (int b2 = 0; b2 < QBW; ++b2) {
      zbits[b2] = 0xFFFFu;
      if constexpr (DROP) {
        zbits[b2] = 0;
#pragma unroll
        for (int gp = 0; gp < 2; ++gp)
          zbits[b2] |= dropout_bits_klane(key, q0 + qw0 + 32 * b2 + 16 * gp + 4 * h, (uint32_t)(bh % a.H),
                                          (uint32_t)b, a.seed_lo, a.seed_hi, a.drop_thr)
                       << (8 * gp);
      }
    }
#pragma unroll
    for (int b2 = 0; b2 < QBW; ++b2)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qr0 = qw0 + 32 * b2 + 8 * g + 4 * h;
        const f32x4 l2 = *reinterpret_cast<const f32x4*>(&stats[BUF][0][qr0]);
        const f32x4 dd = *reinterpret_cast<const f32x4*>(&stats[BUF][1][qr0]);
        const uint32_t keep = (zbits[b2] >> (4 * g)) & 0xFu;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g + e;
          const float p = fast_exp2(__builtin_fmaf(s[b2][i], a.c2s, -l2[e]));
          if constexpr (DROP) {
            const bool kept = (keep >> e) & 1u;
            s[b2][i] = kept ? p : 0.f;
            dp[b2][i] = p * ((kept ? dp[b2][i] * a.drop_scale : 0.f) - dd[e]);
          } else {
            s[b2][i] = p;
            dp[b2][i] = p * (dp[b2][i] - dd[e]);
          }
        }
      }
    // Tiles that cross the causal diagonal or the key padding (a wave-uniform test): the
    // masked pairs get P = dS = 0, by selection, so whatever was computed there is dropped.
    const int kk0 = k0 + 32 * kg, qa = q0 + qw0;  // the wave's first key and first query
    if ((kk0 + 31 >= kv_end) || (a.wr >= 0 && kk0 + 31 > qa + a.wr) ||
        (a.wl >= 0 && kk0 < qa + 32 * QBW - 1 - a.wl)) {
#pragma unroll
      for (int b2 = 0; b2 < QBW; ++b2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qrow = q0 + qw0 + 32 * b2 + 8 * (i >> 2) + 4 * h + (i & 3);
          const bool masked = key >= kv_end || (a.wr >= 0 && key > qrow + a.wr) || (a.wl >= 0 && key < qrow - a.wl);
          s[b2][i] = masked ? 0.f : s[b2][i];
          dp[b2][i] = masked ? 0.f : dp[b2][i];
        }
    }
    // dV^T += dO^T P, dK^T += Q^T dS (16 queries per k-step).
    // Pipelined like the score products: transpose reads of item j + 1 (item = 16-query
    // step s4 x d-block md) are requested before the products of item j.
    bf16x8 pb[2 * QBW], sb[2 * QBW];
#pragma unroll
    for (int s4 = 0; s4 < 2 * QBW; ++s4) {
      pb[s4] = pack8(s[s4 >> 1], 8 * (s4 & 1));
      sb[s4] = pack8(dp[s4 >> 1], 8 * (s4 & 1));
    }
    constexpr int NJ = 2 * QBW * MD;
    struct TOps {
      bf16x8 d, q;
    };
    auto load_t = [&](int j, TOps& o) {
      const int s4 = j / MD, md = j % MD;
      const int ro = 16 * s4 * 2 * D;
      const int lo = (tl0 ^ (64 * md)) + ro, hi = (th0 ^ (64 * md)) + ro;
      o.d = lds_tr8(db + lo, db + hi);
      o.q = lds_tr8(qb + lo, qb + hi);
    };
    TOps to[2];
    load_t(0, to[0]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j + 1 < NJ) load_t(j + 1, to[(j + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      const int s4 = j / MD, md = j % MD;
      dvt[md] = mfma32(to[j & 1].d, pb[s4], dvt[md]);
      dkt[md] = mfma32(to[j & 1].q, sb[s4], dkt[md]);
    }
    // Wait for the staged tile, publish it and its statistics.
    wait_loads();
    store_stats(BUF ^ 1);
    __syncthreads();
    asm volatile("" ::: "memory");
  };
  for (int t = 0; t < nq; t += 2) {
    step(std::integral_constant<int, 0>{}, t);
    if (t + 1 < nq) step(std::integral_constant<int, 1>{}, t + 1);
  }

  wait_loads();  // the last step's look-ahead staging must land before LDS is reused
  if constexpr (QH == 2) {
    __syncthreads();
    // Sum the two query halves' partials through LDS (all tiles are free now): the upper
    // half stores dK^T, dV^T in fp32 in its accumulator layout, the lower half adds them.
    // [MD][16 regs][64 lanes] per key group
    float* const kred = reinterpret_cast<float*>(kvt) + kg * RED + l;
    float* const vred = reinterpret_cast<float*>(kg < 2 ? qd0 : qd1) + (kg & 1) * RED + l;
    if (qh == 1) {
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          kred[(md * 16 + i) * 64] = dkt[md][i];
          vred[(md * 16 + i) * 64] = dvt[md][i];
        }
    }
    __syncthreads();
    if (qh == 0) {
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          dkt[md][i] += kred[(md * 16 + i) * 64];
          dvt[md][i] += vred[(md * 16 + i) * 64];
        }
    }
  }
  if (qh == 0 && key < N) {
    __bf16* dK = reinterpret_cast<__bf16*>(a.dk) + hoff + (size_t)key * rs;
    __bf16* dV = reinterpret_cast<__bf16*>(a.dv) + hoff + (size_t)key * rs;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 kv4, vv4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g + e;
          kv4[e] = (__bf16)(dkt[md][i] * a.scale);
          vv4[e] = (__bf16)(dvt[md][i] * (DROP ? a.drop_scale : 1.0f));
        }
        if (32 * md + 8 * g < DG) {
          *reinterpret_cast<bf16x4*>(dK + 32 * md + 8 * g + 4 * h) = kv4;
          *reinterpret_cast<bf16x4*>(dV + 32 * md + 8 * g + 4 * h) = vv4;
        }
      }
  }
}

// ---------------------------------------------------------------------------------------
// 2. dQ kernel: one workgroup per (b, h, 128-query tile), 4 waves of 32 queries; key tiles
//    of 64 keys stream through double-buffered LDS. The orientation is the forward's:
//    scores are formed transposed so each lane owns one query and lse, D are per-lane
//    scalars.
//   S^T, dP^T = K Q^T, V dO^T   (A = K / V rows from LDS, B = the wave's Q / dO rows held
//                                 in registers)
//   dS^T      = P^T o (dP^T - D),  P^T = exp2(S^T scale log2e - lse log2e)
//   dQ^T     += K^T dS^T          (A = K^T transpose reads, B = dS^T from the accumulator)
//   dQ = scale dQ^T^T, written once in bf16.
//   K and V tiles are staged by direct buffer -> LDS loads bounded at row N (rows past the
//   end arrive as zeros), one tile ahead, so no staging registers are needed.
// ---------------------------------------------------------------------------------------
constexpr int kDqRows = 128;  // query rows per workgroup
constexpr int kDqKeys = 64;   // keys per tile

template <int D, bool DROP, int DG = D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdArgs a) {
  static_assert(DG == D || (D == 32 && DG == 16), "narrow heads run on 32-wide tiles");
  constexpr int KSG = (DG + 15) / 16;               // k-steps that carry data
  constexpr int CH = D / 8;                         // 16-byte chunks per row
  constexpr int TILE = kDqKeys * D * 2;             // bytes of one K or V tile
  constexpr int KS = D / 16;                        // k-steps over d
  constexpr int MD = D / 32;                        // 32-row blocks of dQ^T
  constexpr int KB = kDqKeys / 32;                  // 32-key blocks of a tile
  constexpr int PS = kDqKeys / 16;                  // k-steps of the dQ^T product
  constexpr int RPB = 1024 / (2 * D);               // tile rows per 1 KB staging block
  constexpr int NDMA = TILE / (kThreads * 16);      // staging instructions per wave per tensor
  static_assert((4 * RPB) % 16 == 0, "staging block step must keep the swizzle");
  // One array per buffer, so that the staging loads into one buffer are known not to
  // touch the other (no wait for them before reading it).
  __shared__ __attribute__((aligned(16))) char kv0[2 * TILE];  // K | V, buffer 0
  __shared__ __attribute__((aligned(16))) char kv1[2 * TILE];  // K | V, buffer 1
  __shared__ uint16_t tlist[kMaxTileList];
  __shared__ int wcount[4];

  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int ntq = (a.N + kDqRows - 1) / kDqRows;
  const int qt = ntq - 1 - blockIdx.x / BH;     // longest (causal) tiles first
  const int b = bh / a.H;
  const int q0 = qt * kDqRows;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, h = l >> 5, ql = l & 31;
  const int qi = q0 + 32 * w + ql;
  const HeadSlice sl = head_slice<DG>(a, bh);
  const int N = sl.N;
  if (q0 >= N) return;  // a query tile past the end of a shorter sequence (uniform)
  const size_t hoff = sl.hoff, rs = (size_t)a.rs;
  const __bf16* __restrict__ Q = reinterpret_cast<const __bf16*>(a.q) + hoff;
  const __bf16* __restrict__ K = reinterpret_cast<const __bf16*>(a.k) + hoff;
  const __bf16* __restrict__ V = reinterpret_cast<const __bf16*>(a.v) + hoff;
  const __bf16* __restrict__ dO = reinterpret_cast<const __bf16*>(a.dout) + hoff;

  int kv_end = N;
  if (a.kv_len) kv_end = min(max(a.kv_len[b], 0), N);
  // Key range of the workgroup's rows under the window: tiles [t0, ntk).
  int hi = kv_end;
  if (a.wr >= 0) hi = min(hi, q0 + kDqRows + a.wr);
  const int t0 = a.wl >= 0 ? max(q0 - a.wl, 0) / kDqKeys : 0;
  const int ntk = (hi + kDqKeys - 1) / kDqKeys;
  int ntiles = max(ntk - t0, 0);
  if (a.mask) {
    // key tiles of this query tile's mask row (128 rows never straddle two mask rows)
    const int rb = q0 / a.mb;
    int count = 0;
    for (int base = 0; base < ntk; base += kThreads) {
      const int j = base + tid;
      const bool keep = j < ntk && a.mask[(size_t)rb * a.nb + (j * kDqKeys) / a.mb] != 0;
      const uint64_t bal = __ballot(keep);
      const int pre = __popcll(bal & ((1ull << l) - 1ull));
      if (l == 0) wcount[w] = __popcll(bal);
      __syncthreads();
      int off = count;
      for (int i = 0; i < w; ++i) off += wcount[i];
      if (keep) tlist[off + pre] = (uint16_t)j;
      count += wcount[0] + wcount[1] + wcount[2] + wcount[3];
      __syncthreads();
    }
    ntiles = __builtin_amdgcn_readfirstlane(count);
  }

  // The wave's Q and dO rows (B operands), and its row statistics in the exp2 domain.
  // Lane (ql, h) holds columns 16 ks + 8 h .. + 7 of its query's row; with the O row in the
  // same layout it also forms that query's D = rowsum(dO o O) (the two halves of the row
  // meet across the half-waves) and publishes it for the dK/dV kernel, which runs next.
  bf16x8 qf[KS], df[KS];
  // The loads are waited for together with the first tile's staging below (one memory
  // latency, not two).
  bf16x8 of[KSG];
  {
    const size_t row = (size_t)min(qi, N - 1) * rs + 8 * h;
    const __bf16* __restrict__ O = reinterpret_cast<const __bf16*>(a.o) + hoff;
#pragma unroll
    for (int ks = 0; ks < KSG; ++ks) {
      qf[ks] = __builtin_bit_cast(bf16x8, gload16(Q + row + 16 * ks));
      df[ks] = __builtin_bit_cast(bf16x8, gload16(dO + row + 16 * ks));
      of[ks] = __builtin_bit_cast(bf16x8, gload16(O + row + 16 * ks));
    }
#pragma unroll
    for (int ks = KSG; ks < KS; ++ks) qf[ks] = df[ks] = bf16x8{};
  }
  const float lse_v = a.lse[sl.loff + min(qi, N - 1)];

  // Per-lane LDS byte offsets (XOR-derived per k-step / d-block, see the dK/dV kernel).
  const int k_off0 = tile_off<D>(ql, 8 * h);  // K / V row operand, k-step 0 (+32 kb rows)
  int t_lo0, t_hi0;                             // K^T transpose reads of d-block 0 (+16 st rows)
  tr8_offsets<D>(0, t_lo0, t_hi0);
  // Staging: instruction c of wave w fills 1 KB block 4c + w of a tile, lane l the 16
  // bytes at 16 l: tile row (4c + w) RPB + l / CH, physical chunk l % CH, which holds the
  // logical chunk (l % CH) ^ swz(row); the row step 4 RPB keeps swz unchanged.
  const int dma_row0 = w * RPB + l / CH;
  const int dma_col = ((l % CH) ^ swz<D>(dma_row0)) * 8;
  int dma_off[NDMA];
#pragma unroll
  for (int c = 0; c < NDMA; ++c) dma_off[c] = ((dma_row0 + 4 * RPB * c) * a.rs + dma_col) * 2;
  if (DG < D && dma_col >= DG) {
#pragma unroll
    for (int c = 0; c < NDMA; ++c) dma_off[c] = (int)0xFFFFFFF0u;  // past any range: reads zero
  }

  f32x16 dq[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) dq[md] = f32x16{};

  auto tile_at = [&](int t) {
    const int tc = min(t, max(ntiles - 1, 0));
    return a.mask ? __builtin_amdgcn_readfirstlane((int)tlist[tc]) : t0 + tc;
  };
  auto stage = [&](int jt, auto bufc) {
    const int key0 = jt * kDqKeys;
    // rows of the tile inside the slice (kept scalar, like the buffer descriptor)
    const int rows = __builtin_amdgcn_readfirstlane(min(max(N - key0, 0), kDqKeys));
    const uint32_t bytes = (uint32_t)rows * (uint32_t)(a.rs * 2);
    const auto rk = make_rsrc(K + (size_t)key0 * rs, bytes);
    const auto rv = make_rsrc(V + (size_t)key0 * rs, bytes);
    FA_LDS char* base = (FA_LDS char*)(decltype(bufc)::value ? kv1 : kv0);
#pragma unroll
    for (int c = 0; c < NDMA; ++c) {
      FA_LDS char* blk = base + (4 * c + w) * 1024;
      const int voff = dma_off[c];  // (a local copy: see the forward's staging)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (FA_LDS void*)blk, 16, voff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (FA_LDS void*)(blk + TILE), 16, voff, 0, 0, 0);
    }
  };

  stage(tile_at(0), std::integral_constant<int, 0>{});
  // The fragments are read in every step: let them land here, so that no wait for them is
  // left inside the loop.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  float dval;
  {
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSG; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) part = __builtin_fmaf((float)df[ks][e], (float)of[ks][e], part);
    dval = part + other_half(part);
    if (h == 0 && qi < N) a.dsum[sl.loff + qi] = dval;
  }
  // an empty row (lse = -inf) and a row past N get lse2 = +inf, so P = 0 there
  const float lse2 = (qi >= N || lse_v == kNegInf) ? __builtin_inff() : lse_v * kLog2e;
  __syncthreads();

  int ko0 = k_off0, tl0 = t_lo0, th0 = t_hi0;
  auto step = [&](auto bufc, int t) {
    constexpr int BUF = decltype(bufc)::value;
    const FA_LDS char* kb = (const FA_LDS char*)(BUF ? kv1 : kv0);
    const FA_LDS char* vb = kb + TILE;
    const int jt = tile_at(t);
    // buffer BUF ^ 1 was last read in step t - 1: stream the next tile into it
    stage(tile_at(t + 1), std::integral_constant<int, BUF ^ 1>{});
    // offset bases made opaque once per step (no copy): keeps the derived offsets from
    // being hoisted into registers
    asm volatile("" : "+v"(ko0), "+v"(tl0), "+v"(th0));
    const int key0 = jt * kDqKeys;
    // A wave whose queries all lie outside the tile's window has nothing to do here.
    const int qw = q0 + 32 * w;
    if (!((a.wr >= 0 && key0 > qw + 31 + a.wr) || (a.wl >= 0 && key0 + kDqKeys - 1 < qw - a.wl))) {
      // S^T, dP^T: items (ks, kb) with the key block innermost, so that four independent
      // accumulations alternate; each item's K / V rows are requested one item ahead.
      f32x16 s[KB], dp[KB];
#pragma unroll
      for (int kbk = 0; kbk < KB; ++kbk) {
        s[kbk] = f32x16{};
        dp[kbk] = f32x16{};
      }
      constexpr int NI = KSG * KB;
      struct SOps {
        bf16x8 k, v;
      };
      auto load_s = [&](int it, SOps& o) {
        const int ks = it / KB, kbk = it % KB;
        const int off = (ko0 ^ (32 * ks)) + kbk * 32 * 2 * D;
        o.k = lds_ld8(kb + off);
        o.v = lds_ld8(vb + off);
      };
      SOps so[2];
      load_s(0, so[0]);
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        if (it + 1 < NI) load_s(it + 1, so[(it + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        const int ks = it / KB, kbk = it % KB;
        s[kbk] = mfma32(so[it & 1].k, qf[ks], s[kbk]);
        dp[kbk] = mfma32(so[it & 1].v, df[ks], dp[kbk]);
      }
      // with dropout, dS = P (Z dP / (1 - p) - D), the keep bits Z as in the forward
#pragma unroll
      for (int kbk = 0; kbk < KB; ++kbk) {
        uint32_t keep = 0xFFFFu;
        if constexpr (DROP)
          keep = dropout_bits_qlane(key0 + 32 * kbk, qi, ql, h, (uint32_t)(bh % a.H), (uint32_t)b, a.seed_lo,
                                    a.seed_hi, a.drop_thr);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(__builtin_fmaf(s[kbk][i], a.c2s, -lse2));
          if constexpr (DROP) dp[kbk][i] = p * ((((keep >> i) & 1u) ? dp[kbk][i] * a.drop_scale : 0.f) - dval);
          else dp[kbk][i] = p * (dp[kbk][i] - dval);
        }
      }
      // Tiles that cross the causal diagonal or the key padding (a wave-uniform test):
      // masked pairs get dS = 0 by selection.
      if ((key0 + kDqKeys > kv_end) || (a.wr >= 0 && key0 + kDqKeys - 1 > qw + a.wr) ||
          (a.wl >= 0 && key0 < qw + 31 - a.wl)) {
#pragma unroll
        for (int kbk = 0; kbk < KB; ++kbk)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + 32 * kbk + 8 * (i >> 2) + 4 * h + (i & 3);
            const bool masked = key >= kv_end || (a.wr >= 0 && key > qi + a.wr) || (a.wl >= 0 && key < qi - a.wl);
            dp[kbk][i] = masked ? 0.f : dp[kbk][i];
          }
      }
      bf16x8 dsb[PS];
#pragma unroll
      for (int kbk = 0; kbk < KB; ++kbk)
#pragma unroll
        for (int i = 0; i < 16; ++i) dsb[2 * kbk + (i >> 3)][i & 7] = (__bf16)dp[kbk][i];
      // dQ^T += K^T dS^T: items (st, md), transpose reads one item ahead.
      constexpr int NJ = PS * MD;
      bf16x8 kt8[2];
      auto load_t = [&](int j) {
        const int st = j / MD, md = j % MD;
        const int ro = st * 16 * 2 * D;
        return lds_tr8(kb + (tl0 ^ (64 * md)) + ro, kb + (th0 ^ (64 * md)) + ro);
      };
      kt8[0] = load_t(0);
      // At d = 64 (no dropout) the wave raises its issue priority for the dQ^T products:
      // 0.9 % faster backward in a same-box A/B; elsewhere it measured no gain.
      constexpr bool kPrioT = D == 64 && !DROP;
      if constexpr (kPrioT) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (j + 1 < NJ) kt8[(j + 1) & 1] = load_t(j + 1);
        __builtin_amdgcn_sched_barrier(0);
        dq[j % MD] = mfma32(kt8[j & 1], dsb[j / MD], dq[j % MD]);
      }
      if constexpr (kPrioT) __builtin_amdgcn_s_setprio(0);
    }
    // the next tile has landed (this wave's part): publish it
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(std::integral_constant<int, 0>{}, t);
    if (t + 1 < ntiles) step(std::integral_constant<int, 1>{}, t + 1);
  }

  if (qi < N) {
    __bf16* dQ = reinterpret_cast<__bf16*>(a.dq) + hoff + (size_t)qi * rs;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(dq[md][4 * g + e] * a.scale);
        if (32 * md + 8 * g < DG) *reinterpret_cast<bf16x4*>(dQ + 32 * md + 8 * g + 4 * h) = v4;
      }
  }
}

}  // namespace

// Dense dK/dV launches without dropout at d = 64 up to this many rows take the three-per-CU
// layout (one 32-query block per wave and step): at these lengths a causal or padded launch
// holds at most three workgroups per CU, so all of them run from the start.
constexpr int kShortBwdMaxQueries = 4096;

hipError_t launch_bwd(const BwdArgs& a, int d, hipStream_t stream, KernelTimer& tm) {
  const dim3 block(kThreads);
  const dim3 gdkdv((unsigned)(((a.N + kBK - 1) / kBK) * a.B * a.H));
  const dim3 gdq((unsigned)(((a.N + kDqRows - 1) / kDqRows) * a.B * a.H));
  tm.mark(stream);
  hipError_t e;
  if (a.order) {
    hipLaunchKernelGGL(bwd_order_kernel, dim3(1), dim3(kOrderThreads), 0, stream, a.mask, a.nb, a.mb,
                       (a.N + kBK - 1) / kBK, a.order);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    tm.mark(stream);
  }
  // dQ first: its prologue writes D, which the dK/dV kernel reads
  if (a.dropout) {
    if (d == 16) hipLaunchKernelGGL((bwd_dq_kernel<32, true, 16>), gdq, block, 0, stream, a);
    else if (d == 32) hipLaunchKernelGGL((bwd_dq_kernel<32, true>), gdq, block, 0, stream, a);
    else if (d == 64) hipLaunchKernelGGL((bwd_dq_kernel<64, true>), gdq, block, 0, stream, a);
    else hipLaunchKernelGGL((bwd_dq_kernel<128, true>), gdq, block, 0, stream, a);
  } else {
    if (d == 16) hipLaunchKernelGGL((bwd_dq_kernel<32, false, 16>), gdq, block, 0, stream, a);
    else if (d == 32) hipLaunchKernelGGL((bwd_dq_kernel<32, false>), gdq, block, 0, stream, a);
    else if (d == 64) hipLaunchKernelGGL((bwd_dq_kernel<64, false>), gdq, block, 0, stream, a);
    else hipLaunchKernelGGL((bwd_dq_kernel<128, false>), gdq, block, 0, stream, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  tm.mark(stream);
  auto dkdv = [&](auto kernel, int qh) { hipLaunchKernelGGL(kernel, gdkdv, dim3(dkdv_threads(qh)), 0, stream, a); };
  if (a.dropout) {  // (the dropout calls take no block mask)
    if (d == 16) dkdv(bwd_dkdv_kernel<32, true, 16>, dkdv_halves<32, true>());
    else if (d == 32) dkdv(bwd_dkdv_kernel<32, true>, dkdv_halves<32, true>());
    else if (d == 64) dkdv(bwd_dkdv_kernel<64, true>, dkdv_halves<64, true>());
    else dkdv(bwd_dkdv_kernel<128, true>, dkdv_halves<128, true>());
  } else if (a.mask) {  // block-sparse: the 8-wave layout (see dkdv_halves)
    if (d == 16) dkdv(bwd_dkdv_kernel<32, false, 16, 2>, 2);
    else if (d == 32) dkdv(bwd_dkdv_kernel<32, false, 32, 2>, 2);
    else if (d == 64) dkdv(bwd_dkdv_kernel<64, false, 64, 2>, 2);
    else dkdv(bwd_dkdv_kernel<128, false, 128, 2>, 2);
  } else {
    if (d == 16) dkdv(bwd_dkdv_kernel<32, false, 16>, dkdv_halves<32, false>());
    else if (d == 32) dkdv(bwd_dkdv_kernel<32, false>, dkdv_halves<32, false>());
    else if (d == 64 && a.N <= kShortBwdMaxQueries) dkdv(bwd_dkdv_kernel<64, false, 64, 1, 1>, 1);
    else if (d == 64) dkdv(bwd_dkdv_kernel<64, false>, dkdv_halves<64, false>());
    else dkdv(bwd_dkdv_kernel<128, false>, dkdv_halves<128, false>());
  }
  e = hipGetLastError();
  if (e == hipSuccess) tm.mark(stream);
  return e;
}

}  // namespace fa
