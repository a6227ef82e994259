// Forward kernels: tiled exact attention with online softmax (gfx950).
//
// Method: aiwiki.page "FlashAttention", section "Tiling and online normalization" — per
// query row keep a running maximum m, a running sum l of exp(s - m) and an accumulator u
// of exp(s - m) v; when a new key tile raises the maximum, rescale l and u by exp(m - m');
// at the end O = u / l. sendsoonai.com "FlashAttention: IO-aware explained", section
// "Tiling and exact softmax": one query block stays on chip while key/value blocks stream
// past, so the N x N score matrix never reaches HBM. Only lse = m + ln l is written.
//
// Work decomposition (one workgroup = 4 waves = 128 query rows, 32 per wave):
//   * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K rows are
//     the A operand (16-byte LDS reads), the wave's Q rows the B operand (registers, loaded
//     once). In the accumulator each lane then owns ONE query (l % 32) and 16 keys per
//     32-key block, so the row max / row sum are in-lane reductions plus one exchange
//     between the two half-waves.
//   * The unnormalised output is accumulated transposed too, O^T += V^T P^T: the
//     probabilities are used straight from the score accumulator as the B operand, and
//     V^T comes from the row-major V tile through ds_read_b64_tr_b16 transpose reads.
//   * K and V tiles (64 keys) are double-buffered in LDS; the next tile's global loads are
//     in flight while the current tile is computed.
//   * The running maximum is refreshed lazily: the accumulator is rescaled only when some
//     row's maximum grew by more than 2^8 in the exp2 domain, which keeps every
//     probability below 256 and leaves the result exact up to rounding (u and l always
//     share the same reference maximum).
//
// The same kernel serves every mask and layout: the (b, h) slice (dense [B, H, N, d] or
// packed [total, H, d] sequences) comes from head_slice(); the causal mask and sliding
// windows set the range of key tiles and the edge masking; block-sparse masks a list of
// key tiles. Template flags add dropout on the probabilities (a Philox4x32-10 mask) and
// run a head dimension of 16 on 32-wide tiles.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kBR = 128;  // query rows per workgroup
constexpr int kBC = 64;   // keys per tile
constexpr int kThreads = 256;
constexpr int kMaxTiles = 4096;  // key-tile list capacity (block-sparse)
constexpr float kRescaleLog2 = 8.0f;

// Builds, in LDS, the list of key tiles [0, ntk) whose mask block is nonzero for mask row
// `rb`. Returns the count (uniform across the workgroup).
__device__ int build_tile_list(uint16_t* list, int* wcount, const uint8_t* mask, int rb, int nb,
                               int mb, int ntk, int bc) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  int count = 0;
  for (int base = 0; base < ntk; base += kThreads) {
    const int j = base + tid;
    const bool keep = j < ntk && mask[(size_t)rb * nb + (j * bc) / mb] != 0;
    const uint64_t bal = __ballot(keep);
    const int pre = __popcll(bal & ((1ull << l) - 1ull));
    if (l == 0) wcount[w] = __popcll(bal);
    __syncthreads();
    int off = count;
    for (int i = 0; i < w; ++i) off += wcount[i];
    if (keep) list[off + pre] = (uint16_t)j;
    count += wcount[0] + wcount[1] + wcount[2] + wcount[3];
    __syncthreads();
  }
  return count;
}

// Ordering hints for the scheduler (masks of __builtin_amdgcn_sched_group_barrier).
constexpr int kSchedMfma = 0x008;
constexpr int kSchedValu = 0x002;
constexpr int kSchedDsRead = 0x100;
// s_waitcnt immediate for vmcnt(0), expcnt and lgkmcnt left free (gfx9 encoding).
constexpr int kWaitVmcnt0 = 0x0F70;
// s_waitcnt immediate for vmcnt(n) (n < 64: low four bits at [3:0], high two at [15:14]).
constexpr int wait_vmcnt(int n) { return kWaitVmcnt0 | (n & 0xF) | ((n >> 4) << 14); }

// DG is the head dimension in memory; D the width of the LDS tiles and MFMA operands. A
// head dimension of 16 runs on 32-wide tiles whose upper half is zero (staged as zeros,
// never stored).
// NS is the number of K and V tile buffers: the loads of a tile are issued NS - 1 steps
// before it is read. Two suffice when most tiles come from L2 (long sequences, where the
// tiles of one head are shared by all its query tiles on an XCD); short sequences read most
// tiles from HBM, whose latency is several steps there. Workgroups staged more than two
// deep serve dense launches only and carry no block-sparse tile list.
template <int D, bool DROP, int DG = D, int NS = 2>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(FwdArgs a) {
  static_assert(DG == D || (D == 32 && DG == 16), "narrow heads run on 32-wide tiles");
  static_assert(NS >= 2 && NS <= 4, "two to four tile buffers");
  constexpr bool LIST = NS == 2;  // block-sparse tile list
  constexpr int KSG = (DG + 15) / 16;          // k-steps that carry data
  constexpr int CH = D / 8;                    // 16-byte chunks per row
  constexpr int TILE = kBC * D * 2;            // bytes of one K or V tile
  constexpr int KS = D / 16;                   // k-steps of the score product
  constexpr int MD = D / 32;                   // 32-row blocks of O^T
  constexpr int KB = kBC / 32;                 // 32-key blocks of a score tile
  constexpr int PS = kBC / 16;                 // k-steps of the O^T product
  constexpr int RPB = 1024 / (2 * D);          // tile rows per 1 KB staging block
  constexpr int NDMA = TILE / (kThreads * 16); // staging instructions per wave per tile
  static_assert((4 * RPB) % 16 == 0, "staging block step must keep the swizzle");
  // LDS: NS K and NS V buffers, each its own array so that the staging loads into one
  // buffer are known not to touch the others (no wait for them before reading those).
  // The score product runs one tile ahead of the value product: step t reads K(t+1), V(t);
  // tile j lives in buffer j mod NS.
  __shared__ __attribute__((aligned(16))) char kb0[TILE];
  __shared__ __attribute__((aligned(16))) char kb1[TILE];
  __shared__ __attribute__((aligned(16))) char kb2[NS > 2 ? TILE : 16];
  __shared__ __attribute__((aligned(16))) char kb3[NS > 3 ? TILE : 16];
  __shared__ __attribute__((aligned(16))) char vb0[TILE];
  __shared__ __attribute__((aligned(16))) char vb1[TILE];
  __shared__ __attribute__((aligned(16))) char vb2[NS > 2 ? TILE : 16];
  __shared__ __attribute__((aligned(16))) char vb3[NS > 3 ? TILE : 16];
  __shared__ uint16_t tlist[LIST ? kMaxTiles : 1];
  __shared__ int wcount[4];

  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int qt = a.ntq - 1 - blockIdx.x / BH;  // longest (causal) tiles first
  const int b = bh / a.H;
  const int q0 = qt * kBR;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, h = l >> 5, ql = l & 31;
  const int qi = q0 + 32 * w + ql;
  const HeadSlice sl = head_slice<DG>(a, bh);
  const int N = sl.N;
  const size_t hoff = sl.hoff, loff = sl.loff;
  if (q0 >= N) return;  // a query tile past the end of a shorter sequence (uniform)
  const size_t rs = (size_t)a.rs;
  const __bf16* __restrict__ Q = reinterpret_cast<const __bf16*>(a.q) + hoff;
  const __bf16* __restrict__ K = reinterpret_cast<const __bf16*>(a.k) + hoff;
  const __bf16* __restrict__ V = reinterpret_cast<const __bf16*>(a.v) + hoff;

  int kv_end = N;
  if (a.kv_len) kv_end = min(max(a.kv_len[b], 0), N);
  // Key range of the workgroup's rows under the window: [lo, hi).
  int hi = kv_end;
  if (a.wr >= 0) hi = min(hi, q0 + kBR + a.wr);
  const int t0 = a.wl >= 0 ? max(q0 - a.wl, 0) / kBC : 0;
  const int ntk = (hi + kBC - 1) / kBC;
  int ntiles = max(ntk - t0, 0);
  if constexpr (LIST) {
    if (a.mask)
      ntiles = __builtin_amdgcn_readfirstlane(build_tile_list(tlist, wcount, a.mask, q0 / a.mb, a.nb, a.mb, ntk, kBC));
  }
  // Key tile of step t, clamped so that the look-ahead of the last steps stays valid.
  auto tile_at = [&](int t) {
    const int tc = min(t, max(ntiles - 1, 0));
    if constexpr (LIST) return a.mask ? __builtin_amdgcn_readfirstlane((int)tlist[tc]) : t0 + tc;
    else return t0 + tc;
  };

  // Q fragments: B operand of S^T = K Q^T, lane holds Q[qi][16 ks + 8h .. +7]. The loads
  // are waited for together with the first tiles' staging (one memory latency, not two).
  bf16x8 qf[KS];
  {
    const __bf16* qrow = Q + (size_t)min(qi, N - 1) * rs + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KSG; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, gload16(qrow + 16 * ks));
#pragma unroll
    for (int ks = KSG; ks < KS; ++ks) qf[ks] = bf16x8{};
  }
  // Scaling by the sign of the softmax scale (or by 0): applied once the fragments landed.
  auto scale_q = [&]() {
    const float qm = qi < N ? a.qmul : 0.f;
    if (qm != 1.0f) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)((float)qf[ks][e] * qm);
    }
  };

  // Per-lane LDS byte offsets, tile-relative, fixed for the whole kernel.
  int k_off[KS];             // S^T A operand: K row ql, columns 16 ks + 8h (+32 kb rows)
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = tile_off<D>(ql, 16 * ks + 8 * h);
  int v_lo[MD], v_hi[MD];    // V^T transpose reads for d-block md (+16 st rows)
#pragma unroll
  for (int md = 0; md < MD; ++md) tr8_offsets<D>(32 * md, v_lo[md], v_hi[md]);
  // Tile staging by direct buffer -> LDS loads bounded at row N (rows past the end arrive
  // as zeros): instruction c of wave w fills 1 KB block 4c + w of a tile, lane l the 16
  // bytes at 16 l: tile row (4c + w) RPB + l / CH, physical chunk l % CH, which holds the
  // logical chunk (l % CH) ^ swz(row); the row step 4 RPB keeps swz unchanged. Global rows
  // are rs elements apart (d for [B, H, N, d], H d for packed tokens).
  const int dma_row0 = w * RPB + l / CH;
  const int dma_col = ((l % CH) ^ swz<D>(dma_row0)) * 8;
  int dma_off[NDMA];
#pragma unroll
  for (int c = 0; c < NDMA; ++c) dma_off[c] = ((dma_row0 + 4 * RPB * c) * a.rs + dma_col) * 2;
  if (DG < D && dma_col >= DG) {
#pragma unroll
    for (int c = 0; c < NDMA; ++c) dma_off[c] = (int)0xFFFFFFF0u;  // past any range: reads zero
  }

  f32x16 o[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) o[md] = f32x16{};
  float m_run = kNegInf, l_run = 0.f, moff = 0.f;
  const float c2 = a.c2;

  auto stage = [&](const __bf16* base, int jt, FA_LDS char* buf) {
    const int key0 = jt * kBC;
    // rows of the tile inside the slice (uniform: kept scalar so that the buffer
    // descriptor stays in scalar registers)
    const int rows = __builtin_amdgcn_readfirstlane(min(max(N - key0, 0), kBC));
    const auto r = make_rsrc(base + (size_t)key0 * rs, (uint32_t)rows * (uint32_t)(a.rs * 2));
#pragma unroll
    for (int c = 0; c < NDMA; ++c) {
      // (an array element passed straight to the builtin makes the host pass silently drop
      // the kernel's launch stub; a local copy does not)
      const int voff = dma_off[c];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FA_LDS void*)(buf + (4 * c + w) * 1024), 16, voff, 0, 0, 0);
    }
  };
  // Buffer of tile j (j mod NS, a compile-time index).
  auto kbuf = [&](auto jc) {
    constexpr int J = decltype(jc)::value % NS;
    if constexpr (J == 0) return (FA_LDS char*)kb0;
    else if constexpr (J == 1) return (FA_LDS char*)kb1;
    else if constexpr (J == 2) return (FA_LDS char*)kb2;
    else return (FA_LDS char*)kb3;
  };
  auto vbuf = [&](auto jc) {
    constexpr int J = decltype(jc)::value % NS;
    if constexpr (J == 0) return (FA_LDS char*)vb0;
    else if constexpr (J == 1) return (FA_LDS char*)vb1;
    else if constexpr (J == 2) return (FA_LDS char*)vb2;
    else return (FA_LDS char*)vb3;
  };
  // vmcnt that leaves the loads of the last NS - 2 steps in flight (each step stages one K
  // and one V tile, NDMA loads each per wave)
  constexpr int kWaitAhead = wait_vmcnt(2 * NDMA * (NS - 2));
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // Score tile S^T = K Q^T of the K tile at `kb` (MFMA phase only).
  auto scores = [&](const FA_LDS char* kb, f32x16 (&s)[KB]) {
#pragma unroll
    for (int kbk = 0; kbk < KB; ++kbk) {
      s[kbk] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KSG; ++ks) s[kbk] = mfma32(lds_ld8(kb + k_off[ks] + kbk * 32 * 2 * D), qf[ks], s[kbk]);
    }
  };
  // Masking of an edge tile, its row maximum and the lazy rescale (a wave-uniform branch).
  auto rowmax_update = [&](int jt, f32x16 (&s)[KB]) {
    const int key0 = jt * kBC;
    const int qw = q0 + 32 * w;  // the wave's first row
    if ((key0 + kBC > kv_end) || (a.wr >= 0 && key0 + kBC - 1 > qw + a.wr) ||
        (a.wl >= 0 && key0 < qw + 31 - a.wl)) {
#pragma unroll
      for (int kbk = 0; kbk < KB; ++kbk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 32 * kbk + 8 * (i >> 2) + 4 * h + (i & 3);
          if (key >= kv_end || (a.wr >= 0 && key > qi + a.wr) || (a.wl >= 0 && key < qi - a.wl))
            s[kbk][i] = kNegInf;
        }
    }
    float tmax = kNegInf;
#pragma unroll
    for (int kbk = 0; kbk < KB; ++kbk)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[kbk][i]);
    tmax = fmaxf(tmax, other_half(tmax));
    const float mcand = fmaxf(m_run, tmax);
    const bool need = (mcand - m_run) * c2 > kRescaleLog2;
    if (__ballot(need)) {
      const float alpha = need ? fast_exp2((m_run - mcand) * c2) : 1.0f;
      if (need) m_run = mcand;
      l_run *= alpha;
#pragma unroll
      for (int md = 0; md < MD; ++md) o[md] *= alpha;
    }
    moff = (m_run == kNegInf) ? 0.f : m_run * c2;
  };

  f32x16 sa[KB], sb[KB];
  if (ntiles > 0) {
    // K(0), V(0), K(1), then V(j), K(j + 1) up to K(NS - 1); wait for the first three and
    // the Q fragments, which were requested before them
    stage(K, tile_at(0), kbuf(I0{}));
    stage(V, tile_at(0), vbuf(I0{}));
    stage(K, tile_at(1), kbuf(I1{}));
    if constexpr (NS > 2) {
      stage(V, tile_at(1), vbuf(I1{}));
      stage(K, tile_at(2), kbuf(std::integral_constant<int, 2>{}));
    }
    if constexpr (NS > 3) {
      stage(V, tile_at(2), vbuf(std::integral_constant<int, 2>{}));
      stage(K, tile_at(3), kbuf(std::integral_constant<int, 3>{}));
    }
    __builtin_amdgcn_s_waitcnt(kWaitAhead);
    scale_q();
    __syncthreads();
    scores(kbuf(I0{}), sa);
    rowmax_update(tile_at(0), sa);
    __syncthreads();  // step 0 overwrites K buffer 0
  } else {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // (the unused Q loads)
  }

  // Step t: S(t+1) from K(t+1) interleaved with the probabilities of tile t; then
  // O^T += V^T P^T from V(t); then find the maximum of tile t+1. At its start the step
  // streams K(t+NS) into the buffer of K(t) and V(t+NS-1) into that of V(t-1), both read
  // in step t - 1; at its end K(t+2) and V(t+1) have landed.
  auto step = [&](auto phc, f32x16 (&cur)[KB], f32x16 (&nxt)[KB], int t) {
    constexpr int P = decltype(phc)::value;  // t mod NS
    const FA_LDS char* kb = kbuf(std::integral_constant<int, P + 1>{});
    const FA_LDS char* vb = vbuf(phc);
    // Deeper staging issues no loads once the last tile is staged (uniform): the step then
    // waits for all. With two buffers the look-ahead tiles are clamped re-loads of the last
    // one and every step waits for all anyway.
    const bool more = NS == 2 || t + NS - 1 < ntiles;
    if (more) {
      stage(K, tile_at(t + NS), kbuf(phc));
      stage(V, tile_at(t + NS - 1), vbuf(std::integral_constant<int, P + NS - 1>{}));
    }
    // -- region A: score MFMAs of the next tile, exp/sum/pack of this tile. At d = 128 the
    // wave raises its issue priority over the other wave of its SIMD for this region and
    // drops it before the value products: the matrix work interleaved with its softmax then
    // wins the arbitration (measured 2.3 % faster at d = 128; at d = 64, where the vector
    // ALU is the first limit, 1 % slower, so it is not done there).
    constexpr bool kPrioA = D == 128 && !DROP;
    if constexpr (kPrioA) __builtin_amdgcn_s_setprio(1);
    scores(kb, nxt);
    // Dropout: bit 16 kbk + i of `keep` says whether this lane's element (kbk, i) of tile t
    // is kept (register i of a block holds key 8 (i / 4) + 4 h + i % 4).
    uint32_t keep = 0xFFFFFFFFu;
    if constexpr (DROP) {
      const int key0 = tile_at(t) * kBC;
      keep = 0;
#pragma unroll
      for (int kbk = 0; kbk < KB; ++kbk)
        keep |= dropout_bits_qlane(key0 + 32 * kbk, qi, ql, h, (uint32_t)(bh % a.H), (uint32_t)b, a.seed_lo,
                                   a.seed_hi, a.drop_thr)
                << (16 * kbk);
    }
    bf16x8 pb[PS];
    float lsum = 0.f;
#pragma unroll
    for (int kbk = 0; kbk < KB; ++kbk)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(__builtin_fmaf(cur[kbk][i], c2, -moff));
        lsum += p;  // the softmax normaliser counts every probability, dropped or not
        if constexpr (DROP) pb[2 * kbk + (i >> 3)][i & 7] = (__bf16)(((keep >> (16 * kbk + i)) & 1u) ? p : 0.f);
        else pb[2 * kbk + (i >> 3)][i & 7] = (__bf16)p;
      }
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
    for (int k = 0; k < KB * KS; ++k) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (k + 4 < KB * KS) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, 7, 0);
    }
    l_run += lsum;
    // -- region B: O^T += V^T P^T, items (st, md), transpose reads one item ahead
    constexpr int NJ = PS * MD;
    bf16x8 vt8[2];
    auto load_v = [&](int j) {
      const int st = j / MD, md = j % MD;
      return lds_tr8(vb + v_lo[md] + st * 16 * 2 * D, vb + v_hi[md] + st * 16 * 2 * D);
    };
    vt8[0] = load_v(0);
    if constexpr (kPrioA) __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j + 1 < NJ) vt8[(j + 1) & 1] = load_v(j + 1);
      __builtin_amdgcn_sched_barrier(0);
      o[j % MD] = mfma32(vt8[j & 1], pb[j / MD], o[j % MD]);
    }
    // -- prepare tile t+1; the staged tiles must have landed before the barrier
    if (t + 1 < ntiles) rowmax_update(tile_at(t + 1), nxt);
    if (more) __builtin_amdgcn_s_waitcnt(kWaitAhead);
    else __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  };
  // Unrolled over a multiple of NS (buffer phase) and of 2 (score register pair).
  constexpr int U = NS % 2 == 0 ? NS : 2 * NS;
  for (int t = 0; t < ntiles; t += U) {
    step(std::integral_constant<int, 0>{}, sa, sb, t);
    if (t + 1 < ntiles) step(std::integral_constant<int, 1 % NS>{}, sb, sa, t + 1);
    if constexpr (U > 2) {
      if (t + 2 < ntiles) step(std::integral_constant<int, 2 % NS>{}, sa, sb, t + 2);
      if (t + 3 < ntiles) step(std::integral_constant<int, 3 % NS>{}, sb, sa, t + 3);
    }
    if constexpr (U > 4) {
      if (t + 4 < ntiles) step(std::integral_constant<int, 4 % NS>{}, sa, sb, t + 4);
      if (t + 5 < ntiles) step(std::integral_constant<int, 5 % NS>{}, sb, sa, t + 5);
    }
  }

  const float l_tot = l_run + other_half(l_run);
  if (qi < N) {
    float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if constexpr (DROP) inv *= a.drop_scale;  // kept probabilities count 1 / (1 - p)
    __bf16* O = reinterpret_cast<__bf16*>(a.o) + hoff + (size_t)qi * rs;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(o[md][4 * g + e] * inv);
        if (32 * md + 8 * g < DG) *reinterpret_cast<bf16x4*>(O + 32 * md + 8 * g + 4 * h) = ov;
      }
    if (h == 0) a.lse[loff + qi] = l_tot > 0.f ? m_run * a.sc_abs + logf(l_tot) : kNegInf;
  }
}

// fp32 forward: same structure on v_mfma_f32_32x32x2_f32, 32-key tiles, one LDS buffer.
template <int D>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(FwdArgs a) {
  constexpr int BC = 32;
  constexpr int LD = D + 1;  // padded row stride (floats)
  constexpr int MD = D / 32;
  __shared__ float kt[BC * LD];
  __shared__ float vt[BC * LD];
  __shared__ uint16_t tlist[kMaxTiles];
  __shared__ int wcount[4];

  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int qt = a.ntq - 1 - blockIdx.x / BH;
  const int b = bh / a.H;
  const int q0 = qt * kBR;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, h = l >> 5, ql = l & 31;
  const int qi = q0 + 32 * w + ql;
  const size_t hoff = (size_t)bh * a.N * D;
  const float* __restrict__ Q = reinterpret_cast<const float*>(a.q) + hoff;
  const float* __restrict__ K = reinterpret_cast<const float*>(a.k) + hoff;
  const float* __restrict__ V = reinterpret_cast<const float*>(a.v) + hoff;

  int kv_end = a.N;
  if (a.kv_len) kv_end = min(max(a.kv_len[b], 0), a.N);
  int hi = kv_end;
  if (a.causal) hi = min(hi, q0 + kBR);
  const int ntk = (hi + BC - 1) / BC;
  int ntiles = ntk;
  if (a.mask)
    ntiles = __builtin_amdgcn_readfirstlane(build_tile_list(tlist, wcount, a.mask, q0 / a.mb, a.nb, a.mb, ntk, BC));

  float qf[D / 2];
#pragma unroll
  for (int s = 0; s < D / 2; ++s) qf[s] = qi < a.N ? Q[(size_t)qi * D + 2 * s + h] * a.qmul : 0.f;

  f32x16 o[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) o[md] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;
  const float c2 = a.c2;

  // Tile t + 1 is read into registers while tile t is computed, then written to LDS after
  // the step's last barrier: one memory latency per launch instead of one per tile.
  constexpr int PER = BC * D / kThreads;  // elements of a tile per thread and tensor
  float kr[PER], vr[PER];
  auto fetch = [&](int t) {
    const int key0 = (a.mask ? __builtin_amdgcn_readfirstlane((int)tlist[t]) : t) * BC;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + i * kThreads, key = key0 + e / D, col = e % D;
      kr[i] = key < a.N ? K[(size_t)key * D + col] : 0.f;
      vr[i] = key < a.N ? V[(size_t)key * D + col] : 0.f;
    }
  };
  auto publish = [&]() {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + i * kThreads, row = e / D, col = e % D;
      kt[row * LD + col] = kr[i];
      vt[row * LD + col] = vr[i];
    }
  };
  if (ntiles > 0) {
    fetch(0);
    publish();
  }
  for (int t = 0; t < ntiles; ++t) {
    const int jt = a.mask ? __builtin_amdgcn_readfirstlane((int)tlist[t]) : t;
    const int key0 = jt * BC;
    __syncthreads();
    if (t + 1 < ntiles) fetch(t + 1);
    if (!(a.causal && key0 > q0 + 32 * w + 31)) {
      f32x16 s = f32x16{};
#pragma unroll
      for (int st = 0; st < D / 2; ++st) s = mfma32_f32(kt[ql * LD + 2 * st + h], qf[st], s);
      float tmax = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key0 + 8 * (i >> 2) + 4 * h + (i & 3);
        if (key >= kv_end || (a.causal && key > qi)) s[i] = kNegInf;
        tmax = fmaxf(tmax, s[i]);
      }
      tmax = fmaxf(tmax, wave_xor32(tmax));
      const float mcand = fmaxf(m_run, tmax);
      const bool need = (mcand - m_run) * c2 > kRescaleLog2;
      if (__ballot(need)) {
        const float alpha = need ? exp2f((m_run - mcand) * c2) : 1.0f;
        if (need) m_run = mcand;
        l_run *= alpha;
#pragma unroll
        for (int md = 0; md < MD; ++md) o[md] *= alpha;
      }
      const float moff = (m_run == kNegInf) ? 0.f : m_run * c2;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = exp2f(__builtin_fmaf(s[i], c2, -moff));
        l_run += s[i];
      }
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          o[md] = mfma32_f32(vt[(8 * (i >> 2) + 4 * h + (i & 3)) * LD + 32 * md + ql], s[i], o[md]);
    }
    __syncthreads();
    if (t + 1 < ntiles) publish();
  }

  const float l_tot = l_run + wave_xor32(l_run);
  if (qi < a.N) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    float* O = reinterpret_cast<float*>(a.o) + hoff + (size_t)qi * D;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = o[md][4 * g + e] * inv;
        *reinterpret_cast<f32x4*>(O + 32 * md + 8 * g + 4 * h) = ov;
      }
    if (h == 0) a.lse[(size_t)bh * a.N + qi] = l_tot > 0.f ? m_run * a.sc_abs + logf(l_tot) : kNegInf;
  }
}

}  // namespace

// Tile buffers of a dense bf16 forward without dropout: deeper staging where the
// workgroups' key ranges are short (their tiles mostly come from HBM).
constexpr int kShortStages = 3;
constexpr int kShortMaxKeys = 4096;  // longest key range (N) that takes it
constexpr int kShortMaxD = 64;       // d = 128 would lose a workgroup per CU to the LDS
int fwd_stages(const FwdArgs& a, int d, bool dropout) {
  return (!a.mask && !dropout && a.N <= kShortMaxKeys && d <= kShortMaxD) ? kShortStages : 2;
}

template <int D, bool DROP, int DG = D>
void launch_bf16(const FwdArgs& a, dim3 grid, dim3 block, hipStream_t stream, int ns) {
  if constexpr (!DROP && D <= kShortMaxD) {
    if (ns == 3) {
      hipLaunchKernelGGL((fwd_bf16_kernel<D, false, DG, 3>), grid, block, 0, stream, a);
      return;
    }
    if (ns == 4) {
      hipLaunchKernelGGL((fwd_bf16_kernel<D, false, DG, 4>), grid, block, 0, stream, a);
      return;
    }
  }
  hipLaunchKernelGGL((fwd_bf16_kernel<D, DROP, DG, 2>), grid, block, 0, stream, a);
}

hipError_t launch_fwd(const FwdArgs& a, fa_dtype dt, int d, hipStream_t stream, KernelTimer& tm,
                      bool dropout) {
  const dim3 grid((unsigned)(a.ntq * a.B * a.H)), block(kThreads);
  tm.mark(stream);
  if (dt == FA_BF16) {
    const int ns = fwd_stages(a, d, dropout);
    if (dropout) {
      if (d == 16) launch_bf16<32, true, 16>(a, grid, block, stream, ns);
      else if (d == 32) launch_bf16<32, true>(a, grid, block, stream, ns);
      else if (d == 64) launch_bf16<64, true>(a, grid, block, stream, ns);
      else launch_bf16<128, true>(a, grid, block, stream, ns);
    } else {
      if (d == 16) launch_bf16<32, false, 16>(a, grid, block, stream, ns);
      else if (d == 32) launch_bf16<32, false>(a, grid, block, stream, ns);
      else if (d == 64) launch_bf16<64, false>(a, grid, block, stream, ns);
      else launch_bf16<128, false>(a, grid, block, stream, ns);
    }
  } else {
    if (d == 32) hipLaunchKernelGGL(fwd_f32_kernel<32>, grid, block, 0, stream, a);
    else if (d == 64) hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, block, 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) tm.mark(stream);
  return e;
}

}  // namespace fa
