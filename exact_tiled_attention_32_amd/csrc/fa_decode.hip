// Attention of a few queries against a key/value cache, split over the keys (gfx950).
//
// Semantics (aiwiki.page "FlashAttention", section "Software integration and
// limitations", lists inference with cached keys and values among the interfaces): the
// Nq queries of (b, h) are the last Nq positions of a sequence whose first L_b keys and
// values are cached; query i attends key j iff j < L_b and, when causal, j <= L_b - Nq + i.
//
// Decoding reads every cached key and value once and does little arithmetic per byte (it
// is bound by HBM bandwidth), so the keys are split evenly over every wave the GPU holds:
//   1. kvc_split_kernel: the valid 32-key tiles of all (b, h) are laid end to end
//      ((b, h) in row-major order, keys in order within one), and wave w of G takes the
//      contiguous tiles [w T / G, (w + 1) T / G) of that sequence (T tiles in all, G <= T,
//      so every wave has work and all waves have the same amount, whatever the cache
//      lengths). A wave streams its tiles through a ring of LDS stages of its own (direct
//      buffer -> LDS loads, no workgroup barrier) without draining it at (b, h) borders,
//      and runs the forward's tiled online softmax for all Nq queries (S^T = K Q^T and
//      O^T += V^T P^T on v_mfma_f32_32x32x16_bf16, one query per lane). Each run of tiles
//      of one (b, h) inside a wave (a "piece") ends with the piece's partial statistics
//      (m, l) and unnormalised output u = sum_j e^(s_j - m) v_j written to slot w + bh:
//      along the sequence w and bh never decrease and one of them grows from a piece to
//      the next, so slots are distinct and fewer than G + B H.
//   2. kvc_merge_kernel: per (b, h, query), finds the waves whose ranges meet the (b, h)
//      (the same arithmetic) and combines their pieces with the online-softmax rule of
//      aiwiki "FlashAttention", section "Tiling and online normalization":
//      m = max_u m_u, l = sum_u e^(m_u - m) l_u, O = sum_u e^(m_u - m) u_u / l, and
//      lse = m + ln l.
#include "fa_device.h"
#include "fa_launch.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace fa {

namespace {

constexpr int kThreads = 256;    // merge kernel
constexpr int kKT = 32;          // keys per tile
constexpr float kRescaleLog2 = 8.0f;
// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8); the unnamed counters are left free.
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int wait_vmcnt(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int kWaitLgkm0 = 0xC07F;
// Cache policy of the streaming key/value loads: non-temporal (each byte is read once,
// in whole 16-byte-per-lane rows, so nothing is lost by not keeping it in the caches).
constexpr int kNonTemporal = 2;

// Pipeline stages S of a key-split wave (one wave per workgroup) and the most waves
// launched per CU, as measured on the decode workloads. A stage holds one K tile and one V
// tile (2 x 32 x D bf16) in LDS; the wave keeps S - 1 tiles in flight while it computes one,
// and reads two sequential streams (its K and V runs). At d = 128 (16 KB stages) 2 waves
// per CU were fastest: filling the CU (5) was 12-16 % slower, 3 or 4 no faster. At d = 64
// 4 were fastest (3: up to 2 % slower; 5, unevenly spread over the four SIMDs: 8-12 %
// slower). At d <= 32 a stage is only 4 KB, and 8 waves keep enough bytes in flight (3 per
// CU: 14-46 % slower).
template <int D> struct SplitShape;
template <> struct SplitShape<32> { static constexpr int S = 3, PER_CU = 8; };
template <> struct SplitShape<64> { static constexpr int S = 3, PER_CU = 4; };
template <> struct SplitShape<128> { static constexpr int S = 2, PER_CU = 2; };

// LDS of one pipeline stage; unused stages shrink to 16 bytes.
template <int D, int STAGE>
struct StageLds {
  static constexpr int BYTES = STAGE < SplitShape<D>::S ? 2 * kKT * D * 2 : 16;
};

// Valid cached keys of batch b, and their 32-key tiles.
__device__ __forceinline__ int cache_len(const DecArgs& a, int b) {
  return a.kv_len ? min(max(a.kv_len[b], 0), a.Nk) : a.Nk;
}
__device__ __forceinline__ int cache_tiles(const DecArgs& a, int b) { return (cache_len(a, b) + kKT - 1) / kKT; }

// Tiles of the batches below `bend` over all heads: H sum_{b < bend} tiles(b) (the lanes of
// the wave share the batches; every lane returns the sum). bend = B gives T.
__device__ int tiles_before(const DecArgs& a, int bend) {
  if (!a.kv_len) return bend * a.H * ((a.Nk + kKT - 1) / kKT);
  int sum = 0;
  for (int c = 0; c < bend; c += 64) {
    const int b = c + lane_id();
    sum += b < bend ? cache_tiles(a, b) : 0;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  return __builtin_amdgcn_readfirstlane(a.H * sum);
}

// Batch b holding tile g of the sequence (0 <= g < T) and the tiles before it, P(b).
__device__ void locate_tile(const DecArgs& a, int g, int& b_out, int& p_out) {
  if (!a.kv_len) {
    const int per = a.H * ((a.Nk + kKT - 1) / kKT);
    b_out = g / per;
    p_out = b_out * per;
    return;
  }
  int base = 0;
  for (int c = 0; c < a.B; c += 64) {
    const int b = c + lane_id();
    const int t = b < a.B ? a.H * cache_tiles(a, b) : 0;
    int incl = t;  // inclusive prefix over the lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane_id() >= off) incl += y;
    }
    const unsigned long long hit = __ballot(b < a.B && base + incl > g);
    if (hit) {
      const int lane = __builtin_ctzll(hit);
      b_out = __builtin_amdgcn_readfirstlane(c + lane);
      p_out = __builtin_amdgcn_readfirstlane(base + __shfl(incl - t, lane));
      return;
    }
    base += __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
  }
  b_out = a.B;  // (g >= T: not reached by the kernels)
  p_out = base;
}

// Wave-uniform position in the tile sequence: batch b, head h, tile j of (b, h), and the
// batch's tile count and valid length. Past the last tile b = B (with tb = 1, L = 0).
struct Cursor {
  int b, h, j, tb, L;
};

__device__ __forceinline__ Cursor cursor_at(const DecArgs& a, int g) {
  Cursor c;
  int p = 0;
  locate_tile(a, g, c.b, p);
  c.L = __builtin_amdgcn_readfirstlane(cache_len(a, c.b));
  c.tb = (c.L + kKT - 1) / kKT;
  const int r = g - p;
  c.h = r / c.tb;
  c.j = r % c.tb;
  return c;
}

__device__ __forceinline__ void cursor_next(const DecArgs& a, Cursor& c) {
  if (++c.j < c.tb) return;
  c.j = 0;
  if (++c.h < a.H) return;
  c.h = 0;
  for (++c.b; c.b < a.B; ++c.b) {  // skip batches with an empty cache
    c.L = __builtin_amdgcn_readfirstlane(cache_len(a, c.b));
    c.tb = (c.L + kKT - 1) / kKT;
    if (c.tb > 0) return;
  }
  c.L = 0;
  c.tb = 1;
}

// Waves that take part: G = min(launched waves, T), so that every range is nonempty.
__device__ __forceinline__ int active_waves(const DecArgs& a, int T) { return min(a.waves, T); }

// DG: head dimension in memory; D: tile width (16 runs on 32-wide tiles, upper half zero).
template <int D, int DG = D>
__global__ __launch_bounds__(64) void kvc_split_kernel(DecArgs a) {
  static_assert(DG == D || (D == 32 && DG == 16), "narrow heads run on 32-wide tiles");
  constexpr int KSG = (DG + 15) / 16;           // k-steps that carry data
  constexpr int S = SplitShape<D>::S;
  static_assert(S >= 2 && S <= 4, "pipeline depth");
  constexpr int KS = D / 16;                    // k-steps of the score product
  constexpr int MD = D / 32;                    // 32-row blocks of O^T
  constexpr int CH = D / 8;                     // 16-byte chunks per row
  constexpr int TILE = kKT * D * 2;             // bytes of a K or V tile
  constexpr int RPB = 1024 / (2 * D);           // tile rows per 1 KB staging block
  constexpr int NB = TILE / 1024;               // staging instructions per tile and tensor
  constexpr int NI = 2 * NB;                    // memory instructions per stage
  // One array per stage, so that the compiler can tell that staging into one stage does
  // not touch the others. Stage layout: [V tile | K tile], both swizzled.
  __shared__ __attribute__((aligned(16))) char st0[StageLds<D, 0>::BYTES];
  __shared__ __attribute__((aligned(16))) char st1[StageLds<D, 1>::BYTES];
  __shared__ __attribute__((aligned(16))) char st2[StageLds<D, 2>::BYTES];
  __shared__ __attribute__((aligned(16))) char st3[StageLds<D, 3>::BYTES];

  const int l = lane_id(), hl = l >> 5, ql = l & 31;
  const int T = tiles_before(a, a.B);
  const int G = active_waves(a, T);
  const int w = blockIdx.x;
  if (w >= G) return;  // (T = 0, or more waves launched than tiles)
  const int s = (int)((long long)w * T / G);
  const int ntiles = (int)((long long)(w + 1) * T / G) - s;

  const __bf16* __restrict__ Q = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* __restrict__ K = reinterpret_cast<const __bf16*>(a.k);
  const __bf16* __restrict__ V = reinterpret_cast<const __bf16*>(a.v);

  // Q fragments (B operand of S^T = K Q^T) of one (b, h): lane holds query ql, columns
  // 16 ks + 8 hl .. + 7; query rows past Nq are zero (their results are never written).
  u32x4 qraw[KS];
  bf16x8 qf[KS];
  auto q_load = [&](int bh) {
    const __bf16* qrow = Q + ((size_t)bh * a.Nq + min(ql, a.Nq - 1)) * DG + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < KSG; ++ks) qraw[ks] = gload16(qrow + 16 * ks);
#pragma unroll
    for (int ks = KSG; ks < KS; ++ks) qraw[ks] = u32x4{};
  };
  auto q_set = [&]() {
    const bool live = ql < a.Nq;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, live ? qraw[ks] : u32x4{});
    if (a.qmul != 1.0f) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)((float)qf[ks][e] * a.qmul);
    }
  };

  // LDS operand offsets: K rows (A operand of S^T), V^T transpose reads (A operand of O^T).
  int k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = TILE + tile_off<D>(ql, 16 * ks + 8 * hl);
  int v_lo[MD], v_hi[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) tr8_offsets<D>(32 * md, v_lo[md], v_hi[md]);
  // Staging: instruction c writes 1 KB block c (rows c RPB .. + RPB - 1), lane l the 16
  // bytes at 16 l: row c RPB + l / CH, physical chunk l % CH, which holds the logical
  // chunk (l % CH) ^ swz(row).
  int st_off[NB];
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int row = c * RPB + l / CH;
    const int chunk = (l % CH) ^ swz<D>(row);
    // a chunk past the head dimension reads zero (offset past any buffer range)
    st_off[c] = 8 * chunk < DG ? (row * DG + chunk * 8) * 2 : (int)0xFFFFFFF0u;
  }
  auto stage = [&](auto si) -> FA_LDS char* {
    if constexpr (decltype(si)::value == 0) return (FA_LDS char*)st0;
    else if constexpr (decltype(si)::value == 1) return (FA_LDS char*)st1;
    else if constexpr (decltype(si)::value == 2) return (FA_LDS char*)st2;
    else return (FA_LDS char*)st3;
  };
  // Tile t of the wave (at cursor c) into a stage. Rows at or past the cache length read
  // as zero (buffer range check), so padding never reaches a sum, and a tile past the
  // wave's range makes no memory access at all; it is issued anyway so that every step
  // issues the same loads and the waits below stay exact. The wave's LDS reads of the
  // stage (the tile computed last) have returned before new values are written into it.
  auto load = [&](int t, const Cursor& c, FA_LDS char* dst) {
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    const int t0 = c.j * kKT;
    const int rows = __builtin_amdgcn_readfirstlane(t < ntiles ? min(c.L - t0, kKT) : 0);  // scalar
    const uint32_t bytes = (uint32_t)rows * (uint32_t)(DG * 2);
    const size_t base = t < ntiles ? ((size_t)(c.b * a.H + c.h) * a.Nk + t0) * DG : 0;
    const auto rv = make_rsrc(V + base, bytes);
    const auto rk = make_rsrc(K + base, bytes);
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const int voff = st_off[blk];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (FA_LDS void*)(dst + blk * 1024), 16, voff, 0, 0, kNonTemporal);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (FA_LDS void*)(dst + TILE + blk * 1024), 16, voff, 0, 0,
                                               kNonTemporal);
    }
  };

  f32x16 o[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) o[md] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;
  const float c2 = a.c2;

  // One tile: keys t0 .. t0 + 31 of a (b, h) whose first L keys are valid.
  auto tile = [&](const FA_LDS char* vt, int t0, int L) {
    f32x16 sc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KSG; ++ks) sc = mfma32(lds_ld8(vt + k_off[ks]), qf[ks], sc);
    const int last = L - a.Nq;  // causal: query i sees keys j <= last + i
    // keys past the valid range, or (causal) past a query's position
    if (t0 + kKT > L || (a.causal && t0 + kKT - 1 > last)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = t0 + 8 * (i >> 2) + 4 * hl + (i & 3);
        if (key >= L || (a.causal && key > last + ql)) sc[i] = kNegInf;
      }
    }
    float tmax = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sc[i]);
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
    const float moff = m_run == kNegInf ? 0.f : m_run * c2;
    bf16x8 pb[2];
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(__builtin_fmaf(sc[i], c2, -moff));
      lsum += p;
      pb[i >> 3][i & 7] = (__bf16)p;
    }
    l_run += lsum;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int md = 0; md < MD; ++md)
        o[md] = mfma32(lds_tr8(vt + v_lo[md] + st * 16 * 2 * D, vt + v_hi[md] + st * 16 * 2 * D), pb[st], o[md]);
  };

  // Partial results of a piece into its slot, then a fresh state for the next piece.
  auto finish_piece = [&](int slot) {
    const float l_tot = l_run + other_half(l_run);
    if (ql < a.Nq) {
      const size_t pu = (size_t)slot * a.Nq + ql;
      float* U = a.part_u + pu * DG;
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = o[md][4 * g + e];
          if (32 * md + 8 * g < DG) *reinterpret_cast<f32x4*>(U + 32 * md + 8 * g + 4 * hl) = v4;
        }
      if (hl == 0) {
        a.part_m[pu] = m_run;
        a.part_l[pu] = l_tot;
      }
    }
#pragma unroll
    for (int md = 0; md < MD; ++md) o[md] = f32x16{};
    m_run = kNegInf;
    l_run = 0.f;
  };

  // Ring of S stages: tile t lives in stage t % S; while it is computed, tiles t + 1 ..
  // t + S - 1 are in flight. `lc` is the position of the next tile to load, `cc` that of
  // the next tile to compute. The loop is unrolled by S so that every stage is a distinct
  // array at every access.
  Cursor lc = cursor_at(a, s);
  Cursor cc = lc;
  q_load(cc.b * a.H + cc.h);
  load(0, lc, stage(std::integral_constant<int, 0>{}));
  cursor_next(a, lc);
  if constexpr (S > 2) {
    load(1, lc, stage(std::integral_constant<int, 1>{}));
    cursor_next(a, lc);
  }
  if constexpr (S > 3) {
    load(2, lc, stage(std::integral_constant<int, 2>{}));
    cursor_next(a, lc);
  }
  // the Q loads, issued before the tiles', have landed once at most the tiles' remain
  __builtin_amdgcn_s_waitcnt(wait_vmcnt((S - 1) * NI));
  q_set();
  for (int t = 0; t < ntiles; t += S) {
    auto step = [&](auto jc) {
      constexpr int J = decltype(jc)::value;
      load(t + J + S - 1, lc, stage(std::integral_constant<int, (J + S - 1) % S>{}));
      cursor_next(a, lc);
      __builtin_amdgcn_s_waitcnt(wait_vmcnt((S - 1) * NI));
      const int tt = t + J;
      if (tt < ntiles) {
        const int bh = cc.b * a.H + cc.h;
        if (tt > 0 && cc.j == 0) {  // a new (b, h): its queries (waits for every load)
          q_load(bh);
          __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
          q_set();
        }
        tile(stage(jc), cc.j * kKT, cc.L);
        if (tt == ntiles - 1 || cc.j == cc.tb - 1) finish_piece(w + bh);
        cursor_next(a, cc);
      }
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    if constexpr (S > 2) step(std::integral_constant<int, 2>{});
    if constexpr (S > 3) step(std::integral_constant<int, 3>{});
  }
  // the last loads (all past the range) must land before the wave ends
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
}

// One workgroup per (b, h, query). The pieces of (b, h) are those of waves w0 .. w1 (the
// waves holding its first and last tile), in slots w + bh. They are spread over the
// threads: first the maximum of their maxima, then groups of D / 4 threads (one 4-column
// slice each) accumulate every G-th piece's weighted output, and the G group sums are
// added in LDS. A (b, h) with an empty cache has no piece: O = 0, lse = -inf.
template <int D>
__global__ __launch_bounds__(kThreads) void kvc_merge_kernel(DecArgs a) {
  constexpr int C4 = D / 4;           // threads per output row
  constexpr int G = kThreads / C4;    // piece groups
  __shared__ float wmax[kThreads / 64];
  __shared__ f32x4 gacc[G][C4];
  __shared__ float gl[G];
  const int bh = blockIdx.x / a.Nq, q = blockIdx.x % a.Nq;
  const int b = bh / a.H, hd = bh % a.H;
  const int tid = threadIdx.x;

  const int T = tiles_before(a, a.B);
  const int tb = __builtin_amdgcn_readfirstlane(cache_tiles(a, b));
  int w0 = 0, np = 0;
  if (tb > 0) {
    const int W = active_waves(a, T);
    const int g0 = tiles_before(a, b) + hd * tb, g1 = g0 + tb - 1;
    w0 = (int)(((long long)(g0 + 1) * W - 1) / T);
    np = (int)(((long long)(g1 + 1) * W - 1) / T) - w0 + 1;
  }
  const size_t base = (size_t)(w0 + bh) * a.Nq + q;  // piece p at base + p Nq

  float m = kNegInf;
  for (int p = tid; p < np; p += kThreads) m = fmaxf(m, a.part_m[base + (size_t)p * a.Nq]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane_id() == 0) wmax[wave_id()] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));

  const int c4 = tid % C4, g = tid / C4;
  f32x4 acc = f32x4{};
  float lsum = 0.f;
  if (m != kNegInf) {
    // a piece whose queries saw no key has m_u = -inf (weight 0), l_u = 0 and u_u = 0
#pragma unroll 4
    for (int p = g; p < np; p += G) {
      const size_t pu = base + (size_t)p * a.Nq;
      const float wgt = fast_exp2((a.part_m[pu] - m) * a.c2);
      lsum += wgt * a.part_l[pu];
      const f32x4 uv = *reinterpret_cast<const f32x4*>(a.part_u + pu * D + 4 * c4);
      acc += wgt * uv;
    }
  }
  gacc[g][c4] = acc;
  if (c4 == 0) gl[g] = lsum;
  __syncthreads();
  if (tid < C4) {
    f32x4 tot = f32x4{};
    float lt = 0.f;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      tot += gacc[i][tid];
      lt += gl[i];
    }
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    bf16x4 ov;
#pragma unroll
    for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(tot[e] * inv);
    __bf16* O = reinterpret_cast<__bf16*>(a.o) + ((size_t)bh * a.Nq + q) * D + 4 * tid;
    *reinterpret_cast<bf16x4*>(O) = ov;
    if (tid == 0) a.lse[(size_t)bh * a.Nq + q] = lt > 0.f ? m * a.sc_abs + logf(lt) : kNegInf;
  }
}

}  // namespace

int kvcache_max_waves(int B, int H, int Nk) {
  const long long tiles = (long long)B * H * ((Nk + kKT - 1) / kKT);
  return (int)std::max(1LL, std::min<long long>(kDecMaxWaves, tiles));
}

namespace {

// Waves of the key-split kernel to launch on the current device: CUs x min(workgroups
// resident per CU, per_cu), looked up once per device and head-dimension variant. 0 if
// unknown.
constexpr int kMaxDevices = 64;
std::atomic<int> g_resident[kMaxDevices][4];

template <typename K>
int resident_waves(K kernel, int variant, int per_cu_max) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = g_resident[dev][variant].load(std::memory_order_relaxed);
  if (n > 0) return n;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel), 64, 0) !=
      hipSuccess)
    return 0;
  n = cus * std::min(per_cu, per_cu_max);
  if (n > 0) g_resident[dev][variant].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace

hipError_t launch_kvcache(const DecArgs& args, int d, hipStream_t stream, KernelTimer& tm) {
  DecArgs a = args;
  const int wmax = kvcache_max_waves(a.B, a.H, a.Nk);
  int res = 0;
  if (d == 16) res = resident_waves(kvc_split_kernel<32, 16>, 0, SplitShape<32>::PER_CU);
  else if (d == 32) res = resident_waves(kvc_split_kernel<32>, 1, SplitShape<32>::PER_CU);
  else if (d == 64) res = resident_waves(kvc_split_kernel<64>, 2, SplitShape<64>::PER_CU);
  else res = resident_waves(kvc_split_kernel<128>, 3, SplitShape<128>::PER_CU);
  a.waves = res > 0 ? std::min(res, wmax) : wmax;
  const dim3 gsplit((unsigned)a.waves), gmerge((unsigned)(a.B * a.H * a.Nq));
  tm.mark(stream);
  if (d == 16) hipLaunchKernelGGL((kvc_split_kernel<32, 16>), gsplit, dim3(64), 0, stream, a);
  else if (d == 32) hipLaunchKernelGGL(kvc_split_kernel<32>, gsplit, dim3(64), 0, stream, a);
  else if (d == 64) hipLaunchKernelGGL(kvc_split_kernel<64>, gsplit, dim3(64), 0, stream, a);
  else hipLaunchKernelGGL(kvc_split_kernel<128>, gsplit, dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  tm.mark(stream);
  if (d == 16) hipLaunchKernelGGL(kvc_merge_kernel<16>, gmerge, dim3(kThreads), 0, stream, a);
  else if (d == 32) hipLaunchKernelGGL(kvc_merge_kernel<32>, gmerge, dim3(kThreads), 0, stream, a);
  else if (d == 64) hipLaunchKernelGGL(kvc_merge_kernel<64>, gmerge, dim3(kThreads), 0, stream, a);
  else hipLaunchKernelGGL(kvc_merge_kernel<128>, gmerge, dim3(kThreads), 0, stream, a);
  e = hipGetLastError();
  if (e == hipSuccess) tm.mark(stream);
  return e;
}

}  // namespace fa
